"""CPU oracle for the ZeRO-1 shard optimizer step (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or runs anything here, and this
package imports nothing from the product.

The arithmetic lives in ``z1_oracle.c`` (plain C, binary64 unless the method
fixes a precision); this module only loads it with ctypes and marshals numpy
arrays.  All arrays are in *packed shard order*: the rank's slices of every
tensor, concatenated in tensor order.

Parity status of each function (what pins it, see ``tests/pins.py``):
  shard_plan   brute force + numpy.array_split boundaries + invariants
  shard_plan_flat  brute force vs numpy.array_split of the concatenation
  shard_plan_dim0  brute force vs torch.chunk along dim 0
  bf16_rne     torch CPU cast on non-NaN patterns + nearest/ties-to-even check
  accumulate   exact binary64 sums rounded once to binary32, per add
  norm_sq      closed form for constant input + math.fsum error bound
  clip_coef    torch.nn.utils.clip_grad_norm_ (binary64)
  adamw        step-1 and constant-gradient closed forms, zero-gradient decay,
               torch.optim.AdamW (binary64), per-group lr / wd
  lr_at        boundary closed forms, torch CosineAnnealingLR
  pack_send    numpy.array_split gather per rank; numpy binary32 division
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "z1_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
             "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(src: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (SSE binary32/64 arithmetic, no contraction)."""
    subprocess.run(["gcc", *GCC_FLAGS, "-o", out, src, "-lm"], check=True)
    return out


class _HP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("clip", ctypes.c_double),
                ("step", ctypes.c_int64)]


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _segments(segments, L):
    """(n_seg, seg_len, lr_scale, wd_scale) arrays for the C side."""
    if segments is None:
        return 0, None, None, None
    sl, ls, ws = (np.ascontiguousarray(np.asarray(x, dt)) for x, dt in
                  zip(segments, (np.int64, np.float64, np.float64)))
    assert sl.size == ls.size == ws.size and int(sl.sum()) == L
    return sl.size, sl, ls, ws


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str = LIB_PATH):
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        L.z1o_shard_plan.argtypes = [ctypes.c_int32, P, ctypes.c_int32, ctypes.c_int32, P, P]
        L.z1o_shard_plan.restype = ctypes.c_int
        L.z1o_shard_plan_flat.argtypes = [ctypes.c_int32, P, ctypes.c_int32, ctypes.c_int32, P, P]
        L.z1o_shard_plan_flat.restype = ctypes.c_int
        L.z1o_shard_plan_dim0.argtypes = [ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int32,
                                          P, P]
        L.z1o_shard_plan_dim0.restype = ctypes.c_int
        L.z1o_bf16_rne.argtypes = [ctypes.c_float]
        L.z1o_bf16_rne.restype = ctypes.c_uint16
        L.z1o_bf16_rne_array.argtypes = [ctypes.c_int64, P, P]
        L.z1o_bf16_rne_array.restype = None
        L.z1o_accumulate.argtypes = [ctypes.c_int64, ctypes.c_int32, P, P]
        L.z1o_accumulate.restype = None
        L.z1o_norm_sq.argtypes = [ctypes.c_int64, P]
        L.z1o_norm_sq.restype = ctypes.c_double
        L.z1o_clip_coef.argtypes = [ctypes.c_double, ctypes.c_double]
        L.z1o_clip_coef.restype = ctypes.c_double
        L.z1o_adamw.argtypes = [ctypes.c_int64, P, P, P, P, P, ctypes.c_double,
                                ctypes.POINTER(_HP)]
        L.z1o_adamw.restype = None
        L.z1o_step.argtypes = [ctypes.c_int64, ctypes.c_int32, P, P, P, P, P, P,
                               ctypes.POINTER(_HP), ctypes.POINTER(ctypes.c_double)]
        L.z1o_step.restype = ctypes.c_double
        L.z1o_adamw_seg.argtypes = [ctypes.c_int64, P, P, P, P, P, ctypes.c_double,
                                    ctypes.POINTER(_HP), ctypes.c_int32, P, P, P]
        L.z1o_adamw_seg.restype = None
        L.z1o_step_seg.argtypes = [ctypes.c_int64, ctypes.c_int32, P, P, P, P, P, P,
                                   ctypes.POINTER(_HP), ctypes.POINTER(ctypes.c_double),
                                   ctypes.c_int32, P, P, P]
        L.z1o_step_seg.restype = ctypes.c_double
        L.z1o_lr_at.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int64,
                                ctypes.c_int64, ctypes.c_int32, ctypes.c_int64]
        L.z1o_lr_at.restype = ctypes.c_double
        L.z1o_pack_send.argtypes = [ctypes.c_int32, P, ctypes.c_int32, P, P, P, ctypes.c_int32, P]
        L.z1o_pack_send.restype = None
        L.z1o_num_threads.argtypes = []
        L.z1o_num_threads.restype = ctypes.c_int
        self.lib = L
        self.path = path

    # O1 ------------------------------------------------------------------
    def shard_plan(self, numel: Sequence[int], dp_size: int, rank: int
                   ) -> Tuple[np.ndarray, np.ndarray]:
        """(start, len) of this rank's contiguous slice of every tensor."""
        n = np.ascontiguousarray(np.asarray(numel, dtype=np.int64))
        start = np.zeros(len(n), np.int64)
        ln = np.zeros(len(n), np.int64)
        rc = self.lib.z1o_shard_plan(len(n), _ptr(n), dp_size, rank, _ptr(start), _ptr(ln))
        if rc != 0:
            raise ValueError("invalid shard plan arguments")
        return start, ln

    def shard_plan_flat(self, numel: Sequence[int], dp_size: int, rank: int
                        ) -> Tuple[np.ndarray, np.ndarray]:
        """Flatten-then-split: the rank's range of the concatenation, per tensor."""
        n = np.ascontiguousarray(np.asarray(numel, dtype=np.int64))
        start = np.zeros(len(n), np.int64)
        ln = np.zeros(len(n), np.int64)
        if self.lib.z1o_shard_plan_flat(len(n), _ptr(n), dp_size, rank, _ptr(start), _ptr(ln)):
            raise ValueError("invalid shard plan arguments")
        return start, ln

    def shard_plan_dim0(self, numel: Sequence[int], rows: Sequence[int], dp_size: int,
                        rank: int) -> Tuple[np.ndarray, np.ndarray]:
        """Dim-0 sharding: ceil(rows/D) rows per rank, in rank order."""
        n = np.ascontiguousarray(np.asarray(numel, dtype=np.int64))
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        start = np.zeros(len(n), np.int64)
        ln = np.zeros(len(n), np.int64)
        if self.lib.z1o_shard_plan_dim0(len(n), _ptr(n), _ptr(r), dp_size, rank, _ptr(start),
                                        _ptr(ln)):
            raise ValueError("invalid shard plan arguments")
        return start, ln

    def plan(self, kind: str, numel, rows, dp_size, rank):
        if kind == "per_tensor":
            return self.shard_plan(numel, dp_size, rank)
        if kind == "flat":
            return self.shard_plan_flat(numel, dp_size, rank)
        if kind == "dim0":
            return self.shard_plan_dim0(numel, rows, dp_size, rank)
        raise ValueError(kind)

    # O2e -----------------------------------------------------------------
    def bf16_rne(self, x: np.ndarray) -> np.ndarray:
        """bf16 bit patterns (uint16) of fp32 values, round-to-nearest-even."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, np.uint16)
        self.lib.z1o_bf16_rne_array(x.size, _ptr(x), _ptr(out))
        return out

    # O2a -----------------------------------------------------------------
    def accumulate(self, g: np.ndarray) -> np.ndarray:
        """In-order binary32 sum of K bf16 micro-gradients; g is uint16 [K, L]."""
        g = np.ascontiguousarray(g, dtype=np.uint16)
        K, L = g.shape
        acc = np.empty(L, np.float32)
        self.lib.z1o_accumulate(L, K, _ptr(g), _ptr(acc))
        return acc

    # O2b -----------------------------------------------------------------
    def norm_sq(self, acc: np.ndarray) -> float:
        """S = sum(acc^2) in binary64."""
        acc = np.ascontiguousarray(acc, dtype=np.float32)
        return float(self.lib.z1o_norm_sq(acc.size, _ptr(acc)))

    # O2c -----------------------------------------------------------------
    def clip_coef(self, S: float, clip: float) -> float:
        """c = min(1, clip / (sqrt(S) + 1e-6)); 1 when clip <= 0."""
        return float(self.lib.z1o_clip_coef(S, clip))

    # O2d / O2e -----------------------------------------------------------
    def adamw(self, acc, p, m, v, c, *, lr, beta1, beta2, eps, weight_decay, step,
              clip=0.0, w: Optional[np.ndarray] = None, segments=None) -> None:
        """In place on fp32 p, m, v (and the bf16 bits w when given).
        segments = (seg_len, lr_scale, wd_scale) per tensor, or None."""
        hp = _HP(lr, beta1, beta2, eps, weight_decay, clip, int(step))
        for a in (acc, p, m, v):
            assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"] and a.size == p.size
        if w is not None:
            assert w.dtype == np.uint16 and w.size == p.size and w.flags["C_CONTIGUOUS"]
        n_seg, sl, ls, ws = _segments(segments, p.size)
        self.lib.z1o_adamw_seg(p.size, _ptr(acc), _ptr(p), _ptr(m), _ptr(v), _ptr(w), c,
                               ctypes.byref(hp), n_seg, _ptr(sl), _ptr(ls), _ptr(ws))

    # whole step ------------------------------------------------------------
    def step(self, g: np.ndarray, p: np.ndarray, m: np.ndarray, v: np.ndarray, *, lr,
             beta1, beta2, eps, weight_decay, clip, step,
             acc: Optional[np.ndarray] = None, w: Optional[np.ndarray] = None,
             segments=None) -> Tuple[float, float, np.ndarray]:
        """O2a..O2e on the packed shard; returns (S, c, acc); p, m, v, w in place."""
        g = np.ascontiguousarray(g, dtype=np.uint16)
        K, L = g.shape
        for a in (p, m, v):
            assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"] and a.size == L
        if acc is None:
            acc = np.empty(L, np.float32)
        if w is not None:
            assert w.dtype == np.uint16 and w.size == L and w.flags["C_CONTIGUOUS"]
        hp = _HP(lr, beta1, beta2, eps, weight_decay, clip, int(step))
        c = ctypes.c_double(0.0)
        n_seg, sl, ls, ws = _segments(segments, L)
        S = self.lib.z1o_step_seg(L, K, _ptr(g), _ptr(acc), _ptr(p), _ptr(m), _ptr(v), _ptr(w),
                                  ctypes.byref(hp), ctypes.byref(c), n_seg, _ptr(sl), _ptr(ls),
                                  _ptr(ws))
        return float(S), float(c.value), acc

    def pack_send(self, numel, rows, kind: str, dp_size: int, acc_full: np.ndarray,
                  divide: bool) -> np.ndarray:
        """Reduce-scatter send buffer: every rank's slices of the full fp32
        accumulated gradient (concatenation order), rank-major, packed."""
        n = np.ascontiguousarray(np.asarray(numel, np.int64))
        starts, lens = [], []
        for r in range(dp_size):
            s_, l_ = self.plan(kind, n, rows, dp_size, r)
            starts.append(s_)
            lens.append(l_)
        st = np.ascontiguousarray(np.stack(starts)) if dp_size else np.zeros((0, n.size), np.int64)
        ln = np.ascontiguousarray(np.stack(lens)) if dp_size else np.zeros((0, n.size), np.int64)
        acc_full = np.ascontiguousarray(acc_full, dtype=np.float32)
        assert acc_full.size == int(n.sum())
        out = np.empty(int(ln.sum()), np.float32)
        self.lib.z1o_pack_send(n.size, _ptr(n), dp_size, _ptr(st), _ptr(ln), _ptr(acc_full),
                               int(bool(divide)), _ptr(out))
        return out

    def lr_at(self, lr_max, lr_min, warmup, decay, style, t) -> float:
        """Learning rate at step t (style 0 none, 1 linear, 2 cosine decay)."""
        return float(self.lib.z1o_lr_at(lr_max, lr_min, warmup, decay, style, t))

    def num_threads(self) -> int:
        return int(self.lib.z1o_num_threads())


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from z1_oracle.c (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default
