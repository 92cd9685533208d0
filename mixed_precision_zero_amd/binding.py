"""Thin ctypes binding of libz1 (include/z1.h): argument marshalling only.

Every step of the optimizer runs in the HIP library; this module converts
torch tensors to device pointers, torch streams to hipStream_t handles and
status codes to exceptions.  There is no fallback: if the library is not
built, importing the binding raises.

torch is imported first so that libz1 binds to the HIP runtime torch has
already loaded (both carry the soname libamdhip64.so.7), which makes torch's
stream handles and device pointers valid inside the library.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libz1.so")

Z1_OK, Z1_EINVAL, Z1_EALIGN, Z1_ENOMEM, Z1_EHIP, Z1_ESTATE = range(6)
_NAMES = {0: "Z1_OK", 1: "Z1_EINVAL", 2: "Z1_EALIGN", 3: "Z1_ENOMEM", 4: "Z1_EHIP",
          5: "Z1_ESTATE"}

EXPORTS = ("z1_abi_version", "z1_strerror", "z1_shard_plan", "z1_shard_plan_kind",
           "z1_plan_create", "z1_plan_destroy", "z1_plan_query", "z1_plan_layout",
           "z1_accum_grads", "z1_grad_norm_sq", "z1_adamw_step", "z1_lr_at", "z1_probe_copy",
           "z1_grad_norm_sq_acc", "z1_pack_layout", "z1_pack_create", "z1_pack_destroy",
           "z1_pack_accum", "z1_probe", "z1_accum_grads_range", "z1_pack_accum_range",
           "z1_probe_plan", "z1_schedule_create", "z1_schedule_destroy", "z1_schedule_query",
           "z1_adamw_step_scheduled", "z1_grad_norm_sq_pair", "z1_norm_combine",
           "z1_grad_norm_sq_flat_noalloc")

PROBES = {"read": 0, "write": 1, "adamw_traffic": 2, "accum_traffic": 3, "slots_traffic": 4,
          "adamw_traffic_wave": 5, "slots_traffic_one": 6}

PLAN_KINDS = {"per_tensor": 0, "flat": 1, "dim0": 2}
LAYOUTS = {"full": 0, "packed": 1}
WALKS = {"auto": 0, "chunks": 1, "arena_tiles": 2}
DECAY_STYLES = {"none": 0, "linear": 1, "cosine": 2}


class Z1Error(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {_NAMES.get(status, status)} ({strerror(status)})")


class Bind(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int32), ("dp_size", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("n_micro", ctypes.c_int32),
                ("numel", ctypes.POINTER(ctypes.c_int64)),
                ("weights", ctypes.POINTER(ctypes.c_void_p)),
                ("grads", ctypes.POINTER(ctypes.c_void_p)),
                ("master", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("acc", ctypes.c_void_p),
                ("arena_elems", ctypes.c_int64), ("chunk_elems", ctypes.c_int64),
                ("max_blocks", ctypes.c_int32), ("plan_kind", ctypes.c_int32),
                ("rows", ctypes.POINTER(ctypes.c_int64)),
                ("lr_scale", ctypes.POINTER(ctypes.c_double)),
                ("wd_scale", ctypes.POINTER(ctypes.c_double)),
                ("layout", ctypes.c_int32), ("walk", ctypes.c_int32)]


class LRSchedule(ctypes.Structure):
    _fields_ = [("lr_max", ctypes.c_double), ("lr_min", ctypes.c_double),
                ("warmup_steps", ctypes.c_int64), ("decay_steps", ctypes.c_int64),
                ("decay_style", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class PackBind(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int32), ("dp_size", ctypes.c_int32),
                ("n_micro", ctypes.c_int32), ("plan_kind", ctypes.c_int32),
                ("numel", ctypes.POINTER(ctypes.c_int64)), ("rows", ctypes.POINTER(ctypes.c_int64)),
                ("grads", ctypes.POINTER(ctypes.c_void_p)), ("send", ctypes.c_void_p),
                ("send_elems", ctypes.c_int64), ("chunk_elems", ctypes.c_int64),
                ("divide", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int32), ("n_micro", ctypes.c_int32),
                ("shard_elems", ctypes.c_int64), ("arena_elems", ctypes.c_int64),
                ("chunk_elems", ctypes.c_int64), ("n_chunks", ctypes.c_int64),
                ("adamw_tiles", ctypes.c_int64), ("boundary_tiles", ctypes.c_int64)]


class AdamWHP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("clip", ctypes.c_double),
                ("step", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libz1 is not built ({LIB_PATH} missing); run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    PI64 = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "z1_abi_version": ([], I32),
        "z1_strerror": ([ctypes.c_int], ctypes.c_char_p),
        "z1_shard_plan": ([I32, PI64, I32, I32, PI64, PI64, PI64, PI64], ctypes.c_int),
        "z1_shard_plan_kind": ([I32, I32, PI64, PI64, I32, I32, PI64, PI64, PI64, PI64],
                               ctypes.c_int),
        "z1_lr_at": ([ctypes.POINTER(LRSchedule), I64, ctypes.POINTER(ctypes.c_double)],
                     ctypes.c_int),
        "z1_plan_create": ([ctypes.POINTER(P), ctypes.POINTER(Bind), P], ctypes.c_int),
        "z1_plan_destroy": ([P], ctypes.c_int),
        "z1_plan_query": ([P, ctypes.POINTER(PlanInfo)], ctypes.c_int),
        "z1_plan_layout": ([P, PI64, PI64, PI64], ctypes.c_int),
        "z1_accum_grads": ([P, I32, P], ctypes.c_int),
        "z1_accum_grads_range": ([P, I32, I32, P], ctypes.c_int),
        "z1_grad_norm_sq": ([P, P, P], ctypes.c_int),
        "z1_adamw_step": ([P, ctypes.POINTER(AdamWHP), P, P], ctypes.c_int),
        "z1_probe_copy": ([P, P, I64, P], ctypes.c_int),
        "z1_grad_norm_sq_acc": ([P, P, P], ctypes.c_int),
        "z1_pack_layout": ([I32, I32, PI64, PI64, I32, PI64], ctypes.c_int),
        "z1_pack_create": ([ctypes.POINTER(P), ctypes.POINTER(PackBind), P], ctypes.c_int),
        "z1_pack_destroy": ([P], ctypes.c_int),
        "z1_pack_accum": ([P, I32, P], ctypes.c_int),
        "z1_pack_accum_range": ([P, I32, I32, P], ctypes.c_int),
        "z1_probe": ([I32, ctypes.POINTER(P), I32, I64, P], ctypes.c_int),
        "z1_probe_plan": ([P, I32, P], ctypes.c_int),
        "z1_grad_norm_sq_pair": ([P, P, P], ctypes.c_int),
        "z1_norm_combine": ([P, I32, P, P], ctypes.c_int),
        "z1_schedule_create": ([ctypes.POINTER(P), ctypes.POINTER(AdamWHP),
                                ctypes.POINTER(LRSchedule), I64, P], ctypes.c_int),
        "z1_schedule_destroy": ([P], ctypes.c_int),
        "z1_schedule_query": ([P, PI64, PI64], ctypes.c_int),
        "z1_adamw_step_scheduled": ([P, P, P, P], ctypes.c_int),
        "z1_grad_norm_sq_flat_noalloc": ([P, I64, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()


def strerror(status: int) -> str:
    return lib.z1_strerror(status).decode()


def _check(status: int, call: str) -> None:
    if status != Z1_OK:
        raise Z1Error(status, call)


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _p64(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _stream(stream) -> Optional[int]:
    """hipStream_t of a torch stream (default: torch's current stream)."""
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _dptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check_tensors(items) -> None:
    """Reject tensors the library would read or write out of bounds or
    misread.  items: (tensor, name, dtype, min_elems) with dtype None meaning
    any dtype and min_elems then counted in bytes.  Every tensor is checked
    for dtype, contiguity and size first, then every tensor for its device
    (the current GPU).  None and int (a raw device address) pass unchecked:
    the caller vouches for them."""
    tensors = []
    for t, name, dtype, min_elems in items:
        if t is None or isinstance(t, int):
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: expected a torch tensor or a device address, "
                            f"got {type(t).__name__}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: not contiguous")
        have = t.numel() if dtype is not None else t.numel() * t.element_size()
        if have < min_elems:
            unit = "elements" if dtype is not None else "bytes"
            raise ValueError(f"{name}: {have} {unit}, the call touches {min_elems}")
        tensors.append((t, name))
    for t, name in tensors:
        if t.device.type != "cuda":
            raise ValueError(f"{name}: on {t.device}, expected the current GPU")
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"{name}: on {t.device}, expected "
                             f"cuda:{torch.cuda.current_device()}")


def _check_tensor(t, name: str, dtype, min_elems: int) -> None:
    _check_tensors([(t, name, dtype, min_elems)])


def z1_abi_version() -> int:
    return int(lib.z1_abi_version())


def z1_shard_plan(numel: Sequence[int], dp_size: int, rank: int, kind: str = "per_tensor",
                  rows: Optional[Sequence[int]] = None):
    """(start, len, arena_off, arena_elems) of this rank's shard plan."""
    n = _i64(numel)
    start = np.zeros(n.size, np.int64)
    ln = np.zeros(n.size, np.int64)
    off = np.zeros(n.size, np.int64)
    ae = np.zeros(1, np.int64)
    if kind == "per_tensor" and rows is None:
        _check(lib.z1_shard_plan(n.size, _p64(n), dp_size, rank, _p64(start), _p64(ln),
                                 _p64(off), _p64(ae)), "z1_shard_plan")
    else:
        r = _i64(rows) if rows is not None else None
        _check(lib.z1_shard_plan_kind(PLAN_KINDS[kind], n.size, _p64(n),
                                      _p64(r) if r is not None else None, dp_size, rank,
                                      _p64(start), _p64(ln), _p64(off), _p64(ae)),
               "z1_shard_plan_kind")
    return start, ln, off, int(ae[0])


def z1_lr_at(step: int, *, lr_max: float, lr_min: float, warmup_steps: int, decay_steps: int,
             decay_style: str = "cosine") -> float:
    sc = LRSchedule(lr_max, lr_min, warmup_steps, decay_steps, DECAY_STYLES[decay_style], 0)
    out = ctypes.c_double()
    _check(lib.z1_lr_at(ctypes.byref(sc), int(step), ctypes.byref(out)), "z1_lr_at")
    return out.value


class Plan:
    """Owner of a z1_plan handle (destroyed with z1_plan_destroy)."""

    def __init__(self, handle: int, info: PlanInfo, keep):
        self.handle = handle
        self.info = info
        # the host arrays the bind pointed at and the bound device tensors:
        # the plan writes into those tensors until it is destroyed, so they
        # must not return to torch's allocator before it is
        self._keep = keep

    def close(self):
        if self.handle:
            _check(lib.z1_plan_destroy(self.handle), "z1_plan_destroy")
            self.handle = 0
            self._keep = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def z1_plan_create(numel: Sequence[int], dp_size: int, rank: int, weights: Sequence,
                   grads: Sequence[Sequence], master, exp_avg, exp_avg_sq, acc,
                   chunk_elems: int = 0, max_blocks: int = 0, stream=None,
                   kind: str = "per_tensor", rows: Optional[Sequence[int]] = None,
                   lr_scale: Optional[Sequence[float]] = None,
                   wd_scale: Optional[Sequence[float]] = None,
                   layout: str = "full", arena_elems: Optional[int] = None,
                   walk: str = "auto") -> Plan:
    """Bind device buffers, the four arenas fp32 of arena_elems.
    layout "full": weights[i] and grads[k][i] are full-size bf16 tensors (or
    raw device addresses).  layout "packed": weights is one packed bf16
    shard and grads[k] one packed bf16 shard per micro-batch, in arena order.
    arena_elems defaults to the smallest arena tensor's length; pass it when
    the arenas are raw device addresses.  walk ("auto", "chunks",
    "arena_tiles"): how the AdamW step walks the shard (z1_walk)."""
    n = _i64(numel)
    K = len(grads)
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    if kind not in PLAN_KINDS:
        raise ValueError(f"unknown plan kind {kind!r}")
    if walk not in WALKS:
        raise ValueError(f"unknown walk {walk!r}")
    # what the plan will touch: slice [start, start+len) of every tensor and
    # arena_elems of every arena (and of each packed bf16 shard)
    st_, ln_, _, need = z1_shard_plan(n, dp_size, rank, kind, rows)
    bf16, f32 = torch.bfloat16, torch.float32
    items = [(a, name, f32, need) for name, a in (("master", master), ("exp_avg", exp_avg),
                                                  ("exp_avg_sq", exp_avg_sq), ("acc", acc))]
    if layout == "packed":
        items.append((weights, "weights (packed shard)", bf16, need))
        items += [(g, f"grads[{k}] (packed shard)", bf16, need) for k, g in enumerate(grads)]
        _check_tensors(items)
        wp = (ctypes.c_void_p * 1)(_dptr(weights))
        gp = (ctypes.c_void_p * max(K, 1))(*[_dptr(g) for g in grads])
    else:
        for gk in grads:
            if len(gk) != n.size:
                raise ValueError("grads[k] must list one tensor per parameter")
        if len(weights) != n.size:
            raise ValueError("weights must list one tensor per parameter")
        for i in range(n.size):
            if ln_[i] == 0:
                continue
            end = int(st_[i] + ln_[i])
            items.append((weights[i], f"weights[{i}]", bf16, end))
            items += [(grads[k][i], f"grads[{k}][{i}]", bf16, end) for k in range(K)]
        _check_tensors(items)
        wp = (ctypes.c_void_p * max(n.size, 1))(*[_dptr(w) for w in weights])
        gp = (ctypes.c_void_p * max(K * n.size, 1))(*[_dptr(g) for gk in grads for g in gk])
    arena = [master, exp_avg, exp_avg_sq, acc]
    sizes = [a.numel() for a in arena if hasattr(a, "numel")]
    if arena_elems is not None:
        sizes = [int(arena_elems)]
    r = _i64(rows) if rows is not None else None
    ls = np.ascontiguousarray(np.asarray(lr_scale, np.float64)) if lr_scale is not None else None
    ws = np.ascontiguousarray(np.asarray(wd_scale, np.float64)) if wd_scale is not None else None
    for a in (r, ls, ws):
        if a is not None and a.size != n.size:
            raise ValueError("rows / lr_scale / wd_scale need one entry per parameter")
    PD = ctypes.POINTER(ctypes.c_double)
    b = Bind(n_tensors=n.size, dp_size=dp_size, rank=rank, n_micro=K, numel=_p64(n),
             weights=ctypes.cast(wp, ctypes.POINTER(ctypes.c_void_p)),
             grads=ctypes.cast(gp, ctypes.POINTER(ctypes.c_void_p)),
             master=_dptr(master), exp_avg=_dptr(exp_avg), exp_avg_sq=_dptr(exp_avg_sq),
             acc=_dptr(acc), arena_elems=min(sizes) if sizes else 0,
             chunk_elems=chunk_elems, max_blocks=max_blocks, plan_kind=PLAN_KINDS[kind],
             rows=_p64(r) if r is not None else None,
             lr_scale=ls.ctypes.data_as(PD) if ls is not None else None,
             wd_scale=ws.ctypes.data_as(PD) if ws is not None else None,
             layout=LAYOUTS[layout], walk=WALKS[walk])
    h = ctypes.c_void_p()
    _check(lib.z1_plan_create(ctypes.byref(h), ctypes.byref(b), _stream(stream)),
           "z1_plan_create")
    info = PlanInfo()
    _check(lib.z1_plan_query(h, ctypes.byref(info)), "z1_plan_query")
    return Plan(h.value, info, (n, wp, gp, r, ls, ws, weights, grads, master, exp_avg,
                                exp_avg_sq, acc))


def z1_plan_layout(plan: Plan):
    n = plan.info.n_tensors
    start = np.zeros(n, np.int64)
    ln = np.zeros(n, np.int64)
    off = np.zeros(n, np.int64)
    _check(lib.z1_plan_layout(plan.handle, _p64(start), _p64(ln), _p64(off)), "z1_plan_layout")
    return start, ln, off


def z1_accum_grads(plan: Plan, k: int, stream=None) -> None:
    _check(lib.z1_accum_grads(plan.handle, k, _stream(stream)), "z1_accum_grads")


def z1_accum_grads_range(plan: Plan, k_begin: int, k_end: int, stream=None) -> None:
    _check(lib.z1_accum_grads_range(plan.handle, k_begin, k_end, _stream(stream)),
           "z1_accum_grads_range")


def z1_grad_norm_sq(plan: Plan, d_S, stream=None) -> None:
    """Writes S into the device float64 tensor d_S (first element)."""
    _check_tensor(d_S, "d_S", torch.float64, 1)
    _check(lib.z1_grad_norm_sq(plan.handle, _dptr(d_S), _stream(stream)), "z1_grad_norm_sq")


def z1_grad_norm_sq_pair(plan: Plan, d_pair, stream=None) -> None:
    """S of this rank as the pair (hi, lo) in the device float64 tensor d_pair[:2]."""
    _check_tensor(d_pair, "d_pair", torch.float64, 2)
    _check(lib.z1_grad_norm_sq_pair(plan.handle, _dptr(d_pair), _stream(stream)),
           "z1_grad_norm_sq_pair")


def z1_norm_combine(d_pairs, n: int, d_S, stream=None) -> None:
    """S from n gathered pairs (device float64 [n, 2]) added in order, into d_S."""
    _check_tensors([(d_pairs, "d_pairs", torch.float64, 2 * int(n)),
                    (d_S, "d_S", torch.float64, 1)])
    _check(lib.z1_norm_combine(_dptr(d_pairs), int(n), _dptr(d_S), _stream(stream)),
           "z1_norm_combine")


def z1_adamw_step(plan: Plan, *, lr, beta1, beta2, eps, weight_decay, clip, step,
                  d_S=None, stream=None) -> None:
    hp = AdamWHP(lr, beta1, beta2, eps, weight_decay, clip, int(step))
    _check_tensor(d_S, "d_S", torch.float64, 1)
    _check(lib.z1_adamw_step(plan.handle, ctypes.byref(hp), _dptr(d_S), _stream(stream)),
           "z1_adamw_step")


class Schedule:
    """Owner of a z1_schedule handle (destroyed with z1_schedule_destroy)."""

    def __init__(self, handle: int, n_steps: int):
        self.handle = handle
        self.n_steps = n_steps

    def close(self):
        if self.handle:
            _check(lib.z1_schedule_destroy(self.handle), "z1_schedule_destroy")
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def z1_schedule_create(*, lr, beta1, beta2, eps, weight_decay, clip, step, n_steps: int,
                       lr_schedule: Optional[dict] = None, stream=None) -> Schedule:
    """Per-step constants for steps step .. step + n_steps - 1; lr_schedule is
    a dict of z1_lr_at's keywords (None: lr every step)."""
    hp = AdamWHP(lr, beta1, beta2, eps, weight_decay, clip, int(step))
    sc = None
    if lr_schedule is not None:
        d = dict(lr_schedule)
        sc = LRSchedule(d["lr_max"], d["lr_min"], d["warmup_steps"], d["decay_steps"],
                        DECAY_STYLES[d.get("decay_style", "cosine")], 0)
    h = ctypes.c_void_p()
    _check(lib.z1_schedule_create(ctypes.byref(h), ctypes.byref(hp),
                                  ctypes.byref(sc) if sc is not None else None, int(n_steps),
                                  _stream(stream)), "z1_schedule_create")
    return Schedule(h.value, int(n_steps))


def z1_schedule_query(sched: Schedule):
    """(next step, overrun count); synchronise the stream that ran the steps first."""
    t = ctypes.c_int64()
    o = ctypes.c_int64()
    _check(lib.z1_schedule_query(sched.handle, ctypes.byref(t), ctypes.byref(o)),
           "z1_schedule_query")
    return t.value, o.value


def z1_adamw_step_scheduled(plan: Plan, sched: Schedule, d_S=None, stream=None) -> None:
    _check_tensor(d_S, "d_S", torch.float64, 1)
    _check(lib.z1_adamw_step_scheduled(plan.handle, sched.handle, _dptr(d_S), _stream(stream)),
           "z1_adamw_step_scheduled")


def z1_grad_norm_sq_acc(plan: Plan, d_S, stream=None) -> None:
    """S of the acc arena as the caller filled it (e.g. by a reduce-scatter)."""
    _check_tensor(d_S, "d_S", torch.float64, 1)
    _check(lib.z1_grad_norm_sq_acc(plan.handle, _dptr(d_S), _stream(stream)),
           "z1_grad_norm_sq_acc")


NORM_FLAT_MAX_ELEMS = 1 << 30


def z1_grad_norm_sq_flat_noalloc(acc, n: int, d_S, stream=None) -> None:
    """S of the first n elements of a contiguous fp32 buffer, into d_S; no
    plan, no device allocation (the library's fixed scratch array)."""
    _check_tensors([(acc, "acc", torch.float32, int(n)), (d_S, "d_S", torch.float64, 1)])
    _check(lib.z1_grad_norm_sq_flat_noalloc(_dptr(acc), int(n), _dptr(d_S), _stream(stream)),
           "z1_grad_norm_sq_flat_noalloc")


def z1_pack_layout(numel: Sequence[int], dp_size: int, kind: str = "per_tensor",
                   rows: Optional[Sequence[int]] = None) -> int:
    """Per-rank segment length of the reduce-scatter send buffer."""
    n = _i64(numel)
    r = _i64(rows) if rows is not None else None
    seg = np.zeros(1, np.int64)
    _check(lib.z1_pack_layout(PLAN_KINDS[kind], n.size, _p64(n),
                              _p64(r) if r is not None else None, dp_size, _p64(seg)),
           "z1_pack_layout")
    return int(seg[0])


class Pack:
    """Owner of a z1_pack handle."""

    def __init__(self, handle: int, seg: int, keep):
        self.handle = handle
        self.seg = seg
        self._keep = keep   # host arrays and the bound device tensors (as Plan)

    def close(self):
        if self.handle:
            _check(lib.z1_pack_destroy(self.handle), "z1_pack_destroy")
            self.handle = 0
            self._keep = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def z1_pack_create(numel: Sequence[int], dp_size: int, grads: Sequence[Sequence], send,
                   kind: str = "per_tensor", rows: Optional[Sequence[int]] = None,
                   divide: bool = False, chunk_elems: int = 0, stream=None) -> Pack:
    n = _i64(numel)
    K = len(grads)
    for gk in grads:
        if len(gk) != n.size:
            raise ValueError("grads[k] must list one tensor per parameter")
    r = _i64(rows) if rows is not None else None
    if kind not in PLAN_KINDS:
        raise ValueError(f"unknown plan kind {kind!r}")
    seg_need = z1_pack_layout(n, dp_size, kind, r)
    _check_tensors([(gk[i], f"grads[{k}][{i}]", torch.bfloat16, int(n[i]))
                    for k, gk in enumerate(grads) for i in range(n.size) if n[i]] +
                   [(send, "send", torch.float32, dp_size * seg_need)])
    gp = (ctypes.c_void_p * max(K * n.size, 1))(*[_dptr(g) for gk in grads for g in gk])
    b = PackBind(n_tensors=n.size, dp_size=dp_size, n_micro=K, plan_kind=PLAN_KINDS[kind],
                 numel=_p64(n), rows=_p64(r) if r is not None else None,
                 grads=ctypes.cast(gp, ctypes.POINTER(ctypes.c_void_p)), send=_dptr(send),
                 send_elems=send.numel() if hasattr(send, "numel") else 0,
                 chunk_elems=chunk_elems, divide=int(bool(divide)), reserved=0)
    h = ctypes.c_void_p()
    _check(lib.z1_pack_create(ctypes.byref(h), ctypes.byref(b), _stream(stream)), "z1_pack_create")
    seg = z1_pack_layout(n, dp_size, kind, r)
    return Pack(h.value, seg, (n, r, gp, grads, send))


def z1_pack_accum(pack: Pack, k: int, stream=None) -> None:
    _check(lib.z1_pack_accum(pack.handle, k, _stream(stream)), "z1_pack_accum")


def z1_pack_accum_range(pack: Pack, k_begin: int, k_end: int, stream=None) -> None:
    _check(lib.z1_pack_accum_range(pack.handle, k_begin, k_end, _stream(stream)),
           "z1_pack_accum_range")


def z1_probe_plan(plan: Plan, kind: str = "adamw", stream=None) -> None:
    """Overwrites the plan's master / m / v arenas and weight slices."""
    _check(lib.z1_probe_plan(plan.handle, {"adamw": 0}[kind], _stream(stream)), "z1_probe_plan")


def z1_probe(kind: str, bufs: Sequence, n_vec: int, stream=None) -> None:
    """Traffic-only streaming kernel (see z1.h); bufs are tensors or addresses."""
    nv = int(n_vec)
    slots = (8 * nv,) * (len(bufs) - 1) + (16 * nv,)
    need = {"read": (16 * nv, 4), "write": (16 * nv,),
            "adamw_traffic": (16 * nv,) * 4 + (8 * nv,),
            "adamw_traffic_wave": (16 * nv,) * 4 + (8 * nv,),
            "accum_traffic": (8 * nv, 16 * nv),
            "slots_traffic": slots, "slots_traffic_one": slots}[kind]
    _check_tensors([(b, f"bufs[{j}]", None, nb) for j, (b, nb) in enumerate(zip(bufs, need))])
    arr = (ctypes.c_void_p * max(len(bufs), 1))(*[_dptr(b) for b in bufs])
    _check(lib.z1_probe(PROBES[kind], arr, len(bufs), int(n_vec), _stream(stream)), "z1_probe")


def z1_probe_copy(src, dst, n_bytes: int, stream=None) -> None:
    _check_tensors([(src, "src", None, int(n_bytes)), (dst, "dst", None, int(n_bytes))])
    _check(lib.z1_probe_copy(_dptr(src), _dptr(dst), int(n_bytes), _stream(stream)),
           "z1_probe_copy")


def hip_runtimes_loaded() -> list:
    """Paths of every libamdhip64 mapped into this process (should be one)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    return sorted(paths)
