"""GPU-vs-oracle parity harness shared by the GPU tests.

Inputs come from ``mixed_precision_zero_amd.workloads`` (seeded, full-size,
generated on the device by torch); the HIP library reads the bound device
tensors, the oracle reads the same bytes copied to the host and cut with the
oracle's own shard plan.  Nothing the HIP path computes is ever fed to the
oracle.
"""
from __future__ import annotations

import math
import sys
import time
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

import oracle
from mixed_precision_zero_amd import workloads as W
from mixed_precision_zero_amd.shard import ShardStep

CANARY = float.fromhex("0x1.5a5a5ap+77")   # a value no step can produce by chance


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def rel_rms_err(x: np.ndarray, y: np.ndarray) -> float:
    """max_e |x_e - y_e| / max(|y_e|, rms(y)): the fp32-state parity metric."""
    if y.size == 0:
        return 0.0
    x = x.astype(np.float64)
    y = y.astype(np.float64)
    rms = math.sqrt(float(np.mean(y * y)))
    den = np.maximum(np.abs(y), rms)
    den[den == 0] = 1.0
    return float(np.max(np.abs(x - y) / den))


def bf16_ord(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns mapped to integers that are ordered like the values."""
    h = h.astype(np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class StepReport:
    step: int
    acc_mismatch: int
    S_gpu: float
    S_ref: float
    S_rel: float
    rel: dict = field(default_factory=dict)          # buffer -> rel_rms_err
    not_bitexact: dict = field(default_factory=dict)  # buffer -> count
    bf16_max_ulp: int = 0
    bf16_self_mismatch: int = 0


class Parity:
    """Runs a workload on the GPU and the oracle side by side."""

    def __init__(self, w: W.Workload, device="cuda", chunk_elems=0, max_blocks=0,
                 seed=0, canaries=True, kind="per_tensor", lr_scale=None, wd_scale=None,
                 ranges=None, layout="full", walk="auto"):
        self.w = w
        self.ranges = ranges     # None: one accumulation call per micro-batch
        self.dev = torch.device(device)
        self.o = oracle.get()
        self.seed = seed
        t0 = time.time()
        self.st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device=self.dev,
                            chunk_elems=chunk_elems, max_blocks=max_blocks,
                            arena_pad=64 if canaries else 0, kind=kind,
                            lr_scale=lr_scale, wd_scale=wd_scale, layout=layout, walk=walk)
        rows = [s[0] if len(s) else 1 for s in w.shapes]
        self.o_start, self.o_len = self.o.plan(kind, w.numel, rows, w.dp_size, w.rank)
        self.segments = None
        if lr_scale is not None or wd_scale is not None:
            n = len(w.shapes)
            self.segments = (self.o_len, lr_scale if lr_scale is not None else [1.0] * n,
                             wd_scale if wd_scale is not None else [1.0] * n)
        self.L = int(self.o_len.sum())
        # canaries in every arena element outside a slice (gaps and tail)
        self.free_mask = None
        if canaries:
            used = torch.zeros(self.st.master.numel(), dtype=torch.bool, device=self.dev)
            for _, _, ln, off in self.st.slices():
                if ln:
                    used[off:off + ln] = True
            self.free_mask = ~used
            for a in (self.st.master, self.st.exp_avg, self.st.exp_avg_sq, self.st.acc):
                a[self.free_mask] = CANARY
            if self.st.w_packed is not None:
                self.st.w_packed[self.free_mask] = CANARY
        master = W.make_master(w, seed=seed, device=self.dev)
        self.st.scatter_to_arena(self.st.master, master)
        self.st.load_weights(master)     # torch's own cast: the weights before any step
        self.p = self._packed_host_f32(master)
        del master
        self.m = np.zeros(self.L, np.float32)
        self.v = np.zeros(self.L, np.float32)
        self.wbits = np.zeros(self.L, np.uint16)
        self.acc = np.zeros(self.L, np.float32)
        self.w_before = None
        if w.dp_size > 1:
            self.w_before = [x.clone() for x in self.st.weights]
        self.t = 0
        log(f"[parity] {w.name}: L={self.L} chunks={self.st.plan.info.n_chunks} "
            f"setup {time.time() - t0:.1f}s")

    def _packed_host_f32(self, full) -> np.ndarray:
        parts = [full[i].reshape(-1)[s:s + n] for i, (s, n) in
                 enumerate(zip(self.o_start, self.o_len)) if n]
        if not parts:
            return np.zeros(0, np.float32)
        return torch.cat(parts).cpu().numpy().astype(np.float32)

    def _packed_host_bf16(self, full) -> np.ndarray:
        parts = [full[i].reshape(-1)[s:s + n] for i, (s, n) in
                 enumerate(zip(self.o_start, self.o_len)) if n]
        if not parts:
            return np.zeros(0, np.uint16)
        return bf16_bits(torch.cat(parts))

    def plan_matches(self) -> bool:
        nz = self.o_len > 0
        return bool((self.st.len == self.o_len).all() and
                    (self.st.start[nz] == self.o_start[nz]).all())

    def step(self, check=True, gpu_step=None, lr=None) -> Optional[StepReport]:
        """One step on both sides from fresh seeded gradients.  gpu_step
        replaces the eager library calls (for example a captured graph's
        replay); lr replaces the workload's learning rate on the oracle side
        (the rate a schedule gives this step)."""
        w, st = self.w, self.st
        self.t += 1
        t = self.t
        t0 = time.time()
        g = np.empty((w.n_micro, self.L), np.uint16)
        for k in range(w.n_micro):
            W.make_micro_grads(w, t, k, seed=self.seed, device=self.dev, out=st.grads[k])
            st.stage_grads(k)
            g[k] = self._packed_host_bf16(st.grads[k])
        t1 = time.time()
        if gpu_step is None:
            st.step(w.hp(), ranges=self.ranges)
        else:
            gpu_step()
        torch.cuda.synchronize()
        t2 = time.time()
        hp = w.hp()
        if lr is not None:
            hp["lr"] = lr
        S, c, _ = self.o.step(g, self.p, self.m, self.v, step=t, acc=self.acc, w=self.wbits,
                              segments=self.segments, **hp)
        del g
        t3 = time.time()
        log(f"[parity] {w.name} step {t}: inputs {t1 - t0:.1f}s gpu {t2 - t1:.2f}s "
            f"oracle {t3 - t2:.1f}s (S={S:.6g}, c={c:.4g})")
        if not check:
            return None
        return self.compare(S)

    def compare(self, S_ref: float) -> StepReport:
        """Bit equality first (cheap); the tolerance metrics are computed only
        for a buffer that is not bit-identical (for identical buffers they
        are 0 by definition)."""
        st = self.st
        acc_g = st.packed(st.acc).cpu().numpy()
        S_g = float(st.d_S.item())
        acc_bad = 0 if np.array_equal(acc_g, self.acc) else int((acc_g != self.acc).sum())
        del acc_g
        rep = StepReport(step=self.t, acc_mismatch=acc_bad, S_gpu=S_g, S_ref=S_ref,
                         S_rel=abs(S_g - S_ref) / S_ref if S_ref else abs(S_g))
        master_exact = True
        x_master = None
        for name, gpu, ref in (("master", st.master, self.p), ("exp_avg", st.exp_avg, self.m),
                               ("exp_avg_sq", st.exp_avg_sq, self.v)):
            x = st.packed(gpu).cpu().numpy()
            if np.array_equal(x.view(np.uint32), ref.view(np.uint32)):
                rep.rel[name] = 0.0
                rep.not_bitexact[name] = 0
            else:
                rep.rel[name] = rel_rms_err(x, ref)
                rep.not_bitexact[name] = int((x.view(np.uint32) != ref.view(np.uint32)).sum())
                if name == "master":
                    master_exact = False
            if name == "master":
                x_master = x
            del x
        wb = bf16_bits(st.packed_weights())
        if wb.size and not np.array_equal(wb, self.wbits):
            rep.bf16_max_ulp = int(np.max(np.abs(bf16_ord(wb) - bf16_ord(self.wbits))))
            rep.not_bitexact["bf16"] = int((wb != self.wbits).sum())
        else:
            rep.not_bitexact["bf16"] = 0
        if wb.size:
            # the GPU's bf16 must be torch's RNE cast of the GPU's own master:
            # every element when anything differs, else a strided sample
            # (exactness against the oracle already implies it)
            sl = slice(None) if (not master_exact or rep.not_bitexact["bf16"]) else slice(None, None, 97)
            own = bf16_bits(torch.from_numpy(np.ascontiguousarray(x_master[sl])).to(torch.bfloat16))
            rep.bf16_self_mismatch = int((wb[sl] != own).sum())
        return rep

    def canaries_intact(self) -> bool:
        if self.free_mask is None:
            return True
        ok = True
        for a in (self.st.master, self.st.exp_avg, self.st.exp_avg_sq, self.st.acc):
            ok &= bool((a[self.free_mask] == CANARY).all())
        if self.st.w_packed is not None:
            c = torch.tensor(CANARY, dtype=torch.bfloat16, device=self.dev)
            ok &= bool((self.st.w_packed[self.free_mask] == c).all())
        return ok

    def weights_outside_slices_intact(self) -> bool:
        if self.w_before is None:
            return True
        for i, s, ln, _ in self.st.slices():
            a = self.st.weights[i].reshape(-1)
            b = self.w_before[i].reshape(-1)
            if not (torch.equal(a[:s], b[:s]) and torch.equal(a[s + ln:], b[s + ln:])):
                return False
        return True

    def close(self):
        self.st.close()


def assert_report(rep: StepReport, tol_state=1e-6, tol_S=1e-5, exact=True) -> None:
    """The contract's tolerances, then (exact=True) bit-exactness: the GPU
    evaluates the oracle's IEEE operation sequence and both round S once, so
    every buffer is expected to match bit for bit."""
    assert rep.acc_mismatch == 0, f"step {rep.step}: {rep.acc_mismatch} acc elements differ"
    assert rep.S_rel <= tol_S, f"step {rep.step}: S rel err {rep.S_rel:.3g}"
    for name, e in rep.rel.items():
        assert e <= tol_state, f"step {rep.step}: {name} rel err {e:.3g} > {tol_state}"
    assert rep.bf16_max_ulp <= 1, f"step {rep.step}: bf16 off by {rep.bf16_max_ulp} ulp"
    assert rep.bf16_self_mismatch == 0, f"step {rep.step}: bf16 != RNE(own master)"
    if exact:
        assert rep.S_gpu == rep.S_ref, f"step {rep.step}: S not bit-exact"
        bad = {k: v for k, v in rep.not_bitexact.items() if v}
        assert not bad, f"step {rep.step}: elements not bit-exact: {bad}"
