"""One rank's device buffers for the ZeRO-1 shard step, wired to a libz1 plan.

This is memory plumbing: it allocates the fp32 arenas (master, m, v, acc),
the full-size bf16 weights and micro-gradient slots and the device norm
scalar with torch, creates the plan, and calls the four library entry points
in step order.  No arithmetic of the step happens here.

layout="packed" binds one packed bf16 weight shard and one packed bf16
gradient shard per micro-batch (arena order) instead of the full tensors;
the full-size tensors then serve only as staging for seeded inputs
(stage_grads copies this rank's slices into the packed slot).
"""
from __future__ import annotations

import time
from typing import List, Optional, Sequence

import torch

from . import binding as B


def flat_views(shapes: Sequence[Sequence[int]], dtype=torch.bfloat16, device="cuda"
               ) -> List[torch.Tensor]:
    """Zeroed tensors of the given shapes as views into one flat buffer.

    Each tensor starts on a 128-byte line (64 bf16 elements), so every view
    keeps the 16-byte alignment the library requires and pieces cut at
    multiples of the chunk size inside a tensor stay line-aligned."""
    numel = [int(torch.Size(s).numel()) for s in shapes]
    starts, o = [], 0
    for n in numel:
        starts.append(o)
        o += (n + 63) // 64 * 64
    flat = torch.zeros(max(o, 1), dtype=dtype, device=device)
    return [flat[a:a + n].view(tuple(shape)) for a, n, shape in zip(starts, numel, shapes)]


class ShardStep:
    def __init__(self, shapes: Sequence[Sequence[int]], dp_size: int, rank: int, n_micro: int,
                 device="cuda", chunk_elems: int = 0, max_blocks: int = 0,
                 weights: Optional[List[torch.Tensor]] = None,
                 grads: Optional[List[List[torch.Tensor]]] = None,
                 arena_pad: int = 0, kind: str = "per_tensor",
                 lr_scale: Optional[Sequence[float]] = None,
                 wd_scale: Optional[Sequence[float]] = None, layout: str = "full",
                 walk: str = "auto"):
        self.shapes = [tuple(s) for s in shapes]
        self.numel = [int(torch.Size(s).numel()) for s in self.shapes]
        self.rows = [int(s[0]) if len(s) else 1 for s in self.shapes]
        self.dp_size, self.rank, self.n_micro = dp_size, rank, n_micro
        self.kind = kind
        self.device = torch.device(device)
        self.start, self.len, self.arena_off, self.arena_elems = B.z1_shard_plan(
            self.numel, dp_size, rank, kind=kind, rows=self.rows if kind == "dim0" else None)
        n = self.arena_elems + arena_pad
        f32 = dict(dtype=torch.float32, device=self.device)
        self.master = torch.zeros(n, **f32)
        self.exp_avg = torch.zeros(n, **f32)
        self.exp_avg_sq = torch.zeros(n, **f32)
        self.acc = torch.zeros(n, **f32)
        bf = dict(dtype=torch.bfloat16, device=self.device)
        # the full-size bf16 weights and each micro-batch's gradients live in
        # one flat buffer per role, one view per tensor (a contiguous
        # parameter / gradient buffer, as data-parallel trainers keep them):
        # one large allocation instead of one per tensor
        self.weights = weights if weights is not None else self._flat_views(bf)
        self.grads = grads if grads is not None else [self._flat_views(bf)
                                                      for _ in range(n_micro)]
        self.d_S = torch.zeros(1, dtype=torch.float64, device=self.device)
        self.layout = layout
        self.w_packed = self.g_packed = None
        bind_w, bind_g = self.weights, self.grads
        if layout == "packed":
            self.w_packed = torch.zeros(n, **bf)
            self.g_packed = [torch.zeros(n, **bf) for _ in range(n_micro)]
            bind_w, bind_g = self.w_packed, self.g_packed
        t0 = time.perf_counter()
        self.plan = B.z1_plan_create(self.numel, dp_size, rank, bind_w, bind_g,
                                     self.master, self.exp_avg, self.exp_avg_sq, self.acc,
                                     chunk_elems=chunk_elems, max_blocks=max_blocks, kind=kind,
                                     rows=self.rows if kind == "dim0" else None,
                                     lr_scale=lr_scale, wd_scale=wd_scale, layout=layout,
                                     walk=walk)
        self.plan_create_s = time.perf_counter() - t0   # plan + chunk table + upload
        self.t = 0

    def _flat_views(self, opts) -> List[torch.Tensor]:
        return flat_views(self.shapes, **opts)

    # -- layout helpers (torch copies; initialisation and inspection only) --
    def slices(self):
        for i in range(len(self.numel)):
            yield i, int(self.start[i]), int(self.len[i]), int(self.arena_off[i])

    def scatter_to_arena(self, arena: torch.Tensor, full: Sequence[torch.Tensor]) -> None:
        """arena[off_i : off_i+len_i] = full_i.flatten()[start_i : start_i+len_i]"""
        for i, s, ln, off in self.slices():
            if ln:
                arena[off:off + ln].copy_(full[i].reshape(-1)[s:s + ln])

    def packed(self, arena: torch.Tensor) -> torch.Tensor:
        """The shard in packed order: the slices of every tensor concatenated."""
        parts = [arena[off:off + ln] for _, _, ln, off in self.slices() if ln]
        if not parts:
            return arena[:0].clone()
        return torch.cat(parts)

    def stage_grads(self, k: int) -> None:
        """Packed layout: copy this rank's slices of the full staging
        gradients of micro-batch k into its packed slot (no-op otherwise)."""
        if self.layout == "packed":
            self.scatter_to_arena(self.g_packed[k], self.grads[k])

    def load_weights(self, full: Sequence[torch.Tensor]) -> None:
        """The bf16 weights before a step, from full-size tensors."""
        if self.layout == "packed":
            self.scatter_to_arena(self.w_packed, full)
        else:
            for wt, x in zip(self.weights, full):
                wt.copy_(x)

    def load_weights_packed_order(self, packed: torch.Tensor) -> None:
        """Inverse of packed_weights(): write this rank's slices of the bf16
        weights from their concatenation."""
        pos = 0
        for i, s, ln, off in self.slices():
            if not ln:
                continue
            if self.layout == "packed":
                self.w_packed[off:off + ln].copy_(packed[pos:pos + ln])
            else:
                self.weights[i].view(-1)[s:s + ln].copy_(packed[pos:pos + ln])
            pos += ln

    def packed_weights(self) -> torch.Tensor:
        if self.layout == "packed":
            return self.packed(self.w_packed)
        parts = [self.weights[i].reshape(-1)[s:s + ln] for i, s, ln, _ in self.slices() if ln]
        if not parts:
            return torch.zeros(0, dtype=torch.bfloat16, device=self.device)
        return torch.cat(parts)

    # -- the step ------------------------------------------------------------
    def accumulate(self, k: int, stream=None) -> None:
        B.z1_accum_grads(self.plan, k, stream)

    def accumulate_range(self, k_begin: int, k_end: int, stream=None) -> None:
        B.z1_accum_grads_range(self.plan, k_begin, k_end, stream)

    def norm(self, stream=None) -> None:
        B.z1_grad_norm_sq(self.plan, self.d_S, stream)

    def adamw(self, hp: dict, step: Optional[int] = None, stream=None) -> None:
        t = self.t + 1 if step is None else step
        B.z1_adamw_step(self.plan, d_S=self.d_S, step=t, stream=stream, **hp)
        self.t = t

    def adamw_scheduled(self, sched, stream=None) -> None:
        """AdamW with the constants of the schedule's current row (the row
        then advances on the device)."""
        B.z1_adamw_step_scheduled(self.plan, sched, d_S=self.d_S, stream=stream)

    def step(self, hp: dict, stream=None, ranges=None) -> None:
        """One optimizer step.  ranges=None accumulates one micro-batch per
        call; otherwise a list of (k_begin, k_end) covering 0..K in order, one
        z1_accum_grads_range call each."""
        if ranges is None:
            for k in range(self.n_micro):
                self.accumulate(k, stream)
        else:
            for a, b in ranges:
                self.accumulate_range(a, b, stream)
        self.norm(stream)
        self.adamw(hp, stream=stream)

    def close(self) -> None:
        self.plan.close()
