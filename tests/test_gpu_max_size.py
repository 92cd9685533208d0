"""The step past 32-bit element indexes: a shard of more than 2^31 elements
whose source offsets inside the full bf16 tensor run past 2^32.

Parameters: one 1-D tensor of 2^32 + 10 elements and one of 1000, D = 2,
rank 1.  Rank 1's slice of the big tensor is elements [2^31 + 5, 2^32 + 10)
of the full tensor (the shard plan of the ZeRO-1 tutorial, section 6.3:
every parameter split evenly, rank r owning one contiguous slice), so the
bf16 source offsets cross 2^31 and 2^32 and the fp32 arena offsets cross
2^31.  About 65 GB of device memory.

The micro-batch gradients are +-2^-4 with seeded random signs, the same in
both micro-batches, so every accumulated element is +-2^-3 and
S = (shard elements) * 2^-6 exactly (a closed form that counts every element
once).  The signs make a wrong gradient index visible in the update.
Step 1 accumulates with resident slots, step 2 with one call per micro-batch.
On about 20k sampled elements (the ends of each slice, the neighbourhoods of
the 2^31 and 2^32 crossings, uniform picks, all of the small tensor) the
accumulated gradient, master, m, v and the bf16 weights must equal the
oracle's bits; weights outside this rank's slices must stay untouched.

The packed case binds packed bf16 shards (gradients and weights at arena
positions past 2^31) and forces AdamW's arena walk, whose tiles then sit
more than 2^31 elements (8 GB of fp32) into the arenas; the padding of the
packed weight shard must stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from mixed_precision_zero_amd.shard import ShardStep

pytestmark = pytest.mark.gpu

BIG = (1 << 32) + 10
SMALL = 1000
HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, clip=1.0)


def _fill_signs(dst, n, gen):
    """dst[0] = +-2^-4 (exact in bf16) with random signs; dst[1:] copies it."""
    bits = torch.randint(0, 2, (n,), generator=gen, device="cuda", dtype=torch.uint8)
    dst[0].copy_(bits)
    del bits
    dst[0].mul_(0.125).sub_(0.0625)
    for d in dst[1:]:
        d.copy_(dst[0])


def _samples(st, rng):
    """(tensor index, element within the slice) pairs to check."""
    out = []
    for i, s, ln, off in st.slices():
        js = [np.arange(min(ln, 4096)), np.arange(max(0, ln - 4096), ln),
              rng.integers(0, ln, 16384 if ln > 100000 else ln)]
        for cross in ((1 << 31) - off, (1 << 32) - s, (1 << 31) - s):
            if -2048 < cross < ln + 2048:
                js.append(np.arange(max(0, cross - 2048), min(ln, cross + 2048)))
        j = np.unique(np.concatenate(js).astype(np.int64))
        out.append((i, s, off, j))
    return out


def _gather(st, picks):
    """Sampled acc / master / m / v (fp32), weights and grads (bf16 bits)."""
    f32 = {name: [] for name in ("acc", "master", "exp_avg", "exp_avg_sq")}
    w, g = [], [[] for _ in range(st.n_micro)]
    packed = st.layout == "packed"
    for i, s, off, j in picks:
        a_idx = torch.from_numpy(off + j).cuda()
        f_idx = torch.from_numpy(s + j).cuda()
        for name in f32:
            f32[name].append(getattr(st, name)[a_idx].cpu().numpy())
        if packed:
            w.append(st.w_packed.view(torch.int16)[a_idx].cpu().numpy().view(np.uint16))
        else:
            w.append(st.weights[i].view(torch.int16)[f_idx].cpu().numpy().view(np.uint16))
        for k in range(st.n_micro):
            src = st.g_packed[k] if packed else st.grads[k][i]
            idx = a_idx if packed else f_idx
            g[k].append(src.view(torch.int16)[idx].cpu().numpy().view(np.uint16))
    cat = {k: np.ascontiguousarray(np.concatenate(v)) for k, v in f32.items()}
    return cat, np.concatenate(w), np.stack([np.concatenate(x) for x in g])


def _bits(x):
    return np.ascontiguousarray(x).view(np.uint32)


@pytest.mark.parametrize("layout", ["full", "packed_arena"])
def test_shard_past_32_bit_indexes_matches_oracle(layout):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    O = oracle.get()
    packed = layout == "packed_arena"
    kw = dict(layout="packed", walk="arena_tiles") if packed else {}
    st = ShardStep([(BIG,), (SMALL,)], 2, 1, 2, device="cuda", **kw)
    try:
        n_shard = int(st.len.sum())
        assert int(st.start[0]) == (1 << 31) + 5 and int(st.len[0]) == (1 << 31) + 5
        assert int(st.arena_off[1]) + int(st.len[1]) > (1 << 31)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(20240607)
        if packed:
            assert st.plan.info.adamw_tiles > (1 << 19)
            _fill_signs(st.g_packed, st.g_packed[0].numel(), gen)
        else:
            for i, shape in enumerate(st.shapes):
                _fill_signs([st.grads[k][i] for k in range(st.n_micro)], shape[0], gen)
        st.master.normal_(0.0, 0.02, generator=gen)
        torch.cuda.synchronize()

        rng = np.random.default_rng(11)
        picks = _samples(st, rng)
        before, _, _ = _gather(st, picks)
        p = before["master"].copy()
        m = np.zeros_like(p)
        v = np.zeros_like(p)

        for t in (1, 2):
            if t == 1:
                st.accumulate_range(0, st.n_micro)
            else:
                for k in range(st.n_micro):
                    st.accumulate(k)
            st.norm()
            st.adamw(HP, step=t)
            torch.cuda.synchronize()
            got, w_got, g_s = _gather(st, picks)

            S = st.d_S.item()
            assert S == n_shard * 2.0 ** -6, f"step {t}: S = {S!r}, want {n_shard} * 2^-6"

            acc = O.accumulate(g_s)
            assert np.all(np.abs(acc) == np.float32(0.125))
            assert np.array_equal(_bits(got["acc"]), _bits(acc)), f"step {t}: acc"

            c = O.clip_coef(S, HP["clip"])
            w_ref = np.zeros(p.size, np.uint16)
            O.adamw(acc, p, m, v, c, w=w_ref, step=t, **HP)
            for name, ref in (("master", p), ("exp_avg", m), ("exp_avg_sq", v)):
                bad = np.flatnonzero(_bits(got[name]) != _bits(ref))
                assert bad.size == 0, f"step {t}: {name} differs at {bad.size} samples"
            assert np.array_equal(w_got, w_ref), f"step {t}: bf16 weights"

        # the other rank's part of every tensor (full layout) or the padding
        # between slices (packed shard) is never written
        if packed:
            wp = st.w_packed.view(torch.int16)
            ends = sorted((off, off + ln) for _, _, ln, off in st.slices() if ln)
            gaps = [(0, ends[0][0])] + [(e0, s1) for (_, e0), (s1, _) in zip(ends, ends[1:])]
            gaps.append((ends[-1][1], wp.numel()))
            for lo, hi in gaps:
                assert not bool(wp[lo:hi].any()), f"packed padding [{lo}, {hi}) written"
        else:
            for i, s, ln, _ in st.slices():
                lo = max(0, s - 4096)
                other = st.weights[i].view(torch.int16)[lo:s].cpu().numpy()
                assert not other.any(), f"tensor {i}: weights outside the slice were written"
    finally:
        st.close()
        del st
        torch.cuda.empty_cache()
