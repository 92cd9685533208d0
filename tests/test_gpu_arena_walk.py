"""GPU parity of AdamW's arena walk (Z1_WALK_ARENA_TILES): plans whose AdamW
step runs one workgroup per 256-element arena tile, tiles inside one slice
straight-line and the slice segments of boundary tiles on workgroups of their
own, with packed bf16 shards and with full-size bf16 tensors (stores placed
through the per-tensor table).  Same bar as the chunk walk (bit-exact against
the oracle; padding and weights outside the slices never written), here on
lists where most tiles are boundary tiles, with per-tensor multipliers, with
an exhausted per-step table, and for the no-arithmetic twin.  Also checks the
walk each plan picks by itself."""
import dataclasses

import numpy as np
import pytest
import torch

from mixed_precision_zero_amd import binding as B
from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu

RAGGED_SMALL = dataclasses.replace(W.RAGGED, name="ragged_small",
                                   shapes=W.ragged_shapes(300, 12, seed=3), n_micro=3,
                                   hot_tensors=(5, 77, 123), steps=2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import harness  # noqa: F401


def _tiles(st):
    """(tiles, boundary tiles) of a plan's arena, recounted here."""
    T = 256
    ae = int(st.arena_elems)
    n_tiles, n_full = (ae + T - 1) // T, ae // T
    inside = np.zeros(n_tiles, dtype=bool)
    for a, ln in zip(st.arena_off, st.len):
        a, ln = int(a), int(ln)
        if ln == 0:
            continue
        j0, j1 = -(-a // T), (a + ln) // T        # tiles wholly inside [a, a + ln)
        inside[j0:min(j1, n_full)] = True
    return n_tiles, int((~inside).sum())


def _run(w, steps, layout="packed", **kw):
    import harness
    h = harness.Parity(w, layout=layout, walk="arena_tiles", **kw)
    try:
        info = h.st.plan.info
        assert info.adamw_tiles > 0
        assert (info.adamw_tiles, info.boundary_tiles) == _tiles(h.st)
        assert h.plan_matches()
        for _ in range(steps):
            rep = h.step()
            harness.log(f"[arena] {w.name} t={rep.step}: tiles={info.adamw_tiles} "
                        f"boundary={info.boundary_tiles} not_bitexact={rep.not_bitexact}")
            harness.assert_report(rep)
        assert h.canaries_intact()
        assert h.weights_outside_slices_intact()
    finally:
        h.close()


def test_tiny_arena_tiles():
    _run(W.TINY, 3)


def test_ragged_small_arena_tiles():
    _run(RAGGED_SMALL, 2, ranges=[(0, 3)])


def test_ragged_full_arena_tiles():
    """4096 tensors, 533 empty and 181 single-element slices: 2832 boundary
    tiles with their segments."""
    _run(W.RAGGED, 2, ranges=[(0, 16)])


# Full-size bf16 tensors on the arena walk: the fp32 streams at arena
# positions, each tile's bf16 store through its tensor's entry of the
# per-tensor table; weights outside the rank's slices untouched.
def test_full_layout_tiny_arena_tiles():
    _run(W.TINY, 3, layout="full")


def test_full_layout_ragged_small_arena_tiles():
    _run(RAGGED_SMALL, 2, layout="full", ranges=[(0, 1), (1, 3)])


def test_full_layout_dim0_smollm_arena_tiles_with_multipliers():
    w = dataclasses.replace(W.SMOLLM_135M, name="smollm_dim0_full", dp_size=8, rank=5, n_micro=2)
    lr_s, wd_s = W.mup_multipliers(w.shapes, 576)
    _run(w, 2, layout="full", kind="dim0", lr_scale=lr_s, wd_scale=wd_s)


def test_full_layout_llama1p7b_arena_tiles():
    _run(W.LLAMA_1P7B, 2, layout="full", ranges=[(0, 8)])


def test_flat_plan_arena_tiles():
    w = dataclasses.replace(RAGGED_SMALL, name="ragged_small_flat", n_micro=4, hot_tensors=())
    _run(w, 2, kind="flat", ranges=[(0, 4)])


def test_dim0_smollm_arena_tiles_with_multipliers():
    w = dataclasses.replace(W.SMOLLM_135M, name="smollm_dim0", dp_size=8, rank=5, n_micro=2)
    lr_s, wd_s = W.mup_multipliers(w.shapes, 576)
    _run(w, 2, kind="dim0", lr_scale=lr_s, wd_scale=wd_s)


def test_ragged_small_arena_tiles_random_multipliers():
    rng = np.random.default_rng(7)
    n = len(RAGGED_SMALL.shapes)
    _run(RAGGED_SMALL, 2, lr_scale=[float(x) for x in rng.uniform(0.05, 2.0, n)],
         wd_scale=[float(x) for x in rng.choice([0.0, 0.5, 1.0], n)])


# A list whose slices are all whole arena tiles (every numel a multiple of
# dp_size * 256): no boundary tile at all.
TILED = W.Workload(name="tiled", shapes=((1024, 64), (4096,), (512, 512), (2048,), (3072, 8)),
                   dp_size=4, rank=2, n_micro=27, grad_sigma=1e-2, lr=1e-3, weight_decay=0.1,
                   clip=1.0, steps=2)


@pytest.mark.parametrize("ranges", [[(0, 2), (2, 5), (5, 9), (9, 14), (14, 20), (20, 27)],
                                    [(0, 7), (7, 13), (13, 18), (18, 22), (22, 25), (25, 27)]])
def test_narrow_passes_in_a_plan_without_boundary_tiles(ranges):
    """Passes of 2, 3, 4, 5, 6 and 7 resident slots (256-lane chunk kernels)
    in a packed plan whose AdamW takes the arena walk, each pass size as a
    step's first, a middle or its last pass: the oracle's bits."""
    import harness
    h = harness.Parity(TILED, layout="packed", walk="arena_tiles", ranges=ranges)
    try:
        info = h.st.plan.info
        assert info.adamw_tiles > 0 and info.boundary_tiles == 0
        for _ in range(TILED.steps):
            harness.assert_report(h.step())
        assert h.canaries_intact()
    finally:
        h.close()


def test_walks_agree_on_the_same_buffers():
    """The chunk walk and the arena walk over the same buffers store the same
    bits (one step from the same state with each)."""
    from mixed_precision_zero_amd.shard import ShardStep
    w = RAGGED_SMALL
    st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device="cuda", layout="packed",
                   walk="chunks")
    other = None
    try:
        assert st.plan.info.adamw_tiles == 0
        other = B.z1_plan_create(st.numel, w.dp_size, w.rank, st.w_packed, st.g_packed, st.master,
                                 st.exp_avg, st.exp_avg_sq, st.acc, layout="packed",
                                 walk="arena_tiles")
        assert other.info.adamw_tiles > 0
        gen = torch.Generator(device="cuda")
        gen.manual_seed(5)
        for t in (st.master, st.acc, st.exp_avg):
            t.copy_(torch.randn(t.numel(), device="cuda", generator=gen) * 1e-2)
        st.exp_avg_sq.copy_(torch.rand(st.exp_avg_sq.numel(), device="cuda", generator=gen) * 1e-4)
        st.w_packed.fill_(3.0)
        bufs = (st.master, st.exp_avg, st.exp_avg_sq, st.w_packed)
        start = [b.clone() for b in bufs]
        outs = []
        for plan in (st.plan, other):
            for b, s0 in zip(bufs, start):
                b.copy_(s0)
            B.z1_grad_norm_sq_acc(plan, st.d_S)
            B.z1_adamw_step(plan, d_S=st.d_S, step=2, **w.hp())
            torch.cuda.synchronize()
            outs.append([b.clone() for b in bufs])
        for a, b in zip(*outs):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    finally:
        if other is not None:
            other.close()
        st.close()


def test_exhausted_table_stores_nothing():
    """Scheduled AdamW on the arena walk: two rows, then a third call finds
    the table exhausted and stores nothing."""
    from mixed_precision_zero_amd.shard import ShardStep
    w = RAGGED_SMALL
    st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device="cuda", layout="packed",
                   walk="arena_tiles")
    sched = None
    try:
        st.master.normal_(0.0, 0.02)
        st.acc.normal_(0.0, 1e-2)
        sched = B.z1_schedule_create(**w.hp(), step=1, n_steps=2)
        for t in range(3):
            B.z1_grad_norm_sq_acc(st.plan, st.d_S)
            before = [b.clone() for b in (st.master, st.exp_avg, st.exp_avg_sq, st.w_packed)]
            st.adamw_scheduled(sched)
            torch.cuda.synchronize()
            after = (st.master, st.exp_avg, st.exp_avg_sq, st.w_packed)
            same = all(torch.equal(a.view(torch.uint8), b.view(torch.uint8))
                       for a, b in zip(after, before))
            assert same == (t == 2), f"call {t}"
        assert B.z1_schedule_query(sched) == (3, 1)
    finally:
        if sched is not None:
            sched.close()
        st.close()


def test_twin_touches_exactly_the_slices():
    """The no-arithmetic twin (z1_probe_plan) on the arena walk adds acc to
    every slice element of master and leaves the padding between slices
    alone."""
    from mixed_precision_zero_amd.shard import ShardStep
    w = dataclasses.replace(RAGGED_SMALL, shapes=((7, 33), (5,), (3, 1000), (1,), (4100,), (9000,)),
                            dp_size=3, rank=1)
    st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device="cuda", arena_pad=64,
                   layout="packed", walk="arena_tiles")
    try:
        canary = float.fromhex("0x1.5a5a5ap+77")
        for a in (st.master, st.exp_avg, st.exp_avg_sq, st.acc):
            a.fill_(canary)
        used = torch.zeros(st.master.numel(), dtype=torch.bool, device="cuda")
        for _, _, ln, off in st.slices():
            used[off:off + ln] = True
        n = int(used.sum())
        st.master[used] = torch.arange(n, device="cuda", dtype=torch.float32)
        st.acc[used] = 0.5
        for a in (st.exp_avg, st.exp_avg_sq):
            a[used] = 1.0
        B.z1_probe_plan(st.plan)
        torch.cuda.synchronize()
        assert torch.equal(st.master[used], torch.arange(n, device="cuda", dtype=torch.float32) + 0.5)
        for a in (st.master, st.exp_avg, st.exp_avg_sq, st.acc):
            assert bool((a[~used] == canary).all())
    finally:
        st.close()


@pytest.mark.parametrize("w,expect_tiles", [(W.LLAMA_7B, True), (W.RAGGED, True),
                                            (W.TINY, False)], ids=["llama7b", "ragged", "tiny"])
def test_automatic_walk(w, expect_tiles):
    """A plan takes the arena walk by itself when at most 1% of its tiles
    cross a slice boundary, with packed shards and with full-size tensors
    alike."""
    from mixed_precision_zero_amd.shard import ShardStep
    st = ShardStep(w.shapes, w.dp_size, w.rank, 1, device="cuda", layout="packed")
    try:
        n_tiles, n_boundary = _tiles(st)
        assert (n_boundary * 100 <= n_tiles) == expect_tiles
        assert st.plan.info.adamw_tiles == (n_tiles if expect_tiles else 0)
        assert st.plan.info.boundary_tiles == (n_boundary if expect_tiles else 0)
    finally:
        st.close()
    full = ShardStep(w.shapes, w.dp_size, w.rank, 1, device="cuda")
    try:
        assert full.plan.info.adamw_tiles == (n_tiles if expect_tiles else 0)
    finally:
        full.close()
