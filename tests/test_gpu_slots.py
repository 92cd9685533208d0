"""GPU parity of multi-slot accumulation (z1_accum_grads_range,
z1_pack_accum_range): several resident micro-batch gradients read in one pass.
The bar is the one of the single-slot path: acc and S bit-exact against the
oracle, the whole step bit-exact, since the binary32 additions happen in the
same order."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_zero_amd import binding as B
from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import harness  # noqa: F401


def _run(w, steps, ranges, **kw):
    import harness
    h = harness.Parity(w, ranges=ranges, **kw)
    try:
        assert h.plan_matches()
        for _ in range(steps):
            rep = h.step()
            harness.log(f"[slots] {w.name} ranges={ranges} t={rep.step}: S_rel={rep.S_rel:.2e} "
                        f"not_bitexact={rep.not_bitexact}")
            harness.assert_report(rep)
        assert h.canaries_intact()
        assert h.weights_outside_slices_intact()
    finally:
        h.close()


def test_tiny_two_slots_one_pass():
    _run(W.TINY, 3, [(0, 2)])


def test_tiny_eleven_slots_one_pass_small_chunks():
    """K = 11 in one pass; 1024-element chunks on 3 workgroups."""
    w = dataclasses.replace(W.TINY, name="tiny_k11", n_micro=11)
    _run(w, 2, [(0, 11)], chunk_elems=1024, max_blocks=3)


def test_tiny_fifteen_slots_wide_pass():
    """K = 15 in one pass (the two-vectors-per-lane form), on 1024-element
    chunks so every workgroup loops and takes partial vectors."""
    w = dataclasses.replace(W.TINY, name="tiny_k15", n_micro=15, shapes=((257, 63), (61,), (1030,)))
    _run(w, 2, [(0, 15)], chunk_elems=1024)


# the full-size layout on the chunk table, and packed shards with the arena
# walk forced (single and wide passes then run on the arena kernels; the
# list's slices leave most 256-element tiles on slice boundaries)
WALKS = {"chunks": {}, "arena": dict(layout="packed", walk="arena_tiles")}


@pytest.mark.parametrize("walk", list(WALKS))
@pytest.mark.parametrize("K,ranges", [
    (33, [(0, 33)]),                     # three passes of 11 slots
    (64, [(0, 64)]),                     # four passes of 16 slots
    (37, [(0, 3), (3, 20), (20, 37)]),   # three calls: 3; 9 + 8; 9 + 8 slots
], ids=["k33", "k64", "k37_three_calls"])
def test_tiny_many_slots_many_passes(K, ranges, walk):
    """Many resident micro-batches: a range longer than 16 slots is split into
    as many passes as it needs, of nearly equal size; every split stores the
    bits of one call per micro-batch (the oracle's in-order binary32 sum)."""
    w = dataclasses.replace(W.TINY, name=f"tiny_k{K}", n_micro=K,
                            shapes=((257, 63), (61,), (1030,)))
    _run(w, 2, ranges, chunk_elems=1024, **WALKS[walk])


def _wide_pass_partitions(K):
    """Per step, the ranges of one step's calls: every pass size from 9 to 16
    once as a step's first pass (it overwrites acc), once between two other
    passes, and once as the last (it also writes the norm partials)."""
    steps = []
    for g in range(9, 17):
        steps.append([(0, g), (g, K)])
        steps.append([(0, 1), (1, 1 + g), (1 + g, K)])
        steps.append([(0, K - g), (K - g, K)])
    return steps


@pytest.mark.parametrize("walk", list(WALKS))
def test_tiny_wide_passes_every_size_and_position(walk):
    """K = 18 on 1024-element chunks: each of the 9- to 16-slot passes as the
    first, a middle and the last pass of a step, 24 steps in a row, every step
    bit-exact against the oracle."""
    import harness
    K = 18
    w = dataclasses.replace(W.TINY, name="tiny_k18", n_micro=K, shapes=((257, 63), (61,), (1030,)))
    steps = _wide_pass_partitions(K)
    h = harness.Parity(w, ranges=steps[0], chunk_elems=1024, **WALKS[walk])
    try:
        assert h.plan_matches()
        for ranges in steps:
            h.ranges = ranges
            rep = h.step()
            harness.log(f"[slots] {w.name} ranges={ranges} t={rep.step}: "
                        f"not_bitexact={rep.not_bitexact}")
            harness.assert_report(rep)
        assert h.canaries_intact()
        assert h.weights_outside_slices_intact()
    finally:
        h.close()


def test_ragged_small_three_slots():
    shapes = W.ragged_shapes(300, 12, seed=3)
    w = dataclasses.replace(W.RAGGED, name="ragged_small", shapes=shapes, n_micro=3,
                            hot_tensors=(5, 77, 123), steps=2)
    _run(w, 2, [(0, 3)])


def test_smollm_mixed_single_and_multi_calls():
    """Single-slot calls around a two-slot range: 1 + 2 + 1 slots."""
    _run(W.SMOLLM_135M, 2, [(0, 1), (1, 3), (3, 4)])


def test_plan_flat_ragged_small_range():
    shapes = W.ragged_shapes(300, 12, seed=4)
    w = dataclasses.replace(W.RAGGED, name="ragged_small_flat", shapes=shapes, n_micro=5,
                            hot_tensors=(), steps=2)
    _run(w, 2, [(0, 2), (2, 5)], kind="flat")


def test_ragged_full_sixteen_slots():
    """K = 16 in one pass; 533 empty and 181 single-element slices."""
    _run(W.RAGGED, 2, [(0, 16)])


def test_llama1p7b_eight_slots():
    _run(W.LLAMA_1P7B, 2, [(0, 8)])


def test_llama7b_four_slots():
    """The benchmarked workload with all K = 4 slots in one pass, every
    element compared."""
    _run(W.LLAMA_7B, 1, [(0, 4)], canaries=False)


def test_range_call_order():
    from mixed_precision_zero_amd.shard import ShardStep
    w = dataclasses.replace(W.TINY, n_micro=4)
    st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device="cuda")
    try:
        for a, b in ((0, 0), (2, 1), (-1, 2), (0, 5)):
            with pytest.raises(B.Z1Error, match="EINVAL"):
                st.accumulate_range(a, b)
        with pytest.raises(B.Z1Error, match="ESTATE"):
            st.accumulate_range(1, 3)          # nothing accumulated yet
        st.accumulate_range(0, 2)
        with pytest.raises(B.Z1Error, match="ESTATE"):
            st.norm()                           # slots 2, 3 missing
        with pytest.raises(B.Z1Error, match="ESTATE"):
            st.accumulate_range(3, 4)           # slot 2 skipped
        st.accumulate(2)
        st.accumulate_range(3, 4)
        st.norm()
        st.adamw(w.hp())
        torch.cuda.synchronize()
    finally:
        st.close()


PACK_CASES = [
    (dataclasses.replace(W.TINY, name="tiny_k5", n_micro=5), "per_tensor", True, [(0, 5)]),
    (dataclasses.replace(W.RAGGED, name="ragged_small", shapes=W.ragged_shapes(300, 12, seed=6),
                         n_micro=3, hot_tensors=()), "flat", True, [(0, 1), (1, 3)]),
    (dataclasses.replace(W.SMOLLM_135M, dp_size=8, rank=0), "per_tensor", False, [(0, 4)]),
    (dataclasses.replace(W.SMOLLM_135M, dp_size=7, rank=0, n_micro=9), "dim0", True, [(0, 9)]),
    (dataclasses.replace(W.TINY, name="tiny_k18", n_micro=18), "per_tensor", True, [(0, 18)]),
    (dataclasses.replace(W.TINY, name="tiny_k16", n_micro=16), "flat", True, [(0, 1), (1, 16)]),
    (dataclasses.replace(W.TINY, name="tiny_k12", n_micro=12), "per_tensor", True, [(0, 12)]),
]


@pytest.mark.parametrize("w,kind,divide,ranges", PACK_CASES,
                         ids=[f"{c[0].name}-{c[1]}-{c[3]}" for c in PACK_CASES])
def test_pack_range_bitexact(w, kind, divide, ranges):
    import test_gpu_pack as P
    o = oracle.get()
    rows = P._rows(w, kind)
    seg = B.z1_pack_layout(w.numel, w.dp_size, kind, rows)
    send = torch.full((w.dp_size * seg + 16,), P.CANARY, dtype=torch.float32, device="cuda")
    grads = P._grads(w)
    pack = B.z1_pack_create(w.numel, w.dp_size, grads, send, kind=kind, rows=rows, divide=divide)
    try:
        for a, b in ranges:
            B.z1_pack_accum_range(pack, a, b)
        torch.cuda.synchronize()
        got, used = P._packed_from_send(w, kind, send, seg)
        g = np.stack([P._host_full(gk) for gk in grads])
        ref = o.pack_send(w.numel, rows, kind, w.dp_size, o.accumulate(g), divide)
        assert got.shape == ref.shape
        assert (got.view(np.uint32) == ref.view(np.uint32)).all()
        assert bool((send[~used] == P.CANARY).all())
    finally:
        pack.close()
