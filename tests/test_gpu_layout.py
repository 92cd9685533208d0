"""GPU parity with the packed bf16 layout (Z1_LAYOUT_PACKED): the weights and
each micro-batch gradient are one packed shard in arena order instead of
full-size tensors.  Same bars as the full layout (bit-exact against the
oracle), plus: the packed weight buffer's padding is never written."""
import dataclasses

import pytest
import torch

from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import harness  # noqa: F401


def _run(w, steps, **kw):
    import harness
    h = harness.Parity(w, layout="packed", **kw)
    try:
        assert h.plan_matches()
        for _ in range(steps):
            rep = h.step()
            harness.log(f"[packed] {w.name} t={rep.step}: S_rel={rep.S_rel:.2e} "
                        f"not_bitexact={rep.not_bitexact}")
            harness.assert_report(rep)
        assert h.canaries_intact()
    finally:
        h.close()


def test_tiny_packed():
    _run(W.TINY, 3)


def test_ragged_small_packed_small_chunks():
    shapes = W.ragged_shapes(300, 12, seed=3)
    w = dataclasses.replace(W.RAGGED, name="ragged_small", shapes=shapes, n_micro=3,
                            hot_tensors=(5, 77, 123), steps=2)
    _run(w, 2, chunk_elems=1024, max_blocks=5)


def test_empty_shard_packed():
    w = dataclasses.replace(W.TINY, name="empty", shapes=((3,), (1,), (5,)), dp_size=8, rank=7)
    _run(w, 2)


def test_plan_flat_packed_resident():
    shapes = W.ragged_shapes(300, 12, seed=4)
    w = dataclasses.replace(W.RAGGED, name="ragged_small_flat", shapes=shapes, n_micro=4,
                            hot_tensors=(), steps=2)
    _run(w, 2, kind="flat", ranges=[(0, 4)])


def test_plan_dim0_smollm_packed():
    w = dataclasses.replace(W.SMOLLM_135M, name="smollm_dim0", dp_size=8, rank=5, n_micro=2)
    _run(w, 2, kind="dim0")


def test_llama1p7b_packed_resident():
    _run(W.LLAMA_1P7B, 2, ranges=[(0, 8)])


def test_llama7b_packed_resident():
    """The benchmarked shard with packed bf16 buffers, every element compared."""
    _run(W.LLAMA_7B, 1, ranges=[(0, 4)], canaries=False)
