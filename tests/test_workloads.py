"""Parameter-list sizes and shard sizes of the synthetic workloads."""
import numpy as np
import pytest

import oracle
from mixed_precision_zero_amd import workloads as W

EXPECT = {
    # name: (tensors, params, shard elements on the stated rank)
    "tiny": (4, 33_088, 8_272),
    "smollm135m": (272, 134_515_008, 134_515_008),
    "llama1p7b": (218, 1_711_376_384, 213_922_048),
    "llama7b": (291, 6_738_415_616, 842_301_952),
    "ragged": (4096, 1_091_452_319, 155_920_055),
}


@pytest.mark.parametrize("name", sorted(EXPECT))
def test_sizes(name):
    w = W.WORKLOADS[name]
    n_t, psi, L = EXPECT[name]
    assert len(w.shapes) == n_t
    assert w.total_params == psi
    _, ln = oracle.get().shard_plan(w.numel, w.dp_size, w.rank)
    assert int(ln.sum()) == L


def test_ragged_edges():
    w = W.RAGGED
    _, ln = oracle.get().shard_plan(w.numel, w.dp_size, w.rank)
    assert int((ln == 0).sum()) == 533 and int((ln == 1).sum()) == 181
    assert len(w.hot_tensors) == 41


def test_generators_are_seeded():
    w = W.TINY
    a = W.make_micro_grads(w, 1, 0, seed=0)
    b = W.make_micro_grads(w, 1, 0, seed=0)
    c = W.make_micro_grads(w, 1, 1, seed=0)
    assert all(x.equal(y) for x, y in zip(a, b))
    assert not all(x.equal(y) for x, y in zip(a, c))
    m = W.make_master(w)
    assert abs(float(np.std(np.concatenate([t.reshape(-1).numpy() for t in m]))) - 0.02) < 1e-3
