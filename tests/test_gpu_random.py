"""Seeded random configurations against the oracle, bit for bit.

Each case draws a parameter list (1-D and 2-D tensors, including empty ones
and single elements), dp size and rank, K, plan kind, bf16 layout, chunk
size, grid cap, how the K accumulations are grouped into calls, per-tensor
multipliers, clip and the gradient scale, then runs two steps through the
C ABI and compares every element with the oracle (the bars of
test_gpu_parity, bit-exact)."""
import os

import numpy as np
import pytest
import torch

from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu
N_CASES = int(os.environ.get("Z1_RANDOM_CASES", "160"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import harness  # noqa: F401


def random_case(i: int):
    rng = np.random.default_rng(1000 + i)
    shapes = []
    for _ in range(int(rng.integers(1, 40))):
        u = rng.random()
        if u < 0.05:
            shapes.append((0,) if rng.random() < 0.5 else (int(rng.integers(1, 9)), 0))
        elif u < 0.55:
            shapes.append((int(2 ** rng.uniform(0, 15)),))
        else:
            shapes.append((int(rng.integers(1, 300)), int(rng.integers(1, 200))))
    dp = int(rng.integers(1, 10))
    K = int(rng.integers(1, 11))
    n = len(shapes)
    if rng.random() < 0.4:
        ranges = None                                   # one call per micro-batch
    else:
        cuts = sorted(set(int(x) for x in rng.integers(1, K, size=int(rng.integers(0, 3))))) if K > 1 else []
        b = [0] + cuts + [K]
        ranges = [(b[j], b[j + 1]) for j in range(len(b) - 1)]
    w = W.Workload(name=f"random{i}", shapes=tuple(shapes), dp_size=dp,
                   rank=int(rng.integers(0, dp)), n_micro=K,
                   grad_sigma=float(10 ** rng.uniform(-4, 0)),
                   lr=float(10 ** rng.uniform(-5, -2)),
                   weight_decay=float(rng.choice([0.0, 0.01, 0.1])),
                   clip=float(rng.choice([1.0, 1.0, 0.0, 1e-3, 1e3])), steps=2)
    kw = dict(kind=str(rng.choice(["per_tensor", "flat", "dim0"])),
              layout=str(rng.choice(["full", "packed"])),
              chunk_elems=int(rng.choice([0, 1024, 2048])),
              max_blocks=int(rng.choice([0, 0, 1, 3, 64])), ranges=ranges)
    if rng.random() < 0.3:
        kw["lr_scale"] = [float(x) for x in rng.uniform(0.1, 2.0, n)]
        kw["wd_scale"] = [float(x) for x in rng.choice([0.0, 1.0], n)]
    # AdamW's walk, from a stream of its own (the draws above stay as they were);
    # both layouts take the arena walk when asked, and under AUTO when boundaries are rare
    if kw["max_blocks"] == 0:
        kw["walk"] = str(np.random.default_rng(5000 + i).choice(["auto", "chunks", "arena_tiles"]))
    return w, kw


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration_bitexact(i):
    import harness
    w, kw = random_case(i)
    harness.log(f"[random] case {i}: n={len(w.shapes)} dp={w.dp_size} rank={w.rank} K={w.n_micro} "
                f"{ {k: v for k, v in kw.items() if k not in ('lr_scale', 'wd_scale')} } "
                f"clip={w.clip} scales={'lr_scale' in kw}")
    h = harness.Parity(w, **kw)
    try:
        assert h.plan_matches()
        for _ in range(w.steps):
            harness.assert_report(h.step())
        assert h.canaries_intact()
        assert h.weights_outside_slices_intact()
    finally:
        h.close()
