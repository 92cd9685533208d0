"""GPU parity at hyperparameter corners of the binary64 update: beta = 0,
lr = 0, a negative lr, wd = 0, eps = 1, beta2 next to 1, a clip so small
that every clipped square underflows the fp32 store of v, a clip and an eps
so small that m lies below 2^-960 (the bias correction of m then takes the
IEEE division instead of the reciprocal with exact remainders) while the
update still moves the weights, and clipping off.
Each runs three steps on a 300-tensor ragged list (K = 3), bit-exact against
the oracle: the GPU evaluates the same IEEE operation sequence whatever the
constants are."""
import dataclasses

import pytest
import torch

from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu

BASE = dataclasses.replace(W.RAGGED, name="ragged_corners", shapes=W.ragged_shapes(300, 14, seed=9),
                           n_micro=3, hot_tensors=(4, 77), steps=3)

CORNERS = {
    "betas_zero": dict(beta1=0.0, beta2=0.0),
    "lr_zero": dict(lr=0.0),
    "lr_negative": dict(lr=-1e-3),
    "wd_zero": dict(weight_decay=0.0),
    "eps_one": dict(eps=1.0),
    "beta2_near_one": dict(beta2=0.999999),
    "clip_tiny": dict(clip=1e-30),
    "clip_eps_below_2e-960": dict(clip=1e-300, eps=1e-300, lr=1.0),
    "clip_off": dict(clip=0.0),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", sorted(CORNERS))
def test_hyperparameter_corner_bitexact(name):
    import harness
    w = dataclasses.replace(BASE, **CORNERS[name])
    h = harness.Parity(w)
    try:
        assert h.plan_matches()
        for _ in range(w.steps):
            rep = h.step()
            harness.log(f"[corner] {name} t={rep.step}: S_rel={rep.S_rel:.2e} "
                        f"not_bitexact={rep.not_bitexact}")
            harness.assert_report(rep)
        assert h.canaries_intact()
        assert h.weights_outside_slices_intact()
    finally:
        h.close()
