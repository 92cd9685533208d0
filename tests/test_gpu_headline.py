"""The headline configuration at its stated length: the 7B Llama-shaped
shard (dp_size 8, rank 3, K = 4) for all 20 steps, in the form the benchmark
times (all K resident gradient slots in one accumulation call, bf16 weights
and gradients as packed shards), every element of every step compared with
the oracle.  About three minutes on one MI355X, most of it the host-side
oracle and the copies it compares."""
import pytest
import torch

from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.timeout(900)
def test_llama7b_all_twenty_steps_resident():
    """20 steps; acc, S, master, m, v and the bf16 weights bit for bit against
    the oracle at every step (on top of the stated tolerances)."""
    import harness
    w = W.LLAMA_7B
    assert w.steps == 20
    h = harness.Parity(w, canaries=True, ranges=[(0, w.n_micro)], layout="packed")
    try:
        assert h.plan_matches()
        for _ in range(w.steps):
            rep = h.step()
            harness.log(f"[headline] {w.name} t={rep.step}: S_rel={rep.S_rel:.2e} "
                        f"not_bitexact={rep.not_bitexact}")
            harness.assert_report(rep)
        assert h.canaries_intact()
    finally:
        h.close()
