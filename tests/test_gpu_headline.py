"""The headline configuration at its stated length: the 7B Llama-shaped
shard (dp_size 8, rank 3, K = 4) for all 20 steps, in the form the benchmark
times (all K resident gradient slots in one accumulation call, bf16 weights
and gradients as packed shards), every element of every step compared with
the oracle.  About three minutes on one MI355X, most of it the host-side
oracle and the copies it compares; the steps run as five tests of four steps
over one module-wide state, so the run reports progress as it goes."""
import pytest
import torch

from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu

STEP_BLOCKS = [(1, 4), (5, 8), (9, 12), (13, 16), (17, 20)]


@pytest.fixture(scope="module")
def headline():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import harness
    w = W.LLAMA_7B
    assert w.steps == 20 and STEP_BLOCKS[-1][1] == w.steps
    h = harness.Parity(w, canaries=True, ranges=[(0, w.n_micro)], layout="packed")
    h.next_step = 1
    try:
        assert h.plan_matches()
        yield h
    finally:
        h.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("first,last", STEP_BLOCKS)
def test_llama7b_all_twenty_steps_resident(headline, first, last):
    """Steps first..last of the 20; acc, S, master, m, v and the bf16 weights
    bit for bit against the oracle at every step (on top of the stated
    tolerances).  Each block continues the state the previous one left."""
    import harness
    h = headline
    assert h.next_step == first, "an earlier block of steps did not complete"
    for t in range(first, last + 1):
        rep = h.step()
        assert rep.step == t
        harness.log(f"[headline] {h.w.name} t={rep.step}: S_rel={rep.S_rel:.2e} "
                    f"not_bitexact={rep.not_bitexact}")
        harness.assert_report(rep)
        h.next_step = t + 1
    if last == h.w.steps:
        assert h.canaries_intact()
