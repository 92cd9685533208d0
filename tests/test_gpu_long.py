"""Long GPU parity runs (minutes), kept out of -m gpu and selected with
-m gpu_long: the configurations' full step counts on the 7B shard."""
import pytest
import torch

from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu_long


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_llama7b_all_twenty_steps_resident():
    """The configuration's 20 steps on the 7B shard in the benchmarked form
    (all K slots in one accumulation call), every element of every step
    compared against the oracle, bit for bit."""
    import harness
    w = W.LLAMA_7B
    h = harness.Parity(w, canaries=False, ranges=[(0, w.n_micro)])
    try:
        assert h.plan_matches()
        for _ in range(w.steps):
            rep = h.step()
            harness.log(f"[long] {w.name} t={rep.step}: S_rel={rep.S_rel:.2e} "
                        f"not_bitexact={rep.not_bitexact}")
            harness.assert_report(rep)
    finally:
        h.close()
