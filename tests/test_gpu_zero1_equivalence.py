"""The ZeRO-1 identity on one GPU: the D ranks' shard steps, each on its own
plan over the same full tensors and given the global S (what an exact
all-reduce of S would deliver), reproduce the unsharded step (dp = 1) bit
for bit.  Every rank's master, m and v equal the unsharded ones restricted
to its slices, and the bf16 slices the ranks write in place form the full
weights the all-gather would distribute.  Σ_r S_r equals the global S up
to the rounding of each S_r ("Distributed Training", ZeRO-1: each rank
keeps its slice of the optimizer state and the step is unchanged)."""
import dataclasses

import pytest
import torch

from mixed_precision_zero_amd import binding as B
from mixed_precision_zero_amd import workloads as W
from mixed_precision_zero_amd.shard import ShardStep

pytestmark = pytest.mark.gpu

CASES = [
    (dataclasses.replace(W.SMOLLM_135M, name="smollm_dp8", dp_size=8, n_micro=2), "per_tensor"),
    (dataclasses.replace(W.SMOLLM_135M, name="smollm_dp8_dim0", dp_size=8, n_micro=2), "dim0"),
    (dataclasses.replace(W.RAGGED, name="ragged_small_dp7", shapes=W.ragged_shapes(300, 12, seed=9),
                         n_micro=3, hot_tensors=(4, 40)), "flat"),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("w,kind", CASES, ids=[f"{w.name}-{k}" for w, k in CASES])
def test_ranks_compose_to_the_unsharded_step(w, kind):
    dev = torch.device("cuda")
    D, K = w.dp_size, w.n_micro
    bf = dict(dtype=torch.bfloat16, device=dev)
    grads = [[torch.empty(s, **bf) for s in w.shapes] for _ in range(K)]
    w_ranks = [torch.zeros(s, **bf) for s in w.shapes]        # written slice by slice
    ref = ShardStep(w.shapes, 1, 0, K, device=dev, grads=grads, kind=kind)
    ranks = [ShardStep(w.shapes, D, r, K, device=dev, grads=grads, weights=w_ranks, kind=kind)
             for r in range(D)]
    try:
        # the D plans partition every tensor
        for i, n in enumerate(ref.numel):
            covered = sorted((int(st.start[i]), int(st.len[i])) for st in ranks if st.len[i])
            pos = 0
            for s, ln in covered:
                assert s == pos
                pos += ln
            assert pos == n
        master = W.make_master(w, seed=0, device=dev)
        for st in [ref] + ranks:
            st.scatter_to_arena(st.master, master)
            st.load_weights(master)
        hp = w.hp()
        for t in (1, 2, 3):
            for k in range(K):
                W.make_micro_grads(w, t, k, seed=0, device=dev, out=grads[k])
            ref.step(hp)
            S_sum = torch.zeros(1, dtype=torch.float64, device=dev)
            for st in ranks:
                st.accumulate_range(0, K)
                st.norm()
                S_sum += st.d_S
                # every rank clips with the global S, as after an all-reduce
                B.z1_adamw_step(st.plan, d_S=ref.d_S, step=t, **hp)
            torch.cuda.synchronize()
            S_ref = float(ref.d_S.item())
            assert abs(float(S_sum.item()) - S_ref) <= 1e-14 * S_ref
        # the state after 3 steps, slice by slice
        for st in ranks:
            for i, s, ln, off in st.slices():
                if not ln:
                    continue
                o_ref = int(ref.arena_off[i]) + s
                for name in ("master", "exp_avg", "exp_avg_sq", "acc"):
                    a = getattr(st, name)[off:off + ln].view(torch.int32)
                    b = getattr(ref, name)[o_ref:o_ref + ln].view(torch.int32)
                    assert torch.equal(a, b), f"rank {st.rank} tensor {i} {name}"
        for i in range(len(w.shapes)):
            assert torch.equal(w_ranks[i].view(torch.int16), ref.weights[i].view(torch.int16)), \
                f"tensor {i}: the ranks' bf16 slices do not form the unsharded weights"
    finally:
        ref.close()
        for st in ranks:
            st.close()
