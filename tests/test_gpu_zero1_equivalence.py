"""The ZeRO-1 identity on one GPU: the D ranks' shard steps, each on its own
plan over the same full tensors, reproduce the unsharded step (dp = 1) bit
for bit ("Distributed Training", ZeRO-1: each rank keeps its slice of the
optimizer state and the step is unchanged).  The ranks exchange their norm
as unrounded pairs (z1_grad_norm_sq_pair; the [D][2] array stands in for
the all-gather) and z1_norm_combine gives every rank the same S, equal to
the unsharded S.  Every rank's master, m, v and acc equal the unsharded ones
restricted to its slices, and the bf16 slices the ranks write in place form
the full weights the all-gather would distribute."""
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
        f64 = dict(dtype=torch.float64, device=dev)
        pairs = torch.zeros(D, 2, **f64)      # row r: rank r's (hi, lo), 16-byte aligned
        ref_pair = torch.zeros(2, **f64)
        S_one = torch.zeros(1, **f64)
        S_global = torch.zeros(1, **f64)
        master = W.make_master(w, seed=0, device=dev)
        for st in [ref] + ranks:
            st.scatter_to_arena(st.master, master)
            st.load_weights(master)
        hp = w.hp()
        for t in (1, 2, 3):
            for k in range(K):
                W.make_micro_grads(w, t, k, seed=0, device=dev, out=grads[k])
            ref.accumulate_range(0, K)
            B.z1_grad_norm_sq_pair(ref.plan, ref_pair)
            B.z1_norm_combine(ref_pair, 1, S_one)
            ref.norm()
            ref.adamw(hp, step=t)
            for r, st in enumerate(ranks):
                st.accumulate_range(0, K)
                B.z1_grad_norm_sq_pair(st.plan, pairs[r])
            B.z1_norm_combine(pairs, D, S_global)
            for st in ranks:
                B.z1_adamw_step(st.plan, d_S=S_global, step=t, **hp)
            torch.cuda.synchronize()
            S_ref = ref.d_S.item()
            assert S_one.item() == S_ref, "one pair combined differs from z1_grad_norm_sq"
            assert S_global.item() == S_ref, (t, S_global.item(), S_ref)
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
