"""z1_grad_norm_sq_flat_noalloc (the entry point that allocates nothing)
against the existing entry point it varies, z1_grad_norm_sq_acc, through the
C ABI: two calls in a row on one GPU's shared scratch array, the second on a
smaller input, each S bit for bit equal to the plan's S (and within the norm
tolerance of 1e-5) and equal to the oracle's S of the same elements."""
import dataclasses

import numpy as np
import pytest
import torch

from mixed_precision_zero_amd import binding as B
from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _plan_with_acc(w, seed):
    """A plan over workload w with a seeded acc arena (padding set to NaN,
    which no norm may read), and the acc shard in packed order."""
    from mixed_precision_zero_amd.shard import ShardStep
    st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device="cuda", arena_pad=64)
    st.acc.fill_(float("nan"))
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for _, _, ln, off in st.slices():
        if ln:
            st.acc[off:off + ln] = torch.randn(ln, generator=g, device="cuda") * 1e-2
    return st, st.packed(st.acc).contiguous()


def _check_same_S(st, flat, n):
    import oracle
    d_ref = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
    d_new = torch.full((1,), -2.0, dtype=torch.float64, device="cuda")
    B.z1_grad_norm_sq_acc(st.plan, d_ref)
    B.z1_grad_norm_sq_flat_noalloc(flat, n, d_new)
    torch.cuda.synchronize()
    S_ref, S_new = float(d_ref.item()), float(d_new.item())
    S_oracle = oracle.get().norm_sq(flat[:n].cpu().numpy())
    assert abs(S_new - S_ref) <= 1e-5 * S_ref
    assert S_new == S_ref, (S_new, S_ref)
    assert S_new == S_oracle, (S_new, S_oracle)
    return S_new


RAGGED_MID = dataclasses.replace(W.RAGGED, name="ragged_mid", shapes=W.ragged_shapes(400, 18, seed=5),
                                 n_micro=1, hot_tensors=())


def test_two_calls_in_a_row_second_smaller():
    big, flat_big = _plan_with_acc(RAGGED_MID, seed=1)     # several thousand tiles, ragged tail
    small, flat_small = _plan_with_acc(W.TINY, seed=2)     # 2 whole tiles and an 80-element tail
    try:
        n_big, n_small = flat_big.numel(), flat_small.numel()
        assert n_big > 100 * n_small and n_small % 4096 == 80
        S1 = _check_same_S(big, flat_big, n_big)
        S2 = _check_same_S(small, flat_small, n_small)
        assert S1 != S2
    finally:
        big.close()
        small.close()


def test_edge_sizes_and_rejections():
    x = torch.randn(3 * 4096 + 5, device="cuda", dtype=torch.float32)
    d_S = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
    for n in (0, 1, 3, 4, 4096, 4097, 2 * 4096, 3 * 4096 + 5):
        B.z1_grad_norm_sq_flat_noalloc(x, n, d_S)
        torch.cuda.synchronize()
        xs = x[:n].double()
        exact = float(torch.sum(xs * xs).item()) if n else 0.0
        got = float(d_S.item())
        assert abs(got - exact) <= 1e-12 * max(exact, 1e-300), (n, got, exact)
    # beyond the stated maximum: refused on the host, nothing enqueued
    d_S.fill_(-7.0)
    rc = B.lib.z1_grad_norm_sq_flat_noalloc(x.data_ptr(), B.NORM_FLAT_MAX_ELEMS + 1,
                                           d_S.data_ptr(), None)
    assert rc == B.Z1_EINVAL
    host = np.zeros(8, np.float32)
    assert B.lib.z1_grad_norm_sq_flat_noalloc(host.ctypes.data, 8, d_S.data_ptr(),
                                              None) == B.Z1_EINVAL
    torch.cuda.synchronize()
    assert float(d_S.item()) == -7.0
