"""GPU parity of the step before the shard path: full-tensor accumulation into
the reduce-scatter send buffer (z1_pack_*), and the norm of an acc arena the
caller filled (z1_grad_norm_sq_acc), against the CPU oracle, bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_zero_amd import binding as B
from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu
CANARY = float.fromhex("0x1.5a5a5ap+77")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _rows(w, kind):
    return [s[0] for s in w.shapes] if kind == "dim0" else None


def _packed_from_send(w, kind, send, seg):
    """The GPU send buffer read back in packed (oracle) order, plus the mask of
    every element it wrote."""
    parts, used = [], torch.zeros(send.numel(), dtype=torch.bool, device=send.device)
    for r in range(w.dp_size):
        start, ln, off, _ = B.z1_shard_plan(w.numel, w.dp_size, r, kind=kind, rows=_rows(w, kind))
        for i in range(len(w.numel)):
            if ln[i]:
                a = r * seg + int(off[i])
                parts.append(send[a:a + int(ln[i])])
                used[a:a + int(ln[i])] = True
    x = torch.cat(parts).cpu().numpy() if parts else np.zeros(0, np.float32)
    return x, used


def _grads(w, step=1):
    out = []
    for k in range(w.n_micro):
        gk = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in w.shapes]
        W.make_micro_grads(w, step, k, seed=0, device="cuda", out=gk)
        out.append(gk)
    return out


def _host_full(gk):
    return torch.cat([x.reshape(-1) for x in gk]).view(torch.int16).cpu().numpy().view(np.uint16)


CASES = [
    (W.TINY, "per_tensor", True),
    (W.TINY, "dim0", False),
    (dataclasses.replace(W.RAGGED, name="ragged_small", shapes=W.ragged_shapes(300, 12, seed=6),
                         n_micro=3, hot_tensors=()), "flat", True),
    (dataclasses.replace(W.SMOLLM_135M, dp_size=8, rank=0), "per_tensor", True),
    (dataclasses.replace(W.SMOLLM_135M, dp_size=7, rank=0, n_micro=2), "dim0", True),
]


@pytest.mark.parametrize("w,kind,divide", CASES,
                         ids=[f"{w.name}-{k}-{'div' if d else 'sum'}" for w, k, d in CASES])
def test_pack_send_bitexact(w, kind, divide):
    o = oracle.get()
    seg = B.z1_pack_layout(w.numel, w.dp_size, kind, _rows(w, kind))
    send = torch.full((w.dp_size * seg + 16,), CANARY, dtype=torch.float32, device="cuda")
    grads = _grads(w)
    pack = B.z1_pack_create(w.numel, w.dp_size, grads, send, kind=kind, rows=_rows(w, kind),
                            divide=divide)
    for k in range(w.n_micro):
        B.z1_pack_accum(pack, k)
    torch.cuda.synchronize()
    got, used = _packed_from_send(w, kind, send, seg)
    g = np.stack([_host_full(gk) for gk in grads])
    acc_full = o.accumulate(g)
    want = o.pack_send(w.numel, _rows(w, kind), kind, w.dp_size, acc_full, divide)
    assert got.size == want.size == sum(w.numel)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        f"{int((got != want).sum())} send elements differ"
    assert bool((send[~used] == CANARY).all()), "padding or tail of the send buffer was written"
    # a second step restarts at k = 0 and overwrites
    grads2 = _grads(w, step=2)
    for gk, gk2 in zip(grads, grads2):
        for a, b in zip(gk, gk2):
            a.copy_(b)
    for k in range(w.n_micro):
        B.z1_pack_accum(pack, k)
    torch.cuda.synchronize()
    got2, _ = _packed_from_send(w, kind, send, seg)
    want2 = o.pack_send(w.numel, _rows(w, kind), kind, w.dp_size,
                        o.accumulate(np.stack([_host_full(gk) for gk in grads])), divide)
    assert np.array_equal(got2.view(np.uint32), want2.view(np.uint32))
    pack.close()


def test_pack_call_order():
    w = W.TINY
    seg = B.z1_pack_layout(w.numel, w.dp_size)
    send = torch.zeros(w.dp_size * seg, dtype=torch.float32, device="cuda")
    pack = B.z1_pack_create(w.numel, w.dp_size, _grads(w), send)
    with pytest.raises(B.Z1Error) as e:
        B.z1_pack_accum(pack, 1)
    assert e.value.status == B.Z1_ESTATE
    with pytest.raises(B.Z1Error) as e:
        B.z1_pack_accum(pack, 2)
    assert e.value.status == B.Z1_EINVAL
    B.z1_pack_accum(pack, 0)
    B.z1_pack_accum(pack, 1)
    with pytest.raises(B.Z1Error) as e:   # the step ended; the next starts at 0
        B.z1_pack_accum(pack, 1)
    assert e.value.status == B.Z1_ESTATE
    torch.cuda.synchronize()
    pack.close()


def test_nanotron_order_pack_then_shard_step():
    """Accumulate full tensors into the send buffer, hand each rank its segment
    as the acc arena (the reduce-scatter's place, one contributor here), then
    z1_grad_norm_sq_acc + z1_adamw_step on every rank: bit-exact vs the oracle."""
    from mixed_precision_zero_amd.shard import ShardStep
    o = oracle.get()
    w = dataclasses.replace(W.TINY, dp_size=4)
    seg = B.z1_pack_layout(w.numel, w.dp_size)
    send = torch.zeros(w.dp_size * seg, dtype=torch.float32, device="cuda")
    grads = _grads(w)
    pack = B.z1_pack_create(w.numel, w.dp_size, grads, send, divide=True)
    for k in range(w.n_micro):
        B.z1_pack_accum(pack, k)
    torch.cuda.synchronize()
    acc_full = o.accumulate(np.stack([_host_full(gk) for gk in grads]))
    want_send = o.pack_send(w.numel, None, "per_tensor", w.dp_size, acc_full, True)
    master = W.make_master(w, seed=0, device="cuda")
    pos = 0
    for r in range(w.dp_size):
        st = ShardStep(w.shapes, w.dp_size, r, w.n_micro, device="cuda")
        st.scatter_to_arena(st.master, master)
        st.acc[:st.arena_elems].copy_(send[r * seg:r * seg + st.arena_elems])
        B.z1_grad_norm_sq_acc(st.plan, st.d_S)
        B.z1_adamw_step(st.plan, d_S=st.d_S, step=1, **w.hp())
        torch.cuda.synchronize()
        o_start, o_len = o.shard_plan(w.numel, w.dp_size, r)
        L = int(o_len.sum())
        acc_r = want_send[pos:pos + L].copy()
        pos += L
        p = np.concatenate([m.reshape(-1)[s:s + n].cpu().numpy()
                            for m, s, n in zip(master, o_start, o_len) if n]).astype(np.float32)
        mm = np.zeros(L, np.float32)
        vv = np.zeros(L, np.float32)
        S = o.norm_sq(acc_r)
        c = o.clip_coef(S, w.clip)
        o.adamw(acc_r, p, mm, vv, c, step=1, **w.hp())
        assert st.d_S.item() == S
        for gpu, ref in ((st.master, p), (st.exp_avg, mm), (st.exp_avg_sq, vv)):
            assert np.array_equal(st.packed(gpu).cpu().numpy().view(np.uint32), ref.view(np.uint32))
        st.close()
    pack.close()


def test_pack_llama7b_sampled():
    """The full 7B parameter list at dp 8 (every element of 6.74e9), divided by
    8: sampled elements against the oracle's in-order sum of the same bytes."""
    w = W.LLAMA_7B
    seg = B.z1_pack_layout(w.numel, w.dp_size)
    send = torch.empty(w.dp_size * seg, dtype=torch.float32, device="cuda")
    grads = _grads(w)
    pack = B.z1_pack_create(w.numel, w.dp_size, grads, send, divide=True)
    for k in range(w.n_micro):
        B.z1_pack_accum(pack, k)
    torch.cuda.synchronize()
    o = oracle.get()
    rng = np.random.default_rng(0)
    for r in (0, 3, 7):
        start, ln, off, _ = B.z1_shard_plan(w.numel, w.dp_size, r)
        os_, ol = o.shard_plan(w.numel, w.dp_size, r)
        assert (start == os_).all() and (ln == ol).all()
        for i in rng.choice(len(w.numel), size=24, replace=False):
            if not ln[i]:
                continue
            e = torch.from_numpy(rng.integers(0, int(ln[i]), size=4096)).cuda()
            src = int(start[i]) + e
            g = np.stack([grads[k][i].reshape(-1)[src].view(torch.int16).cpu().numpy().view(np.uint16)
                          for k in range(w.n_micro)])
            want = o.accumulate(g) / np.float32(w.dp_size)
            got = send[r * seg + int(off[i]) + e].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (r, i)
    pack.close()


@pytest.mark.parametrize("resident", [False, True], ids=["per_call", "resident"])
def test_pack_divide_exhaustive_over_all_bf16_pairs(resident):
    """send = (f32(g0) + f32(g1)) / 7 for every pair of bf16 patterns (2^32
    pairs, four 2^30-element tensors), against the correctly rounded binary32
    quotient: the binary32 sum divided in binary64 and rounded once to
    binary32 (double rounding is harmless for one division, since 53 >= 2*24+2).
    NaN exactly where the reference is NaN."""
    n, D = 1 << 30, 7
    g0 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    g1 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    seg = B.z1_pack_layout([n], D)
    send = torch.empty(D * seg, dtype=torch.float32, device="cuda")
    pack = B.z1_pack_create([n], D, [[g0], [g1]], send, divide=True)
    try:
        slices = []
        for r in range(D):
            s, ln, off, _ = B.z1_shard_plan([n], D, r)
            slices.append((int(s[0]), int(ln[0]), r * seg + int(off[0])))
        bad = 0
        for c in range(4):
            bits = torch.arange(c * n, (c + 1) * n, dtype=torch.int64, device="cuda")
            g0.view(torch.int16).copy_((bits >> 16).to(torch.int16))
            g1.view(torch.int16).copy_((bits & 0xFFFF).to(torch.int16))
            del bits
            if resident:
                B.z1_pack_accum_range(pack, 0, 2)
            else:
                B.z1_pack_accum(pack, 0)
                B.z1_pack_accum(pack, 1)
            torch.cuda.synchronize()
            ref = ((g0.float() + g1.float()).double() / D).float()
            for s, ln, o in slices:
                got = send[o:o + ln]
                want = ref[s:s + ln]
                nan = torch.isnan(want)
                bad += int((torch.isnan(got) != nan).sum())
                bad += int(((got.view(torch.int32) != want.view(torch.int32)) & ~nan).sum())
            del ref
        assert bad == 0, f"{bad} quotients differ from the correctly rounded binary32 value"
    finally:
        pack.close()
