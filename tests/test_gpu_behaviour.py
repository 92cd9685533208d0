"""GPU behaviour beyond parity: determinism, call order, resume."""
import dataclasses
import math

import numpy as np
import pytest
import torch

from mixed_precision_zero_amd import binding as B
from mixed_precision_zero_amd import workloads as W
from mixed_precision_zero_amd.shard import ShardStep

pytestmark = pytest.mark.gpu

RAGGED_SMALL = dataclasses.replace(
    W.RAGGED, name="ragged_small", shapes=W.ragged_shapes(300, 14, seed=5), n_micro=3,
    hot_tensors=(3, 50), steps=3)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _fresh(w, **kw):
    st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device="cuda", **kw)
    master = W.make_master(w, seed=0, device="cuda")
    st.scatter_to_arena(st.master, master)
    for wt, mt in zip(st.weights, master):
        wt.copy_(mt)
    return st


def _run_steps(st, w, t0, t1):
    for t in range(t0, t1):
        for k in range(w.n_micro):
            W.make_micro_grads(w, t, k, seed=0, device="cuda", out=st.grads[k])
        st.step(w.hp())
    torch.cuda.synchronize()


def _state(st):
    return [st.packed(a).cpu().numpy().view(np.uint32) for a in
            (st.master, st.exp_avg, st.exp_avg_sq, st.acc)] + \
           [st.packed_weights().view(torch.int16).cpu().numpy(),
            np.array([st.d_S.item()]).view(np.uint64)]


@pytest.mark.parametrize("w", [W.TINY, RAGGED_SMALL], ids=["tiny", "ragged_small"])
def test_bitwise_deterministic_across_launch_shapes(w):
    """Same inputs, different chunk sizes and grids: identical bits, S included."""
    ref = None
    for chunk, mb in ((0, 0), (1024, 0), (4096, 7), (65536, 1), (0, 1)):
        st = _fresh(w, chunk_elems=chunk, max_blocks=mb)
        _run_steps(st, w, 1, 3)
        got = _state(st)
        st.close()
        if ref is None:
            ref = got
            continue
        for a, b in zip(ref, got):
            assert np.array_equal(a, b), f"chunk={chunk} max_blocks={mb} changed the result"


def test_repeat_runs_identical():
    w = RAGGED_SMALL
    outs = []
    for _ in range(3):
        st = _fresh(w)
        _run_steps(st, w, 1, 3)
        outs.append(_state(st))
        st.close()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


def test_resume_is_bitexact():
    """T steps straight equal T1 steps, save caller-owned state, new plan, reload, T-T1 steps."""
    w = RAGGED_SMALL
    st = _fresh(w)
    _run_steps(st, w, 1, 5)
    straight = _state(st)
    st.close()

    st = _fresh(w)
    _run_steps(st, w, 1, 3)
    saved = {k: getattr(st, k).cpu().clone() for k in ("master", "exp_avg", "exp_avg_sq")}
    saved_w = [x.cpu().clone() for x in st.weights]
    st.close()
    del st
    st = _fresh(w)
    for k, v in saved.items():
        getattr(st, k).copy_(v)
    for x, v in zip(st.weights, saved_w):
        x.copy_(v)
    st.t = 2
    _run_steps(st, w, 3, 5)
    resumed = _state(st)
    st.close()
    for a, b in zip(straight, resumed):
        assert np.array_equal(a, b)


def test_call_order_errors():
    w = W.TINY
    st = _fresh(w)
    hp = dict(w.hp())
    with pytest.raises(B.Z1Error) as e:
        B.z1_accum_grads(st.plan, 1)
    assert e.value.status == B.Z1_ESTATE
    with pytest.raises(B.Z1Error) as e:
        B.z1_grad_norm_sq(st.plan, st.d_S)
    assert e.value.status == B.Z1_ESTATE
    with pytest.raises(B.Z1Error) as e:
        B.z1_adamw_step(st.plan, d_S=st.d_S, step=1, **hp)
    assert e.value.status == B.Z1_ESTATE
    st.accumulate(0)
    with pytest.raises(B.Z1Error) as e:          # norm before the last pass
        st.norm()
    assert e.value.status == B.Z1_ESTATE
    st.accumulate(0)                            # k = 0 restarts the step
    st.accumulate(1)
    with pytest.raises(B.Z1Error) as e:          # clipping on: norm first
        B.z1_adamw_step(st.plan, d_S=st.d_S, step=1, **hp)
    assert e.value.status == B.Z1_ESTATE
    with pytest.raises(B.Z1Error) as e:
        B.z1_accum_grads(st.plan, 2)             # k out of range
    assert e.value.status == B.Z1_EINVAL
    st.norm()
    bad = dict(hp, beta1=1.0)
    with pytest.raises(B.Z1Error) as e:
        B.z1_adamw_step(st.plan, d_S=st.d_S, step=1, **bad)
    assert e.value.status == B.Z1_EINVAL
    with pytest.raises(B.Z1Error) as e:
        B.z1_adamw_step(st.plan, d_S=st.d_S, step=0, **hp)
    assert e.value.status == B.Z1_EINVAL
    with pytest.raises(B.Z1Error) as e:
        B.z1_adamw_step(st.plan, d_S=None, step=1, **hp)
    assert e.value.status == B.Z1_EINVAL
    with pytest.raises(B.Z1Error) as e:
        B.z1_grad_norm_sq(st.plan, st.d_S.data_ptr() + 4)
    assert e.value.status == B.Z1_EALIGN
    B.z1_adamw_step(st.plan, d_S=st.d_S, step=1, **hp)
    with pytest.raises(B.Z1Error) as e:          # a new step starts at k = 0
        B.z1_accum_grads(st.plan, 1)
    assert e.value.status == B.Z1_ESTATE
    # clipping off: the norm is optional
    st.accumulate(0)
    st.accumulate(1)
    B.z1_adamw_step(st.plan, d_S=None, step=2, **dict(hp, clip=0.0))
    torch.cuda.synchronize()
    st.close()


def test_probe_copy():
    n = (1 << 24) + 48
    src = torch.randn(n // 4, device="cuda")
    dst = torch.zeros_like(src)
    B.z1_probe_copy(src, dst, n)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_traffic_probes_run():
    """The measurement kernels run on odd sizes (tails) and leave the
    buffers they should not touch alone."""
    n = 1024 * 7 + 13
    bufs = [torch.ones(n * 4, device="cuda") for _ in range(4)]
    half = torch.zeros(n * 4, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(4, device="cuda")
    B.z1_probe("read", [bufs[0], sink], n)
    B.z1_probe("write", [bufs[1]], n)
    B.z1_probe("adamw_traffic", [bufs[0], bufs[1], bufs[2], bufs[3], half], n)
    B.z1_probe("adamw_traffic_wave", [bufs[0], bufs[1], bufs[2], bufs[3], half], n)
    B.z1_probe("accum_traffic", [half, bufs[2]], n)
    torch.cuda.synchronize()
    assert float(sink.sum()) == 0.0 and bool((bufs[0] == 1).all())
    # the slot mixes write sum_j bf16(g_j) into every vector of the fp32
    # stream, in both shapes and for every slot count up to 16
    halves = [torch.full((n * 4,), 0.5, dtype=torch.bfloat16, device="cuda") for _ in range(16)]
    out = torch.zeros(n * 4 + 4, device="cuda")
    for kind in ("slots_traffic", "slots_traffic_one"):
        for G in (2, 7, 16):
            out.zero_()
            B.z1_probe(kind, halves[:G] + [out], n)
            torch.cuda.synchronize()
            v = out[:n * 4].view(n, 4)
            assert bool((v[:, 0] == 0.5 * G).all()) and bool((v[:, 1] == 0.5 * G).all())
            assert float(out[n * 4:].abs().sum()) == 0.0
    with pytest.raises(B.Z1Error):
        B.z1_probe("adamw_traffic", [bufs[0]], n)
    # both AdamW-mix shapes add a to p, m and v over exactly n vectors
    for kind in ("adamw_traffic", "adamw_traffic_wave"):
        a = torch.ones(n * 4 + 8, device="cuda")
        pmv = [torch.full((n * 4 + 8,), 2.0, device="cuda") for _ in range(3)]
        wh = torch.zeros(n * 4 + 8, dtype=torch.bfloat16, device="cuda")
        B.z1_probe(kind, [a] + pmv + [wh], n)
        torch.cuda.synchronize()
        for t in pmv:
            assert bool((t[:n * 4] == 3.0).all()) and bool((t[n * 4:] == 2.0).all())
        assert float(wh[n * 4:].float().abs().sum()) == 0.0


def test_plan_probe_covers_exactly_the_slices():
    """z1_probe_plan walks the AdamW kernel's chunks over the plan's buffers:
    every slice element gets p + acc (an exact fp32 add here), nothing outside
    the slices is touched."""
    w = dataclasses.replace(W.TINY, shapes=((7, 33), (5,), (3, 1000), (1,)), dp_size=3, rank=1)
    st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device="cuda", arena_pad=64)
    try:
        canary = float.fromhex("0x1.5a5a5ap+77")
        for a in (st.master, st.exp_avg, st.exp_avg_sq, st.acc):
            a.fill_(canary)
        used = torch.zeros(st.master.numel(), dtype=torch.bool, device="cuda")
        for _, _, ln, off in st.slices():
            used[off:off + ln] = True
        n = int(used.sum())
        st.master[used] = torch.arange(n, device="cuda", dtype=torch.float32)
        st.acc[used] = 0.5
        for a in (st.exp_avg, st.exp_avg_sq):
            a[used] = 1.0
        for wt in st.weights:
            wt.fill_(3.0)
        B.z1_probe_plan(st.plan)
        torch.cuda.synchronize()
        assert torch.equal(st.master[used], torch.arange(n, device="cuda", dtype=torch.float32) + 0.5)
        assert bool((st.exp_avg[used] == 1.5).all()) and bool((st.exp_avg_sq[used] == 1.5).all())
        for a in (st.master, st.exp_avg, st.exp_avg_sq, st.acc):
            assert bool((a[~used] == canary).all())
        for i, s, ln, _ in st.slices():
            flat = st.weights[i].reshape(-1)
            assert bool((flat[:s] == 3.0).all()) and bool((flat[s + ln:] == 3.0).all())
            if ln:
                assert not bool((flat[s:s + ln] == 3.0).any())
        assert B.lib.z1_probe_plan(st.plan.handle, 1, None) == B.Z1_EINVAL   # unknown kind
    finally:
        st.close()


def _nan_aware_equal_f32(x: np.ndarray, y: np.ndarray) -> bool:
    nx, ny = np.isnan(x), np.isnan(y)
    return bool(np.array_equal(nx, ny) and
                np.array_equal(x[~nx].view(np.uint32), y[~ny].view(np.uint32)))


def _bf16_nan(h: np.ndarray) -> np.ndarray:
    return ((h & 0x7F80) == 0x7F80) & ((h & 0x7F) != 0)


@pytest.mark.parametrize("resident", [False, True], ids=["per_call", "resident"])
@pytest.mark.parametrize("bad", ["inf", "nan"])
def test_nonfinite_gradient_matches_oracle(bad, resident):
    """A non-finite gradient element propagates exactly as in the oracle:
    Inf gives S = Inf and c = 0 (only that element turns NaN, 0 * Inf); NaN
    gives S = NaN and c = NaN (every element turns NaN).  NaN positions must
    agree and every other element must match bit for bit (NaN payloads are
    not compared)."""
    import oracle
    o = oracle.get()
    w = W.TINY
    st = _fresh(w)
    try:
        for k in range(w.n_micro):
            W.make_micro_grads(w, 1, k, seed=0, device="cuda", out=st.grads[k])
        i, s0, ln, _ = next(x for x in st.slices() if x[2] > 8)
        st.grads[1][i].view(-1)[s0 + ln // 2] = float(bad)
        p = st.packed(st.master).cpu().numpy().copy()
        m = np.zeros_like(p)
        v = np.zeros_like(p)
        wb = np.zeros(p.size, np.uint16)
        acc = np.zeros_like(p)
        g = np.stack([torch.cat([st.grads[k][j].reshape(-1)[s:s + n] for j, s, n, _ in st.slices()
                                 if n]).view(torch.int16).cpu().numpy().view(np.uint16)
                      for k in range(w.n_micro)])
        st.step(w.hp(), ranges=[(0, w.n_micro)] if resident else None)
        torch.cuda.synchronize()
        with np.errstate(invalid="ignore", over="ignore"):
            S, c, _ = o.step(g, p, m, v, step=1, acc=acc, w=wb, **w.hp())
        S_gpu = float(st.d_S.item())
        if bad == "inf":
            assert S == math.inf and S_gpu == math.inf and c == 0.0
        else:
            assert math.isnan(S) and math.isnan(S_gpu) and math.isnan(c)
        for name, gpu, ref in (("acc", st.acc, acc), ("master", st.master, p),
                               ("exp_avg", st.exp_avg, m), ("exp_avg_sq", st.exp_avg_sq, v)):
            assert _nan_aware_equal_f32(st.packed(gpu).cpu().numpy(), ref), name
        wg = st.packed_weights().view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(_bf16_nan(wg), _bf16_nan(wb))
        assert np.array_equal(wg[~_bf16_nan(wg)], wb[~_bf16_nan(wb)])
        n_nan = int(np.isnan(p).sum())
        assert (n_nan == 1) if bad == "inf" else (n_nan == p.size)
    finally:
        st.close()


def test_two_plans_on_two_streams_are_independent():
    """Two plans (their own chunk tables, norm partials and arrival counters)
    stepping concurrently on two streams give the bits each gives alone."""
    wa = RAGGED_SMALL
    wb = dataclasses.replace(W.TINY, n_micro=3)

    def run(concurrent):
        sa, sb = _fresh(wa), _fresh(wb)
        try:
            for k in range(wa.n_micro):
                W.make_micro_grads(wa, 1, k, seed=0, device="cuda", out=sa.grads[k])
            for k in range(wb.n_micro):
                W.make_micro_grads(wb, 1, k, seed=0, device="cuda", out=sb.grads[k])
            torch.cuda.synchronize()
            s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
            for t in range(1, 4):
                if concurrent:
                    with torch.cuda.stream(s1):
                        sa.step(wa.hp(), ranges=[(0, wa.n_micro)])
                    with torch.cuda.stream(s2):
                        sb.step(wb.hp())
                else:
                    with torch.cuda.stream(s1):
                        sa.step(wa.hp(), ranges=[(0, wa.n_micro)])
                    s1.synchronize()
                    with torch.cuda.stream(s1):
                        sb.step(wb.hp())
                    s1.synchronize()
            torch.cuda.synchronize()
            return _state(sa) + _state(sb)
        finally:
            sa.close()
            sb.close()

    ref = run(False)
    for _ in range(2):
        got = run(True)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)


def test_adamw_runs_at_the_memory_limit_of_its_buffers():
    """Performance guard that does not depend on where the buffers land:
    AdamW must take no more than 15% longer than its no-arithmetic twin
    (z1_probe_plan: the same walk, loads and stores; here the arena walk of
    a full-size-tensor plan) on the same buffers.  Measured ratios are
    1.0-1.03; an update that became compute-bound or a broken access
    pattern would fail this."""
    w = dataclasses.replace(W.LLAMA_1P7B, n_micro=1)
    st = _fresh(w)
    try:
        W.make_micro_grads(w, 1, 0, seed=0, device="cuda", out=st.grads[0])
        stream = torch.cuda.current_stream()

        def timed(fn):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        step_ms, twin_ms = [], []
        for t in range(1, 9):
            st.accumulate(0)
            st.norm()
            step_ms.append(timed(lambda: st.adamw(w.hp(), step=t)))
            twin_ms.append(timed(lambda: B.z1_probe_plan(st.plan)))
        ratio = float(np.median(step_ms[2:])) / float(np.median(twin_ms[2:]))
        print(f"k_adamw / twin = {ratio:.3f}")
        assert ratio <= 1.15, f"k_adamw takes {ratio:.2f}x its no-arithmetic twin"
    finally:
        st.close()


def test_bf16_cast_in_the_kernel_exhaustive():
    """With lr = 0, weight decay 0, zero gradients and no clipping the update
    leaves every master value as it is (p * 1 - 0), so one step writes
    bf16_RNE(p) of arbitrary bit patterns through k_adamw's own cast.  All
    2^32 fp32 patterns, in four 2^30-element steps: equal to torch's cast for
    every non-NaN pattern (master unchanged too), a quiet NaN of the same sign
    for every NaN."""
    n = 1 << 30
    st = ShardStep([(n,)], 1, 0, 1, device="cuda")
    try:
        hp = dict(lr=0.0, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, clip=0.0)
        st.grads[0][0].zero_()
        bad = bad_nan = 0
        for c in range(4):
            bits = torch.arange(c * n, (c + 1) * n, dtype=torch.int64, device="cuda").to(torch.int32)
            st.master.copy_(bits.view(torch.float32))
            st.exp_avg.zero_()
            st.exp_avg_sq.zero_()
            st.accumulate(0)
            st.adamw(hp, step=1)
            torch.cuda.synchronize()
            f = bits.view(torch.float32)
            nan = torch.isnan(f)
            ref = f.to(torch.bfloat16).view(torch.int16)
            got = st.weights[0].view(torch.int16)
            bad += int(((got != ref) & ~nan).sum())
            bad += int(((st.master.view(torch.int32) != bits) & ~nan).sum())
            h = got[nan].to(torch.int32) & 0xFFFF
            sign = (bits[nan] >> 31) & 1
            bad_nan += int((((h & 0x7FC0) != 0x7FC0) | ((h >> 15) != sign)).sum())
            del bits, f, nan, ref, h, sign
        assert bad == 0, f"{bad} patterns differ from torch's cast (or the master changed)"
        assert bad_nan == 0, f"{bad_nan} NaN patterns did not give a quiet NaN of the same sign"
    finally:
        st.close()


@pytest.mark.parametrize("resident", [False, True], ids=["per_call", "resident"])
def test_accumulation_exhaustive_over_all_bf16_pairs(resident):
    """acc = f32(g0) + f32(g1) for every pair of bf16 bit patterns (2^32
    pairs, four 2^30-element passes): equal to torch's binary32 addition of
    the two widened values for every non-NaN sum, NaN exactly where it is
    NaN."""
    n = 1 << 30
    st = ShardStep([(n,)], 1, 0, 2, device="cuda")
    try:
        g0, g1 = st.grads[0][0], st.grads[1][0]
        bad = 0
        for c in range(4):
            bits = torch.arange(c * n, (c + 1) * n, dtype=torch.int64, device="cuda")
            g0.view(torch.int16).copy_((bits >> 16).to(torch.int16))
            g1.view(torch.int16).copy_((bits & 0xFFFF).to(torch.int16))
            del bits
            if resident:
                st.accumulate_range(0, 2)
            else:
                st.accumulate(0)
                st.accumulate(1)
            torch.cuda.synchronize()
            ref = g0.float() + g1.float()
            nan = torch.isnan(ref)
            bad += int((torch.isnan(st.acc[:n]) != nan).sum())
            bad += int(((st.acc[:n].view(torch.int32) != ref.view(torch.int32)) & ~nan).sum())
            del ref, nan
        assert bad == 0, f"{bad} bf16 pairs sum differently from torch's binary32 addition"
    finally:
        st.close()


def _finite_patterns(rng, n, bits, nonneg_frac=None):
    """Random bit patterns with every finite exponent (subnormals and zero
    included), as uint32 (fp32) or uint16 (bf16)."""
    if bits == 32:
        u = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
        e = rng.integers(0, 255, size=n, dtype=np.uint32)
        u = (u & np.uint32(0x807FFFFF)) | (e << np.uint32(23))
        if nonneg_frac is not None:
            neg = rng.random(n) >= nonneg_frac
            u = np.where(neg, u | np.uint32(0x80000000), u & np.uint32(0x7FFFFFFF))
        return u
    u = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    e = rng.integers(0, 255, size=n, dtype=np.uint16)
    return (u & np.uint16(0x807F)) | (e << np.uint16(7))


@pytest.mark.parametrize("clip,step", [(0.0, 1), (1.0, 7)])
def test_adamw_wide_range_matches_oracle(clip, step):
    """p, m, v and the gradient drawn over every finite fp32 / bf16 exponent
    (subnormals, zero, near-overflow; 1% of v negative, so its square root is
    NaN): one step on the GPU stores the oracle's bits for every element that
    is not NaN, and NaN exactly where the oracle has NaN."""
    import oracle
    o = oracle.get()
    n = 1 << 22
    rng = np.random.default_rng(77 + step)
    p = _finite_patterns(rng, n, 32).view(np.float32)
    m = _finite_patterns(rng, n, 32).view(np.float32)
    v = _finite_patterns(rng, n, 32, nonneg_frac=0.99).view(np.float32)
    g = _finite_patterns(rng, n, 16)
    st = ShardStep([(n,)], 1, 0, 1, device="cuda")
    try:
        st.master[:n].copy_(torch.from_numpy(p.copy()))
        st.exp_avg[:n].copy_(torch.from_numpy(m.copy()))
        st.exp_avg_sq[:n].copy_(torch.from_numpy(v.copy()))
        st.grads[0][0].view(torch.int16).copy_(torch.from_numpy(g.view(np.int16).copy()))
        hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, clip=clip)
        st.accumulate(0)
        st.norm()
        st.adamw(hp, step=step)
        torch.cuda.synchronize()
        wb = np.zeros(n, np.uint16)
        with np.errstate(all="ignore"):
            S, c, _ = o.step(g.reshape(1, n), p, m, v, step=step, w=wb, **hp)
        assert float(st.d_S.item()) == S
        for name, gpu, ref in (("master", st.master, p), ("exp_avg", st.exp_avg, m),
                               ("exp_avg_sq", st.exp_avg_sq, v)):
            x = gpu[:n].cpu().numpy()
            assert np.array_equal(np.isnan(x), np.isnan(ref)), f"{name}: NaN positions differ"
            keep = ~np.isnan(ref)
            assert np.array_equal(x[keep].view(np.uint32), ref[keep].view(np.uint32)), name
        wg = st.weights[0].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(_bf16_nan(wg), _bf16_nan(wb))
        keep = ~_bf16_nan(wb)
        assert np.array_equal(wg[keep], wb[keep])
        assert np.isnan(p).any()          # the negative-v elements took the NaN path
    finally:
        st.close()


# (beta1, beta2, step): bias-correction divisors 1 - beta^t from 0.5 down to
# about 1e-6 and up to 1 - 1e-300 (the kernel divides by them through their
# reciprocals with exact remainders); beta2 = 0 keeps v finite where m is
# infinite, so an infinite quotient there reaches the weight as an infinity.
BIAS_DIVISORS = [(0.9, 0.95, 1), (0.9, 0.95, 2), (0.9, 0.95, 3), (0.9, 0.95, 13),
                 (0.9, 0.95, 1000), (0.9, 0.999, 10), (0.9, 0.999, 65537),
                 (0.5, 0.999999, 1), (0.5, 0.999999, 3000), (0.3, 0.99, 7),
                 (0.99, 0.0, 5), (0.0, 0.999, 1_000_000)]


def test_adamw_bias_divisors_match_oracle():
    """m / (1 - beta1^t) and v / (1 - beta2^t) for many divisors: p, m and v
    over every finite fp32 exponent plus 0.1% infinities in m and v, one
    step each, the oracle's bits for every element that is not NaN and NaN
    exactly where the oracle has NaN (clipping off, so the infinities reach
    the quotients)."""
    import oracle
    o = oracle.get()
    n = 1 << 20
    st = ShardStep([(n,)], 1, 0, 1, device="cuda")
    try:
        for i, (b1, b2, step) in enumerate(BIAS_DIVISORS):
            rng = np.random.default_rng(500 + i)
            p = _finite_patterns(rng, n, 32).view(np.float32)
            m = _finite_patterns(rng, n, 32).view(np.float32)
            v = _finite_patterns(rng, n, 32, nonneg_frac=0.99).view(np.float32)
            g = _finite_patterns(rng, n, 16)
            for x in (m, v):
                hit = rng.random(n) < 1e-3
                x[hit] = np.where(rng.random(int(hit.sum())) < 0.5, np.inf, -np.inf)
            st.master[:n].copy_(torch.from_numpy(p.copy()))
            st.exp_avg[:n].copy_(torch.from_numpy(m.copy()))
            st.exp_avg_sq[:n].copy_(torch.from_numpy(v.copy()))
            st.grads[0][0].view(torch.int16).copy_(torch.from_numpy(g.view(np.int16).copy()))
            hp = dict(lr=1e-3, beta1=b1, beta2=b2, eps=1e-8, weight_decay=0.1, clip=0.0)
            st.accumulate(0)
            st.norm()
            st.adamw(hp, step=step)
            torch.cuda.synchronize()
            wb = np.zeros(n, np.uint16)
            with np.errstate(all="ignore"):
                o.step(g.reshape(1, n), p, m, v, step=step, w=wb, **hp)
            for name, gpu, ref in (("master", st.master, p), ("exp_avg", st.exp_avg, m),
                                   ("exp_avg_sq", st.exp_avg_sq, v)):
                x = gpu[:n].cpu().numpy()
                assert np.array_equal(np.isnan(x), np.isnan(ref)), \
                    f"{name}: NaN positions differ (beta1 {b1}, beta2 {b2}, t {step})"
                keep = ~np.isnan(ref)
                assert np.array_equal(x[keep].view(np.uint32), ref[keep].view(np.uint32)), \
                    f"{name} (beta1 {b1}, beta2 {b2}, t {step})"
            wg = st.weights[0].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(_bf16_nan(wg), _bf16_nan(wb))
            keep = ~_bf16_nan(wb)
            assert np.array_equal(wg[keep], wb[keep]), f"weights (beta1 {b1}, beta2 {b2}, t {step})"
            if b2 == 0.0:
                assert np.isinf(p).any()    # an infinite m over a finite v: an infinite weight
    finally:
        st.close()


def _plan_from_temporaries(w):
    """A plan over tensors that nothing but the plan references."""
    start, ln, off, ae = B.z1_shard_plan(w.numel, w.dp_size, w.rank)
    master_full = W.make_master(w, seed=0, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    master = torch.zeros(ae, **f32)
    for i in range(len(w.shapes)):
        if ln[i]:
            master[off[i]:off[i] + ln[i]].copy_(
                master_full[i].reshape(-1)[start[i]:start[i] + ln[i]])
    weights = [m.to(torch.bfloat16) for m in master_full]
    grads = [W.make_micro_grads(w, 1, k, seed=0, device="cuda") for k in range(w.n_micro)]
    return B.z1_plan_create(w.numel, w.dp_size, w.rank, weights, grads, master,
                            torch.zeros(ae, **f32), torch.zeros(ae, **f32), torch.zeros(ae, **f32))


def test_plan_keeps_its_bound_tensors_alive():
    """The binding holds every tensor a plan is bound to until the plan is
    closed: a plan built from temporaries, stepped after same-sized NaN
    tensors were allocated (they would take any freed block), stores the
    bits of the same step on tensors the caller kept, and the NaN tensors
    stay untouched."""
    w = W.TINY
    ref = _fresh(w)
    plan = None
    try:
        _run_steps(ref, w, 1, 2)
        plan = _plan_from_temporaries(w)
        torch.cuda.synchronize()
        junk = [torch.full((ref.arena_elems,), float("nan"), device="cuda") for _ in range(8)]
        junk += [torch.full(s, float("nan"), dtype=torch.bfloat16, device="cuda")
                 for s in w.shapes for _ in range(1 + w.n_micro)]
        d_S = torch.zeros(1, dtype=torch.float64, device="cuda")
        B.z1_accum_grads_range(plan, 0, w.n_micro)
        B.z1_grad_norm_sq(plan, d_S)
        B.z1_adamw_step(plan, d_S=d_S, step=1, **w.hp())
        torch.cuda.synchronize()
        weights, _, master, m, v, acc = plan._keep[6:12]
        for got, want in ((master, ref.master), (m, ref.exp_avg), (v, ref.exp_avg_sq),
                          (acc, ref.acc)):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32))
        for got, want in zip(weights, ref.weights):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        assert d_S.item() == ref.d_S.item()
        assert all(bool(torch.isnan(j.float()).all()) for j in junk)
    finally:
        if plan is not None:
            plan.close()
        ref.close()
