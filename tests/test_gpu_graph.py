"""The step captured once in a HIP graph (torch.cuda.CUDAGraph over the
C-ABI calls, which only enqueue kernels on the current stream) and replayed
several times, with eager work and synchronisations between the replays:
every replay must store the same bits as the eager step from the same state.
Nothing in the step records a memset; the norm's arrival counter is reset by
the kernel that consumes it."""
import dataclasses

import pytest
import torch

from mixed_precision_zero_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


RAGGED_SMALL = dataclasses.replace(W.RAGGED, name="ragged_small", shapes=W.ragged_shapes(300, 12, seed=3),
                                   n_micro=3, hot_tensors=(5, 77), steps=1)


@pytest.mark.parametrize("w", [W.TINY, RAGGED_SMALL], ids=lambda w: w.name)
@pytest.mark.parametrize("resident", [False, True], ids=["per_call", "resident"])
def test_step_graph_replays_bitexact(w, resident):
    from mixed_precision_zero_amd.shard import ShardStep
    dev = torch.device("cuda")
    st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device=dev)
    try:
        master = W.make_master(w, seed=0, device=dev)
        st.scatter_to_arena(st.master, master)
        for wt, mt in zip(st.weights, master):
            wt.copy_(mt)
        for k in range(w.n_micro):
            W.make_micro_grads(w, 1, k, seed=0, device=dev, out=st.grads[k])
        bufs = [st.master, st.exp_avg, st.exp_avg_sq, st.acc] + list(st.weights)
        init = [b.clone() for b in bufs]
        hp = w.hp()

        def restore():
            for b, x in zip(bufs, init):
                b.copy_(x)

        def step():
            if resident:
                st.accumulate_range(0, w.n_micro)
            else:
                for k in range(w.n_micro):
                    st.accumulate(k)
            st.norm()
            st.adamw(hp, step=1)

        step()
        torch.cuda.synchronize()
        ref = [b.clone() for b in bufs] + [st.d_S.clone()]

        restore()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        for rep in range(3):
            restore()
            st.d_S.fill_(-1.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = bufs + [st.d_S]
            for i, (a, b) in enumerate(zip(got, ref)):
                assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float64 else a,
                                   b.view(torch.uint8) if b.dtype != torch.float64 else b), \
                    f"replay {rep}: buffer {i} differs from the eager step"
        del g
    finally:
        st.close()


@pytest.mark.parametrize("w,mup", [(W.TINY, False), (RAGGED_SMALL, False), (W.TINY, True)],
                         ids=["tiny", "ragged_small", "tiny_mup"])
def test_scheduled_step_captured_once_trains_over_steps(w, mup):
    """[accumulate all slots, norm, z1_adamw_step_scheduled] captured once and
    replayed for 6 steps of a warmup + cosine learning-rate schedule, with
    fresh gradients written between replays: every replay stores the bits of
    the eager step with that step's t and z1_lr_at(t).  A 7th replay finds
    the table exhausted: master, m, v and the weights stay as they were.
    With mup, both plans carry per-tensor lr / weight-decay multipliers,
    which the scheduled kernel applies to each row's constants."""
    from mixed_precision_zero_amd import binding as B
    from mixed_precision_zero_amd.shard import ShardStep
    dev = torch.device("cuda")
    T = 6
    lr_sched = dict(lr_max=w.lr, lr_min=w.lr / 10, warmup_steps=2, decay_steps=3,
                    decay_style="cosine")
    hp = w.hp()
    lr_s = wd_s = None
    if mup:
        lr_s, wd_s = W.mup_multipliers(w.shapes, w.shapes[0][1])
    gs = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device=dev, lr_scale=lr_s,
                   wd_scale=wd_s)
    es = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device=dev, lr_scale=lr_s,
                   wd_scale=wd_s)
    sched = None
    try:
        master = W.make_master(w, seed=0, device=dev)
        for st in (gs, es):
            st.scatter_to_arena(st.master, master)
            st.load_weights(master)
        sched = B.z1_schedule_create(**hp, step=1, n_steps=T, lr_schedule=lr_sched)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gs.accumulate_range(0, w.n_micro)
            gs.norm()
            gs.adamw_scheduled(sched)
        torch.cuda.synchronize()
        assert B.z1_schedule_query(sched) == (1, 0)

        def state(st):
            return [st.master.view(torch.int32).clone(), st.exp_avg.view(torch.int32).clone(),
                    st.exp_avg_sq.view(torch.int32).clone(), st.acc.view(torch.int32).clone(),
                    st.packed_weights().view(torch.int16).clone(), st.d_S.clone()]

        for t in range(1, T + 2):
            for k in range(w.n_micro):
                W.make_micro_grads(w, t, k, seed=0, device=dev, out=gs.grads[k])
                for a, b in zip(es.grads[k], gs.grads[k]):
                    a.copy_(b)
            torch.cuda.synchronize()
            before = state(gs)
            g.replay()
            torch.cuda.synchronize()
            if t <= T:
                es.accumulate_range(0, w.n_micro)
                es.norm()
                lr_t = B.z1_lr_at(t, **lr_sched)
                B.z1_adamw_step(es.plan, **{**hp, "lr": lr_t}, step=t, d_S=es.d_S)
                torch.cuda.synchronize()
                for i, (a, b) in enumerate(zip(state(gs), state(es))):
                    assert torch.equal(a, b), f"step {t}: buffer {i} differs from the eager step"
                assert B.z1_schedule_query(sched) == (t + 1, 0)
            else:
                after = state(gs)
                for i in (0, 1, 2, 4):          # master, m, v, weights untouched
                    assert torch.equal(after[i], before[i]), f"exhausted table changed buffer {i}"
                assert B.z1_schedule_query(sched) == (T + 1, 1)
        del g
    finally:
        if sched is not None:
            sched.close()
        gs.close()
        es.close()


def test_scheduled_step_graph_7b_matches_eager():
    """The benchmarked form at full size: [all 4 slots, norm, scheduled AdamW]
    captured once on the 7B shard and replayed for steps 1 and 2; each replay
    stores the bits of the eager step taken from the same state."""
    from mixed_precision_zero_amd import binding as B
    from mixed_precision_zero_amd.shard import ShardStep
    w = W.LLAMA_7B
    dev = torch.device("cuda")
    st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device=dev)
    sched = None
    try:
        master = W.make_master(w, seed=0, device=dev)
        st.scatter_to_arena(st.master, master)
        st.load_weights(master)
        del master
        hp = w.hp()
        sched = B.z1_schedule_create(**hp, step=1, n_steps=2)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st.accumulate_range(0, w.n_micro)
            st.norm()
            st.adamw_scheduled(sched)
        torch.cuda.synchronize()

        def snap():
            return [st.master.clone(), st.exp_avg.clone(), st.exp_avg_sq.clone(),
                    st.packed_weights().clone()]

        def restore(s):
            st.master.copy_(s[0])
            st.exp_avg.copy_(s[1])
            st.exp_avg_sq.copy_(s[2])
            st.load_weights_packed_order(s[3])

        state = snap()
        for t in (1, 2):
            for k in range(w.n_micro):
                W.make_micro_grads(w, t, k, seed=0, device=dev, out=st.grads[k])
            restore(state)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = snap() + [st.acc.clone(), st.d_S.clone()]
            restore(state)
            st.accumulate_range(0, w.n_micro)
            st.norm()
            st.adamw(hp, step=t)
            torch.cuda.synchronize()
            ref = snap() + [st.acc.clone(), st.d_S.clone()]
            for i, (a, b) in enumerate(zip(got, ref)):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                    f"step {t}: buffer {i} differs between replay and eager"
            state = ref[:4]
            del got
        assert B.z1_schedule_query(sched) == (3, 0)
        del g
    finally:
        if sched is not None:
            sched.close()
        st.close()


def _random_multipliers(n, seed):
    """Seeded per-tensor lr / weight-decay multipliers (inputs of the step:
    any finite lr scale, any non-negative wd scale, some tensors kept out of
    decay)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    lr_s = [float(x) for x in rng.uniform(0.05, 2.0, n)]
    wd_s = [float(x) for x in rng.choice([0.0, 0.5, 1.0, 2.0], n)]
    return lr_s, wd_s


@pytest.mark.parametrize("w,mult,style,walk,layout", [
    (W.TINY, None, "cosine", None, "full"),
    (W.TINY, "mup", "cosine", None, "full"),
    (RAGGED_SMALL, None, "linear", None, "full"),
    (RAGGED_SMALL, "random", "cosine", None, "full"),
    (W.SMOLLM_135M, "mup", "cosine", None, "full"),
    (W.TINY, "mup", "cosine", "arena_tiles", "packed"),
    (RAGGED_SMALL, "random", "linear", "arena_tiles", "packed"),
    (RAGGED_SMALL, "random", "cosine", "arena_tiles", "full"),
], ids=["tiny_cosine", "tiny_mup_cosine", "ragged_small_linear", "ragged_small_mult_cosine",
        "smollm135m_mup_cosine", "tiny_mup_cosine_packed_arena",
        "ragged_small_mult_linear_packed_arena", "ragged_small_mult_cosine_full_arena"])
def test_scheduled_graph_matches_oracle(w, mult, style, walk, layout):
    """[accumulate all slots, norm, z1_adamw_step_scheduled] captured once and
    replayed for 8 steps of a learning-rate schedule (3 warmup steps, 4 decay
    steps, then the minimum), with fresh gradients before every replay.  Each
    replay is compared element by element with the oracle's step t at the
    oracle's own rate lr_at(t) (Nanotron Guide, config.yaml: learning_rate,
    lr_warmup_steps, lr_decay_steps, min_decay_lr), with the per-tensor
    multipliers as oracle segments: acc, S, master, m, v and the bf16 weights
    bit for bit.  With walk set, AdamW takes that walk in the given bf16
    layout (full-size tensors: its bf16 stores placed through the per-tensor
    table, and its boundary segments by the chunk table); without, the plan
    chooses."""
    import harness
    from mixed_precision_zero_amd import binding as B
    T, warm, decay = 8, 3, 4
    lr_min = w.lr / 10
    style_id = {"none": 0, "linear": 1, "cosine": 2}[style]
    lr_sched = dict(lr_max=w.lr, lr_min=lr_min, warmup_steps=warm, decay_steps=decay,
                    decay_style=style)
    lr_s = wd_s = None
    if mult == "mup":
        lr_s, wd_s = W.mup_multipliers(w.shapes, w.shapes[0][1])
    elif mult == "random":
        lr_s, wd_s = _random_multipliers(len(w.shapes), seed=11)
    layout = dict(layout=layout, walk=walk) if walk else dict(layout=layout)
    h = harness.Parity(w, lr_scale=lr_s, wd_scale=wd_s, ranges=[(0, w.n_micro)], **layout)
    sched = None
    try:
        assert h.plan_matches()
        if walk == "arena_tiles":
            assert h.st.plan.info.adamw_tiles > 0
        sched = B.z1_schedule_create(**w.hp(), step=1, n_steps=T, lr_schedule=lr_sched)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            h.st.accumulate_range(0, w.n_micro)
            h.st.norm()
            h.st.adamw_scheduled(sched)
        torch.cuda.synchronize()
        for t in range(1, T + 1):
            lr_t = h.o.lr_at(w.lr, lr_min, warm, decay, style_id, t)
            rep = h.step(gpu_step=g.replay, lr=lr_t)
            harness.log(f"[sched] {w.name} t={t} lr={lr_t:.6g}: S_rel={rep.S_rel:.2e} "
                        f"not_bitexact={rep.not_bitexact}")
            harness.assert_report(rep)
            assert B.z1_schedule_query(sched) == (t + 1, 0)
        assert h.canaries_intact()
        if layout == "full":
            assert h.weights_outside_slices_intact()
        del g
    finally:
        if sched is not None:
            sched.close()
        h.close()
