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
