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
