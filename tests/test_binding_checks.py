"""The binding rejects tensors the library would read or write out of bounds
or misread, before any call reaches the C ABI: wrong dtype, not contiguous,
fewer elements than the call touches, not on the GPU.  Every case here is
decided on the host (CPU tensors, no GPU needed)."""
import ctypes

import pytest
import torch

from mixed_precision_zero_amd import binding as B

NUMEL = [300, 64, 1030]          # tiny three-tensor list
D, R, K = 4, 1, 2


def _plan_args(layout="full", **over):
    start, ln, off, A = B.z1_shard_plan(NUMEL, D, R)
    bf, f32 = torch.bfloat16, torch.float32
    if layout == "packed":
        weights = torch.zeros(A, dtype=bf)
        grads = [torch.zeros(A, dtype=bf) for _ in range(K)]
    else:
        weights = [torch.zeros(n, dtype=bf) for n in NUMEL]
        grads = [[torch.zeros(n, dtype=bf) for n in NUMEL] for _ in range(K)]
    args = dict(numel=NUMEL, dp_size=D, rank=R, weights=weights, grads=grads,
                master=torch.zeros(A, dtype=f32), exp_avg=torch.zeros(A, dtype=f32),
                exp_avg_sq=torch.zeros(A, dtype=f32), acc=torch.zeros(A, dtype=f32),
                layout=layout)
    args.update(over)
    return args, A


def _create(args):
    return B.z1_plan_create(**args)


def test_right_tensors_on_the_cpu_are_refused_for_their_device():
    for layout in ("full", "packed"):
        args, _ = _plan_args(layout)
        with pytest.raises(ValueError, match="expected the current GPU"):
            _create(args)


@pytest.mark.parametrize("layout", ["full", "packed"])
@pytest.mark.parametrize("arena", ["master", "exp_avg", "exp_avg_sq", "acc"])
def test_arena_checks(layout, arena):
    args, A = _plan_args(layout)
    bad = dict(args, **{arena: torch.zeros(A, dtype=torch.bfloat16)})
    with pytest.raises(TypeError, match=f"{arena}: dtype"):
        _create(bad)
    bad = dict(args, **{arena: torch.zeros(2 * A, dtype=torch.float32)[::2]})
    with pytest.raises(ValueError, match=f"{arena}: not contiguous"):
        _create(bad)
    bad = dict(args, **{arena: torch.zeros(A - 1, dtype=torch.float32)})
    with pytest.raises(ValueError, match=f"{arena}: {A - 1} elements"):
        _create(bad)


def test_full_layout_weight_and_grad_checks():
    start, ln, _, _ = B.z1_shard_plan(NUMEL, D, R)
    i = 2                                   # a tensor this rank touches
    end = int(start[i] + ln[i])
    args, _ = _plan_args("full")
    w = list(args["weights"])
    w[i] = torch.zeros(NUMEL[i], dtype=torch.float16)
    with pytest.raises(TypeError, match=rf"weights\[{i}\]: dtype"):
        _create(dict(args, weights=w))
    w[i] = torch.zeros(end - 1, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=rf"weights\[{i}\]: {end - 1} elements"):
        _create(dict(args, weights=w))
    w[i] = torch.zeros(NUMEL[i], 2, dtype=torch.bfloat16)[:, 0]
    with pytest.raises(ValueError, match=rf"weights\[{i}\]: not contiguous"):
        _create(dict(args, weights=w))
    g = [list(gk) for gk in args["grads"]]
    g[1][i] = torch.zeros(NUMEL[i], dtype=torch.float32)
    with pytest.raises(TypeError, match=rf"grads\[1\]\[{i}\]: dtype"):
        _create(dict(args, grads=g))
    g[1][i] = torch.zeros(end - 1, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=rf"grads\[1\]\[{i}\]: {end - 1} elements"):
        _create(dict(args, grads=g))


def test_packed_layout_shard_checks():
    args, A = _plan_args("packed")
    with pytest.raises(ValueError, match=rf"weights \(packed shard\): {A - 1} elements"):
        _create(dict(args, weights=torch.zeros(A - 1, dtype=torch.bfloat16)))
    with pytest.raises(TypeError, match=r"weights \(packed shard\): dtype"):
        _create(dict(args, weights=torch.zeros(A, dtype=torch.int32)))
    g = list(args["grads"])
    g[0] = torch.zeros(A - 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"grads\[0\] \(packed shard\)"):
        _create(dict(args, grads=g))


def test_raw_addresses_reach_the_library_unchecked():
    """An int is a device address the caller vouches for: the binding passes
    it on and the library's own host checks decide (here: misaligned)."""
    args, A = _plan_args("full")
    args = dict(args, master=0x10004, exp_avg=0x20000, exp_avg_sq=0x30000, acc=0x40000,
                weights=[0x50000, 0x60000, 0x70000],
                grads=[[0x80000, 0x90000, 0xA0000], [0xB0000, 0xC0000, 0xD0000]],
                arena_elems=A, stream=0)
    with pytest.raises(B.Z1Error) as e:
        _create(args)
    assert e.value.status == B.Z1_EALIGN


def test_norm_and_step_scalars():
    bad_dtype = torch.zeros(1, dtype=torch.float32)
    with pytest.raises(TypeError, match="d_S: dtype"):
        B.z1_grad_norm_sq(None, bad_dtype)
    with pytest.raises(TypeError, match="d_S: dtype"):
        B.z1_grad_norm_sq_acc(None, bad_dtype)
    with pytest.raises(ValueError, match="d_pair: 1 elements"):
        B.z1_grad_norm_sq_pair(None, torch.zeros(1, dtype=torch.float64))
    with pytest.raises(ValueError, match="d_pairs: 5 elements"):
        B.z1_norm_combine(torch.zeros(5, dtype=torch.float64), 3,
                          torch.zeros(1, dtype=torch.float64))
    with pytest.raises(ValueError, match="d_pairs: on cpu"):
        B.z1_norm_combine(torch.zeros(6, dtype=torch.float64), 3,
                          torch.zeros(1, dtype=torch.float64))
    with pytest.raises(TypeError, match="d_S: dtype"):
        B.z1_adamw_step(None, lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
                        clip=1.0, step=1, d_S=bad_dtype)


def test_pack_checks():
    seg = B.z1_pack_layout(NUMEL, D)
    grads = [[torch.zeros(n, dtype=torch.bfloat16) for n in NUMEL] for _ in range(K)]
    send = torch.zeros(D * seg, dtype=torch.float32)
    g = [list(gk) for gk in grads]
    g[0][1] = torch.zeros(NUMEL[1] - 1, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"grads\[0\]\[1\]: 63 elements"):
        B.z1_pack_create(NUMEL, D, g, send)
    with pytest.raises(ValueError, match=f"send: {D * seg - 1} elements"):
        B.z1_pack_create(NUMEL, D, grads, torch.zeros(D * seg - 1, dtype=torch.float32))
    with pytest.raises(TypeError, match="send: dtype"):
        B.z1_pack_create(NUMEL, D, grads, torch.zeros(D * seg, dtype=torch.float64))
    with pytest.raises(ValueError, match="expected the current GPU"):
        B.z1_pack_create(NUMEL, D, grads, send)


def test_probe_checks():
    nv = 100
    f = torch.zeros(4 * nv, dtype=torch.float32)
    half = torch.zeros(4 * nv, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"bufs\[4\]: 798 bytes"):
        B.z1_probe("adamw_traffic", [f, f, f, f, half[:-1]], nv)
    with pytest.raises(ValueError, match=r"bufs\[4\]: 798 bytes"):
        B.z1_probe("adamw_traffic_wave", [f, f, f, f, half[:-1]], nv)
    with pytest.raises(ValueError, match=r"bufs\[2\]: 1596 bytes"):
        B.z1_probe("slots_traffic_one", [half, half, f[:-1]], nv)
    with pytest.raises(ValueError, match=r"bufs\[0\]: 1596 bytes"):
        B.z1_probe("read", [f[:-1], f], nv)
    with pytest.raises(ValueError, match="src: 1596 bytes"):
        B.z1_probe_copy(f[:-1], f, 16 * nv)
    with pytest.raises(ValueError, match="expected the current GPU"):
        B.z1_probe("write", [f], nv)


def test_norm_combine_host_checks():
    """z1_norm_combine's host-side checks: NULL or n < 1 give Z1_EINVAL and a
    misaligned pointer Z1_EALIGN before any device query; without a current
    GPU the call returns Z1_EHIP rather than enqueue (with one, pointers that
    are not its device memory give Z1_EINVAL: GPU test)."""
    L = B.lib
    assert L.z1_norm_combine(None, 1, 0x2000, None) == B.Z1_EINVAL
    assert L.z1_norm_combine(0x1000, 1, None, None) == B.Z1_EINVAL
    assert L.z1_norm_combine(0x1000, 0, 0x2000, None) == B.Z1_EINVAL
    assert L.z1_norm_combine(0x1000, -3, 0x2000, None) == B.Z1_EINVAL
    assert L.z1_norm_combine(0x1008, 1, 0x2000, None) == B.Z1_EALIGN
    assert L.z1_norm_combine(0x1000, 1, 0x2004, None) == B.Z1_EALIGN
    if not torch.cuda.is_available():
        assert L.z1_norm_combine(0x1000, 1, 0x2000, None) == B.Z1_EHIP


def test_norm_flat_noalloc_host_checks():
    """The entry point that allocates nothing refuses, before any device
    query, a size beyond its stated maximum, a negative size and NULL."""
    L = B.lib
    assert L.z1_grad_norm_sq_flat_noalloc(0x1000, (1 << 30) + 1, 0x2000, None) == B.Z1_EINVAL
    assert L.z1_grad_norm_sq_flat_noalloc(0x1000, -1, 0x2000, None) == B.Z1_EINVAL
    assert L.z1_grad_norm_sq_flat_noalloc(None, 5, 0x2000, None) == B.Z1_EINVAL
    assert L.z1_grad_norm_sq_flat_noalloc(0x1000, 5, None, None) == B.Z1_EINVAL
    assert L.z1_grad_norm_sq_flat_noalloc(0x1004, 5, 0x2000, None) == B.Z1_EALIGN
    assert L.z1_grad_norm_sq_flat_noalloc(0x1000, 5, 0x2004, None) == B.Z1_EALIGN
    with pytest.raises(ValueError, match="acc: 9 elements"):
        B.z1_grad_norm_sq_flat_noalloc(torch.zeros(9), 10, torch.zeros(1, dtype=torch.float64))
