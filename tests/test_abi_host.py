"""Host-side checks of libz1 (no GPU needed): symbols, shard plan, errors."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from mixed_precision_zero_amd import binding as B
from mixed_precision_zero_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "z1.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(z1_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "z1_shard_plan" in names and "z1_adamw_step" in names
    for name in names:
        assert hasattr(B.lib, name), f"{name} declared in z1.h but not exported"
    assert set(names) == set(B.EXPORTS)


def test_abi_version_and_strerror():
    assert B.z1_abi_version() == 10
    for s in range(6):
        assert B.strerror(s)
    assert B.strerror(99) == "unknown status"


def test_single_hip_runtime():
    """libz1 binds to the HIP runtime torch already loaded."""
    rts = B.hip_runtimes_loaded()
    assert len(rts) == 1, rts


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_plan_bitexact_vs_oracle(name):
    w = W.WORKLOADS[name]
    start, ln, off, arena = B.z1_shard_plan(w.numel, w.dp_size, w.rank)
    o_start, o_len = oracle.get().shard_plan(w.numel, w.dp_size, w.rank)
    assert (start == o_start).all() and (ln == o_len).all()
    _check_arena(start, ln, off, arena)


def _check_arena(start, ln, off, arena):
    assert (off % 64 == start % 64).all(), "arena offset must share the slice's residue mod 64"
    end = off + ln
    assert (off[1:] >= end[:-1]).all(), "arena slices overlap or go backwards"
    assert (off >= 0).all() and (end <= arena).all()
    assert arena - int(ln.sum()) <= 63 * len(ln), "more padding than 63 per tensor"
    if len(ln):
        assert arena == int(end[-1])


def test_plan_bruteforce_vs_oracle():
    o = oracle.get()
    n = np.arange(300, dtype=np.int64)
    for D in range(1, 18):
        for r in range(D):
            s, l, off, arena = B.z1_shard_plan(n, D, r)
            os_, ol = o.shard_plan(n, D, r)
            assert (s == os_).all() and (l == ol).all()
            _check_arena(s, l, off, arena)


def test_plan_large_numel():
    numel = [2 ** 40 + 3, 2 ** 33 - 1, 7, 0, 1]
    for D in (1, 7, 8, 1000):
        for r in (0, D // 2, D - 1):
            s, l, _, _ = B.z1_shard_plan(numel, D, r)
            os_, ol = oracle.get().shard_plan(numel, D, r)
            assert (s == os_).all() and (l == ol).all()


def test_plan_errors():
    P = ctypes.POINTER(ctypes.c_int64)
    buf = (ctypes.c_int64 * 4)()
    ae = ctypes.c_int64()
    numel = (ctypes.c_int64 * 2)(5, 7)
    cast = lambda a: ctypes.cast(a, P)  # noqa: E731
    L = B.lib
    assert L.z1_shard_plan(2, cast(numel), 0, 0, cast(buf), cast(buf), cast(buf), ctypes.byref(ae)) == B.Z1_EINVAL
    assert L.z1_shard_plan(2, cast(numel), 4, 4, cast(buf), cast(buf), cast(buf), ctypes.byref(ae)) == B.Z1_EINVAL
    assert L.z1_shard_plan(2, cast(numel), 4, -1, cast(buf), cast(buf), cast(buf), ctypes.byref(ae)) == B.Z1_EINVAL
    assert L.z1_shard_plan(-1, cast(numel), 4, 0, cast(buf), cast(buf), cast(buf), ctypes.byref(ae)) == B.Z1_EINVAL
    assert L.z1_shard_plan(2, None, 4, 0, cast(buf), cast(buf), cast(buf), ctypes.byref(ae)) == B.Z1_EINVAL
    assert L.z1_shard_plan(2, cast(numel), 4, 0, cast(buf), cast(buf), cast(buf), None) == B.Z1_EINVAL
    neg = (ctypes.c_int64 * 2)(5, -1)
    assert L.z1_shard_plan(2, cast(neg), 4, 0, cast(buf), cast(buf), cast(buf), ctypes.byref(ae)) == B.Z1_EINVAL
    assert L.z1_shard_plan(0, None, 1, 0, None, None, None, ctypes.byref(ae)) == B.Z1_OK and ae.value == 0


def _bind(**over):
    numel = (ctypes.c_int64 * 1)(1024)
    w = (ctypes.c_void_p * 1)(0x10000)
    g = (ctypes.c_void_p * 2)(0x20000, 0x30000)
    b = B.Bind(n_tensors=1, dp_size=1, rank=0, n_micro=2,
               numel=ctypes.cast(numel, ctypes.POINTER(ctypes.c_int64)),
               weights=ctypes.cast(w, ctypes.POINTER(ctypes.c_void_p)),
               grads=ctypes.cast(g, ctypes.POINTER(ctypes.c_void_p)),
               master=0x40000, exp_avg=0x50000, exp_avg_sq=0x60000, acc=0x70000,
               arena_elems=1024, chunk_elems=0, max_blocks=0, plan_kind=0)
    for k, v in over.items():
        if k in ("w0", "g1"):
            (w if k == "w0" else g)[0 if k == "w0" else 1] = v
        else:
            setattr(b, k, v)
    return b, (numel, w, g)


@pytest.mark.parametrize("over,status", [
    (dict(n_micro=0), B.Z1_EINVAL), (dict(dp_size=0), B.Z1_EINVAL),
    (dict(rank=1), B.Z1_EINVAL), (dict(plan_kind=3), B.Z1_EINVAL),
    (dict(plan_kind=2), B.Z1_EINVAL),  # dim0 without rows
    (dict(chunk_elems=1000), B.Z1_EINVAL), (dict(chunk_elems=1 << 21), B.Z1_EINVAL),
    (dict(arena_elems=1023), B.Z1_EINVAL), (dict(max_blocks=-1), B.Z1_EINVAL),
    (dict(master=0), B.Z1_EINVAL), (dict(w0=0), B.Z1_EINVAL), (dict(g1=0), B.Z1_EINVAL),
    (dict(w0=0x10008), B.Z1_EALIGN), (dict(g1=0x30002), B.Z1_EALIGN),
    (dict(acc=0x70004), B.Z1_EALIGN),
    (dict(layout=2), B.Z1_EINVAL), (dict(walk=3), B.Z1_EINVAL), (dict(walk=-1), B.Z1_EINVAL),
    (dict(walk=2, max_blocks=4), B.Z1_EINVAL),             # arena tiles run one workgroup
    (dict(walk=2, layout=1, max_blocks=4), B.Z1_EINVAL),   # per tile, in either layout
    (dict(layout=1, w0=0), B.Z1_EINVAL), (dict(layout=1, g1=0), B.Z1_EINVAL),
    (dict(layout=1, w0=0x10008), B.Z1_EALIGN), (dict(layout=1, g1=0x30002), B.Z1_EALIGN),
])
def test_plan_create_rejects_before_device_work(over, status):
    """Validation happens on the host: fake addresses never reach the device."""
    b, keep = _bind(**over)
    h = ctypes.c_void_p(1)
    assert B.lib.z1_plan_create(ctypes.byref(h), ctypes.byref(b), None) == status
    assert h.value is None


def test_null_plan_calls():
    L = B.lib
    assert L.z1_plan_create(None, None, None) == B.Z1_EINVAL
    assert L.z1_accum_grads(None, 0, None) == B.Z1_EINVAL
    assert L.z1_accum_grads_range(None, 0, 1, None) == B.Z1_EINVAL
    assert L.z1_pack_accum_range(None, 0, 1, None) == B.Z1_EINVAL
    assert L.z1_probe_plan(None, 0, None) == B.Z1_EINVAL
    assert L.z1_adamw_step_scheduled(None, None, None, None) == B.Z1_EINVAL
    assert L.z1_schedule_query(None, None, None) == B.Z1_EINVAL
    assert L.z1_schedule_destroy(None) == B.Z1_OK
    assert L.z1_grad_norm_sq_pair(None, None, None) == B.Z1_EINVAL
    assert L.z1_norm_combine(None, 1, None, None) == B.Z1_EINVAL
    assert L.z1_norm_combine(0x1000, 0, 0x2000, None) == B.Z1_EINVAL
    assert L.z1_norm_combine(0x1008, 1, 0x2000, None) == B.Z1_EALIGN
    assert L.z1_grad_norm_sq(None, None, None) == B.Z1_EINVAL
    hp = B.AdamWHP(1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, 1)
    assert L.z1_adamw_step(None, ctypes.byref(hp), None, None) == B.Z1_EINVAL
    assert L.z1_plan_query(None, None) == B.Z1_EINVAL
    assert L.z1_plan_destroy(None) == B.Z1_OK
    assert L.z1_probe_copy(None, None, 16, None) == B.Z1_EINVAL
    assert L.z1_probe_copy(0x1000, 0x2000, 15, None) == B.Z1_EINVAL
    assert L.z1_probe_copy(0x1008, 0x2000, 16, None) == B.Z1_EALIGN
    bufs = (ctypes.c_void_p * 5)(0x1000, 0x2000, 0x3000, 0x4000, 0x5000)
    assert L.z1_probe(7, bufs, 5, 16, None) == B.Z1_EINVAL        # unknown kind
    assert L.z1_probe(-1, bufs, 5, 16, None) == B.Z1_EINVAL
    assert L.z1_probe(2, bufs, 4, 16, None) == B.Z1_EINVAL        # adamw traffic needs 5
    assert L.z1_probe(0, bufs, 2, -1, None) == B.Z1_EINVAL
    assert L.z1_probe(0, None, 2, 16, None) == B.Z1_EINVAL
    odd = (ctypes.c_void_p * 2)(0x1008, 0x2000)
    assert L.z1_probe(0, odd, 2, 16, None) == B.Z1_EALIGN
    assert L.z1_probe(1, bufs, 1, 0, None) == B.Z1_OK              # nothing to do
    assert L.z1_probe(5, bufs, 4, 16, None) == B.Z1_EINVAL        # one-wave AdamW mix needs 5
    assert L.z1_probe(6, bufs, 2, 16, None) == B.Z1_EINVAL        # slots need G >= 2
    many = (ctypes.c_void_p * 18)(*[0x1000 * (j + 1) for j in range(18)])
    assert L.z1_probe(6, many, 18, 16, None) == B.Z1_EINVAL       # G = 17 > 16
    assert L.z1_probe(4, many, 18, 16, None) == B.Z1_EINVAL
    assert L.z1_probe(2, bufs, 5, (1 << 31) * 256, None) == B.Z1_EINVAL   # grid too large
    assert L.z1_probe(2, bufs, 5, (1 << 31) * 64, None) == B.Z1_EINVAL    # 2^31 one-wave groups


@pytest.mark.parametrize("over,n_steps", [
    (dict(), 0), (dict(), -3), (dict(), (1 << 24) + 1), (dict(step=0), 4),
    (dict(beta1=1.0), 4), (dict(eps=0.0), 4), (dict(lr=float("nan")), 4),
    (dict(weight_decay=-0.1), 4), (dict(clip=float("nan")), 4),
])
def test_schedule_create_rejects_before_device_work(over, n_steps):
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, clip=1.0, step=1)
    hp.update(over)
    h = ctypes.c_void_p(1)
    a = B.AdamWHP(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["clip"],
                  hp["step"])
    assert B.lib.z1_schedule_create(ctypes.byref(h), ctypes.byref(a), None, n_steps,
                                    None) == B.Z1_EINVAL
    assert h.value is None
    bad_lr = B.LRSchedule(1e-3, 1e-4, -1, 10, 2, 0)         # negative warmup
    assert B.lib.z1_schedule_create(ctypes.byref(h), ctypes.byref(B.AdamWHP(
        1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, 1)), ctypes.byref(bad_lr), 4, None) == B.Z1_EINVAL


@pytest.mark.parametrize("kind", ["flat", "dim0"])
@pytest.mark.parametrize("name", ["tiny", "smollm135m", "llama7b", "ragged"])
def test_plan_kinds_bitexact_vs_oracle(kind, name):
    w = W.WORKLOADS[name]
    rows = [s[0] for s in w.shapes]
    for D, r in ((w.dp_size, w.rank), (7, 6), (8, 0), (3, 1)):
        start, ln, off, arena = B.z1_shard_plan(w.numel, D, r, kind=kind,
                                                rows=rows if kind == "dim0" else None)
        o_start, o_len = oracle.get().plan(kind, w.numel, rows, D, r)
        assert (ln == o_len).all()
        assert (start[ln > 0] == o_start[ln > 0]).all()
        _check_arena(start, ln, off, arena)


def test_plan_kinds_bruteforce_vs_oracle():
    o = oracle.get()
    rng = np.random.default_rng(3)
    for _ in range(40):
        rows = rng.integers(0, 30, size=6)
        cols = rng.integers(1, 5, size=6)
        numel = rows * cols
        for D in range(1, 10):
            for r in range(D):
                for kind in ("flat", "dim0"):
                    s, l, off, arena = B.z1_shard_plan(numel, D, r, kind=kind, rows=rows)
                    os_, ol = o.plan(kind, numel, rows, D, r)
                    assert (l == ol).all() and (s[l > 0] == os_[l > 0]).all(), (kind, numel, D, r)
                    _check_arena(s, l, off, arena)


def test_plan_kind_errors():
    with pytest.raises(B.Z1Error):
        B.z1_shard_plan([6, 4], 2, 0, kind="dim0", rows=[4, 2])    # 6 not a multiple of 4
    with pytest.raises(B.Z1Error):
        B.z1_shard_plan([6, 4], 2, 0, kind="dim0", rows=[3, 0])    # elements without rows
    s, l, _, _ = B.z1_shard_plan([6, 0], 2, 1, kind="dim0", rows=[3, 5])   # a (5, 0) tensor
    assert list(l) == [2, 0]
    with pytest.raises(B.Z1Error):
        B.z1_shard_plan([6, 4], 2, 0, kind="dim0")                 # rows missing


@pytest.mark.parametrize("style", ["linear", "cosine", "none"])
def test_lr_schedule_bitexact_vs_oracle(style):
    o = oracle.get()
    code = {"none": 0, "linear": 1, "cosine": 2}[style]
    for (lmax, lmin, W_, D) in ((3e-3, 3e-4, 2000, 100000), (1e-3, 0.0, 0, 10), (5e-4, 1e-5, 7, 0)):
        for t in list(range(0, 40)) + [W_, W_ + 1, W_ + D // 2, W_ + D, W_ + D + 9, 123456]:
            got = B.z1_lr_at(t, lr_max=lmax, lr_min=lmin, warmup_steps=W_, decay_steps=D,
                             decay_style=style)
            assert got == o.lr_at(lmax, lmin, W_, D, code, t), (style, t)


def test_lr_schedule_errors():
    with pytest.raises(B.Z1Error):
        B.z1_lr_at(-1, lr_max=1.0, lr_min=0.0, warmup_steps=1, decay_steps=1)
    with pytest.raises(B.Z1Error):
        B.z1_lr_at(1, lr_max=1.0, lr_min=0.0, warmup_steps=-1, decay_steps=1)


@pytest.mark.parametrize("kind", ["per_tensor", "flat", "dim0"])
def test_pack_layout_is_largest_rank_arena(kind):
    for name in ("tiny", "ragged", "llama7b"):
        w = W.WORKLOADS[name]
        rows = [s[0] for s in w.shapes]
        for D in (1, 3, 8):
            seg = B.z1_pack_layout(w.numel, D, kind, rows if kind == "dim0" else None)
            arenas = [B.z1_shard_plan(w.numel, D, r, kind=kind,
                                      rows=rows if kind == "dim0" else None)[3] for r in range(D)]
            assert seg % 64 == 0 and seg - 64 < max(arenas) <= seg


def test_pack_create_rejects_before_device_work():
    numel = (ctypes.c_int64 * 1)(1024)
    g = (ctypes.c_void_p * 2)(0x20000, 0x30000)
    def bind(**over):
        b = B.PackBind(n_tensors=1, dp_size=2, n_micro=2, plan_kind=0,
                       numel=ctypes.cast(numel, ctypes.POINTER(ctypes.c_int64)), rows=None,
                       grads=ctypes.cast(g, ctypes.POINTER(ctypes.c_void_p)), send=0x40000,
                       send_elems=1024, chunk_elems=0, divide=1, reserved=0)
        for k, v in over.items():
            setattr(b, k, v)
        return b
    h = ctypes.c_void_p(1)
    for over, status in ((dict(send_elems=1023), B.Z1_EINVAL), (dict(send=0x40004), B.Z1_EALIGN),
                         (dict(n_micro=0), B.Z1_EINVAL), (dict(reserved=2), B.Z1_EINVAL),
                         (dict(plan_kind=2), B.Z1_EINVAL), (dict(send=0), B.Z1_EINVAL)):
        b = bind(**over)
        assert B.lib.z1_pack_create(ctypes.byref(h), ctypes.byref(b), None) == status, over
    g[1] = 0x30002
    b = bind()
    assert B.lib.z1_pack_create(ctypes.byref(h), ctypes.byref(b), None) == B.Z1_EALIGN
    assert B.lib.z1_pack_accum(None, 0, None) == B.Z1_EINVAL
    assert B.lib.z1_pack_destroy(None) == B.Z1_OK
    assert B.lib.z1_grad_norm_sq_acc(None, None, None) == B.Z1_EINVAL


from hypothesis import given, settings, strategies as st


@settings(max_examples=150, deadline=None)
@given(shapes=st.lists(st.tuples(st.integers(0, 40), st.integers(1, 6)), min_size=0, max_size=12),
       D=st.integers(1, 12), kind=st.sampled_from(["per_tensor", "flat", "dim0"]))
def test_plan_kinds_cover_every_element_once(shapes, D, kind):
    """Across all ranks every element of every tensor is owned exactly once,
    and every rank's arena layout is valid."""
    rows = [r for r, _ in shapes]
    numel = [r * c for r, c in shapes]
    owned = [np.zeros(n, np.int64) for n in numel]
    for r in range(D):
        s, l, off, arena = B.z1_shard_plan(numel, D, r, kind=kind, rows=rows)
        _check_arena(s, l, off, arena)
        for i in range(len(numel)):
            owned[i][s[i]:s[i] + l[i]] += 1
    assert all((o == 1).all() for o in owned)


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No CPU fallback: a copy of the package without libz1.so cannot be
    imported (ImportError naming the missing library)."""
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "mixed_precision_zero_amd")
    dst = tmp_path / "mixed_precision_zero_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "*.so.tmp", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import mixed_precision_zero_amd.binding"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=120,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libz1" in r.stderr


def test_host_allocation_failure_is_a_status():
    """No C++ exception crosses the C interface: a host allocation failure
    inside an entry point returns Z1_ENOMEM.  A child process caps its
    address space just above what it uses, then asks z1_schedule_create for
    the largest table the header allows (2^24 steps, 1.3 GB of host
    staging); the call must return Z1_ENOMEM, not abort."""
    import subprocess
    import sys
    code = "\n".join([
        "import ctypes, resource, sys",
        f"sys.path.insert(0, {ROOT!r})",
        "from mixed_precision_zero_amd import binding as B",
        "vm = [int(l.split()[1]) for l in open('/proc/self/status') if l.startswith('VmSize')][0]",
        "resource.setrlimit(resource.RLIMIT_AS, (vm * 1024 + (256 << 20), resource.RLIM_INFINITY))",
        "hp = B.AdamWHP(1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, 1)",
        "h = ctypes.c_void_p()",
        "st = B.lib.z1_schedule_create(ctypes.byref(h), ctypes.byref(hp), None, 1 << 24, None)",
        "print('status', st, flush=True)",
    ])
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    assert f"status {B.Z1_ENOMEM}" in r.stdout, r.stdout
