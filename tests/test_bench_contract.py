"""bench.py's command-line contract, checked without a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_exits_with_a_message():
    """The step is one rank's shard on one GPU: --gpus N > 1 prints one
    JSON line saying so and exits non-zero, before touching a GPU."""
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
    assert "one GPU" in r.stderr


def test_help_lists_the_run_flags():
    r = subprocess.run([sys.executable, BENCH, "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_kernel_hash_ignores_comments_and_whitespace_only(tmp_path):
    """The hash that attaches counter runs to a kernel source survives
    comment and whitespace edits and changes with any edit to the code."""
    bench = _bench_module()
    base = bench.kernel_source_hash()
    copies = []
    for path in bench.KERNEL_SRCS:
        dst = tmp_path / os.path.basename(path)
        with open(path) as f:
            dst.write_text(f.read())
        copies.append(str(dst))
    bench.KERNEL_SRCS = tuple(copies)
    assert bench.kernel_source_hash() == base
    with open(copies[-1], "a") as f:
        f.write("\n// a trailing comment\n/* and a block\n   comment */\n\n\t \n")
    assert bench.kernel_source_hash() == base
    with open(copies[-1], "a") as f:
        f.write("static int z1_unused_marker;\n")
    assert bench.kernel_source_hash() != base


def test_committed_counters_belong_to_the_kernel_source():
    """profiles/pmc_adamw_llama7b.json was taken on the kernel source as it
    is now, so bench.py reports its traffic; the bytes per AdamW launch lie
    within 1% above the algorithmic 30 B per element of the 7B shard (the
    per-tile tags), and the copy probe that scales the counters moved its
    stated bytes."""
    bench = _bench_module()
    path = os.path.join(ROOT, "profiles", "pmc_adamw_llama7b.json")
    with open(path) as f:
        d = json.load(f)
    assert d["kernel_source_sha"] == bench.kernel_source_hash()
    shard_elems = 842_301_952
    traffic = bench.traffic_from_profiles("llama7b", "adamw")
    assert traffic == d["hbm_bytes_per_launch"]
    assert 1.0 <= traffic / (30 * shard_elems) < 1.01
    k = d["kernels"]["k_copy"]
    assert abs(k["read_bytes"] / d["copy_bytes"] - 1) < 1e-3
    assert abs(k["write_bytes"] / d["copy_bytes"] - 1) < 1e-3
    for name, e in d["kernels"].items():
        if name.startswith("k_adamw_tiles"):
            assert (e["alg_read"], e["alg_write"]) == (16 * shard_elems, 14 * shard_elems), name
            assert 1.0 <= e["ratio"] < 1.01, name
