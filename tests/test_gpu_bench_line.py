"""bench.py on a GPU, run as a child process on the tiny workload: the one
JSON line carries every field of its contract (value, timing, roofline with
its HBM peak, the CPU oracle's baseline, the workload's config)."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.parametrize("walk", ["auto", "arena_tiles"])
def test_bench_line_contract(walk):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, BENCH, "--workload", "tiny", "--steps", "3", "--warmup", "1",
                        "--cpu-steps", "1", "--copy-gb", "0.25", "--layout-steps", "2",
                        "--graph-steps", "2", "--walk", walk],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["unit"] == "params/s" and d["value"] > 0 and d["higher_is_better"] is True
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 3, 1)
    assert d["ms_per_step"] > 0 and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["dtype"] == "f64" and "synthetic" in d["data"]
    c = d["config"]
    assert c["workload"] == "tiny" and c["layout"] == "packed"
    assert c["adamw_walk"] == ("arena_tiles" if walk == "arena_tiles" else "chunks")
    assert (c["adamw_tiles"] > 0) == (walk == "arena_tiles")
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    assert rf["kernel"] == ("k_adamw_tiles" if walk == "arena_tiles" else "k_adamw")
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["unit"] == "params/s" and "whole-shard" in cb["sample"]
    rates = d["rates"]
    assert rates["adamw"]["same_mix_probe"] in ("adamw_traffic", "adamw_traffic_wave")
    # both forms of the whole step: the headline (resident slots) and the one
    # with an accumulation call per micro-batch, each over its own bytes
    v = d["accum_variants"]
    assert abs(rates["H3_step"]["GBps"] - v["resident"]["step_hbm_GBps"]) < 1e-9 * v["resident"]["step_hbm_GBps"]
    assert abs(rates["H3_per_call"]["GBps"] - v["slot"]["step_hbm_GBps"]) < 1e-9 * v["slot"]["step_hbm_GBps"]
