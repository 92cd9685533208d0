#!/usr/bin/env python3
"""Throughput of the ZeRO-1 shard optimizer step on one MI355X.

One step = the whole path over one batch of synthetic input: the fp32
accumulation of the K micro-batch gradients, the norm (z1_grad_norm_sq) and
the clipped AdamW with the bf16 cast (z1_adamw_step), all through the C ABI.
The default workload is the 7B Llama-shaped list at dp_size 8, rank 3
(842,301,952 shard elements, K = 4).  Inputs are generated on the device
before timing and stay resident in HBM; every timed step does all of the work.

The K gradients are resident, so by default one z1_accum_grads_range(0, K)
call reads all of them in one pass (12 bytes per element for K = 4); the
same step with one z1_accum_grads call per micro-batch (36 bytes per element)
is timed after it and reported under accum_variants.  Both store the same
bits.  --accum slot makes the per-micro-batch form the headline.

Prints ONE JSON line (rank 0).  Besides metric, value, unit, timing and the
workload's config it carries
  roofline      the dominant kernel (AdamW) against the 8 TB/s HBM peak, with
                algorithmic bytes per launch / its mean duration measured with
                events on the launch stream, and the HBM bytes the committed
                counter runs measured for the same kernel source;
  rates         each part of the step (accumulation, AdamW, norm + AdamW, the
                whole step in both accumulation forms) against the peak and
                against the fastest traffic-only probe of the same mix run on
                the step's own buffers;
  cpu_baseline  the CPU oracle timed on --cpu-steps whole-shard steps of the
                same workload on the host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, vendor figure
BYTES_ADAMW = 30                 # read acc, p, m, v (16); write p, m, v (12) + bf16 (2)
BYTES_ACC_FIRST = 6              # read bf16 g (2); write acc (4)
BYTES_ACC_NEXT = 10              # read bf16 g (2) + acc (4); write acc (4)
MAX_SLOTS = 16                   # micro-batch slots per multi-slot pass
PROFILE_DIR = os.path.join(ROOT, "profiles")
# the kernels and the constants that fix their launch shapes
KERNEL_SRCS = tuple(os.path.join(ROOT, "mixed_precision_zero_amd", "csrc", f)
                    for f in ("z1_internal.h", "z1_kernels.hip"))


def accum_bytes(K: int, resident: bool) -> int:
    """Algorithmic bytes per shard element of the K accumulation passes."""
    if not resident:
        return BYTES_ACC_FIRST + BYTES_ACC_NEXT * (K - 1)
    total, k = 0, 0
    while k < K:   # the library's split: passes of at most 16 slots, as even as possible
        left = K - k
        passes = (left + MAX_SLOTS - 1) // MAX_SLOTS
        g = (left + passes - 1) // passes
        total += 2 * g + (4 if k == 0 else 8)
        k += g
    return total


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama7b")
    ap.add_argument("--chunk", type=int, default=0, help="chunk_elems (0 = library default)")
    ap.add_argument("--max-blocks", type=int, default=0)
    ap.add_argument("--cpu-steps", type=int, default=3,
                    help="whole-shard steps of the CPU oracle timed on the host cores "
                         "(0 = skip)")
    ap.add_argument("--copy-gb", type=float, default=4.0, help="probe-copy size for the ceiling")
    ap.add_argument("--plan", default="per_tensor", choices=["per_tensor", "flat", "dim0"],
                    help="shard plan kind")
    ap.add_argument("--mup", action="store_true",
                    help="per-tensor muP lr multipliers and no decay on norms")
    ap.add_argument("--accum", default="resident", choices=["resident", "slot"],
                    help="resident (default): the K resident micro-batch gradients in one "
                         "z1_accum_grads_range call (up to 16 slots per pass); slot: one "
                         "z1_accum_grads call per micro-batch; the other form is timed too "
                         "and reported beside")
    ap.add_argument("--layout", default="packed", choices=["full", "packed"],
                    help="bf16 weights and gradients as packed shards in arena order "
                         "(default: the reduce-scatter's output and the all-gather's input) "
                         "or as full-size tensors; the other layout is timed too and "
                         "reported beside")
    ap.add_argument("--walk", default="auto", choices=["auto", "chunks", "arena_tiles"],
                    help="how the AdamW step walks the shard (z1_walk; auto: the arena "
                         "tiles of a plan with at most 1%% boundary tiles, else the chunk "
                         "table)")
    ap.add_argument("--layout-steps", type=int, default=10,
                    help="steps timed with the other bf16 layout over the same arenas, "
                         "reported beside the headline (0 = skip)")
    ap.add_argument("--graph-steps", type=int, default=10,
                    help="steps replayed from one captured HIP graph (z1_adamw_step_scheduled), "
                         "reported beside the eager headline; 0 = skip")
    ap.add_argument("--mode", default="step", choices=["step", "pack"],
                    help="step: the shard step (default); pack: full-tensor accumulation into "
                         "the reduce-scatter send buffer, every element of the model")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """sha256[:16] of the kernel sources (z1_internal.h, then z1_kernels.hip)
    with comments and whitespace removed, so that counters taken on a kernel
    stay attached to it through comment edits and are dropped after any
    change to the code."""
    src = ""
    for path in KERNEL_SRCS:
        with open(path) as f:
            src += f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = re.sub(r"\s+", "", src)
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def traffic_from_profiles(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the kernel source as it is now (else None)."""
    path = os.path.join(PROFILE_DIR, f"pmc_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the shard step is measured on one GPU only; "
                                   "--gpus must be 1", "n_gpus": args.gpus}), flush=True)
        print("bench.py: one rank's ZeRO-1 shard step runs on one GPU; the collectives "
              "around it (reduce-scatter / all-gather over RCCL) are not implemented",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixed_precision_zero_amd import binding as B
    from mixed_precision_zero_amd import workloads as W
    from mixed_precision_zero_amd.shard import ShardStep

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.workload]
    log = lambda m: print(m, file=sys.stderr, flush=True)  # noqa: E731
    if args.mode == "pack":
        return bench_pack(args, w, dev, log)

    t0 = time.time()
    lr_s = wd_s = None
    if args.mup:
        lr_s, wd_s = W.mup_multipliers(w.shapes, w.shapes[0][1])
    st = ShardStep(w.shapes, w.dp_size, w.rank, w.n_micro, device=dev,
                   chunk_elems=args.chunk, max_blocks=args.max_blocks, kind=args.plan,
                   lr_scale=lr_s, wd_scale=wd_s, layout=args.layout, walk=args.walk)
    L = int(st.plan.info.shard_elems)
    master_full = W.make_master(w, seed=0, device=dev)
    st.scatter_to_arena(st.master, master_full)
    st.load_weights(master_full)
    del master_full
    for k in range(w.n_micro):
        W.make_micro_grads(w, 1, k, seed=0, device=dev, out=st.grads[k])
        st.stage_grads(k)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: L={L} chunks={st.plan.info.n_chunks} setup {time.time() - t0:.1f}s")

    hp = w.hp()
    stream = torch.cuda.current_stream()

    def one_step(t, resident, ev=None):
        # events: before the accumulation, after it, after the norm, after AdamW
        if ev is not None:
            ev[0].record(stream)
        if resident:
            st.accumulate_range(0, w.n_micro)
        else:
            for k in range(w.n_micro):
                st.accumulate(k)
        if ev is not None:
            ev[1].record(stream)
        st.norm()
        if ev is not None:
            ev[2].record(stream)
        st.adamw(hp, step=t)
        if ev is not None:
            ev[3].record(stream)

    def timed(resident, warmup, steps, t0):
        for t in range(t0, t0 + warmup):
            one_step(t, resident)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record(stream)
        for s_ in range(steps):
            one_step(t0 + warmup + s_, resident, evs[s_])
        stop.record(stream)
        torch.cuda.synchronize()
        wall_ = time.perf_counter() - wall0
        span = lambda a, b: np.array([e[a].elapsed_time(e[b]) for e in evs])  # noqa: E731
        return {"ms_step": start.elapsed_time(stop) / steps, "wall": wall_,
                "accum": span(0, 1), "norm": span(1, 2), "adamw": span(2, 3),
                "step": span(0, 3), "t_next": t0 + warmup + steps}

    head_resident = args.accum == "resident"
    r = timed(head_resident, args.warmup, args.steps, 1)
    alt_steps = min(args.steps, 10)
    alt = timed(not head_resident, min(args.warmup, 3), alt_steps, r["t_next"]) \
        if alt_steps > 0 else None
    ms_step, wall = r["ms_step"], r["wall"]
    norm_ms, adam_ms = r["norm"], r["adamw"]
    adam_avg = float(adam_ms.mean())
    log("[bench] per-step ms: " + " ".join(f"{x:.3f}" for x in r["step"]))
    log(f"[bench] k_adamw ms: mean {adam_avg:.4f} median {float(np.median(adam_ms)):.4f} "
        f"min {float(adam_ms.min()):.4f} max {float(adam_ms.max()):.4f}")
    accum_ms = float(r["accum"].mean())

    def variant(x, resident):
        b = (accum_bytes(w.n_micro, resident) + BYTES_ADAMW) * L
        return {"calls": "one z1_accum_grads_range(0, K)" if resident
                else "one z1_accum_grads per micro-batch",
                "steps": len(x["step"]), "ms_per_step": x["ms_step"],
                "params_per_s": L / (x["ms_step"] / 1e3),
                "accum_ms": float(x["accum"].mean()), "adamw_ms": float(x["adamw"].mean()),
                "bytes_per_param": b // L if L else None,
                "step_hbm_GBps": b / (x["ms_step"] / 1e3) / 1e9,
                "accum_hbm_GBps": accum_bytes(w.n_micro, resident) * L /
                (float(x["accum"].mean()) / 1e3) / 1e9}
    variants = {("resident" if head_resident else "slot"): variant(r, head_resident)}
    if alt is not None:
        variants["slot" if head_resident else "resident"] = variant(alt, not head_resident)

    # the headline step captured once in a HIP graph (with a per-step schedule
    # for t and lr) and replayed: same work, no host enqueue per step
    graph = None
    if args.graph_steps > 0:
        t0 = (alt["t_next"] if alt is not None else r["t_next"])
        warm = 2
        sched = B.z1_schedule_create(**hp, step=t0, n_steps=warm + args.graph_steps)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            if head_resident:
                st.accumulate_range(0, w.n_micro)
            else:
                for k in range(w.n_micro):
                    st.accumulate(k)
            st.norm()
            st.adamw_scheduled(sched)
        for _ in range(warm):
            gr.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.graph_steps):
            gr.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        next_t, overrun = B.z1_schedule_query(sched)
        gms = g0.elapsed_time(g1) / args.graph_steps
        graph = {"steps": args.graph_steps, "ms_per_step": gms, "params_per_s": L / (gms / 1e3),
                 "schedule_next_step": next_t, "schedule_overrun": overrun}
        del gr
        sched.close()

    # the other bf16 layout over the same fp32 arenas: a second plan, the
    # headline step (resident or per call) for a few steps, reported beside
    other_layout = "full" if args.layout == "packed" else "packed"
    layout_variants = {args.layout: {"ms_per_step": ms_step, "adamw_ms": adam_avg,
                                     "accum_ms": accum_ms}}
    if args.layout_steps > 0:
        rows = st.rows if args.plan == "dim0" else None
        if other_layout == "full":
            w2, g2 = st.weights, st.grads
        else:
            w2 = torch.zeros(st.arena_elems, dtype=torch.bfloat16, device=dev)
            g2 = [torch.zeros(st.arena_elems, dtype=torch.bfloat16, device=dev)
                  for _ in range(w.n_micro)]
            for k in range(w.n_micro):
                st.scatter_to_arena(g2[k], st.grads[k])
        plan2 = B.z1_plan_create(st.numel, w.dp_size, w.rank, w2, g2, st.master, st.exp_avg,
                                 st.exp_avg_sq, st.acc, chunk_elems=args.chunk,
                                 max_blocks=args.max_blocks, kind=args.plan, rows=rows,
                                 lr_scale=lr_s, wd_scale=wd_s, layout=other_layout)
        t2 = (alt["t_next"] if alt is not None else r["t_next"])
        ev2 = []
        for j in range(2 + args.layout_steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            if head_resident:
                B.z1_accum_grads_range(plan2, 0, w.n_micro)
            else:
                for k in range(w.n_micro):
                    B.z1_accum_grads(plan2, k)
            B.z1_grad_norm_sq(plan2, st.d_S)
            e[1].record(stream)
            B.z1_adamw_step(plan2, d_S=st.d_S, step=t2 + j, **hp)
            e[2].record(stream)
            if j >= 2:
                ev2.append(e)
        torch.cuda.synchronize()
        step2 = np.array([e[0].elapsed_time(e[2]) for e in ev2])
        adam2 = np.array([e[1].elapsed_time(e[2]) for e in ev2])
        layout_variants[other_layout] = {"ms_per_step": float(step2.mean()),
                                         "adamw_ms": float(adam2.mean()),
                                         "accum_norm_ms": float((step2 - adam2).mean()),
                                         "steps": args.layout_steps}
        plan2.close()
        del w2, g2

    # the CPU oracle on the whole shard, from the GPU's current state and the
    # step's gradients (copied to the host before the probes below overwrite
    # the arenas)
    cpu = None
    if args.cpu_steps > 0:
        import oracle
        o = oracle.get()
        c_copy = time.perf_counter()

        def shard_grads(k):
            if st.layout == "packed":
                return st.packed(st.g_packed[k])
            return torch.cat([st.grads[k][i].reshape(-1)[a:a + n]
                              for i, a, n, _ in st.slices() if n])
        g_host = np.empty((w.n_micro, L), np.uint16)
        for k in range(w.n_micro):
            g_host[k] = shard_grads(k).view(torch.int16).cpu().numpy().view(np.uint16)
        p_h, m_h, v_h = (st.packed(x).cpu().numpy() for x in (st.master, st.exp_avg,
                                                               st.exp_avg_sq))
        acc_h = np.empty(L, np.float32)
        w_h = np.empty(L, np.uint16)
        segments = None
        if args.mup:
            rows_o = [s_[0] if len(s_) else 1 for s_ in w.shapes]
            _, o_len = o.plan(args.plan, w.numel, rows_o, w.dp_size, w.rank)
            segments = (o_len, lr_s, wd_s)
        c_copy = time.perf_counter() - c_copy
        t_cpu = (alt["t_next"] if alt is not None else r["t_next"]) + 100
        c0 = time.perf_counter()
        for j in range(args.cpu_steps):
            o.step(g_host, p_h, m_h, v_h, step=t_cpu + j, acc=acc_h, w=w_h,
                   segments=segments, **hp)
        cpu_s = (time.perf_counter() - c0) / args.cpu_steps
        cpu = {"value": L / cpu_s, "unit": "params/s", "cores": o.num_threads(),
               "kind": "oracle",
               "sample": f"{args.cpu_steps} whole-shard steps of the {w.name} shard "
                         f"({L} elements, K={w.n_micro}): accumulate, norm, clip, AdamW, "
                         f"bf16 cast; binary64 C oracle, not a tuned CPU optimizer",
               "ms_per_step": cpu_s * 1e3, "host_copy_s": c_copy,
               "cpu_model": _cpu_model()}
        del g_host, p_h, m_h, v_h, acc_h, w_h
        log(f"[bench] cpu oracle: {cpu_s * 1e3:.0f} ms per whole-shard step "
            f"({cpu['cores']} threads)")

    value = L / (ms_step / 1e3)
    adam_bytes = BYTES_ADAMW * L
    achieved = adam_bytes / (adam_avg / 1e3) / 1e9
    traffic = traffic_from_profiles(w.name, "adamw")
    h3_bytes = (accum_bytes(w.n_micro, head_resident) + BYTES_ADAMW) * L

    # ceilings: traffic-only streaming kernels (z1_probe*) on this machine, after the
    # timed steps (they overwrite the step's buffers)
    def timed_gbps(fn, nbytes, reps=6):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9

    ceilings = None
    if args.copy_gb > 0:
        nbytes = int(args.copy_gb * 1e9) // 16 * 16
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        sink = torch.zeros(4, dtype=torch.float32, device=dev)
        nv = nbytes // 16
        ceilings = {
            "read": timed_gbps(lambda: B.z1_probe("read", [src, sink], nv), nbytes),
            "write": timed_gbps(lambda: B.z1_probe("write", [dst], nv), nbytes),
            "copy": timed_gbps(lambda: B.z1_probe_copy(src, dst, nbytes), 2 * nbytes),
        }
        del src, dst
        nvL = L // 4
        half = torch.empty(nvL * 4, dtype=torch.bfloat16, device=dev)
        # the AdamW mix over the step's own buffers: the four fp32 arenas and
        # the bf16 weight buffer the step writes (the packed shard, or the
        # start of the flat full-size weight buffer), so placement is shared
        w_buf = (st.w_packed if st.layout == "packed"
                 else st.weights[0].untyped_storage().data_ptr())
        adam_bufs = [st.acc, st.master, st.exp_avg, st.exp_avg_sq, w_buf]
        for kind in ("adamw_traffic", "adamw_traffic_wave"):
            ceilings[kind] = timed_gbps(lambda: B.z1_probe(kind, adam_bufs, nvL), 30 * 4 * nvL)
        ceilings["accum_traffic"] = timed_gbps(
            lambda: B.z1_probe("accum_traffic", [half, st.acc], nvL), 10 * 4 * nvL)
        if head_resident and 2 <= w.n_micro <= MAX_SLOTS:
            # the step's own gradient slots (packed shards, or the start of
            # each flat full-size gradient buffer) and acc arena
            slots = ([g for g in st.g_packed] if st.layout == "packed" else
                     [st.grads[k][0].untyped_storage().data_ptr() for k in range(w.n_micro)])
            for kind in ("slots_traffic", "slots_traffic_one"):
                ceilings[kind] = timed_gbps(lambda: B.z1_probe(kind, slots + [st.acc], nvL),
                                            (2 * w.n_micro + 4) * 4 * nvL)
            del slots
        del half
    # k_adamw's own chunk walk over the step's own buffers with no arithmetic
    # (z1_probe_plan): the same-traffic ceiling on exactly this placement
    twin_gbps = None
    if args.copy_gb > 0:
        twin_gbps = timed_gbps(lambda: B.z1_probe_plan(st.plan), BYTES_ADAMW * L)
    copy_gbps = ceilings["copy"] if ceilings else None

    # GB/s of each timed piece: algorithmic bytes / mean time, as a fraction of
    # the 8 TB/s peak and of the fastest traffic-only probe with the same
    # read/write mix measured in this process (where one exists)
    def rate(nbytes, ms, probes=()):
        gbps = nbytes / (ms / 1e3) / 1e9
        have = [(ceilings[k], k) for k in probes if ceilings and ceilings.get(k)]
        ref, name = max(have) if have else (None, None)
        return {"GBps": gbps, "frac_of_peak": gbps / HBM_PEAK_GBPS,
                "same_mix_probe": name,
                "frac_of_same_mix_probe": (gbps / ref) if ref else None}
    acc_b = accum_bytes(w.n_micro, head_resident) * L
    norm_avg = float(norm_ms.mean())
    acc_probes = (("slots_traffic", "slots_traffic_one")
                  if head_resident and 2 <= w.n_micro <= MAX_SLOTS
                  else () if head_resident else ("accum_traffic",))
    adam_probes = ("adamw_traffic", "adamw_traffic_wave")
    rates = {"accum_all_K": rate(acc_b, accum_ms, acc_probes),
             "adamw": rate(BYTES_ADAMW * L, adam_avg, adam_probes),
             "H1_norm_plus_adamw": rate(BYTES_ADAMW * L, adam_avg + norm_avg, adam_probes),
             "H3_step": rate(acc_b + BYTES_ADAMW * L, ms_step)}
    if "slot" in variants:
        # the step with one accumulation call per micro-batch (10K + 26 bytes
        # per element), timed in the same process beside the headline
        x = alt if head_resident else r
        rates["H3_per_call"] = rate((accum_bytes(w.n_micro, False) + BYTES_ADAMW) * L,
                                    x["ms_step"])

    out = {
        "metric": ("optimizer-step params/s and achieved HBM GB/s (% of MI355X peak), 7B shard"
                   if w.name == "llama7b" else
                   f"optimizer-step params/s and achieved HBM GB/s (% of MI355X peak), "
                   f"{w.name} shard"),
        "metric_detail": "value = shard params / step time; the step is K accumulations + "
                         "norm + clipped AdamW + bf16 cast; GB/s and % of peak are under "
                         "roofline (dominant kernel) and rates (each part of the step)",
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "dtype_detail": "binary64 AdamW update (the dominant kernel) on fp32 master/m/v; "
                        "binary32 accumulation of bf16 gradients; bf16 weights out",
        "data": "synthetic",
        "config": {"workload": w.name, "params": w.total_params, "shard_elems": L,
                   "dp_size": w.dp_size, "rank": w.rank, "micro_batches": w.n_micro,
                   "chunk_elems": int(st.plan.info.chunk_elems),
                   "n_chunks": int(st.plan.info.n_chunks), "plan": args.plan,
                   "mup": bool(args.mup), "accum": args.accum, "layout": args.layout,
                   "adamw_walk": "arena_tiles" if st.plan.info.adamw_tiles else "chunks",
                   "adamw_tiles": int(st.plan.info.adamw_tiles),
                   "boundary_tiles": int(st.plan.info.boundary_tiles)},
        "roofline": {"bound": "hbm",
                     "kernel": "k_adamw_tiles" if st.plan.info.adamw_tiles else "k_adamw",
                     "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "bytes_per_param": BYTES_ADAMW,
                     "launch_ms": adam_avg,
                     "same_traffic_twin_GBps": twin_gbps,
                     "vs_same_traffic_ceiling": (achieved / twin_gbps) if twin_gbps else None},
        "plan_create_ms": st.plan_create_s * 1e3,
        "plan_create_detail": "the shard plan and chunk table built on the host and uploaded "
                              "once per parameter list (z1_plan_create); not part of the step",
        "kernels_ms": {"accum_all_K": accum_ms, "norm_fin": float(norm_ms.mean()),
                       "adamw": adam_avg, "adamw_median": float(np.median(adam_ms))},
        "rates": rates,
        "accum_variants": variants,
        "layout_variants": layout_variants,
        "graph_replay": graph,
        "step_hbm_GBps": h3_bytes / (ms_step / 1e3) / 1e9,
        "step_bytes_per_param": h3_bytes // L if L else None,
        "optimizer_step_params_per_s": L / ((adam_avg + float(norm_ms.mean())) / 1e3),
        "adamw_34B_equivalent_GBps": 34 * L / (adam_avg / 1e3) / 1e9,
        "copy_probe_GBps": copy_gbps,
        "ceilings_GBps": ceilings,
        "wall_s": wall,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    st.close()


def bench_pack(args, w, dev, log):
    """Full-tensor accumulation into the reduce-scatter send buffer (the step
    before the shard path): every element of the model, K passes, the last
    dividing by dp_size."""
    import numpy as np
    import torch

    from mixed_precision_zero_amd import binding as B
    from mixed_precision_zero_amd import workloads as W
    from mixed_precision_zero_amd.shard import flat_views
    rows = [s[0] for s in w.shapes] if args.plan == "dim0" else None
    seg = B.z1_pack_layout(w.numel, w.dp_size, args.plan, rows)
    send = torch.zeros(w.dp_size * seg, dtype=torch.float32, device=dev)
    grads = []
    for k in range(w.n_micro):
        gk = flat_views(w.shapes, dtype=torch.bfloat16, device=dev)   # one buffer per slot
        W.make_micro_grads(w, 1, k, seed=0, device=dev, out=gk)
        grads.append(gk)
    pack = B.z1_pack_create(w.numel, w.dp_size, grads, send, kind=args.plan, rows=rows,
                            divide=True, chunk_elems=args.chunk)
    stream = torch.cuda.current_stream()
    K = w.n_micro

    resident = args.accum == "resident"

    def one(ev=None):
        if resident:
            if ev is not None:
                ev[0].record(stream)
            B.z1_pack_accum_range(pack, 0, K)
            if ev is not None:
                ev[1].record(stream)
            return
        for k in range(K):
            if ev is not None:
                ev[k].record(stream)
            B.z1_pack_accum(pack, k)
        if ev is not None:
            ev[K].record(stream)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    n_ev = 2 if resident else K + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
           for _ in range(args.steps)]
    for s in range(args.steps):
        one(evs[s])
    torch.cuda.synchronize()
    per = np.array([[evs[s][k].elapsed_time(evs[s][k + 1]) for k in range(n_ev - 1)]
                    for s in range(args.steps)])
    step_ms = float(per.sum(1).mean())
    psi = w.total_params
    byts = accum_bytes(K, resident) * psi
    if resident:
        kernels = {"pack_all_K": step_ms}
        kname, achieved = "k_accum_slots (pack)", byts / (step_ms / 1e3) / 1e9
    else:
        first_ms = float(per[:, 0].mean())
        next_ms = float(per[:, 1:].mean()) if K > 1 else None
        kernels = {"pack_first": first_ms, "pack_next": next_ms}
        kname = "k_accum (pack, k>=1)"
        achieved = (10 * psi / (next_ms / 1e3) / 1e9) if next_ms else \
            (6 * psi / (first_ms / 1e3) / 1e9)
    out = {"metric": "pack params/s (full-tensor fp32 accumulation into the reduce-scatter "
                     "send buffer, last pass / dp_size)",
           "value": psi / (step_ms / 1e3), "unit": "params/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "dtype_detail": "binary32 accumulation of bf16 gradients",
           "data": "synthetic",
           "config": {"workload": w.name, "params": psi, "dp_size": w.dp_size,
                      "micro_batches": K, "plan": args.plan, "seg_elems": seg,
                      "accum": args.accum},
           "kernels_ms": kernels,
           "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved,
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "traffic": None},
           "bytes_per_param": byts // psi,
           "step_hbm_GBps": byts / (step_ms / 1e3) / 1e9}
    out["roofline"]["frac"] = out["roofline"]["achieved"] / HBM_PEAK_GBPS
    print(json.dumps(out), flush=True)
    pack.close()


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
