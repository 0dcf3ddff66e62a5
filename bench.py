#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer served from per-layer GPU expert slots.

    python bench.py [--steps K] [--warmup W] [--workload gemma|qwen|qwen_b2|qwen_b4|large|prefill|tiny]

One step = one batch (decode: one token per stream; prefill: one ubatch) through
every layer of the workload, layer after layer, through the C ABI.  The default
workload is the Gemma-4-26B-A4B-like decode (30 layers, d_model 2816, d_ff 704,
128 experts, top-8, 32 slots per layer, LRU, batch 1, misses computed on the
host cores while their slot fills stream in the background; `--miss-mode
stream` streams them into slots first).

Prints one JSON line.  `value` = MoE-layer tokens/s (tokens x layers / wall
time) over exactly K timed steps, inputs resident in HBM and expert weights in
the library's page-locked host arena before the timed region starts.  Then the
same number of further steps runs with the library bracketing every kernel
launch with HIP events on the stream it launches on (recording them inside the
timed region would cost ~30% of the throughput, since the host enqueues on the
critical path).  `roofline` is the decode expert GEMV (gate/up + SwiGLU and
down launches of a call taken together: expert bytes read / their device time)
against HBM, or for prefill the grouped GEMM against the fp16 matrix-core peak;
`roofline_fill` is the slot-fill kernel against PCIe Gen5 x16 when misses are
streamed (it then holds the most device time, `dominant_kernel_by_device_time`);
with host misses the fills run on the copy engines
(`extra.fill_copy_engine_GB_per_s`).  `traffic` comes from the
rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in profiles/pmc_traffic.json
and is null when the kernel source changed since.  The oracle is timed on a
bounded sample of the same workload as the CPU baseline.

    python bench.py --copy-calibration   # plain 256 MiB device copies, for PMC scaling
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
PCIE_PEAK_GBS = 64.0             # PCIe Gen5 x16, one direction
MFMA_F16_PEAK_TFLOPS = 2500.0    # dense fp16 / bf16 matrix cores
KERNEL_SRC = os.path.join(ROOT, "expert_cache_host_amd", "csrc", "kernels.hip")
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
# the library's kernel ids -> kernel names in rocprofv3 output
KERNEL_SYMBOL = {"gateup": "q4_gateup_kernel", "down": "q4_down_kernel", "fill": "pull_kernel",
                 "router": "router_decode_kernel", "topk": "topk_decode_kernel", "combine": "combine_kernel"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pick_workload(name):
    import synth
    if name.startswith("qwen_b"):
        return synth.qwen_batch(int(name[len("qwen_b"):]))
    return synth.WORKLOADS[name]


def describe(wl):
    kind = "prefill ubatch" if wl.rho is None else f"decode b={wl.batch}"
    miss = wl.miss_mode + " misses"
    sh = f" + {wl.n_shared} shared" if wl.n_shared else ""
    return (f"{wl.name}: {wl.layers} layers, d_model {wl.d_model}, d_ff {wl.d_ff}, "
            f"{wl.n_experts} experts{sh}, top-{wl.top_k}, {wl.slots} slots/layer, {kind} "
            f"({wl.batch} tokens/call), {miss}")


def kernel_source_hash() -> str:
    import hashlib
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def pmc_traffic(workload: str, kernel: str, launches: int, bytes_per_launch: float):
    """Calibrated FETCH+WRITE bytes per launch for `kernel`, or None."""
    try:
        data = json.load(open(PMC_FILE))
    except (OSError, ValueError):
        return None
    if data.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    ent = data.get("workloads", {}).get(workload, {}).get(kernel)
    if not ent:
        return None
    return (ent["fetch_KiB"] * data["fetch_scale"] + ent["write_KiB"] * data["write_scale"]) * 1024.0


def copy_calibration():
    """Plain device-to-device copies of known size (rocprofv3 --pmc scaling)."""
    import torch
    n = 256 << 20
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}))


def probes(torch, dev, launch_bytes, record_bytes):
    """References measured on this GPU outside the timed region, each operation
    timed alone between two events on its stream: device-to-device copies
    (torch copy_, the runtime's copy kernel; read + write bytes counted, the
    STREAM convention) of `launch_bytes` (the bytes one decode GEMV pair reads)
    and of 1 GiB, every slice fresh (rotating over 2 x 2 GiB, far more than the
    256 MB last-level cache), and page-locked host -> device copies of one
    expert record."""
    res = {"op": "torch copy_ device-to-device (read + write bytes) and from pinned host memory"}
    pool = torch.empty((4 << 30) // 4, dtype=torch.float32, device=dev)
    half = pool.numel() // 2

    def timed(fn, reps):
        evs = []
        for i in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(i)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) * 1e-3 / reps

    def copy_rate(nbytes, reps):
        n = max(1, nbytes // 4)
        k = half // n
        fn = lambda i: pool[half + (i % k) * n:half + (i % k + 1) * n].copy_(
            pool[((i + 1) % k) * n:((i + 1) % k + 1) * n])
        fn(0)
        return 2 * n * 4 / timed(fn, reps) / 1e9

    if launch_bytes:
        res["copy_bytes_per_op"] = int(launch_bytes)
        res["copy_GB_per_s"] = copy_rate(int(launch_bytes), 12)
    res["copy_GB_per_s_1GiB"] = copy_rate(1 << 30, 6)
    del pool
    src = torch.empty(record_bytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(record_bytes, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    res["h2d_record_bytes"] = record_bytes
    res["h2d_GB_per_s"] = record_bytes / timed(lambda i: dst.copy_(src, non_blocking=True), 8) / 1e9
    return res


def cpu_baseline(wl, weights, routers, hidden, budget_s=12.0, max_calls=64):
    """The oracle, as it stands, on the first calls of layer 0 until ~budget_s."""
    from oracle.layer import moe_layer
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    lb = weights[:wl.layer_bytes]
    w_r, b = routers[0]
    n = 0
    t0 = time.perf_counter()
    while n < max_calls and n < hidden[0].shape[0]:
        moe_layer(hidden[0][n], w_r, b, lb, wl.d_model, wl.d_ff, wl.n_experts, wl.top_k,
                  n_shared=wl.n_shared)
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": n * wl.batch / dt, "unit": "layer-tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {n} calls of layer 0 ({n * wl.batch} tokens), fp64 numpy, {dt:.1f} s"}


def preload_study(args, first=32, profile_calls=128):
    """The usage-profile preload on the workload's own routing: a profile gathered
    on the last `profile_calls` calls of every layer (standing in for earlier runs)
    is preloaded into a fresh cache, and the hit rate of the first `first` calls is
    compared with a cold cache (slot s holds expert s)."""
    import torch
    import expert_cache_host_amd as m
    import synth
    wl = pick_workload(args.workload)
    if args.miss_mode is not None:
        import dataclasses
        wl = dataclasses.replace(wl, miss_mode=args.miss_mode)
    n = wl.calls_per_layer
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    weights = synth.gen_all_weights(wl)
    routers = [synth.gen_router(wl, l) for l in range(wl.layers)]
    hidden = [synth.gen_hidden(wl, l, n) for l in range(wl.layers)]
    w_d = [torch.from_numpy(w).to(dev) for w, _ in routers]
    b_d = [torch.from_numpy(b).to(dev) if b is not None else None for _, b in routers]
    x_d = [torch.from_numpy(h).to(dev) for h in hidden]
    out = torch.empty((wl.batch, wl.d_model), dtype=torch.float32, device=dev)

    def new_cache():
        return m.MoECache(wl.layers, wl.n_experts, wl.slots, wl.d_model, wl.d_ff, weights,
                          top_k=wl.top_k, miss_mode=wl.miss_mode, n_shared=wl.n_shared,
                          policy=args.policy, max_fills_per_call=args.max_fills)

    def run(cache, calls):
        cache.reset_stats()
        for s in calls:
            for l in range(wl.layers):
                cache.forward(l, x_d[l][s], w_d[l], b_d[l], out=out)
        torch.cuda.synchronize()
        cache.sync()
        st = cache.stats()
        return st["hits"] / max(1, st["selections"])

    c = new_cache()
    run(c, range(n - profile_calls, n))
    counts = c.usage()
    c.close()
    c = new_cache()
    cold = run(c, range(first))
    c.close()
    c = new_cache()
    c.preload(counts)
    warm = run(c, range(first))
    c.close()
    print(json.dumps({"study": "usage-profile preload", "workload": describe(wl),
                      "slot_policy": args.policy, "profile": f"calls {n - profile_calls}..{n - 1} of every layer",
                      "first_calls": first, "hit_rate_cold": cold, "hit_rate_preloaded": warm}), flush=True)


def preheat_study(args, prompt_ubatches=24, decode_tokens=256, adopts=(-1, 500, 1000)):
    """Prefill preheat: a prompt of `prompt_ubatches` ubatches of 512 tokens, then
    `decode_tokens` single-token decode calls, through every layer of the large
    shape (stream misses), with the decode workload's router (Zipf bias, so
    expert popularity persists) in both phases.  Reports per adopt share (-1 =
    off) the prompt time, the decode hit rate and the decode layer-tokens/s."""
    import torch
    import expert_cache_host_amd as m
    import synth
    dec = synth.WORKLOADS["large"]
    pre = synth.WORKLOADS["prefill"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    weights = synth.gen_all_weights(dec)
    routers = [synth.gen_router(dec, l) for l in range(dec.layers)]
    w_d = [torch.from_numpy(w).to(dev) for w, _ in routers]
    b_d = [torch.from_numpy(b).to(dev) if b is not None else None for _, b in routers]
    xp = [torch.from_numpy(synth.gen_hidden(pre, l, prompt_ubatches)).to(dev)
          for l in range(dec.layers)]
    xd = [torch.from_numpy(synth.gen_hidden(dec, l, decode_tokens)).to(dev)
          for l in range(dec.layers)]
    out_p = torch.empty((pre.batch, dec.d_model), dtype=torch.float32, device=dev)
    out_d = torch.empty((1, dec.d_model), dtype=torch.float32, device=dev)
    rows = []
    for adopt in adopts:
        c = m.MoECache(dec.layers, dec.n_experts, dec.slots, dec.d_model, dec.d_ff, weights,
                       top_k=dec.top_k, miss_mode="stream", n_shared=dec.n_shared, adopt=adopt)
        log(f"preheat study: adopt={adopt}, prompt")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for u in range(prompt_ubatches):
            for l in range(dec.layers):
                c.forward(l, xp[l][u], w_d[l], b_d[l], out=out_p)
        torch.cuda.synchronize()
        c.sync()
        t1 = time.perf_counter()
        stp = c.stats()
        c.reset_stats()
        log(f"preheat study: adopt={adopt}, decode")
        first = None
        for s in range(decode_tokens):
            if s == 32:
                torch.cuda.synchronize()
                c.sync()
                st32 = c.stats()
                first = st32["hits"] / max(1, st32["selections"])
            for l in range(dec.layers):
                c.forward(l, xd[l][s], w_d[l], b_d[l], out=out_d)
        torch.cuda.synchronize()
        c.sync()
        t2 = time.perf_counter()
        st = c.stats()
        rows.append({"adopt": adopt, "prompt_s": t1 - t0,
                     "prompt_stages_per_call": stp["stages"] / max(1, stp["calls"]),
                     "prompt_fills": stp["fills"],
                     "decode_hit_rate": st["hits"] / max(1, st["selections"]),
                     "decode_hit_rate_first32": first,
                     "decode_layer_tokens_per_s": decode_tokens * dec.layers / (t2 - t1),
                     "decode_fills_per_call": st["fills"] / max(1, st["calls"])})
        c.close()
    print(json.dumps({"study": "prefill preheat", "shape": describe(dec),
                      "prompt": f"{prompt_ubatches} ubatches of {pre.batch} i.i.d. tokens",
                      "decode": f"{decode_tokens} AR(1) tokens, one per call",
                      "miss_mode": "stream", "results": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="gemma")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--miss-mode", choices=["stream", "host"], default=None,
                    help="override the workload's miss mode")
    ap.add_argument("--policy", choices=["lru", "score"], default="lru",
                    help="slot policy: LRU, or the decayed usage score with admission")
    ap.add_argument("--max-fills", type=int, default=-1,
                    help="host mode: slot fills per call (-1 = every admitted miss)")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without per-kernel events (no roofline)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--preload-study", action="store_true",
                    help="first-call hit rates cold and after preloading a usage profile")
    ap.add_argument("--preheat-study", action="store_true",
                    help="decode after a long prompt, with and without prefill preheat")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.preload_study:
        preload_study(args)
        return
    if args.preheat_study:
        preheat_study(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU (the layer and its cache live on one device); --gpus must be 1"}))
        sys.exit(2)

    import torch
    import expert_cache_host_amd as m
    import synth

    wl = pick_workload(args.workload)
    if args.miss_mode is not None:
        import dataclasses
        wl = dataclasses.replace(wl, miss_mode=args.miss_mode)
    per_layer = wl.calls_per_layer
    if wl.rho is None:
        steps = args.steps if args.steps is not None else 6
        warmup = args.warmup if args.warmup is not None else 1
    else:
        steps = args.steps if args.steps is not None else 224
        warmup = args.warmup if args.warmup is not None else 16
    ev_steps = 0 if args.no_kernel_events else min(steps, per_layer - warmup - steps)
    need = warmup + steps + ev_steps
    if need > per_layer:
        raise SystemExit(f"{wl.name} has {per_layer} calls per layer; warmup+steps = {need}")

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    weights = synth.gen_all_weights(wl)
    log(f"[bench] generated {wl.total_bytes / 1e9:.2f} GB of Q4 experts in "
        f"{time.perf_counter() - t0:.1f} s")
    routers = [synth.gen_router(wl, l) for l in range(wl.layers)]
    hidden = [synth.gen_hidden(wl, l, need) for l in range(wl.layers)]
    t0 = time.perf_counter()
    cache = m.MoECache(wl.layers, wl.n_experts, wl.slots, wl.d_model, wl.d_ff, weights,
                       top_k=wl.top_k, miss_mode=wl.miss_mode, n_shared=wl.n_shared,
                       policy=args.policy, max_fills_per_call=args.max_fills)
    log(f"[bench] cache created (pinned arena + slot preload) in {time.perf_counter() - t0:.1f} s")
    w_d = [torch.from_numpy(w).to(dev) for w, _ in routers]
    b_d = [torch.from_numpy(b).to(dev) if b is not None else None for _, b in routers]
    x_d = [torch.from_numpy(h).to(dev) for h in hidden]          # [calls, batch, d] per layer
    out = torch.empty((wl.batch, wl.d_model), dtype=torch.float32, device=dev)

    def run(step0, n):
        for s in range(step0, step0 + n):
            for l in range(wl.layers):
                cache.forward(l, x_d[l][s], w_d[l], b_d[l], out=out)

    # Warm-up, untimed.  Each call's routing is read back (which waits for the
    # call) for the stickiness |S_t & S_t-1| / k of every stream (decode).
    prev = [None] * wl.layers
    acc = [0, 0]
    for s_ in range(warmup):
        for l in range(wl.layers):
            cache.forward(l, x_d[l][s_], w_d[l], b_d[l], out=out)
            if wl.rho is None:
                continue
            idx, _ = cache.routing(l)
            if prev[l] is not None:
                for b_ in range(idx.shape[0]):
                    acc[0] += len(set(idx[b_].tolist()) & set(prev[l][b_].tolist()))
                    acc[1] += wl.top_k
            prev[l] = idx
    stick = acc[0] / acc[1] if acc[1] else None
    torch.cuda.synchronize()
    st0 = cache.stats()  # the warm-up calls: slots start from the preload
    cache.reset_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(warmup, steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cache.sync()
    st = cache.stats()
    log(f"[bench] timed {steps} steps in {wall:.3f} s")
    ks = {k: (0, 0.0, 0.0) for k in cache.KERNELS}
    if ev_steps > 0:
        cache.reset_stats()
        cache.set_timing(True)
        run(warmup + steps, ev_steps)
        torch.cuda.synchronize()
        cache.set_timing(False)
        cache.sync()
        ks = cache.kernel_stats()
        st2 = cache.stats()
        log(f"[bench] kernel-event pass of {ev_steps} steps done")
    layer_tokens = steps * wl.batch * wl.layers
    value = layer_tokens / wall
    sel = max(1, st["selections"])
    extra = {
        "stack_tokens_per_s": steps * wl.batch / wall,
        "hit_rate": st["hits"] / sel,
        "hit_rate_warmup_calls": st0["hits"] / max(1, st0["selections"]),
        "warmup_calls_per_layer": warmup,
        "stickiness_warmup_calls": stick,
        "fills_per_call": st["fills"] / max(1, st["calls"]),
        "fill_GB": st["fill_bytes"] / 1e9,
        "stages_per_call": st["stages"] / max(1, st["calls"]),
        "plan_us_per_call": 1e6 * st["plan_s"] / max(1, st["calls"]),
        "host_ms_per_call": 1e3 * st["host_s"] / max(1, st["calls"]),
    }
    if ev_steps > 0 and st2["h2d_s"] > 0:
        extra["fill_copy_engine_GB_per_s"] = st2["fill_bytes"] / st2["h2d_s"] / 1e9
    if ks["fill"][0]:
        extra["fill_kernel_GB_per_s"] = ks["fill"][2] / ks["fill"][1] / 1e9

    kernels = {}
    for name, (n, sec, by) in ks.items():
        if n:
            kernels[name] = {"launches": n, "avg_us": 1e6 * sec / n,
                             "GB_per_s": by / sec / 1e9 if sec > 0 else None,
                             "bytes_per_launch": by / n, "device_s": sec}

    def roof_pair(a, b):
        """Two kernels launched back to back per call, taken as one: algorithmic bytes / time."""
        na, sa, ba = ks[a]
        nb_, sb, bb = ks[b]
        if not na or sa + sb <= 0:
            return None
        ach = (ba + bb) / (sa + sb) / 1e9
        tr = [pmc_traffic(f"{wl.name}/{wl.miss_mode}", k, 0, 0) for k in (a, b)]
        traffic = None if None in tr else (tr[0] * na + tr[1] * nb_) / na
        return {"bound": "hbm", "kernel": f"{KERNEL_SYMBOL[a]} + {KERNEL_SYMBOL[b]}",
                "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                "traffic": traffic, "avg_launch_us": 1e6 * (sa + sb) / na, "launches": na,
                "algorithmic_bytes_per_launch": (ba + bb) / na,
                "per_kernel": {a: roof(a, "hbm", HBM_PEAK_GBS, "GB/s"),
                               b: roof(b, "hbm", HBM_PEAK_GBS, "GB/s")}}

    def roof(name, bound, peak, unit):
        n, sec, by = ks[name]
        if not n or sec <= 0:
            return None
        if unit == "TFLOP/s":
            ach = by / sec / 1e12
        else:
            ach = by / sec / 1e9
        tr = pmc_traffic(f"{wl.name}/{wl.miss_mode}", name, n, by / n)
        return {"bound": bound, "kernel": KERNEL_SYMBOL.get(name, name), "achieved": ach,
                "peak": peak, "unit": unit, "frac": ach / peak,
                "traffic": tr, "avg_launch_us": 1e6 * sec / n, "launches": n,
                "algorithmic_bytes_per_launch": by / n}

    roofline = roofline_fill = roofline_mfma = None
    dominant = None
    if kernels:
        dominant = KERNEL_SYMBOL.get(max(kernels, key=lambda k: kernels[k]["device_s"]))
        if wl.batch <= 4:
            # decode: the expert GEMV (gate/up + SwiGLU, then down) on the bytes it reads
            roofline = roof_pair("gateup", "down")
        roofline_fill = roof("fill", "pcie", PCIE_PEAK_GBS, "GB/s")
        if wl.batch > 4 and ks["gateup"][0]:
            # algorithmic flops of the grouped GEMM: 2 * tokens * rows * K per expert
            n, sec, by = ks["gateup"]
            n2, sec2, by2 = ks["down"]
            flops = 2.0 * wl.batch * (wl.top_k + wl.n_shared) * 3 * wl.d_model * wl.d_ff * ev_steps * wl.layers
            t_mm = sec + sec2
            roofline_mfma = {"bound": "mfma", "kernel": "q4_mfma_kernel", "achieved": flops / t_mm / 1e12,
                             "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": flops / t_mm / 1e12 / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                             "avg_launch_us": 1e6 * t_mm / max(1, n + n2), "launches": n + n2,
                             "hbm_GB_per_s": (by + by2) / t_mm / 1e9,
                             "hbm_frac": (by + by2) / t_mm / 1e9 / HBM_PEAK_GBS}
            roofline = roofline_mfma

    launch_bytes = None
    if wl.batch <= 4 and ks["gateup"][0]:
        launch_bytes = (ks["gateup"][2] + ks["down"][2]) / ks["gateup"][0]
    extra["probes"] = probes(torch, dev, launch_bytes, wl.expert_bytes)
    if roofline is not None and launch_bytes and extra["probes"].get("copy_GB_per_s"):
        roofline["vs_copy_probe"] = roofline["achieved"] / extra["probes"]["copy_GB_per_s"]
    if roofline_fill is not None:
        roofline_fill["vs_h2d_probe"] = roofline_fill["achieved"] / extra["probes"]["h2d_GB_per_s"]
    if "fill_copy_engine_GB_per_s" in extra:
        extra["fill_copy_engine_vs_h2d_probe"] = (extra["fill_copy_engine_GB_per_s"] /
                                                  extra["probes"]["h2d_GB_per_s"])

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, weights, routers, hidden)

    line = {
        "metric": "MoE-layer tokens/s (decode b=1)" if wl.rho is not None else
                  "MoE-layer tokens/s (prefill ub=512)",
        "value": value,
        "unit": "layer-tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": 1e3 * wall / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Q4_0 experts ~N(0,0.02), AR(1) hidden states, Zipf router bias)",
        "config": {"workload": describe(wl), "layers": wl.layers, "tokens_per_call": wl.batch,
                   "slot_policy": args.policy, "max_fills_per_call": args.max_fills,
                   "steps_are": "one batch through every layer",
                   "kernel_timing": f"HIP events per launch over {ev_steps} further steps"},
        "roofline": roofline,
        "dominant_kernel_by_device_time": dominant,
        "roofline_fill": roofline_fill,
        "cpu_baseline": cpu,
        "extra": extra,
        "kernels": kernels,
    }
    cache.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
