#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer served from per-layer GPU expert slots.

    python bench.py [--steps K] [--warmup W] [--workload large|prefill|gemma|qwen|qwen_b2|qwen_b4|tiny]

One step = one batch (decode: one token per stream; prefill: one ubatch of 512)
through every layer of the workload, layer after layer, through the C ABI.  The
default workload is the large-expert decode: 8 layers, d_model 6144, d_ff 2048,
256 routed experts + 1 resident shared expert, top-8, 64 slots per layer, LRU,
batch 1, misses computed on the host cores while their slot fills stream over
PCIe in the background (`--miss-mode stream` streams them into slots first).

Prints one JSON line.  `value` = MoE-layer tokens/s (tokens x layers / wall
time) over exactly K timed steps, with inputs resident in HBM and the expert
weights in the library's page-locked host arena before the timed region
starts.  Inside the timed region the two expert GEMV launches of every call
are timed with HIP events on the stream they run on, and nothing else is: a
start / stop pair the launch itself carries (hipExtLaunchKernel) and one event
recorded just before it, each launch's time running from the later start to
the stop: `roofline` is the gate/up + SwiGLU
kernel (the one with the most device time) on the bytes it reads, against HBM;
`roofline_down` the down projection.  A further pass of the same length times
every kernel (`extra.kernels_breakdown_pass`, `dominant_kernel_by_device_time`).
Unless --no-legs, the same line carries two more workloads under `legs`: the
prefill of a 12288-token prompt in ubatches of 512 through the same layer shape
(matrix-core grouped GEMM; HBM and MFMA fractions on algorithmic bytes and
flops) and the Gemma-4-26B-A4B-like decode.  `traffic` comes from the rocprofv3
FETCH_SIZE / WRITE_SIZE runs recorded in profiles/pmc_traffic.json and is null
when the kernel source changed since.  The oracle is timed on a bounded sample
of the headline workload as the CPU baseline, with as many BLAS threads as the
process may use cores.

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
# batches beyond the decode path (more than 4 tokens) take these instead
KERNEL_SYMBOL_GEMM = {**KERNEL_SYMBOL, "gateup": "q4_mfma_kernel<true>", "down": "q4_mfma_kernel<false>",
                      "router": "router_kernel", "topk": "topk_kernel", "remap": "remap_kernel",
                      "prep": "prep_pairs_kernel"}


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


def host_cores():
    """Cores this process may run on; BLAS threads are set to the same count."""
    n = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(n)
    except Exception:  # pragma: no cover
        pass
    return n


def cpu_baseline(wl, weights, routers, hidden, budget_s=15.0, max_calls=64):
    """The oracle, as it stands, on the first calls of layer 0 until ~budget_s."""
    from oracle.layer import moe_layer
    cores = host_cores()
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
    return {"value": n * wl.batch / dt, "unit": "layer-tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {n} calls of layer 0 of {wl.name} ({n * wl.batch} tokens), fp64 "
                      f"numpy with {cores} BLAS threads, {dt:.1f} s"}


DECODE_DTYPE = "int4 x int16 dot (int32 per block, fp32 across blocks); fp32 router, gating, combine"
PREFILL_DTYPE = "fp16 (exact q-8) x fp16 hi+lo MFMA, fp32 accumulate"


def run_leg(wl, weights, steps, warmup, policy="lru", max_fills=-1, breakdown=True,
            with_probes=False, with_cpu=False):
    """One workload through the library: `warmup` untimed steps, then exactly
    `steps` timed steps (one batch through every layer each) with HIP events
    around the expert GEMV launches only, then (breakdown) as many further
    steps with every kernel and the fills timed."""
    import torch
    import expert_cache_host_amd as m
    import synth
    dev = torch.device("cuda:0")
    per_layer = wl.calls_per_layer
    ev_steps = min(steps, per_layer - warmup - steps) if breakdown else 0
    need = warmup + steps + max(0, ev_steps)
    if need > per_layer:
        raise SystemExit(f"{wl.name} has {per_layer} calls per layer; warmup+steps = {need}")
    routers = [synth.gen_router(wl, l) for l in range(wl.layers)]
    hidden = [synth.gen_hidden(wl, l, need) for l in range(wl.layers)]
    t0 = time.perf_counter()
    cache = m.MoECache(wl.layers, wl.n_experts, wl.slots, wl.d_model, wl.d_ff, weights,
                       top_k=wl.top_k, miss_mode=wl.miss_mode, n_shared=wl.n_shared,
                       policy=policy, max_fills_per_call=max_fills)
    log(f"[bench] {wl.name}: cache created (pinned arena + slot preload) in "
        f"{time.perf_counter() - t0:.1f} s")
    w_d = [torch.from_numpy(w).to(dev) for w, _ in routers]
    b_d = [torch.from_numpy(b).to(dev) if b is not None else None for _, b in routers]
    x_d = [torch.from_numpy(h).to(dev) for h in hidden]          # [calls, batch, d] per layer
    del hidden
    out = torch.empty((wl.batch, wl.d_model), dtype=torch.float32, device=dev)
    decode = wl.rho is not None

    def run(step0, n):
        for s_ in range(step0, step0 + n):
            for l in range(wl.layers):
                cache.forward(l, x_d[l][s_], w_d[l], b_d[l], out=out)

    # Warm-up, untimed.  Each decode call's routing is read back (which waits
    # for the call) for the stickiness |S_t & S_t-1| / k of every stream.
    prev = [None] * wl.layers
    acc = [0, 0]
    for s_ in range(warmup):
        for l in range(wl.layers):
            cache.forward(l, x_d[l][s_], w_d[l], b_d[l], out=out)
            if not decode:
                continue
            idx, _ = cache.routing(l)
            if prev[l] is not None:
                for b_ in range(idx.shape[0]):
                    acc[0] += len(set(idx[b_].tolist()) & set(prev[l][b_].tolist()))
                    acc[1] += wl.top_k
            prev[l] = idx
    stick = acc[0] / acc[1] if acc[1] else None
    torch.cuda.synchronize()
    cache.sync()
    st0 = cache.stats()  # the warm-up calls: slots start from the preload
    cache.reset_stats()
    cache.set_kernel_timing(["gateup", "down"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(warmup, steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cache.set_kernel_timing([])
    cache.sync()
    st = cache.stats()
    ks = cache.kernel_stats()
    log(f"[bench] {wl.name}: timed {steps} steps in {wall:.3f} s")
    ks_all, st2 = None, None
    if ev_steps > 0:
        cache.reset_stats()
        cache.set_timing(True)
        run(warmup + steps, ev_steps)
        torch.cuda.synchronize()
        cache.set_timing(False)
        cache.sync()
        ks_all = cache.kernel_stats()
        st2 = cache.stats()
        log(f"[bench] {wl.name}: breakdown pass of {ev_steps} steps done")
    cache.close()

    sel = max(1, st["selections"])
    leg = {
        "workload": describe(wl),
        "value": steps * wl.batch * wl.layers / wall,
        "unit": "layer-tokens/s",
        "stack_tokens_per_s": steps * wl.batch / wall,
        "steps": steps, "warmup": warmup, "ms_per_step": 1e3 * wall / steps,
        "slot_policy": policy, "max_fills_per_call": max_fills,
        "dtype": DECODE_DTYPE if decode and wl.batch * (wl.top_k + wl.n_shared) <= 64 else PREFILL_DTYPE,
        "hit_rate": st["hits"] / sel,
        "hit_rate_warmup_calls": st0["hits"] / max(1, st0["selections"]),
        "warmup_calls_per_layer": warmup,
        "stickiness_warmup_calls": stick,
        "fills_per_call": st["fills"] / max(1, st["calls"]),
        "fill_GB": st["fill_bytes"] / 1e9,
        "fill_GB_per_s_over_timed_region": st["fill_bytes"] / wall / 1e9,
        "stages_per_call": st["stages"] / max(1, st["calls"]),
        "plan_us_per_call": 1e6 * st["plan_s"] / max(1, st["calls"]),
        "host_ms_per_call": 1e3 * st["host_s"] / max(1, st["calls"]),
    }

    names = KERNEL_SYMBOL if decode and wl.batch <= 4 else KERNEL_SYMBOL_GEMM

    def entry(k, src):
        n, sec, by = src[k]
        if not n or sec <= 0:
            return None
        return {"kernel": names.get(k, k), "launches": n, "avg_us": 1e6 * sec / n,
                "algorithmic_bytes_per_launch": by / n, "GB_per_s": by / sec / 1e9, "device_s": sec}

    def hbm_roof(k):
        e = entry(k, ks)
        if e is None:
            return None
        ach = e["GB_per_s"]
        return {"bound": "hbm", "kernel": e["kernel"], "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                "traffic": pmc_traffic(f"{wl.name}/{wl.miss_mode}", k, 0, 0),
                "avg_launch_us": e["avg_us"], "launches": e["launches"],
                "algorithmic_bytes_per_launch": e["algorithmic_bytes_per_launch"],
                "timed": "HIP events on the launch's stream, inside the timed region: the "
                         "launch's own start / stop (hipExtLaunchKernel) and one recorded "
                         "before it, from the later start to the stop"}

    if decode:
        leg["roofline"] = hbm_roof("gateup")
        leg["roofline_down"] = hbm_roof("down")
    else:
        ng, sg, bg = ks["gateup"]
        nd, sd, bd = ks["down"]
        if ng and sg + sd > 0:
            pairs = wl.batch * (wl.top_k + wl.n_shared)
            flops = 2.0 * pairs * 3 * wl.d_model * wl.d_ff * steps * wl.layers
            t_mm = sg + sd
            hbm = (bg + bd) / t_mm / 1e9
            leg["roofline"] = {
                "bound": "hbm", "kernel": "q4_mfma_kernel (gate/up + down, every stage)",
                "achieved": hbm, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": hbm / HBM_PEAK_GBS,
                "traffic": pmc_traffic(f"{wl.name}/{wl.miss_mode}", "mfma", 0, 0),
                "algorithmic_bytes_per_launch": (bg + bd) / max(1, ng + nd), "launches": ng + nd,
                "avg_launch_us": 1e6 * t_mm / max(1, ng + nd),
                "mfma_achieved_TFLOP_per_s": flops / t_mm / 1e12,
                "mfma_peak_TFLOP_per_s": MFMA_F16_PEAK_TFLOPS,
                "mfma_frac": flops / t_mm / 1e12 / MFMA_F16_PEAK_TFLOPS,
                "algorithmic_flops_per_ubatch_layer": flops / (steps * wl.layers),
                "gemm_ms_per_ubatch_layer": 1e3 * t_mm / (steps * wl.layers),
                "per_kernel": {"gateup": entry("gateup", ks), "down": entry("down", ks)},
                "timed": "HIP events on the launch's stream, inside the timed region: the "
                         "launch's own start / stop (hipExtLaunchKernel) and one recorded "
                         "before it, from the later start to the stop"}
    if ks_all is not None:
        kernels = {k: entry(k, ks_all) for k in ks_all if entry(k, ks_all)}
        leg["kernels_breakdown_pass"] = kernels
        if kernels:
            leg["dominant_kernel_by_device_time"] = kernels[max(
                kernels, key=lambda k: kernels[k]["device_s"])]["kernel"]
        if st2 and st2["h2d_s"] > 0:
            leg["fill_copy_spans_GB_per_s"] = st2["fill_bytes"] / st2["h2d_s"] / 1e9
    if with_probes:
        e = entry("gateup", ks)
        leg["probes"] = probes(torch, dev, e["algorithmic_bytes_per_launch"] if e else None,
                               wl.expert_bytes)
        if leg.get("roofline") and leg["probes"].get("copy_GB_per_s"):
            leg["roofline"]["vs_copy_probe"] = leg["roofline"]["achieved"] / leg["probes"]["copy_GB_per_s"]
    if with_cpu:
        leg["cpu_baseline"] = cpu_baseline(wl, weights, routers, [x.cpu().numpy() for x in x_d[:1]])
    del x_d
    torch.cuda.empty_cache()
    return leg


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="large")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="only the headline workload (no prefill / Gemma legs)")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the pass that times every kernel")
    ap.add_argument("--miss-mode", choices=["stream", "host"], default=None,
                    help="override the workload's miss mode")
    ap.add_argument("--policy", choices=["lru", "score"], default="lru",
                    help="slot policy: LRU, or the decayed usage score with admission")
    ap.add_argument("--max-fills", type=int, default=-1,
                    help="host mode: slot fills per call (-1 = every admitted miss)")
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
        print(json.dumps({"error": "this benchmark runs on one GPU (each layer's cache lives on one "
                                   "device; sharding over GPUs is designed, not built): use --gpus 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    import synth

    torch.cuda.set_device(0)
    wl = pick_workload(args.workload)
    if args.miss_mode is not None:
        import dataclasses
        wl = dataclasses.replace(wl, miss_mode=args.miss_mode)
    if wl.rho is None:
        steps = args.steps if args.steps is not None else 6
        warmup = args.warmup if args.warmup is not None else 1
    else:
        steps = args.steps if args.steps is not None else 112
        warmup = args.warmup if args.warmup is not None else 16
    t0 = time.perf_counter()
    weights = synth.gen_all_weights(wl)
    log(f"[bench] generated {wl.total_bytes / 1e9:.2f} GB of Q4 experts in "
        f"{time.perf_counter() - t0:.1f} s")
    head = run_leg(wl, weights, steps, warmup, args.policy, args.max_fills,
                   breakdown=not args.no_breakdown, with_probes=True,
                   with_cpu=not args.no_cpu_baseline)
    legs = {}
    if not args.no_legs and wl.name == "large":
        # the prefill workload reads the same expert bytes (same layer shape and seeds)
        pre = synth.WORKLOADS["prefill"]
        log("[bench] leg: prefill ub=512 through the same layer shape")
        legs["prefill_ub512"] = run_leg(pre, weights, 6, 1, breakdown=not args.no_breakdown)
        del weights
        g = synth.WORKLOADS["gemma"]
        t0 = time.perf_counter()
        gw = synth.gen_all_weights(g)
        log(f"[bench] leg: gemma-like decode ({g.total_bytes / 1e9:.2f} GB generated in "
            f"{time.perf_counter() - t0:.1f} s)")
        legs["gemma_decode"] = run_leg(g, gw, 112, 16, breakdown=not args.no_breakdown)
        del gw

    line = {
        "metric": "MoE-layer tokens/s (decode b=1)" if wl.rho is not None else
                  "MoE-layer tokens/s (prefill ub=512)",
        "value": head["value"],
        "unit": "layer-tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded Q4_0 experts ~N(0,0.02), AR(1) hidden states, Zipf router bias)",
        "config": {"workload": head["workload"], "layers": wl.layers, "tokens_per_call": wl.batch,
                   "slot_policy": args.policy, "max_fills_per_call": args.max_fills,
                   "steps_are": "one batch through every layer"},
        "roofline": head.get("roofline"),
        "roofline_down": head.get("roofline_down"),
        "dominant_kernel_by_device_time": head.get("dominant_kernel_by_device_time"),
        "cpu_baseline": head.get("cpu_baseline"),
        "hit_rate": head["hit_rate"],
        "hit_rate_warmup_calls": head["hit_rate_warmup_calls"],
        "legs": legs,
        "extra": {k: v for k, v in head.items() if k not in (
            "roofline", "roofline_down", "dominant_kernel_by_device_time", "cpu_baseline", "value",
            "unit", "steps", "warmup", "ms_per_step", "workload", "dtype", "hit_rate",
            "hit_rate_warmup_calls")},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
