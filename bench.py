"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
                    [--others NAME,NAME,... | --others none]

A step is one whole layer forward (gate projection, top-k, grouping, grouped expert
FFN, combine) over one batch of synthetic inputs resident in HBM.  The headline
workload is the largest configuration that fits one GPU: the fine-grained, skewed
layer (8192 tokens, hidden 7168, 256 SwiGLU experts of d_ff 2048, top-8, a Zipf-by-
rank logit bias), bf16 with fp32 routing.

Prints one JSON line: tokens/s, the roofline figures of the dominant grouped-GEMM kernel
(timed live with HIP events that moe_forward_timed records at its stage boundaries on
its stream; the other projection is reported beside it), per-stage times and rates, the
layer time's median and p10/p90 with and without a 256 MB MALL flush before each step,
peak rates measured on this GPU (bf16 MFMA loop, HBM read and copy) beside the published
ones, the CPU oracle timed on a bounded sample of the same workload, and under
"workloads" the same per-workload figures (tokens/s, grouped-GEMM TFLOP/s and % of bf16
peak, per-projection rooflines, stages) for the other layer shapes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA peak) on 1 MI355X"
HEADLINE = "fine_grained_skewed"
OTHERS = ["pages_worked_shape", "mixtral_style", "decode"]


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--others", default=",".join(OTHERS),
                    help="comma-separated workloads measured beside the headline ('none': no others)")
    ap.add_argument("--other-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens of the workload the CPU oracle is timed on")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (reference for HBM byte counters)")
    ap.add_argument("--flush-steps", type=int, default=5,
                    help="extra steps, each after a 1 GiB write that evicts the MALL (0: none)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the peak-rate microbenchmarks")
    return ap.parse_args(argv)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}); the layer is "
              "data-parallel with no exchange, so N GPUs each run this same step on their own "
              "tokens.", file=sys.stderr)
        return 2

    import torch

    from mixture_experts_layer_46_amd import _lib
    from workloads import preset

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _lib.load()

    if args.copy_calibration:
        src = torch.full((1 << 30,), 7, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cfg = preset(args.config)
    head = measure(cfg, dev, args.steps, args.warmup, args.flush_steps,
                   cpu_tokens=None if args.no_cpu_baseline else args.cpu_tokens)
    others = [] if args.others in ("", "none") else [o for o in args.others.split(",") if o != cfg.name]
    extra = {}
    for name in others:
        r = measure(preset(name), dev, args.other_steps, max(2, args.warmup // 2), 0, None)
        extra[name] = {k: r[k] for k in ("tokens_per_s", "ms_per_step", "layer_ms", "config", "dtype",
                                         "grouped_gemm_tflops", "grouped_gemm_pct_bf16_peak",
                                         "grouped_ffn_ms", "grouped_ffn_pct_roofline", "touched_experts",
                                         "projections", "stages")}
        extra[name]["steps"] = args.other_steps

    result = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": head["config"],
        "grouped_gemm_tflops": head["grouped_gemm_tflops"],
        "grouped_gemm_pct_bf16_peak": head["grouped_gemm_pct_bf16_peak"],
        "grouped_ffn_ms": head["grouped_ffn_ms"],
        "grouped_ffn_pct_roofline": head["grouped_ffn_pct_roofline"],
        "touched_experts": head["touched_experts"],
        "roofline": head["roofline"],
        "projections": head["projections"],
        "layer_ms": head["layer_ms"],
        "layer_ms_mall_flushed": head["layer_ms_mall_flushed"],
        "stages": head["stages"],
        "workloads": extra,
        "measured_peaks": None if args.no_peaks else measured_peaks(dev),
        "cpu_baseline": head["cpu_baseline"],
    }
    print(json.dumps(result), flush=True)
    return 0


def measure(cfg, dev, steps, warmup, flush_steps, cpu_tokens):
    """Time `steps` layer forwards of workload `cfg` (after `warmup` untimed ones) with
    stage events; returns the figures of one workload (and, with cpu_tokens, the CPU
    oracle on that many of its tokens)."""
    import numpy as np
    import torch

    import mixture_experts_layer_46_amd as M
    from mixture_experts_layer_46_amd import _lib
    from mixture_experts_layer_46_amd import accounting as A
    from workloads import generate

    inp = generate(cfg, device=dev)
    x, wg, b = inp["x"], inp["w_gate"], inp["bias"]
    w_in, w_up, w_out = inp["w_in"], inp["w_up"], inp["w_out"]
    out = torch.empty_like(x)
    ws = M.Workspace(dev)
    torch.cuda.synchronize()

    def step(events=None):
        M.forward(x, wg, w_in, w_up, w_out, cfg.k, bias=b, out=out, workspace=ws, events=events)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the routing this batch takes (the forward's own, from its workspace; not timed)
    mid = M.forward_intermediates(ws, x, wg, w_in, w_up, cfg.k)
    counts = mid["counts"].cpu().numpy()
    touched = int((counts > 0).sum())

    K = steps
    NS = _lib.MOE_STAGE_EVENTS

    def new_events(n):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(NS)] for _ in range(n)]
        for row in evs:          # materialise the event handles
            for e in row:
                e.record()
        return evs

    ev = new_events(K)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(K):
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_step = (t1 - t0) * 1e3 / K
    # stage durations per step: [route, group, ffn up, ffn down, combine]
    per = np.array([[row[j].elapsed_time(row[j + 1]) for j in range(NS - 1)] for row in ev])
    layer = np.array([row[0].elapsed_time(row[-1]) for row in ev])
    up_ms = float(per[:, 2].mean())
    down_ms = float(per[:, 3].mean())
    ffn_ms = up_ms + down_ms
    tokens_per_s = cfg.T * K / (t1 - t0)

    # the same steps after a 1 GiB write each, so x and the routing tensors start out of the
    # 256 MB MALL (not part of the timed loop above)
    flushed = None
    if flush_steps > 0:
        junk = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        evf = new_events(flush_steps)
        torch.cuda.synchronize()
        for i in range(flush_steps):
            junk.fill_(i & 0xFF)
            step(evf[i])
        torch.cuda.synchronize()
        flushed = _spread([row[0].elapsed_time(row[-1]) for row in evf])
        del junk

    sb = A.stage_bytes(cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.ffn, cfg.dtype, touched)
    flops = A.ffn_flops(cfg.T, cfg.k, cfg.H, cfg.F, cfg.ffn)
    peak_flops = A.PEAK_BF16_FLOPS if cfg.dtype == "bf16" else A.PEAK_FP32_FLOPS
    kernels = {
        "up": dict(name=_gemm_kernel_name(cfg, True, counts), ms=up_ms,
                   flops=A.ffn_up_flops(cfg.T, cfg.k, cfg.H, cfg.F, cfg.ffn), bytes=sb.ffn_up,
                   designed_bytes=sb.ffn_up_designed),
        "down": dict(name=_gemm_kernel_name(cfg, False, counts), ms=down_ms,
                     flops=A.ffn_down_flops(cfg.T, cfg.k, cfg.H, cfg.F), bytes=sb.ffn_down,
                     designed_bytes=sb.ffn_down_designed),
    }
    projections = {}
    for which, kd in kernels.items():
        r = _roofline(kd, peak_flops)
        r.update(kernel=kd["name"], ms=kd["ms"], algorithmic_bytes=kd["bytes"], algorithmic_flops=kd["flops"],
                 as_designed_bytes=kd["designed_bytes"],
                 as_designed_GBps=kd["designed_bytes"] / (kd["ms"] * 1e-3) / 1e9,
                 tflops=kd["flops"] / (kd["ms"] * 1e-3) / 1e12,
                 pct_bf16_peak=kd["flops"] / (kd["ms"] * 1e-3) / A.PEAK_BF16_FLOPS * 100,
                 traffic=_traffic(cfg.name, which, kd["name"]))
        projections[which] = r
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    roof = {k: projections[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof.update(kernel=kernels[dom]["name"], projection=dom, ms=kernels[dom]["ms"],
                algorithmic_bytes=kernels[dom]["bytes"], algorithmic_flops=kernels[dom]["flops"],
                roofline_ms=projections[dom]["roofline_ms"])
    t_ffn_roof = max(flops / peak_flops, (sb.ffn_up + sb.ffn_down) / A.PEAK_HBM_BPS)
    sec = ffn_ms * 1e-3

    def hbm_stage(ms, nbytes):
        return {"ms": ms, "algorithmic_bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9,
                "pct_hbm_peak": nbytes / (ms * 1e-3) / A.PEAK_HBM_BPS * 100}

    stages = {
        "route": dict(hbm_stage(float(per[:, 0].mean()), sb.route),
                      gate_tflops=A.gate_flops(cfg.T, cfg.H, cfg.E) / (per[:, 0].mean() * 1e-3) / 1e12),
        "group": hbm_stage(float(per[:, 1].mean()), sb.group),
        "ffn_up": dict(hbm_stage(up_ms, sb.ffn_up), tflops=projections["up"]["tflops"]),
        "ffn_down": dict(hbm_stage(down_ms, sb.ffn_down), tflops=projections["down"]["tflops"]),
        "combine": hbm_stage(float(per[:, 4].mean()), sb.combine),
    }
    res = {
        "tokens_per_s": tokens_per_s, "ms_per_step": ms_step, "dtype": cfg.dtype,
        "config": {"workload": cfg.name, "tokens": cfg.T, "batch": cfg.batch, "seq_len": cfg.seq,
                   "hidden": cfg.H, "experts": cfg.E, "top_k": cfg.k, "d_ff": cfg.F,
                   "ffn": cfg.ffn, "bias": cfg.bias, "global_batch": cfg.T, "parallelism": "none (1 GPU)"},
        "grouped_gemm_tflops": flops / sec / 1e12,
        "grouped_gemm_pct_bf16_peak": flops / sec / A.PEAK_BF16_FLOPS * 100,
        "grouped_ffn_ms": ffn_ms,
        "grouped_ffn_pct_roofline": t_ffn_roof / sec * 100,
        "touched_experts": touched,
        "roofline": roof,
        "projections": projections,
        "layer_ms": _spread(layer.tolist()),
        "layer_ms_mall_flushed": flushed,
        "stages": stages,
        "cpu_baseline": None,
    }
    if cpu_tokens:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, cpu_tokens)
    del inp, x, wg, b, w_in, w_up, w_out, out, ws, mid
    torch.cuda.empty_cache()
    return res


def _spread(ms):
    """Median and 10th/90th percentiles of per-step times (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def measured_peaks(dev):
    """Peak rates measured on this GPU with the library's microbenchmark kernels, beside
    the published MI355X figures the roofline uses (best of several runs each)."""
    import torch
    from mixture_experts_layer_46_amd import _lib
    from mixture_experts_layer_46_amd import accounting as A

    def timed(fn, reps):
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            t = a.elapsed_time(b) * 1e-3
            best = t if best is None else min(best, t)
        return best

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks, iters = 2 * cus, 1000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    khz = _lib.peak_mfma_bf16(blocks, 10, sink, clocks)            # warm-up
    t = timed(lambda: _lib.peak_mfma_bf16(blocks, iters, sink, clocks), 3)
    flops = blocks * 4 * iters * 32 * 16384
    cyc, ticks = (int(v) for v in clocks.cpu())
    clock_ghz = cyc / (ticks / (khz * 1e3)) / 1e9 if ticks > 0 and khz > 0 else None

    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    rblocks = 8 * cus
    rsink = torch.empty(rblocks * 256, dtype=torch.float32, device=dev)
    _lib.peak_hbm_read(buf, n, rblocks, rsink)
    t_read = timed(lambda: _lib.peak_hbm_read(buf, n, rblocks, rsink), 5)
    half = n // 2
    src, dst = buf[:half], buf[half:]
    t_copy = timed(lambda: _lib.peak_hbm_copy(src, dst, half, rblocks), 5)
    del buf
    return {"bf16_mfma_tflops": flops / t / 1e12,
            "mfma_loop_clock_ghz": clock_ghz,
            "hbm_read_GBps": n / t_read / 1e9,
            "hbm_copy_GBps": 2 * half / t_copy / 1e9,
            "published": {"bf16_mfma_tflops": A.PEAK_BF16_FLOPS / 1e12, "hbm_GBps": A.PEAK_HBM_BPS / 1e9},
            "how": f"MFMA-only loop {blocks} workgroups x {iters} x 32 MFMA per wavefront; "
                   f"4 GiB streaming read and 2 GiB copy (read + write bytes), {rblocks} workgroups; "
                   "best of 3 / 5 runs"}


def _host_info():
    """CPU model, usable cores and RAM of the host."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    ram = None
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal:"):
                ram = int(line.split()[1]) / (1 << 20)
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": len(os.sched_getaffinity(0)), "host_ram_gib": ram}


def _tile_height(cfg, counts) -> int:
    """The row-tile height the library's tile builder picks for these per-expert counts
    (256 or 320 rows: the one needing fewer work items, 256 on a tie)."""
    import math
    swiglu = cfg.ffn == "swiglu"

    def blocks(bn1, bn2):
        return math.ceil(cfg.F / bn1) + math.ceil(cfg.H / bn2)
    wa = blocks(128 if swiglu else 256, 256)
    wb = blocks(96 if swiglu else 192, 192)
    ta = sum(math.ceil(int(c) / 256) for c in counts) * wa
    tb = sum(math.ceil(int(c) / 320) for c in counts) * wb
    return 320 if tb < ta else 256


def _gemm_kernel_name(cfg, up: bool, counts) -> str:
    """Name of the grouped-GEMM kernel a projection runs (as rocprofv3 lists it): the
    kernel follows the mean rows per expert, and above 160 rows the tile height the
    tile builder picks (256-row tiles run in the ping-pong kernel, 320-row ones in the
    four-wavefront kernel)."""
    if cfg.dtype != "bf16":
        return "k_grouped_gemm_f32<%d, %d, %s>" % ((2 if cfg.ffn == "swiglu" else 1) if up else 1,
                                                    1 if up else 0, "true" if up else "false")
    mean = cfg.T * cfg.k / cfg.E
    nmat = (2 if cfg.ffn == "swiglu" else 1) if up else 1
    act, gather = (1, "true") if up else (0, "false")
    if mean <= 24:
        return "k_grouped_gemm_bf16<16, 256, %d, 1, %d, %s>" % (nmat, act, gather)
    if mean <= 80:
        return "k_grouped_gemm_lds<64, 64, %d, %d, %s>" % (nmat, act, gather)
    if mean <= 160:
        return "k_grouped_gemm_lds<128, 128, %d, %d, %s>" % (nmat, act, gather)
    if _tile_height(cfg, counts) == 320:
        return "k_grouped_gemm_lds<320, 320, %d, %d, %s>" % (nmat, act, gather)
    # the second projection runs the split-capable instance where K = F allows two parts
    # of 64 K steps of 32
    split = "true" if (not up and (cfg.F + 31) // 32 >= 128) else "false"
    return "k_grouped_gemm_pp<256, %d, %d, %s, %s>" % (nmat, act, gather, split)


def _roofline(kd, peak_flops):
    """Roofline figures of one kernel from its algorithmic flops/bytes and its mean time."""
    import mixture_experts_layer_46_amd.accounting as A
    sec = kd["ms"] * 1e-3
    t_mfma = kd["flops"] / peak_flops
    t_hbm = kd["bytes"] / A.PEAK_HBM_BPS
    if t_hbm >= t_mfma:
        r = {"bound": "hbm", "achieved": kd["bytes"] / sec / 1e9, "peak": A.PEAK_HBM_BPS / 1e9,
             "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": kd["flops"] / sec / 1e12, "peak": peak_flops / 1e12,
             "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["roofline_ms"] = max(t_mfma, t_hbm) * 1e3
    return r


def _traffic(workload: str, which: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed PMC summary of this workload
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), or None when there is no
    summary or the GEMM source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    src = os.path.join(ROOT, "mixture_experts_layer_46_amd", "csrc", "grouped_gemm.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("grouped_gemm.hip sha256") != digest:
        return None
    if fields.get(f"{which} kernel") != kernel:
        return None
    try:
        return float(fields[f"{which} hbm bytes per launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, inp, n_tokens):
    """The CPU oracle (numpy float64) on the first n_tokens tokens of the same inputs.
    Expert weights those tokens use are copied to host memory first (not timed); the
    timed oracle converts each expert to float64 as it streams through them."""
    import numpy as np
    import oracle.moe_oracle as O
    from threadpoolctl import threadpool_info
    from workloads import to_numpy

    x = to_numpy(inp["x"][:n_tokens])
    wg = to_numpy(inp["w_gate"])
    b = to_numpy(inp["bias"])
    _, idx, _ = O.route(x, wg, b, cfg.k)
    used = sorted(set(int(e) for e in idx.reshape(-1)))
    host = {}
    for e in used:
        host[e] = tuple(None if inp[n] is None else inp[n][e].to("cpu")
                        for n in ("w_in", "w_up", "w_out"))

    def weights(e):
        return tuple(None if t is None else t.float().numpy().astype(np.float64) for t in host[e])

    t0 = time.perf_counter()
    O.forward(x, wg, b, weights, cfg.k, cfg.ffn)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": dt, **_host_info(),
            "sample": f"first {n_tokens} tokens of {cfg.name} ({len(used)} experts touched), "
                      f"numpy float64, experts streamed and widened to fp64 one at a time"}


if __name__ == "__main__":
    sys.exit(main())
