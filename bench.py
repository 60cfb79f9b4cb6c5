"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

A step is one whole layer forward (gate projection, top-k, grouping, grouped expert
FFN, combine) over one batch of synthetic inputs resident in HBM.  The default
workload is the pages' worked shape: 8192 tokens (batch 4 x seq 2048), hidden 4096,
64 experts, top-2, two-layer SiLU FFN 4096 -> 16384 -> 4096, bf16 with fp32 routing.

Prints one JSON line: tokens/s, the roofline figures of the dominant grouped-GEMM kernel
(timed live with HIP events that moe_forward records around each projection's launch on
its stream; the other projection is reported beside it) and the CPU oracle timed on a
bounded sample of the same workload.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="pages_worked_shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1536,
                    help="tokens of the workload the CPU oracle is timed on")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (reference for HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}); the layer is "
              "data-parallel with no exchange, so N GPUs each run this same step on their own "
              "tokens.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mixture_experts_layer_46_amd as M
    from mixture_experts_layer_46_amd import _lib
    from mixture_experts_layer_46_amd import accounting as A
    from workloads import generate, preset

    cfg = preset(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _lib.load()
    inp = generate(cfg, device=dev)
    x, wg, b = inp["x"], inp["w_gate"], inp["bias"]
    w_in, w_up, w_out = inp["w_in"], inp["w_up"], inp["w_out"]
    out = torch.empty_like(x)
    ws = M.Workspace(dev)
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.full((1 << 30,), 7, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # routing statistics of this batch (outside the timed region)
    logits, idx, _ = M.route(x, wg, cfg.k, bias=b)
    grp = M.permute(idx, cfg.E)
    counts = grp["counts"].cpu().numpy()
    touched = int((counts > 0).sum())

    def step():
        M.forward(x, wg, w_in, w_up, w_out, cfg.k, bias=b, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(K)]
    for trio in ev:              # materialise the event handles
        for e in trio:
            e.record()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(K):
        _lib.set_ffn_events(*ev[i])
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _lib.set_ffn_events()

    ms_step = (t1 - t0) * 1e3 / K
    up_ms = float(np.mean([a.elapsed_time(m) for a, m, _ in ev]))
    down_ms = float(np.mean([m.elapsed_time(c) for _, m, c in ev]))
    ffn_ms = up_ms + down_ms
    tokens_per_s = cfg.T * K / (t1 - t0)

    sb = A.stage_bytes(cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.ffn, cfg.dtype, touched)
    flops = A.ffn_flops(cfg.T, cfg.k, cfg.H, cfg.F, cfg.ffn)
    peak_flops = A.PEAK_BF16_FLOPS if cfg.dtype == "bf16" else A.PEAK_FP32_FLOPS
    kernels = {
        "up": dict(name=_gemm_kernel_name(cfg, True, counts), ms=up_ms,
                   flops=A.ffn_up_flops(cfg.T, cfg.k, cfg.H, cfg.F, cfg.ffn), bytes=sb.ffn_up),
        "down": dict(name=_gemm_kernel_name(cfg, False, counts), ms=down_ms,
                     flops=A.ffn_down_flops(cfg.T, cfg.k, cfg.H, cfg.F), bytes=sb.ffn_down),
    }
    for kd in kernels.values():
        kd["roofline"] = _roofline(kd, peak_flops)
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    roof = dict(kernels[dom]["roofline"])
    roof["traffic"] = _traffic(cfg.name, dom, kernels[dom]["name"])
    roof["kernel"] = kernels[dom]["name"]
    roof["ms"] = kernels[dom]["ms"]
    roof["algorithmic_bytes"] = kernels[dom]["bytes"]
    roof["algorithmic_flops"] = kernels[dom]["flops"]
    other = "down" if dom == "up" else "up"
    roof["other_projection"] = dict(kernels[other]["roofline"], kernel=kernels[other]["name"],
                                    ms=kernels[other]["ms"])
    t_ffn_roof = max(flops / peak_flops, (sb.ffn_up + sb.ffn_down) / A.PEAK_HBM_BPS)
    sec = ffn_ms * 1e-3

    result = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "batch": cfg.batch, "seq_len": cfg.seq,
                   "hidden": cfg.H, "experts": cfg.E, "top_k": cfg.k, "d_ff": cfg.F,
                   "ffn": cfg.ffn, "bias": cfg.bias, "global_batch": cfg.T, "parallelism": "none (1 GPU)"},
        "grouped_gemm_tflops": flops / sec / 1e12,
        "grouped_gemm_pct_bf16_peak": flops / sec / A.PEAK_BF16_FLOPS * 100,
        "grouped_ffn_ms": ffn_ms,
        "grouped_ffn_pct_roofline": t_ffn_roof / sec * 100,
        "touched_experts": touched,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_tokens)
    print(json.dumps(result), flush=True)
    return 0


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
    return "k_grouped_gemm_pp<%d, %d, %s>" % (nmat, act, gather)


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
            "seconds": dt,
            "sample": f"first {n_tokens} tokens of {cfg.name} ({len(used)} experts touched), "
                      f"numpy float64, experts streamed and widened to fp64 one at a time"}


if __name__ == "__main__":
    sys.exit(main())
