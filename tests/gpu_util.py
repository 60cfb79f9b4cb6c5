"""Shared helpers of the GPU parity tests (not a test module)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle.moe_oracle as O
from workloads import MoEConfig, generate, to_numpy


def say(*a):
    """Name the case before any GPU step, flushed, so a failing run shows where it was."""
    print(*a, flush=True)
    sys.stdout.flush()


def normwise(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def tol_for(cfg: MoEConfig) -> float:
    """Normwise tolerance of the layer output: 1e-5 for fp32 layers, 2e-2 for bf16
    (h, y rows and the output are each rounded to bf16 once: 3 roundings of 2^-9
    relative, well inside 2e-2)."""
    return 1e-5 if cfg.dtype == "f32" else 2e-2


def gpu_inputs(cfg: MoEConfig, where="cpu"):
    """Inputs drawn on `where` then placed on the GPU (identical bits on both sides)."""
    d = generate(cfg, device=where)
    return {k: (None if v is None else v.to("cuda")) for k, v in d.items()}


def weights_numpy(inp):
    return (to_numpy(inp["w_in"]), to_numpy(inp["w_up"]), to_numpy(inp["w_out"]))


def near_tie_tau(scores_row) -> float:
    return 1e-4 * max(1.0, float(np.abs(scores_row).max()))


def check_selection(gpu_idx, oracle_scores, k):
    """GPU top-k vs the oracle's fp64 scores: equal where the k-th/(k+1)-th gap is
    clear; where it is within tau, the GPU's choice must be one of the oracle's
    tie-tolerant alternatives.  Returns {token: the oracle's alternative the GPU took}
    for the tokens a near tie decided differently."""
    ref_idx = O.select_topk(oracle_scores, k)
    flips = {}
    for t in np.nonzero((gpu_idx != ref_idx).any(axis=1))[0]:
        alts = O.topk_alternatives(oracle_scores[t], k, near_tie_tau(oracle_scores[t]))
        match = [a for a in alts if np.array_equal(gpu_idx[t], a)]
        assert match, f"token {t}: GPU picked {gpu_idx[t].tolist()}, oracle {ref_idx[t].tolist()}"
        flips[int(t)] = match[0]
    return flips


def run_forward(cfg: MoEConfig, inp, capacity_factor=None, flags=0):
    import mixture_experts_layer_46_amd as M
    out = M.forward(inp["x"], inp["w_gate"], inp["w_in"], inp["w_up"], inp["w_out"], cfg.k,
                    bias=inp["bias"], flags=flags, capacity_factor=capacity_factor)
    torch.cuda.synchronize()
    return out
