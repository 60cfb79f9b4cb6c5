"""Seeded input generators (no layer arithmetic here).

Every tensor gets its own generator seeded with ``subseed(seed, tag, e)`` so that a
single expert's weights can be drawn, or re-drawn, on their own.

Distributions (the variance is the second argument of N):
  x        ~ N(0, 1)                      [T, H]   dtype of the config
  w_gate   ~ N(0, 1/H)                    [H, E]   always fp32 (the gate runs in fp32)
  w_in     ~ N(0, 1/H)   per expert       [E, H, F] (W1 of the SiLU FFN, W_gate of SwiGLU)
  w_up     ~ N(0, 1/H)   per expert       [E, H, F] (SwiGLU only)
  w_out    ~ N(0, 1/F)   per expert       [E, F, H]
  bias     "none"       : no bias
           "normal0.5"  : b_e ~ N(0, 0.5), fp32
           "zipf1.1"    : b_e = -1.1 * ln(r_e) with r = 1 + a seeded permutation of
                          0..E-1, so exp(b) is a Zipf(1.1) prior over experts by rank.
bf16 tensors are drawn in fp32 and rounded to bf16 once (round-to-nearest-even).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .configs import MoEConfig

TAG_X, TAG_WG, TAG_BIAS, TAG_WIN, TAG_WUP, TAG_WOUT, TAG_PERM = 1, 2, 3, 4, 5, 6, 7


def subseed(seed: int, tag: int, e: int = 0) -> int:
    return seed * (1 << 20) + tag * (1 << 12) + e


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _normal(shape, std: float, s: int, device, out_dtype) -> torch.Tensor:
    t = torch.randn(*shape, generator=_gen(device, s), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(out_dtype)


def torch_dtype(cfg: MoEConfig):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def make_bias(cfg: MoEConfig, device="cpu"):
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal0.5":
        return _normal((cfg.E,), math.sqrt(0.5), subseed(cfg.seed, TAG_BIAS), device, torch.float32)
    if cfg.bias == "zipf1.1":
        perm = torch.randperm(cfg.E, generator=_gen("cpu", subseed(cfg.seed, TAG_PERM)))
        r = (perm + 1).to(torch.float64)
        return (-1.1 * torch.log(r)).to(torch.float32).to(device)
    raise ValueError(f"unknown bias kind {cfg.bias!r}")


def generate(cfg: MoEConfig, device="cpu", experts: bool = True) -> dict:
    """Draw all inputs of one layer call on ``device`` (torch tensors)."""
    dt = torch_dtype(cfg)
    s = cfg.seed
    out = {
        "x": _normal((cfg.T, cfg.H), 1.0, subseed(s, TAG_X), device, dt),
        "w_gate": _normal((cfg.H, cfg.E), 1.0 / math.sqrt(cfg.H), subseed(s, TAG_WG), device,
                          torch.float32),
        "bias": make_bias(cfg, device),
    }
    if not experts:
        return out
    swiglu = cfg.ffn == "swiglu"
    w_in = torch.empty((cfg.E, cfg.H, cfg.F), dtype=dt, device=device)
    w_up = torch.empty((cfg.E, cfg.H, cfg.F), dtype=dt, device=device) if swiglu else None
    w_out = torch.empty((cfg.E, cfg.F, cfg.H), dtype=dt, device=device)
    for e in range(cfg.E):
        w_in[e] = _normal((cfg.H, cfg.F), 1.0 / math.sqrt(cfg.H), subseed(s, TAG_WIN, e), device, dt)
        if swiglu:
            w_up[e] = _normal((cfg.H, cfg.F), 1.0 / math.sqrt(cfg.H), subseed(s, TAG_WUP, e), device, dt)
        w_out[e] = _normal((cfg.F, cfg.H), 1.0 / math.sqrt(cfg.F), subseed(s, TAG_WOUT, e), device, dt)
    out.update(w_in=w_in, w_up=w_up, w_out=w_out)
    return out


def to_numpy(t) -> np.ndarray | None:
    """Exact host copy of a tensor as float64 (bf16 -> fp32 -> fp64 is exact) or int."""
    if t is None:
        return None
    t = t.detach().to("cpu")
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.to(torch.float32)
    a = t.numpy()
    return a.astype(np.float64) if a.dtype.kind == "f" else a


def expert_numpy(inputs: dict, e: int):
    """(w_in[e], w_up[e] or None, w_out[e]) as exact float64 host arrays."""
    w_up = inputs.get("w_up")
    return (to_numpy(inputs["w_in"][e]),
            None if w_up is None else to_numpy(w_up[e]),
            to_numpy(inputs["w_out"][e]))
