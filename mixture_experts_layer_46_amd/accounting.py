"""Algorithmic FLOP and byte counts of the MoE layer forward (no GPU needed).

These are the figures the benchmark divides by measured time.  They count the work
and the HBM traffic the method needs at minimum, not what a kernel happens to move.

Pages cited (by title and section):
  [FourStage]  "MoE显存与计算开销四阶段手算指南" (bjdmk.com.cn/news/5154310)
  [Principles] "MoE混合专家模型计算原理与推理部署实战解析" (sheratonhq.com/news/207562)

* one projection of one token through one expert matrix [H, F] costs 2*H*F FLOPs;
  SwiGLU has three such matrices, the two-layer SiLU FFN two ([Principles §3.4]).
* expert weights take n_mat * H * F * bytes per expert ([FourStage §2.3]).
"""
from __future__ import annotations

from dataclasses import dataclass

# MI355X published peaks (dense, no sparsity).
PEAK_BF16_FLOPS = 2.5e15        # bf16 MFMA
PEAK_FP32_FLOPS = 157.3e12      # fp32 (vector and MFMA)
PEAK_HBM_BPS = 8.0e12           # HBM3E


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "f16": 2, "i32": 4}[dtype]


def n_mats(ffn: str) -> int:
    return 3 if ffn == "swiglu" else 2


def ffn_flops_per_pair(H: int, F: int, ffn: str) -> int:
    """FLOPs of one token through one expert."""
    return n_mats(ffn) * 2 * H * F


def ffn_flops(T: int, k: int, H: int, F: int, ffn: str) -> int:
    """FLOPs of the grouped expert FFN over all T*k token-expert pairs."""
    return T * k * ffn_flops_per_pair(H, F, ffn)


def ffn_up_flops(T: int, k: int, H: int, F: int, ffn: str) -> int:
    """FLOPs of the first grouped projection (W_in, and W_up for SwiGLU)."""
    return T * k * (n_mats(ffn) - 1) * 2 * H * F


def ffn_down_flops(T: int, k: int, H: int, F: int) -> int:
    """FLOPs of the second grouped projection (W_out)."""
    return T * k * 2 * F * H


def gate_flops(T: int, H: int, E: int) -> int:
    return 2 * T * H * E


def expert_weight_bytes(H: int, F: int, ffn: str, dtype: str) -> int:
    return n_mats(ffn) * H * F * elem_bytes(dtype)


@dataclass
class StageBytes:
    """HBM bytes of each stage, given the number of experts touched.

    Algorithmic bytes are the least the layer must move: every touched expert's
    weights once, x read once, out written once.  Split over the two projections, the
    first takes its weights and x, the second its weights and out (the grouped rows in
    between, h and the y rows, are the design's, not the method's).  The as-designed
    figures add them: h written by the first projection and read by the second, the y
    rows written by the second (and read by the combine)."""
    route: int
    permute: int       # the explicit grouping with the row gather (moe_permute with x)
    group: int         # moe_forward's grouping: top-k indices in, the two maps out
    ffn_up: int        # first projection, algorithmic: touched W_in (+W_up) + x
    ffn_down: int      # second projection, algorithmic: touched W_out + out
    ffn_up_designed: int     # + h written
    ffn_down_designed: int   # + h read + y rows written
    combine: int
    layer: int         # the whole layer: touched weights once + x in + out


def stage_bytes(T: int, H: int, E: int, k: int, F: int, ffn: str, dtype: str,
                touched: int) -> StageBytes:
    b = elem_bytes(dtype)
    P = T * k
    route = T * H * b + H * E * 4 + P * 8
    permute = T * H * b + P * H * b + P * 16
    w_up_side = (n_mats(ffn) - 1) * H * F * b * touched
    w_down_side = F * H * b * touched
    ffn_up = w_up_side + T * H * b
    ffn_down = w_down_side + T * H * b
    group = P * 4 + P * 8
    combine = P * H * b + T * H * b + P * 8
    layer = w_up_side + w_down_side + 2 * T * H * b
    return StageBytes(route, permute, group, ffn_up, ffn_down,
                      w_up_side + T * H * b + P * F * b,
                      w_down_side + P * F * b + P * H * b, combine, layer)
