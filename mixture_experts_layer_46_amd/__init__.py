"""MI355X-native token-choice Mixture-of-Experts layer forward.

The layer runs in libmoe.so (hand-written HIP kernels for gfx950 behind a C ABI,
include/moe.h).  This module only allocates torch device tensors for outputs and
workspace and passes pointers and the current stream; it has no other compute path.

    out = forward(x, w_gate, w_in, w_up, w_out, top_k, bias=None)

x [T, H] (bf16 or fp32), w_gate [H, E] fp32, w_in / w_up [E, H, F], w_out [E, F, H]
(w_up None for the two-layer SiLU FFN), bias [E] fp32 or None.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_F32, MOE_FFN_SILU2, MOE_FFN_SWIGLU, MOE_FLAG_BIAS_SELECT_ONLY,
                   MOE_FLAG_NO_RENORM, MoeError, Shape, capacity_rows)

__all__ = ["forward", "route", "route_from_logits", "permute", "grouped_ffn", "combine",
           "router_stats", "make_shape", "Workspace", "Shape", "MoeError", "forward_intermediates",
           "MOE_FLAG_BIAS_SELECT_ONLY", "MOE_FLAG_NO_RENORM", "capacity_rows"]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported element type {t.dtype}")


def _need(t, name, dtype, shape):
    """Raise ValueError unless tensor `t` has this dtype and shape."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_layer(x, w_gate, bias, w_in=None, w_up=None, w_out=None, out=None, top_k=None,
                 experts=True):
    """Element types and shapes the C ABI assumes (it sees only pointers): x [T, H] bf16
    or fp32; w_gate [H, E] and bias [E] fp32; w_in / w_up [E, H, F] and w_out [E, F, H]
    in x's type; out [T, H] in x's type.  Returns (T, H, E, F)."""
    if x is None or x.dim() != 2:
        raise ValueError("x must be a [T, H] tensor")
    _dtype_code(x)
    T, H = x.shape
    if w_gate is None or w_gate.dim() != 2:
        raise ValueError("w_gate must be a [H, E] tensor")
    E = w_gate.shape[1]
    _need(w_gate, "w_gate", torch.float32, (H, E))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    if top_k is not None and not 1 <= top_k <= E:
        raise ValueError(f"top_k = {top_k} must be in [1, E = {E}]")
    F = 0
    if experts:
        if w_in is None or w_in.dim() != 3:
            raise ValueError("w_in must be an [E, H, F] tensor")
        F = w_in.shape[2]
        _need(w_in, "w_in", x.dtype, (E, H, F))
        if w_up is not None:
            _need(w_up, "w_up", x.dtype, (E, H, F))
        _need(w_out, "w_out", x.dtype, (E, F, H))
    if out is not None:
        _need(out, "out", x.dtype, (T, H))
    devs = {t.device for t in (x, w_gate, bias, w_in, w_up, w_out, out) if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors are on different devices: {sorted(map(str, devs))}")
    return T, H, E, F


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU (the layer has no CPU path)")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def make_shape(T, H, E, k, F, dtype=torch.bfloat16, swiglu=True, flags=0, capacity=0) -> Shape:
    return Shape(T=T, H=H, E=E, k=k, F=F,
                 dtype=MOE_BF16 if dtype == torch.bfloat16 else MOE_F32,
                 ffn=MOE_FFN_SWIGLU if swiglu else MOE_FFN_SILU2, flags=flags, capacity=capacity)


class Workspace:
    """A device byte buffer that grows to what a shape needs and is then reused."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, shape: Shape) -> torch.Tensor:
        n = _lib.workspace_size(shape)
        if self.buf is None or self.buf.numel() < n:
            self.buf = torch.empty(max(n, 256), dtype=torch.uint8,
                                   device=self.device or torch.cuda.current_device())
        return self.buf


def forward(x, w_gate, w_in, w_up, w_out, top_k, bias=None, out=None, workspace=None,
            flags=0, capacity_factor=None, events=None):
    """The whole layer on the current stream; returns out [T, H] (x's dtype).
    `events`: MOE_STAGE_EVENTS timing events recorded at the stage boundaries."""
    T, H, E, F = _check_layer(x, w_gate, bias, w_in, w_up, w_out, out, top_k)
    _need_cuda(x, w_gate, w_in, w_up, w_out, bias, out)
    shape = Shape(T=T, H=H, E=E, k=top_k, F=F, dtype=_dtype_code(x),
                  ffn=MOE_FFN_SWIGLU if w_up is not None else MOE_FFN_SILU2, flags=flags,
                  capacity=capacity_rows(capacity_factor, T, top_k, E))
    if out is None:
        out = torch.empty_like(x)
    ws = (workspace or Workspace(x.device)).get(shape)
    _lib.forward(shape, x, w_gate, bias, w_in, w_up, w_out, out, ws, events=events)
    return out


def forward_intermediates(workspace, x, w_gate, w_in, w_up, top_k, flags=0, capacity_factor=None):
    """Views into `workspace` (a Workspace after a finished forward() on these tensors)
    of the intermediates that call left there (moe_workspace_layout): logit_parts
    [splits, T, E] fp32, topk_idx [T, k] int32, topk_w [T, k] fp32, counts [E],
    offsets [E+1], sorted_token [T*k], row_of_pair [T*k], h [T*k, F], y [T*k, H]."""
    T, H = x.shape
    E = w_gate.shape[1]
    F = w_in.shape[2]
    shape = Shape(T=T, H=H, E=E, k=top_k, F=F, dtype=_dtype_code(x),
                  ffn=MOE_FFN_SWIGLU if w_up is not None else MOE_FFN_SILU2, flags=flags,
                  capacity=capacity_rows(capacity_factor, T, top_k, E))
    lay = _lib.workspace_layout(shape)
    buf = workspace.buf
    if buf is None or buf.numel() < lay["total"]:
        raise ValueError("workspace is smaller than this layer's")
    P = T * top_k

    def part(name, dtype, shp):
        n = 1
        for d in shp:
            n *= d
        nb = n * torch.empty((), dtype=dtype).element_size()
        return buf[lay[name]:lay[name] + nb].view(dtype).view(*shp)

    return dict(logit_parts=part("logit_parts", torch.float32, (lay["logit_splits"], T, E)),
                topk_idx=part("topk_idx", torch.int32, (T, top_k)),
                topk_w=part("topk_w", torch.float32, (T, top_k)),
                counts=part("counts", torch.int32, (E,)),
                offsets=part("offsets", torch.int32, (E + 1,)),
                sorted_token=part("sorted_token", torch.int32, (P,)),
                row_of_pair=part("row_of_pair", torch.int32, (P,)),
                h=part("h", x.dtype, (P, F)), y=part("y", x.dtype, (P, H)))


def route(x, w_gate, top_k, bias=None, flags=0):
    """Gate projection + top-k + gates: (logits [T,E] fp32, topk_idx [T,k] i32, topk_w [T,k] f32)."""
    _check_layer(x, w_gate, bias, top_k=top_k, experts=False)
    _need_cuda(x, w_gate, bias)
    T, H = x.shape
    E = w_gate.shape[1]
    shape = Shape(T=T, H=H, E=E, k=top_k, F=8, dtype=_dtype_code(x), flags=flags)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    idx = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    _lib.route(shape, x, w_gate, bias, logits, idx, w)
    return logits, idx, w


def route_from_logits(logits, top_k, bias=None, flags=0):
    """Top-k + gates from given fp32 logits [T, E]: (topk_idx, topk_w)."""
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    _need(logits, "logits", torch.float32, logits.shape)
    if bias is not None:
        _need(bias, "bias", torch.float32, (logits.shape[1],))
    _need_cuda(logits, bias)
    T, E = logits.shape
    shape = Shape(T=T, H=8, E=E, k=top_k, F=8, dtype=MOE_F32, flags=flags)
    idx = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _lib.route(shape, None, None, bias, logits, idx, w)
    return idx, w


def permute(topk_idx, E, x=None, capacity=0, workspace=None, H=None, dtype=None):
    """Group pairs by expert: dict(counts, offsets, sorted_token, row_of_pair, x_perm)."""
    _need_cuda(topk_idx, x)
    T, k = topk_idx.shape
    if x is not None:
        H, dtype = x.shape[1], x.dtype
    H = H or 8
    dtype = dtype or torch.bfloat16
    shape = Shape(T=T, H=H, E=E, k=k, F=8, dtype=MOE_BF16 if dtype == torch.bfloat16 else MOE_F32,
                  capacity=capacity)
    dev = topk_idx.device
    P = T * k
    res = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               sorted_token=torch.empty(max(P, 1), dtype=torch.int32, device=dev),
               row_of_pair=torch.empty(max(P, 1), dtype=torch.int32, device=dev),
               x_perm=None if x is None else torch.empty((max(P, 1), H), dtype=dtype, device=dev))
    ws = (workspace or Workspace(dev)).get(shape)
    _lib.permute(shape, topk_idx, x, res["counts"], res["offsets"], res["sorted_token"],
                 res["row_of_pair"], res["x_perm"], ws)
    return res


def grouped_ffn(x_perm, offsets, w_in, w_up, w_out, top_k, T, workspace=None, y_perm=None):
    """Grouped expert FFN over x_perm [T*k, H] -> y_perm [T*k, H]."""
    _need_cuda(x_perm, offsets, w_in, w_up, w_out, y_perm)
    E, H, F = w_in.shape
    shape = Shape(T=T, H=H, E=E, k=top_k, F=F, dtype=_dtype_code(x_perm),
                  ffn=MOE_FFN_SWIGLU if w_up is not None else MOE_FFN_SILU2)
    if y_perm is None:
        y_perm = torch.empty((max(T * top_k, 1), H), dtype=x_perm.dtype, device=x_perm.device)
    ws = (workspace or Workspace(x_perm.device)).get(shape)
    _lib.grouped_ffn(shape, x_perm, offsets, w_in, w_up, w_out, y_perm, ws)
    return y_perm


def combine(y_perm, row_of_pair, topk_w, out=None):
    """out[t] = sum_j topk_w[t, j] * y_perm[row_of_pair[t*k + j]]."""
    _need_cuda(y_perm, row_of_pair, topk_w, out)
    T, k = topk_w.shape
    H = y_perm.shape[1]
    shape = Shape(T=T, H=H, E=max(k, 1), k=k, F=8, dtype=_dtype_code(y_perm))
    if out is None:
        out = torch.empty((T, H), dtype=y_perm.dtype, device=y_perm.device)
    _lib.combine(shape, y_perm, row_of_pair, topk_w, out)
    return out


def router_stats(logits, counts, top_k, bias=None, offsets=None, capacity=0):
    """Router monitoring statistics: (P [E], balance, entropy, top1_mean, drop_fraction)."""
    _need_cuda(logits, counts, bias, offsets)
    T, E = logits.shape
    shape = Shape(T=T, H=8, E=E, k=top_k, F=8, dtype=MOE_F32, capacity=capacity)
    stats = torch.empty(E + 4, dtype=torch.float32, device=logits.device)
    _lib.router_stats(shape, logits, bias, counts, offsets, stats)
    return stats
