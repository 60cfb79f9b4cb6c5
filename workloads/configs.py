"""The five layer shapes the layer is checked and timed on.

Pages cited (by title and section):
  [FourStage]  "MoE显存与计算开销四阶段手算指南" (bjdmk.com.cn/news/5154310)
  [Principles] "MoE混合专家模型计算原理与推理部署实战解析" (sheratonhq.com/news/207562)

* tiny_f32            - a small fp32 layer the oracle finishes in well under a second.
* pages_worked_shape  - [FourStage §2]: input [4, 2048, 4096], 64 experts, top-2, each
                        expert a standard FFN hidden -> 4*hidden -> hidden (SiLU reading).
* mixtral_style       - the shape of [Principles §3.4]'s FLOP estimate (d=4096,
                        d_ff=14336, 8 experts, top-2, 4096 tokens) with SwiGLU experts
                        ([Principles §3.1]) and a mild per-expert logit bias.
* decode              - 64 tokens against the same SwiGLU experts with 64 experts: the
                        matrix-vector regime of [Principles §3.2].
* fine_grained_skewed - 256 small SwiGLU experts, top-8, with a Zipf-by-rank logit bias
                        that makes per-expert row counts heavily uneven ([FourStage §2.2],
                        [Principles §3.2] on load imbalance).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens = batch * seq_len
    H: int          # hidden size
    E: int          # number of experts
    k: int          # experts per token
    F: int          # expert intermediate size (d_ff)
    ffn: str        # "silu2" (SiLU two-layer FFN) or "swiglu"
    dtype: str      # "f32" or "bf16": x, expert weights, intermediates and output
    bias: str       # "none", "normal0.5" (variance 0.5) or "zipf1.1"
    seed: int = 0
    batch: int = 0  # batch/seq factorisation of T, for display only (0 = not given)
    seq: int = 0

    @property
    def pairs(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


PRESETS = {
    "tiny_f32": MoEConfig("tiny_f32", T=256, H=128, E=8, k=2, F=256, ffn="swiglu",
                          dtype="f32", bias="none"),
    "pages_worked_shape": MoEConfig("pages_worked_shape", T=8192, H=4096, E=64, k=2,
                                    F=16384, ffn="silu2", dtype="bf16", bias="none",
                                    batch=4, seq=2048),
    "mixtral_style": MoEConfig("mixtral_style", T=4096, H=4096, E=8, k=2, F=14336,
                               ffn="swiglu", dtype="bf16", bias="normal0.5"),
    "decode": MoEConfig("decode", T=64, H=4096, E=64, k=2, F=14336, ffn="swiglu",
                        dtype="bf16", bias="none"),
    "fine_grained_skewed": MoEConfig("fine_grained_skewed", T=8192, H=7168, E=256, k=8,
                                     F=2048, ffn="swiglu", dtype="bf16", bias="zipf1.1"),
}

ORDER = ["tiny_f32", "pages_worked_shape", "mixtral_style", "decode", "fine_grained_skewed"]


def preset(name: str) -> MoEConfig:
    return PRESETS[name]
