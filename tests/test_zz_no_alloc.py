"""moe_forward_noalloc (intermediates in the library's static per-GPU scratch, no
workspace argument) against moe_forward (a caller workspace), through the C ABI.

Both run the same kernels on the same inputs, so the outputs must be bit-identical.
Two calls in a row, the second on a smaller layer, check that nothing a call needs
depends on what the previous call left in the shared scratch; a layer larger than the
scratch is refused before anything is enqueued."""
import ctypes

import pytest
import torch

from workloads import MoEConfig, generate

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_layer_46_amd as M
    from mixture_experts_layer_46_amd import _lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _lib.load()
    return M


def _shape(cfg):
    from mixture_experts_layer_46_amd import _lib
    return _lib.Shape(T=cfg.T, H=cfg.H, E=cfg.E, k=cfg.k, F=cfg.F,
                      dtype=_lib.MOE_F32 if cfg.dtype == "f32" else _lib.MOE_BF16,
                      ffn=_lib.MOE_FFN_SWIGLU if cfg.ffn == "swiglu" else _lib.MOE_FFN_SILU2)


# the first on 256-row tiles (split of the last round and the per-XCD fetch counters in
# the scratch), the second smaller (128-row tiles), then a small fp32 layer
CASES = [
    MoEConfig("noalloc_big", T=2048, H=512, E=8, k=2, F=4096, ffn="swiglu", dtype="bf16", bias="zipf1.1"),
    MoEConfig("noalloc_small", T=300, H=256, E=8, k=2, F=384, ffn="silu2", dtype="bf16", bias="normal0.5"),
    MoEConfig("noalloc_f32", T=100, H=64, E=4, k=2, F=96, ffn="swiglu", dtype="f32", bias="none"),
]


def test_noalloc_matches_forward_on_consecutive_calls(lib):
    from mixture_experts_layer_46_amd import _lib
    M = lib
    for cfg in CASES:
        shape = _shape(cfg)
        need = _lib.workspace_size(shape)
        assert need <= _lib.NOALLOC_SCRATCH_BYTES, (cfg.name, need)
        say(f"noalloc {cfg.name}: workspace {need} bytes")
        d = {k: (None if v is None else v.cuda()) for k, v in generate(cfg).items()}
        ref = M.forward(d["x"], d["w_gate"], d["w_in"], d["w_up"], d["w_out"], cfg.k, bias=d["bias"])
        out = torch.full_like(d["x"], float("nan"))
        _lib.forward_noalloc(shape, d["x"], d["w_gate"], d["bias"], d["w_in"], d["w_up"], d["w_out"], out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), cfg.name
        # a second call on the same layer, after the others' contents
        out2 = torch.full_like(d["x"], float("nan"))
        _lib.forward_noalloc(shape, d["x"], d["w_gate"], d["bias"], d["w_in"], d["w_up"], d["w_out"], out2)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref), cfg.name


def test_noalloc_refuses_a_layer_beyond_the_scratch(lib):
    from mixture_experts_layer_46_amd import _lib
    cfg = MoEConfig("too_big", T=8192, H=4096, E=64, k=2, F=16384, ffn="silu2", dtype="bf16", bias="none")
    shape = _shape(cfg)
    assert _lib.workspace_size(shape) > _lib.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")      # never read: refused first
    with pytest.raises(_lib.MoeError) as e:
        _lib.forward_noalloc(shape, x, x, None, x, None, x, x)
    assert e.value.code == 5 and "static scratch" in e.value.detail
