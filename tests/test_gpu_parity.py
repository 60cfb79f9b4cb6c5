"""GPU path vs the CPU oracle, stage by stage and end to end, at sizes the oracle
finishes in seconds (several tiles plus ragged tails in every dimension).

Bar: routing indices, counts, offsets, the permutation and x_perm bit-exact (fed
identical fp32 logits / indices); gates within 1e-6; expert FFN and layer outputs
within a normwise 1e-5 (fp32) or 2e-2 (bf16).
"""
import math

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from workloads import MoEConfig, PRESETS, generate, to_numpy

from gpu_util import (check_selection, gpu_inputs, normwise, run_forward, say, tol_for,
                      weights_numpy)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    import mixture_experts_layer_46_amd as M
    from mixture_experts_layer_46_amd import _lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _lib.load()          # fails loudly when the library is missing: no fallback
    return M


# --------------------------------------------------------------------------- routing

ROUTE_CASES = [  # T, E, k, bias, flags
    (300, 8, 2, False, 0), (257, 64, 2, True, 0), (129, 256, 8, True, 0), (64, 1, 1, False, 0),
    (77, 5, 5, True, 0), (100, 100, 3, False, 0), (65, 256, 1, False, 0),
    (90, 16, 4, True, 1), (90, 16, 4, True, 2), (90, 16, 4, True, 3),
]


@pytest.mark.parametrize("T,E,k,use_bias,flags", ROUTE_CASES)
def test_route_from_logits_bit_exact(lib, T, E, k, use_bias, flags):
    say(f"route_from_logits T={T} E={E} k={k} bias={use_bias} flags={flags}")
    g = torch.Generator().manual_seed(1000 + T + E + k)
    # quantised logits: many exact ties, and both signs of zero
    L = torch.round(torch.randn(T, E, generator=g) * 3) / 4
    L[::7, : min(E, 3)] = -0.0
    L[::5, -1] = 0.0
    L = L.float()
    b = (torch.round(torch.randn(E, generator=g) * 2) / 8).float() if use_bias else None
    idx, w = lib.route_from_logits(L.cuda(), k, bias=None if b is None else b.cuda(), flags=flags)
    torch.cuda.synchronize()
    _, ridx, rg = O.route_from_f32_logits(L.numpy(), None if b is None else b.numpy(), k,
                                          select_only=bool(flags & 1), renorm=not (flags & 2))
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(w.cpu().numpy(), rg, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("E,k", [(256, 8), (100, 3), (64, 2)])
def test_route_nonfinite_scores(lib, E, k):
    """Scores of +inf, -inf and NaN: the selection is still the oracle's order (score
    descending, NaN below every number, equal scores to the lower index)."""
    say(f"route_nonfinite E={E} k={k}")
    T = 96
    g = torch.Generator().manual_seed(77 + E + k)
    L = (torch.round(torch.randn(T, E, generator=g) * 2) / 4).float()
    L[0::4, 5::9] = float("nan")
    L[1::4, 3::7] = float("inf")
    L[2::4, :: 2] = float("-inf")
    L[3::4, :] = float("nan")
    L[3::4, E - 1] = 1.0
    L[3::8, 0] = float("-inf")
    idx, _ = lib.route_from_logits(L.cuda(), k)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        _, ridx, _ = O.route_from_f32_logits(L.numpy(), None, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)


@pytest.mark.parametrize("E,k", [(256, 8), (200, 8), (48, 3)])
def test_route_winners_in_one_lane(lib, E, k):
    """The k largest scores of a token all on experts that share e mod 16 (one lane of
    the selection holds them), some of them equal: the order is still score
    descending, then index ascending."""
    say(f"route_one_lane E={E} k={k}")
    T = 80
    g = torch.Generator().manual_seed(4242 + E + k)
    L = (torch.round(torch.randn(T, E, generator=g) * 2) / 8).float()
    for r in range(T):
        lane = r % 16
        owned = list(range(lane, E, 16))
        for i, e in enumerate(owned[:k + 1]):
            L[r, e] = 10.0 - (i // 2)          # pairs of equal scores
    idx, w = lib.route_from_logits(L.cuda(), k)
    torch.cuda.synchronize()
    _, ridx, rg = O.route_from_f32_logits(L.numpy(), None, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(w.cpu().numpy(), rg, rtol=1e-6, atol=1e-7)


# T > 256 with bf16 x takes the split-weight bf16 MFMA gate (128-token tiles); ragged
# K (H = 200), several expert tiles (E = 256) and a ragged expert count (E = 37)
ROUTE_X_CASES = [(333, 200, 64, 2), (1000, 4096, 256, 8), (700, 64, 37, 3), (200, 512, 64, 2),
                 (257, 8, 3, 1)]


@pytest.mark.parametrize("T,H,E,k", ROUTE_X_CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_route_from_x(lib, dtype, T, H, E, k):
    cfg = MoEConfig("r", T=T, H=H, E=E, k=k, F=8, ffn="swiglu", dtype=dtype, bias="normal0.5")
    say(f"route_from_x {cfg}")
    d = generate(cfg, experts=False)
    x, wg, b = d["x"].cuda(), d["w_gate"].cuda(), d["bias"].cuda()
    logits, idx, w = lib.route(x, wg, cfg.k, bias=b)
    torch.cuda.synchronize()
    ref = O.gate_logits(to_numpy(d["x"]), to_numpy(d["w_gate"]))
    got = logits.cpu().numpy().astype(np.float64)
    assert np.abs(got - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())
    scores, ridx, rg = O.route(to_numpy(d["x"]), to_numpy(d["w_gate"]), to_numpy(d["bias"]), cfg.k)
    flips = check_selection(idx.cpu().numpy(), scores, cfg.k)
    assert len(flips) <= max(2, cfg.T // 200)
    same = np.setdiff1d(np.arange(cfg.T), list(flips))
    np.testing.assert_allclose(w.cpu().numpy()[same], rg[same], rtol=2e-5, atol=1e-6)


# -------------------------------------------------------------------------- grouping

PERMUTE_CASES = [  # T, E, k, H, capacity
    (1, 4, 2, 64, 0), (37, 5, 2, 72, 0), (600, 8, 2, 128, 0), (1100, 64, 3, 40, 0),
    (513, 256, 8, 16, 0), (700, 16, 4, 24, 0), (700, 16, 4, 24, 150), (300, 8, 2, 8, 40),
]


@pytest.mark.parametrize("T,E,k,H,cap", PERMUTE_CASES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_permute_bit_exact(lib, T, E, k, H, cap, dtype):
    say(f"permute T={T} E={E} k={k} H={H} cap={cap} {dtype}")
    g = torch.Generator().manual_seed(T * 31 + E)
    # skewed distinct picks per token
    w = torch.linspace(3.0, 0.1, E)
    idx = torch.stack([torch.multinomial(w, k, replacement=False, generator=g) for _ in range(T)]).int()
    x = torch.randn(T, H, generator=g).to(dtype)
    r = lib.permute(idx.cuda(), E, x=x.cuda(), capacity=cap)
    torch.cuda.synchronize()
    counts, offsets, st, rop = O.group_by_expert(idx.numpy(), E)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    if cap == 0:
        assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
        P = T * k
        assert np.array_equal(r["sorted_token"].cpu().numpy()[:P], st)
        assert np.array_equal(r["row_of_pair"].cpu().numpy()[:P], rop)
        assert torch.equal(r["x_perm"][:P].cpu(), x[torch.from_numpy(st).long()])
    else:
        kept = np.minimum(counts, cap)
        offs = np.concatenate([[0], np.cumsum(kept)])
        assert np.array_equal(r["offsets"].cpu().numpy(), offs)
        # expected: the first `cap` pairs (token order) of each expert keep rows
        want_rop = np.full(T * k, -1)
        for e in range(E):
            a, b = offsets[e], offsets[e + 1]
            for i in range(min(cap, b - a)):
                want_rop[st[a + i] * k + int(np.nonzero(idx.numpy()[st[a + i]] == e)[0][0])] = offs[e] + i
        got_rop = r["row_of_pair"].cpu().numpy()[: T * k]
        assert np.array_equal(got_rop, want_rop)
        R = int(offs[-1])
        got_st = r["sorted_token"].cpu().numpy()[:R]
        for e in range(E):
            assert np.array_equal(got_st[offs[e]:offs[e + 1]], st[offsets[e]:offsets[e] + kept[e]])


# -------------------------------------------------------------------------- expert FFN

FFN_CASES = [  # T, H, E, k, F, ffn, dtype  (mean rows per expert picks the row tile)
    (256, 128, 8, 2, 256, "swiglu", "f32"), (37, 72, 5, 2, 40, "silu2", "f32"),
    (24, 256, 16, 2, 512, "swiglu", "bf16"), (200, 200, 8, 2, 320, "silu2", "bf16"),
    # decode-sized (16-row tiles) two-layer SiLU, F ragged against 256-column blocks
    (40, 256, 16, 2, 384, "silu2", "bf16"),
    (512, 264, 4, 2, 136, "swiglu", "bf16"), (100, 128, 1, 1, 128, "silu2", "bf16"),
    (300, 128, 256, 8, 64, "swiglu", "bf16"), (700, 192, 4, 2, 2056, "swiglu", "bf16"),
    # ~275 rows per expert: the tile builder picks 320 x 192 tiles (8 items against ~16 x
    # the column blocks of 256-row tiles); ragged K and N against 192 (96 per SwiGLU matrix)
    (1100, 520, 8, 2, 392, "silu2", "bf16"), (1100, 264, 8, 2, 200, "swiglu", "bf16"),
    # split of the second projection's last round along K (on 256 workgroups, at least 64
    # K steps of 32 per part): 320-row tiles with 24 items, split in 3 (K = 6400) and in 2
    # (K = 4608); 128-row tiles with ~48 items, split in 2; 256-row tiles (the ping-pong
    # kernel, ~512 rows per expert) with ~48 items, split in 2 (K = 4096 and 4608)
    (1100, 520, 8, 2, 6400, "silu2", "bf16"), (1100, 520, 8, 2, 4608, "swiglu", "bf16"),
    (1024, 512, 16, 2, 4096, "silu2", "bf16"),
    (2048, 512, 8, 2, 4096, "silu2", "bf16"), (2048, 512, 8, 2, 4608, "swiglu", "bf16"),
    # 256-row tiles with K >= 4096 in both projections: both take the ordered per-XCD fetch
    (2048, 4096, 8, 2, 4096, "silu2", "bf16"),
]


@pytest.mark.parametrize("T,H,E,k,F,ffn,dtype", FFN_CASES)
def test_grouped_ffn(lib, T, H, E, k, F, ffn, dtype):
    cfg = MoEConfig("g", T=T, H=H, E=E, k=k, F=F, ffn=ffn, dtype=dtype, bias="none", seed=3)
    say(f"grouped_ffn {cfg}")
    d = generate(cfg)
    g = torch.Generator().manual_seed(T + F)
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).int().numpy()
    counts, offsets, st, rop = O.group_by_expert(idx, E)
    x_perm = d["x"][torch.from_numpy(st).long()]
    y = lib.grouped_ffn(x_perm.cuda(), torch.from_numpy(offsets).cuda(), d["w_in"].cuda(),
                        None if d["w_up"] is None else d["w_up"].cuda(), d["w_out"].cuda(), k, T)
    torch.cuda.synchronize()
    ref = O.grouped_ffn(to_numpy(x_perm), offsets, weights_numpy(d), ffn)
    err = normwise(to_numpy(y[: T * k]), ref)
    say(f"  normwise error {err:.3e}")
    assert err <= tol_for(cfg)


# Skewed per-expert counts on 256-row tiles (mean above 160 rows): tiles of at most 64 rows
# (single-tile experts, and the ragged last tile of a long expert) take the ping-pong
# kernel's thin-tile loop, the others its full K loop; empty experts, 1-row experts and the
# 64 / 65-row boundary included; ragged K and N.  Then the same at K = 4096 (ordered
# per-XCD fetch) and with a split-capable second projection (K = 4608).
THIN_CASES = [  # counts per expert, H, F, ffn
    ([1200, 1, 16, 17, 64, 65, 0, 300, 33, 5, 256, 63, 2000, 700, 40, 8], 264, 392, "swiglu"),
    ([1200, 1, 16, 17, 64, 65, 0, 300, 33, 5, 256, 63, 2000, 700, 40, 8], 200, 520, "silu2"),
    ([900, 3, 64, 1, 0, 48, 600, 17], 4096, 512, "swiglu"),
    ([700, 20, 1, 64, 500, 2, 33, 9], 256, 4608, "silu2"),
]


@pytest.mark.parametrize("counts,H,F,ffn", THIN_CASES)
def test_grouped_ffn_thin_tiles(lib, counts, H, F, ffn):
    E, k = len(counts), 2
    R = sum(counts)
    T = (R + k - 1) // k
    assert T * k / E > 160                     # 256-row tiles
    cfg = MoEConfig("thin", T=T, H=H, E=E, k=k, F=F, ffn=ffn, dtype="bf16", bias="none", seed=5)
    say(f"grouped_ffn thin tiles: counts {counts} H={H} F={F} {ffn}")
    d = generate(cfg)
    g = torch.Generator().manual_seed(R + H + F)
    x_perm = torch.randn(T * k, H, generator=g).to(torch.bfloat16)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    y = lib.grouped_ffn(x_perm.cuda(), torch.from_numpy(offsets).cuda(), d["w_in"].cuda(),
                        None if d["w_up"] is None else d["w_up"].cuda(), d["w_out"].cuda(), k, T)
    torch.cuda.synchronize()
    ref = O.grouped_ffn(to_numpy(x_perm[:R]), offsets, weights_numpy(d), ffn)
    got = to_numpy(y[:R])
    err = normwise(got, ref)
    # every expert's rows on their own, so a wrong thin tile cannot hide behind the big ones
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            assert normwise(got[a:b], ref[a:b]) <= tol_for(cfg), f"expert {e} ({b - a} rows)"
    say(f"  normwise error {err:.3e}")
    assert err <= tol_for(cfg)


# ---------------------------------------------------------------------------- combine

@pytest.mark.parametrize("T,k,H,dtype", [(1, 1, 8, torch.float32), (333, 2, 4096, torch.bfloat16),
                                         (100, 8, 7168, torch.bfloat16), (50, 3, 120, torch.float32)])
def test_combine(lib, T, k, H, dtype):
    say(f"combine T={T} k={k} H={H} {dtype}")
    g = torch.Generator().manual_seed(T * k)
    P = T * k
    y = torch.randn(P, H, generator=g).to(dtype)
    rop = torch.randperm(P, generator=g).int()
    rop[::5] = -1                                    # dropped pairs add nothing
    w = torch.rand(T, k, generator=g)
    out = lib.combine(y.cuda(), rop.cuda(), w.cuda())
    torch.cuda.synchronize()
    ynp = to_numpy(y)
    ynp = np.concatenate([ynp, np.zeros((1, H))])    # row -1 -> zeros
    ref = O.combine(ynp, np.where(rop.numpy() < 0, P, rop.numpy()), w.numpy().astype(np.float64))
    tol = 1e-6 if dtype == torch.float32 else 8e-3
    assert normwise(to_numpy(out), ref) <= tol


# --------------------------------------------------------------------------- end to end

E2E = [
    PRESETS["tiny_f32"],
    MoEConfig("f32_ragged", T=37, H=72, E=5, k=2, F=40, ffn="silu2", dtype="f32", bias="normal0.5"),
    MoEConfig("decode_small", T=24, H=256, E=16, k=2, F=512, ffn="swiglu", dtype="bf16", bias="none"),
    MoEConfig("mid_silu2", T=200, H=200, E=8, k=2, F=320, ffn="silu2", dtype="bf16", bias="none"),
    MoEConfig("two_tiles", T=512, H=264, E=4, k=2, F=136, ffn="swiglu", dtype="bf16", bias="normal0.5"),
    MoEConfig("k_eq_E", T=64, H=128, E=4, k=4, F=256, ffn="swiglu", dtype="bf16", bias="none"),
    MoEConfig("one_expert", T=100, H=128, E=1, k=1, F=128, ffn="silu2", dtype="bf16", bias="none"),
    MoEConfig("skew_256", T=300, H=128, E=256, k=8, F=64, ffn="swiglu", dtype="bf16", bias="zipf1.1"),
    MoEConfig("one_token", T=1, H=64, E=8, k=2, F=64, ffn="swiglu", dtype="bf16", bias="none"),
    # 320-row tiles with skewed counts: hot experts span several tiles, cold ones a few rows
    MoEConfig("tiles_320_skew", T=1200, H=520, E=16, k=3, F=392, ffn="silu2", dtype="bf16", bias="zipf1.1"),
    # bf16 above 256 tokens: the gate's per-call weight planes with a ragged expert count (37,
    # a partial 64-expert tile and a partial 4-expert group) and H not a multiple of 64
    MoEConfig("planes_ragged_E", T=700, H=136, E=37, k=3, F=200, ffn="swiglu", dtype="bf16", bias="normal0.5"),
    # 128-expert gate tiles (E > 64) with a ragged last tile, zipf-skewed 256-row GEMM tiles
    MoEConfig("planes_E200", T=2600, H=264, E=200, k=8, F=136, ffn="swiglu", dtype="bf16", bias="zipf1.1"),
    # a single expert (E = k = 1) above 256 tokens: dense FFN through the bf16 path
    MoEConfig("one_expert_bf16", T=300, H=256, E=1, k=1, F=512, ffn="silu2", dtype="bf16", bias="none"),
]


def _oracle_forward(cfg, d, **kw):
    return O.forward(to_numpy(d["x"]), to_numpy(d["w_gate"]), to_numpy(d["bias"]), weights_numpy(d),
                     cfg.k, cfg.ffn, **kw)


@pytest.mark.parametrize("cfg", E2E, ids=[c.name for c in E2E])
def test_forward_matches_oracle(lib, cfg):
    """The layer against the oracle on every token.  The routing checked is the forward's
    own (read back from its workspace): its top-k equals the oracle's selection of its
    own partial gate sums added in the kernel's order (bit-exact, split-K included), and
    a token that a near tie routed differently from the float64 oracle is compared with
    the oracle's output for the GPU's selection."""
    say(f"forward {cfg}")
    d = generate(cfg)
    inp = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    ws = lib.Workspace()
    out = lib.forward(inp["x"], inp["w_gate"], inp["w_in"], inp["w_up"], inp["w_out"], cfg.k,
                      bias=inp["bias"], workspace=ws)
    torch.cuda.synchronize()
    mid = lib.forward_intermediates(ws, inp["x"], inp["w_gate"], inp["w_in"], inp["w_up"], cfg.k)
    parts = mid["logit_parts"].cpu().numpy()
    L32 = parts[0].copy()
    for q in parts[1:]:
        L32 = (L32 + q).astype(np.float32)
    idx = mid["topk_idx"].cpu().numpy()
    _, ridx, rg = O.route_from_f32_logits(L32, None if d["bias"] is None else d["bias"].numpy(), cfg.k)
    assert np.array_equal(idx, ridx)
    np.testing.assert_allclose(mid["topk_w"].cpu().numpy(), rg, rtol=1e-6, atol=1e-7)
    ref = _oracle_forward(cfg, d)
    flips = check_selection(idx, ref["logits"], cfg.k)
    got = to_numpy(out)
    keep = np.setdiff1d(np.arange(cfg.T), list(flips))
    err = normwise(got[keep], ref["out"][keep])
    say(f"  normwise error {err:.3e}, near-tie tokens {len(flips)}, gate splits {parts.shape[0]}")
    assert err <= tol_for(cfg)
    for t, alt in flips.items():   # a near tie went the other way: output of that selection
        want = O.token_output(to_numpy(d["x"])[t], ref["logits"][t], alt, weights_numpy(d), cfg.ffn)
        assert normwise(got[t], want) <= tol_for(cfg)


POISON_CASES = [
    # 256-row tiles with zipf-skewed counts: the ping-pong kernel's per-XCD queues, the
    # stealing between them, thin tiles beside full ones
    MoEConfig("poison_pp_skew", T=2048, H=264, E=16, k=2, F=392, ffn="swiglu", dtype="bf16", bias="zipf1.1"),
    # a second projection with K = 4096: the split of the last round along K
    MoEConfig("poison_pp_split", T=1024, H=136, E=4, k=2, F=4096, ffn="silu2", dtype="bf16", bias="none"),
    # 320-row tiles with skewed counts (the four-wavefront kernel)
    MoEConfig("poison_320", T=1200, H=520, E=16, k=3, F=392, ffn="silu2", dtype="bf16", bias="zipf1.1"),
]


@pytest.mark.parametrize("cfg", POISON_CASES, ids=[c.name for c in POISON_CASES])
def test_forward_writes_every_row(lib, cfg):
    """Every work item runs and nothing is read before this call writes it: after a clean
    run (checked against the oracle), the workspace and the output are filled with 0xFF
    bytes (NaN in bf16 and fp32) and the layer runs again, twice.  Every grouped row of h
    and y and every output value must then be finite and the output equal, bit for bit,
    to the clean run's (a skipped item would leave NaN rows; a counter or buffer read
    before it is written would pick up the poison)."""
    say(f"poisoned workspace {cfg}")
    d = generate(cfg)
    inp = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    ws = lib.Workspace()
    args = (inp["x"], inp["w_gate"], inp["w_in"], inp["w_up"], inp["w_out"], cfg.k)
    clean = lib.forward(*args, bias=inp["bias"], workspace=ws)
    torch.cuda.synchronize()
    mid = lib.forward_intermediates(ws, inp["x"], inp["w_gate"], inp["w_in"], inp["w_up"], cfg.k)
    ref = _oracle_forward(cfg, d)
    flips = check_selection(mid["topk_idx"].cpu().numpy(), ref["logits"], cfg.k)
    got = to_numpy(clean)
    keep = np.setdiff1d(np.arange(cfg.T), list(flips))
    err = normwise(got[keep], ref["out"][keep])
    say(f"  clean run: normwise error {err:.3e}, near-tie tokens {len(flips)}")
    assert err <= tol_for(cfg)
    clean = clean.clone()
    out = torch.empty_like(clean)
    for rep in range(2):
        ws.buf.fill_(255)
        out.view(torch.uint8).fill_(255)
        lib.forward(*args, bias=inp["bias"], workspace=ws, out=out)
        torch.cuda.synchronize()
        mid = lib.forward_intermediates(ws, inp["x"], inp["w_gate"], inp["w_in"], inp["w_up"], cfg.k)
        assert bool(torch.isfinite(mid["h"]).all()), f"run {rep}: rows of h left unwritten"
        assert bool(torch.isfinite(mid["y"]).all()), f"run {rep}: rows of y left unwritten"
        assert bool(torch.isfinite(out).all()), f"run {rep}: output values left unwritten"
        assert torch.equal(out, clean), f"run {rep}: output differs from the clean run"


@pytest.mark.parametrize("dtype,ffn", [("bf16", "silu2"), ("bf16", "swiglu"), ("f32", "swiglu")])
def test_forward_all_tokens_to_two_experts(lib, dtype, ffn):
    """Degenerate routing: a logit bias of 40 on experts 3 and 6 sends every token to both, so
    six experts are empty (before, between and after the two) and each chosen one holds all
    700 tokens in several row tiles (a ragged last one)."""
    cfg = MoEConfig("collapsed", T=700, H=136, E=8, k=2, F=264, ffn=ffn, dtype=dtype, bias="none")
    say(f"collapsed routing {cfg}")
    d = generate(cfg)
    d["bias"] = torch.zeros(cfg.E, dtype=torch.float32)
    d["bias"][[3, 6]] = 40.0
    inp = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    _, idx, _ = lib.route(inp["x"], inp["w_gate"], cfg.k, bias=inp["bias"])
    assert set(np.unique(idx.cpu().numpy()).tolist()) == {3, 6}
    out = run_forward(cfg, inp)
    ref = _oracle_forward(cfg, d)
    err = normwise(to_numpy(out), ref["out"])
    say(f"  normwise error {err:.3e}")
    assert err <= tol_for(cfg)


def test_forward_is_deterministic(lib):
    cfg = MoEConfig("det", T=500, H=256, E=32, k=4, F=384, ffn="swiglu", dtype="bf16", bias="zipf1.1")
    say(f"determinism {cfg}")
    inp = gpu_inputs(cfg)
    a = run_forward(cfg, inp).clone()
    b = run_forward(cfg, inp)
    assert torch.equal(a, b)


CAP_CASES = [  # capacity factor, layer (mean rows per expert picks the row tile)
    (0.5, MoEConfig("cap", T=300, H=128, E=8, k=2, F=192, ffn="swiglu", dtype="bf16", bias="normal0.5")),
    (1.0, MoEConfig("cap", T=300, H=128, E=8, k=2, F=192, ffn="swiglu", dtype="bf16", bias="normal0.5")),
    # 300 rows per expert on average: the 256- and 320-row tile kernels, capped experts full
    (1.0, MoEConfig("cap_big", T=1200, H=264, E=8, k=2, F=392, ffn="silu2", dtype="bf16", bias="normal0.5")),
    # skewed counts on 256-row tiles, capped: thin tiles beside capped full ones
    (1.25, MoEConfig("cap_skew", T=2048, H=264, E=16, k=2, F=392, ffn="swiglu", dtype="bf16", bias="zipf1.1")),
]


@pytest.mark.parametrize("cf,cfg", CAP_CASES, ids=[f"{c.name}-cf{f}" for f, c in CAP_CASES])
def test_forward_with_capacity(lib, cf, cfg):
    say(f"capacity cf={cf} {cfg}")
    d = generate(cfg)
    inp = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    out = run_forward(cfg, inp, capacity_factor=cf)
    ref = _oracle_forward(cfg, d, capacity_factor=cf)
    assert ref["keep"] is not None and not ref["keep"].all()
    assert normwise(to_numpy(out), ref["out"]) <= tol_for(cfg)


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_forward_routing_variants(lib, flags):
    cfg = MoEConfig("var", T=200, H=128, E=16, k=3, F=128, ffn="silu2", dtype="f32", bias="normal0.5")
    say(f"routing variant flags={flags}")
    d = generate(cfg)
    inp = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    out = run_forward(cfg, inp, flags=flags)
    ref = _oracle_forward(cfg, d, select_only=bool(flags & 1), renorm=not (flags & 2))
    assert normwise(to_numpy(out), ref["out"]) <= tol_for(cfg)


def test_router_stats(lib):
    cfg = MoEConfig("st", T=999, H=64, E=40, k=3, F=8, ffn="swiglu", dtype="f32", bias="normal0.5")
    say("router stats")
    d = generate(cfg, experts=False)
    # both sides start from the same fp32 logits (made on the CPU)
    L32 = O.gate_logits(to_numpy(d["x"]), to_numpy(d["w_gate"])).astype(np.float32)
    b32 = d["bias"].numpy()
    logits = torch.from_numpy(L32).cuda()
    idx, _ = lib.route_from_logits(logits, cfg.k, bias=d["bias"].cuda())
    r = lib.permute(idx, cfg.E)
    s = lib.router_stats(logits, r["counts"], cfg.k, bias=d["bias"].cuda())
    torch.cuda.synchronize()
    s = s.cpu().numpy().astype(np.float64)
    l, ridx, _ = O.route_from_f32_logits(L32, b32, cfg.k)
    ref = O.router_stats(l.astype(np.float64), ridx, cfg.E)
    np.testing.assert_allclose(s[:cfg.E], ref["P"], rtol=1e-4, atol=1e-7)
    assert s[cfg.E] == pytest.approx(ref["balance"], rel=1e-4)
    assert s[cfg.E + 1] == pytest.approx(ref["entropy"], rel=1e-4)
    assert s[cfg.E + 2] == pytest.approx(ref["top1_mean"], rel=1e-4)
    assert s[cfg.E + 3] == 0.0
