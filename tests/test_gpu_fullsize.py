"""GPU path vs the CPU oracle at the full layer shapes the benchmark times.

Each case draws the workload on the GPU with the seeded generators (the same inputs
the benchmark uses) and runs moe_forward at full size, so the tile height, split-K
gate and work order are the ones that are timed.  The oracle cannot evaluate every
output row at these sizes, so the checks are:

* routing for every token: the GPU's top-k from x equals the oracle's float64
  selection wherever the k-th/(k+1)-th gap is clear, and is one of the oracle's
  tie-tolerant alternatives elsewhere; its gates match the oracle's;
* grouping for every pair: the oracle's own indices, fed to moe_permute, give
  counts, offsets and both maps bit-equal to the oracle's grouping;
* the layer output on sampled tokens (clear selections only), each evaluated by the
  oracle token by token from host copies of the few experts the sample uses; the
  sample includes the first and last grouped row of each of those experts (the row
  tile edges and the ragged tail of the expert's last tile).
"""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from workloads import preset, generate, to_numpy

from gpu_util import check_selection, normwise, say, tol_for

pytestmark = pytest.mark.gpu

# workload, number of sampled tokens, cap on the experts the sample may touch
CASES = [("pages_worked_shape", 12, 6), ("mixtral_style", 12, 4), ("decode", 8, 8),
         ("fine_grained_skewed", 8, 24)]


@pytest.fixture(scope="module", autouse=True)
def lib():
    import mixture_experts_layer_46_amd as M
    from mixture_experts_layer_46_amd import _lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _lib.load()
    return M


def _clear(scores, k):
    """Tokens whose k-th and (k+1)-th scores are further apart than the near-tie band."""
    T, E = scores.shape
    if k == E:
        return np.ones(T, bool)
    s = -np.sort(-scores, axis=1)
    gap = s[:, k - 1] - s[:, k]
    tau = 1e-4 * np.maximum(1.0, np.abs(scores).max(axis=1))
    return gap > tau


def _sample(idx, clear, n, max_experts, seed):
    """Tokens with clear selections, drawn so that together they touch at most
    max_experts experts; then the first and last token of each touched expert."""
    rng = np.random.default_rng(seed)
    chosen, experts = [], set()
    for t in rng.permutation(idx.shape[0]):
        if not clear[t]:
            continue
        new = experts | set(int(e) for e in idx[t])
        if len(new) > max_experts:
            continue
        chosen.append(int(t))
        experts = new
        if len(chosen) == n:
            break
    assert chosen, "no token fits the expert cap"
    for e in sorted(experts):
        toks = np.nonzero((idx == e).any(axis=1) & clear)[0]
        for t in (toks[0], toks[-1]):
            if set(int(v) for v in idx[t]) <= experts and int(t) not in chosen:
                chosen.append(int(t))
    return sorted(chosen), sorted(experts)


@pytest.mark.parametrize("name,n_tokens,max_experts", CASES)
def test_full_size_layer(lib, name, n_tokens, max_experts):
    M = lib
    cfg = preset(name)
    say(f"full-size {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} F={cfg.F} {cfg.ffn} {cfg.dtype}")
    dev = torch.device("cuda:0")
    inp = generate(cfg, device=dev)
    out = M.forward(inp["x"], inp["w_gate"], inp["w_in"], inp["w_up"], inp["w_out"], cfg.k,
                    bias=inp["bias"])
    _, idx_g, w_g = M.route(inp["x"], inp["w_gate"], cfg.k, bias=inp["bias"])
    torch.cuda.synchronize()
    say(f"  {name}: GPU forward and route done")

    x64 = to_numpy(inp["x"])
    wg = to_numpy(inp["w_gate"])
    b = None if inp["bias"] is None else to_numpy(inp["bias"])
    scores, idx, gates = O.route(x64, wg, b, cfg.k)

    # routing, every token
    gi = idx_g.cpu().numpy()
    flips = check_selection(gi, scores, cfg.k)
    assert len(flips) <= max(2, cfg.T // 200), f"{len(flips)} near-tie flips"
    keep = np.ones(cfg.T, bool)
    keep[list(flips)] = False
    np.testing.assert_allclose(w_g.cpu().numpy()[keep], gates[keep], rtol=0, atol=1e-4)
    say(f"  {name}: routing ok ({len(flips)} near-tie flips)")

    # grouping, every pair, from the oracle's indices
    grp = M.permute(torch.from_numpy(idx).to(dev), cfg.E)
    counts, offsets, sorted_token, row_of_pair = O.group_by_expert(idx, cfg.E)
    P = cfg.T * cfg.k
    assert np.array_equal(grp["counts"].cpu().numpy(), counts)
    assert np.array_equal(grp["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(grp["sorted_token"].cpu().numpy()[:P], sorted_token)
    assert np.array_equal(grp["row_of_pair"].cpu().numpy()[:P], row_of_pair)
    say(f"  {name}: grouping bit-exact ({int((counts > 0).sum())} experts touched)")

    # layer output on sampled tokens
    toks, experts = _sample(idx, _clear(scores, cfg.k), n_tokens, max_experts, seed=7)
    host = {}
    for e in experts:
        host[e] = tuple(None if inp[n] is None else to_numpy(inp[n][e])
                        for n in ("w_in", "w_up", "w_out"))
    got = to_numpy(out[torch.tensor(toks, device=dev)])
    ref = np.stack([O.token_output(x64[t], scores[t], idx[t], host.__getitem__, cfg.ffn)
                    for t in toks])
    err = normwise(got, ref)
    say(f"  {name}: {len(toks)} sampled tokens over experts {experts}: normwise {err:.2e}")
    assert err <= tol_for(cfg)
    del inp, out
    torch.cuda.empty_cache()
