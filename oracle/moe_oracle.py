"""CPU oracle of the token-choice MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
module.  The product path (the HIP library and its Python binding) never does, and
shares no code with it: this file is plain numpy in float64, written from the pages.

Pages cited (by title and section):
  [FourStage]  "MoE显存与计算开销四阶段手算指南" (bjdmk.com.cn/news/5154310)
  [Principles] "MoE混合专家模型计算原理与推理部署实战解析" (sheratonhq.com/news/207562)

What the layer computes, for every token t with hidden state x_t:
  1. router logits  l_t = x_t @ W_g (+ b)                    [FourStage §2.1], [Principles §2.1]
  2. probabilities  p_t = softmax(l_t) over all E experts     [FourStage §2.2], [Principles §2.1]
  3. the k experts with the largest p_t, their probabilities renormalised to sum
     to 1                                                     [Principles §2.2]
  4. each selected expert runs its FFN on x_t: SwiGLU         [Principles §3.1]
     or the two-layer SiLU FFN (hidden -> d_ff -> hidden)     [FourStage §2, §2.3]
  5. y_t = sum_j g'_j * Expert_{e_j}(x_t)                     [Principles §2.2], [FourStage §2.4]
Grouping tokens by expert (count, prefix sum, permutation, [Principles §5.1]) is an
exact reordering of step 4; the oracle performs it too so that the GPU's grouping
tensors can be compared bit for bit.

Readings of points the pages leave open:
  * selection is made on the logits (after the bias), not on rounded probabilities:
    softmax is strictly increasing, so the chosen set is the same in exact
    arithmetic; equal values go to the lower expert index; -0 equals +0.
  * the logit bias is added before the softmax (a gate bias).
  * experts have no bias vectors; weights are [in, out] and used as h @ W.
  * SiLU(z) = z / (1 + exp(-z)); the two-layer FFN is SiLU(x @ W1) @ W2.
  * no capacity limit unless ``capacity_factor`` is given (then [Principles §4.3]).
"""
from __future__ import annotations

import itertools
import math

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------- routing

def gate_logits(x, w_gate, bias=None):
    """Router logits l = x @ W_g (+ b), float64.  [FourStage §2.1], [Principles §2.1]"""
    l = np.asarray(x, F64) @ np.asarray(w_gate, F64)
    if bias is not None:
        l = l + np.asarray(bias, F64)[None, :]
    return l


def softmax(l):
    """Row softmax over the expert axis (max-shifted).  [Principles §2.1]"""
    l = np.asarray(l, F64)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def select_topk(scores, k):
    """Indices of the k largest scores per row, largest first; equal scores go to
    the lower index (IEEE equality, so -0 == +0).  [FourStage §2.2], [Principles §2.1]"""
    scores = np.asarray(scores, F64)
    T, E = scores.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    eidx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((eidx, -scores), axis=-1)   # primary: score desc; then index asc
    return order[:, :k].astype(np.int32)


def renormalised_gates(logits, idx, renorm=True):
    """Softmax over all experts, then the selected probabilities divided by their
    sum: g'_j = p_{e_j} / sum_j' p_{e_j'}.  [Principles §2.1, §2.2]
    With renorm=False the selected probabilities are returned as they are, as in the
    walk-through of [FourStage §3]."""
    p = softmax(logits)
    sel = np.take_along_axis(p, np.asarray(idx, np.int64), axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True) if renorm else sel


def route(x, w_gate, bias, k, select_only=False, renorm=True):
    """Full-precision routing from the hidden states: (scores, idx, gates).
    The ranking score is l + b.  With select_only the bias only picks the experts and
    the gates come from the unbiased logits l ([Principles §4.4])."""
    l = gate_logits(x, w_gate, None)
    s = l if bias is None else l + np.asarray(bias, F64)[None, :]
    idx = select_topk(s, k)
    return s, idx, renormalised_gates(l if select_only else s, idx, renorm)


def route_from_f32_logits(logits32, bias32, k, select_only=False, renorm=True):
    """Routing from given fp32 logits, the way the bit-exact check feeds both sides:
    the biased score is one IEEE fp32 add, l' = fp32(L + b); the set is then chosen
    on l' and the gates computed in float64 from l' (or from L with select_only)."""
    L = np.asarray(logits32, np.float32)
    l = L
    if bias32 is not None:
        l = (L + np.asarray(bias32, np.float32)[None, :]).astype(np.float32)
    idx = select_topk(l.astype(F64), k)
    return l, idx, renormalised_gates((L if select_only else l).astype(F64), idx, renorm)


def topk_alternatives(logits_row, k, tol):
    """All top-k selections of one token that are correct when logits within ``tol``
    of the k-th largest are taken as tied: experts clearly above the boundary are
    always in, and the remaining slots are filled from the boundary band.  Each
    alternative is returned in slot order (score desc, then index asc)."""
    l = np.asarray(logits_row, F64)
    order = select_topk(l[None, :], l.size)[0]
    kth = l[order[k - 1]]
    sure = [e for e in order if l[e] > kth + tol]
    band = [e for e in order if abs(l[e] - kth) <= tol]
    need = k - len(sure)
    alts = []
    for pick in itertools.combinations(band, need):
        chosen = set(sure) | set(pick)
        alts.append(np.array([e for e in order if e in chosen], np.int32))
    return alts


# ---------------------------------------------------------------------------- grouping

def group_by_expert(idx, E):
    """Count, prefix-sum and permute the token-expert pairs into expert-major order.
    [FourStage §2.3], [Principles §5.1 steps 2-3]

    Pair p = t*k + j.  Returns
      counts[e]          number of pairs routed to expert e (sums to T*k)
      offsets[e]         start row of expert e in the grouped buffer; offsets[E] = T*k
      sorted_token[r]    token whose row sits at grouped row r (ascending t within e)
      row_of_pair[p]     grouped row of pair p
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")        # grouped row r -> pair p
    sorted_token = (order // k).astype(np.int32)
    row_of_pair = np.empty(T * k, np.int32)
    row_of_pair[order] = np.arange(T * k, dtype=np.int32)
    return counts, offsets, sorted_token, row_of_pair


# --------------------------------------------------------------------------- expert FFN

def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(X, w_in, w_up, w_out, ffn):
    """One expert on its rows X [n, H].
    swiglu: (SiLU(X @ W_gate) * (X @ W_up)) @ W_down      [Principles §3.1]
    silu2:  SiLU(X @ W1) @ W2  (hidden -> d_ff -> hidden)  [FourStage §2, §2.3]"""
    X = np.asarray(X, F64)
    a = X @ np.asarray(w_in, F64)
    if ffn == "swiglu":
        h = silu(a) * (X @ np.asarray(w_up, F64))
    elif ffn == "silu2":
        h = silu(a)
    else:
        raise ValueError(ffn)
    return h @ np.asarray(w_out, F64)


def _expert_weights(weights, e):
    """weights: (w_in, w_up, w_out) arrays stacked over experts, or a callable e -> tuple."""
    if callable(weights):
        return weights(e)
    w_in, w_up, w_out = weights
    return w_in[e], (None if w_up is None else w_up[e]), w_out[e]


def grouped_ffn(x_perm, offsets, weights, ffn):
    """Expert e runs on grouped rows [offsets[e], offsets[e+1]).  [Principles §3.2, §5.1 step 4]"""
    x_perm = np.asarray(x_perm, F64)
    y = np.zeros_like(x_perm)
    E = len(offsets) - 1
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            w_in, w_up, w_out = _expert_weights(weights, e)
            y[r0:r1] = expert_ffn(x_perm[r0:r1], w_in, w_up, w_out, ffn)
    return y


def combine(y_perm, row_of_pair, gates):
    """y_t = sum_j g'_{t,j} * y_perm[row_of_pair[t*k + j]], in slot order j.
    [FourStage §2.4], [Principles §2.2, §5.1 step 5]"""
    gates = np.asarray(gates, F64)
    T, k = gates.shape
    rop = np.asarray(row_of_pair).reshape(T, k)
    y_perm = np.asarray(y_perm, F64)
    out = np.zeros((T, y_perm.shape[1]), F64)
    for j in range(k):
        out += gates[:, j, None] * y_perm[rop[:, j]]
    return out


# ------------------------------------------------------------------------- whole layer

def forward(x, w_gate, bias, weights, k, ffn, capacity_factor=None, select_only=False,
            renorm=True):
    """The layer forward on all tokens of x [T, H]; returns every intermediate.

    ``logits`` in the result is the ranking score l + b.
    ``weights`` is (w_in, w_up, w_out) stacked over experts, or a callable that
    returns one expert's (w_in, w_up, w_out) -- so large layers can be streamed one
    expert at a time.  With ``capacity_factor`` the grouped rows of an expert beyond
    C = ceil(cf * T * k / E) (later tokens first to go) contribute nothing
    ([Principles §4.3]; "total_tokens" read as token-expert pairs)."""
    x = np.asarray(x, F64)
    E = np.asarray(w_gate).shape[1]
    logits, idx, gates = route(x, w_gate, bias, k, select_only, renorm)
    counts, offsets, sorted_token, row_of_pair = group_by_expert(idx, E)
    x_perm = x[sorted_token]
    y_perm = grouped_ffn(x_perm, offsets, weights, ffn)
    keep = None
    if capacity_factor is not None:
        cap = capacity(capacity_factor, x.shape[0], k, E)
        keep = np.zeros(len(sorted_token), bool)
        for e in range(E):
            keep[offsets[e]:offsets[e] + min(cap, int(counts[e]))] = True
        y_perm = np.where(keep[:, None], y_perm, 0.0)
    out = combine(y_perm, row_of_pair, gates)
    return dict(logits=logits, idx=idx, gates=gates, counts=counts, offsets=offsets,
                sorted_token=sorted_token, row_of_pair=row_of_pair, x_perm=x_perm,
                y_perm=y_perm, out=out, keep=keep)


def capacity(capacity_factor, T, k, E):
    """Per-expert row limit C = ceil(cf * T * k / E).  [Principles §4.3]"""
    return int(math.ceil(capacity_factor * (T * k) / E))


def token_output(x_row, logits_row, sel, weights, ffn):
    """Output of one token for a given selection ``sel`` (slot order), gates
    renormalised over that selection from the token's own logits."""
    x_row = np.asarray(x_row, F64)[None, :]
    p = softmax(np.asarray(logits_row, F64)[None, :])[0]
    g = p[sel] / p[sel].sum()
    out = np.zeros(x_row.shape[1], F64)
    for j, e in enumerate(sel):
        w_in, w_up, w_out = _expert_weights(weights, int(e))
        out += g[j] * expert_ffn(x_row, w_in, w_up, w_out, ffn)[0]
    return out


def dense_masked(x, w_gate, bias, weights, k, ffn):
    """Brute force for tiny layers: every expert on every token, then a dense
    [T, E] gate mask that is zero outside each token's top-k.  No grouping code."""
    x = np.asarray(x, F64)
    E = np.asarray(w_gate).shape[1]
    logits, idx, gates = route(x, w_gate, bias, k)
    mask = np.zeros((x.shape[0], E), F64)
    np.put_along_axis(mask, idx.astype(np.int64), gates, axis=-1)
    out = np.zeros_like(x)
    for e in range(E):
        w_in, w_up, w_out = _expert_weights(weights, e)
        out += mask[:, e, None] * expert_ffn(x, w_in, w_up, w_out, ffn)
    return out


# ---------------------------------------------------------------------- router statistics

def router_stats(logits, idx, E):
    """Monitoring statistics over one batch ([Principles §4.2, §5.2]):
      f_i        share of token-expert pairs routed to expert i
      P_i        mean softmax probability of expert i over the tokens
      balance    N * sum_i f_i * P_i  (1 for perfectly uniform routing)
      entropy    entropy (nats) of the per-expert load f
      top1_mean  mean over tokens of the largest softmax probability."""
    p = softmax(logits)
    counts = np.bincount(np.asarray(idx).reshape(-1), minlength=E).astype(F64)
    f = counts / counts.sum()
    P = p.mean(axis=0)
    nz = f[f > 0]
    return dict(f=f, P=P, balance=float(E * np.sum(f * P)),
                entropy=float(-np.sum(nz * np.log(nz))), top1_mean=float(p.max(axis=-1).mean()))
