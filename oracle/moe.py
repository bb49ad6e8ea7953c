"""Routed-MoE layer written out step by step in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the layer computes (readings in brackets are where the pages are silent):

1. Router logits  L[t,e] = sum_c x[t,c] * Wr[e,c] (+ bias[e])
   ("Strata-DSV4.1", §How it works: the router runs with the dense half on
   the GPU; 384 experts, top-6 per §DeepSeek-V4.1-Flash.)
2. p = softmax(L[t,:]);  S_t = the k largest logits in descending order,
   [exact ties -> lower expert index];  w_tj = p[S_tj] / sum_i p[S_ti]
   (softmax then renormalise over the selected experts).
3. Plan: per-expert counts, exclusive offsets, the pair permutation sorted
   stably by expert, and the ascending union of selected experts
   ("Feature Request: support DeepSeek V4.1 Flash ...", §Stack progress:
   request-union planning; "Strata-DSV4.1", §Latest (10-14): a verify pass
   serves the union of its experts once per layer).
4. Expert FFN per pair: g = Wg x, u = Wu x, h = silu(g) * u, y = Wd h
   (SwiGLU with the gate as the SiLU operand, per the commit notes of "run the
   DeepSeek-V4-Flash-Vision tower on CUDA"; [no clamp: no constant on the
   pages]).
5. Combine: out[t] = sum_{j=0..k-1} w_tj * y_tj + y_shared[t], in that fixed
   order ("Strata-DSV4.1", §How it works: shared expert + routed sum;
   "Feature Request ...", §Runtime stack progress: keep a single expert
   reduction order).  [The shared expert has weight 1; no routed scaling
   factor appears on the pages.]

All arithmetic is float64 on exactly dequantised weights.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

from . import formats


@dataclass
class Layer:
    """One MoE layer as the oracle sees it.

    ``expert_bytes(kind, e)`` returns the raw Q2 bytes of expert e's matrix
    ``kind`` in {"gate", "up", "down"} (gate/up: [d_ff][d_model],
    down: [d_model][d_ff]).  ``shared_bytes(kind)`` returns the Q8_0 bytes of
    the shared expert's matrix of the same shape, or is None.
    """

    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    w_router: np.ndarray  # float32 [E][d_model]
    expert_bytes: Callable[[str, int], np.ndarray]
    shared_bytes: Optional[Callable[[str], np.ndarray]] = None
    _cache: dict = field(default_factory=dict, repr=False)

    def expert_matrix(self, kind: str, e: int) -> np.ndarray:
        key = (kind, e)
        if key not in self._cache:
            rows, cols = (self.d_model, self.d_ff) if kind == "down" else (self.d_ff, self.d_model)
            self._cache[key] = formats.q2_matrix(self.expert_bytes(kind, e), rows, cols)
        return self._cache[key]

    def shared_matrix(self, kind: str) -> np.ndarray:
        key = ("shared", kind)
        if key not in self._cache:
            rows, cols = (self.d_model, self.d_ff) if kind == "down" else (self.d_ff, self.d_model)
            self._cache[key] = formats.q8_0_matrix(self.shared_bytes(kind), rows, cols)
        return self._cache[key]


# ---------------------------------------------------------------- routing


def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """L = x . Wr^T (+ bias) in float64; x [T][d], Wr [E][d]."""
    L = np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float64)[None, :]
    return L


def softmax(L: np.ndarray) -> np.ndarray:
    """Row softmax, max-subtracted."""
    z = L - L.max(axis=-1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=-1, keepdims=True)


def topk_ids(L: np.ndarray, k: int) -> np.ndarray:
    """The k largest logits per row, in descending order; an exact tie goes to
    the lower expert index.  Returns int64 [T][k]."""
    T, E = L.shape
    out = np.empty((T, k), dtype=np.int64)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -L[t]))  # primary key -L, secondary key e
        out[t] = order[:k]
    return out


def route(x, w_router, k: int, bias=None):
    """Steps 1-2.  Returns (ids int64 [T][k], weights float64 [T][k],
    logits float64 [T][E])."""
    L = router_logits(x, w_router, bias)
    p = softmax(L)
    ids = topk_ids(L, k)
    ps = np.take_along_axis(p, ids, axis=1)
    w = ps / ps.sum(axis=1, keepdims=True)
    return ids, w, L


def weights_for_selection(L: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Renormalised softmax weights of a given selection (used when a routing
    tie lets the GPU pick a different, equally valid selection)."""
    p = softmax(L)
    ps = np.take_along_axis(p, np.asarray(ids, dtype=np.int64), axis=1)
    return ps / ps.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------- router variants
# "Strata-DSV4.1", §Results: decode routes with selection-only biases whose
# mixing weights stay exact; "DeepSeek-V4-Flash" (what this is): hash routing
# on the first layers; the commit notes of the DeepSeek-V4-Flash-Vision
# bias work: a row routed by a table or by a biased learned top-k gathers its
# weights from the UNBIASED scores, and the scoring there is sqrt(softplus).
# Readings where the pages stop: the selection bias is added to the score
# (softmax probability or sqrt-softplus value) of every expert, the top-k of
# that sum is taken with the tie rule above, and the weights are the unbiased
# scores of the selected experts divided by their sum (for softmax scores this
# is the same renormalisation as step 2).

SCORE_SOFTMAX = "softmax"
SCORE_SQRT_SOFTPLUS = "sqrt_softplus"


def softplus(L: np.ndarray) -> np.ndarray:
    """log(1 + e^L) in float64, written so that large |L| neither overflows nor
    loses the small term: max(L, 0) + log1p(e^-|L|)."""
    L = np.asarray(L, dtype=np.float64)
    return np.maximum(L, 0.0) + np.log1p(np.exp(-np.abs(L)))


def route_scores(L: np.ndarray, score: str) -> np.ndarray:
    """Per-expert routing score of logits L [T][E]."""
    if score == SCORE_SOFTMAX:
        return softmax(L)
    if score == SCORE_SQRT_SOFTPLUS:
        return np.sqrt(softplus(L))
    raise ValueError(score)


def route_variant(x, w_router, k: int, logit_bias=None, select_bias=None, score: str = SCORE_SOFTMAX,
                  hash_ids=None):
    """Routing with the pages' variants.  hash_ids [T][k] (a hash-routed layer:
    the rows of its token-id table for the tokens) replaces the selection.
    Returns (ids int64 [T][k], weights float64 [T][k], logits [T][E],
    selection score [T][E])."""
    L = router_logits(x, w_router, logit_bias)
    sc = route_scores(L, score)
    sel = sc if select_bias is None else sc + np.asarray(select_bias, dtype=np.float64)[None, :]
    if hash_ids is not None:
        ids = np.asarray(hash_ids, dtype=np.int64)
    else:
        ids = topk_ids(sel, k)
    # a table row may name an expert outside [0, E) or repeat one: such slots
    # are not served (see served_pairs) and get weight 0; the row's weights
    # are renormalised over the slots that are
    keep = served_pairs(ids, L.shape[1])
    g = np.where(keep, np.take_along_axis(sc, np.clip(ids, 0, L.shape[1] - 1), axis=1), 0.0)
    tot = g.sum(axis=1, keepdims=True)
    return ids, np.divide(g, tot, out=np.zeros_like(g), where=tot > 0), L, sel


# ---------------------------------------------------------------- plan


@dataclass
class Plan:
    counts: np.ndarray  # int64 [E]
    offsets: np.ndarray  # int64 [E+1], exclusive prefix sums
    perm: np.ndarray  # int64 [T*k] pair indices (t*k + j), grouped by expert, stable
    union: np.ndarray  # int64 [U], ascending experts with count > 0

    @property
    def n_union(self) -> int:
        return int(self.union.size)


def served_pairs(ids: np.ndarray, n_experts: int) -> np.ndarray:
    """Which (token, slot) pairs are served, bool [T][k].  [Reading: the pages
    route a token to k distinct experts and do not say what a selection that
    names an expert twice (a hand-written hash-routing table row, a caller's
    ids) means.  Taken here: the token gets that expert once, at its first
    slot; a later slot naming it again, or an id outside [0, E), contributes
    nothing and is reported.]"""
    ids = np.atleast_2d(np.asarray(ids, dtype=np.int64))
    T, k = ids.shape
    ok = np.zeros((T, k), dtype=bool)
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < n_experts and e not in seen:
                ok[t, j] = True
            seen.add(e)
    return ok


def plan(ids: np.ndarray, n_experts: int) -> Plan:
    """Step 3.  Pairs are numbered p = t*k + j; ``perm`` lists the served
    pairs (:func:`served_pairs`) grouped by expert in ascending expert order,
    and in ascending p inside a group."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    keep = served_pairs(ids, n_experts).reshape(-1)
    counts = np.zeros(n_experts, dtype=np.int64)
    for p, e in enumerate(flat):
        if keep[p]:
            counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    perm = np.empty(int(offsets[-1]), dtype=np.int64)
    fill = offsets[:-1].copy()
    for p, e in enumerate(flat):
        if not keep[p]:
            continue
        perm[fill[e]] = p
        fill[e] += 1
    union = np.array([e for e in range(n_experts) if counts[e] > 0], dtype=np.int64)
    return Plan(counts, offsets, perm, union)


# ---------------------------------------------------------------- FFN / combine


def silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def ffn(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """Step 4 for one or more tokens: x [n][d] -> y [n][d]."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    g = x @ wg.T
    u = x @ wu.T
    h = silu(g) * u
    return h @ wd.T


def ffn_hidden(x: np.ndarray, wg: np.ndarray, wu: np.ndarray) -> np.ndarray:
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return silu(x @ wg.T) * (x @ wu.T)


def expert_outputs(layer: Layer, x: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """y[t][j] = FFN_{ids[t,j]}(x_t) for every pair, float64 [T][k][d]."""
    T, k = ids.shape
    y = np.zeros((T, k, layer.d_model))
    pl = plan(ids, layer.n_experts)
    for e in pl.union:
        pairs = pl.perm[pl.offsets[e]:pl.offsets[e + 1]]
        toks = pairs // k
        ye = ffn(x[toks], layer.expert_matrix("gate", e), layer.expert_matrix("up", e),
                 layer.expert_matrix("down", e))
        for r, p in enumerate(pairs):
            y[p // k, p % k] = ye[r]
    return y


def shared_output(layer: Layer, x: np.ndarray) -> np.ndarray:
    if layer.shared_bytes is None:
        return np.zeros((x.shape[0], layer.d_model))
    return ffn(x, layer.shared_matrix("gate"), layer.shared_matrix("up"), layer.shared_matrix("down"))


def combine(w: np.ndarray, y: np.ndarray, y_shared: np.ndarray) -> np.ndarray:
    """Step 5: out[t] = sum_j w[t,j] y[t,j] + y_shared[t], j in order."""
    T, k = w.shape
    out = np.zeros((T, y.shape[2]))
    for t in range(T):
        acc = np.zeros(y.shape[2])
        for j in range(k):
            acc = acc + w[t, j] * y[t, j]
        out[t] = acc + y_shared[t]
    return out


@dataclass
class LayerResult:
    ids: np.ndarray
    weights: np.ndarray
    logits: np.ndarray
    out: np.ndarray


def moe_layer(layer: Layer, x: np.ndarray, bias=None, ids=None) -> LayerResult:
    """Steps 1-5 for tokens x [T][d] (float64 values of the inputs).

    ``ids`` may force a selection (a valid alternative at a routing tie); the
    weights are then those of that selection.
    """
    x = np.asarray(x, dtype=np.float64)
    r_ids, r_w, L = route(x, layer.w_router, layer.top_k, bias)
    if ids is not None:
        r_ids = np.asarray(ids, dtype=np.int64)
        r_w = weights_for_selection(L, r_ids)
    y = expert_outputs(layer, x, r_ids)
    ysh = shared_output(layer, x)
    return LayerResult(r_ids, r_w, L, combine(r_w, y, ysh))


def dense_moe(layer: Layer, x: np.ndarray, bias=None) -> np.ndarray:
    """Brute force: every expert on every token, mixed by a dense [T][E]
    gate matrix that is zero outside the selected experts.  Independent of
    :func:`plan` and :func:`combine`; must equal :func:`moe_layer`."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    L = router_logits(x, layer.w_router, bias)
    p = softmax(L)
    G = np.zeros((T, layer.n_experts))
    order = np.argsort(-L, axis=1, kind="stable")  # stable -> lower index first on ties
    for t in range(T):
        sel = order[t, :layer.top_k]
        G[t, sel] = p[t, sel] / p[t, sel].sum()
    out = shared_output(layer, x).copy()
    for e in range(layer.n_experts):
        ye = ffn(x, layer.expert_matrix("gate", e), layer.expert_matrix("up", e), layer.expert_matrix("down", e))
        out += G[:, e:e + 1] * ye
    return out


def residual_rescale(x_bf16_values: np.ndarray, out: np.ndarray) -> np.ndarray:
    """Residual step of the 40-layer stack [reading of "per-layer RMS
    rescale": r = x + out; x' = bf16(r / sqrt(mean(r^2) + 1e-6)), no learned
    weight].  Returns BF16 bits."""
    r = np.asarray(x_bf16_values, dtype=np.float64) + np.asarray(out, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + 1e-6)
    return formats.bf16_array_from_f64(r / rms)
