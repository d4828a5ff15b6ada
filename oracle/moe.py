"""Router, experts, combine, prefill bucketing and the residual stack (oracle).

Test infrastructure only; see the package docstring. Float64 throughout,
except where the definition itself rounds (the router logit is rounded once
to fp32, the stack re-rounds its activations to bf16).

Pages:
* Each layer sends a token to 10 of 512 experts (80B) or 8 of 256 (35B); the
  router and the shared experts belong to the always-resident dense core
  (paotong.dev commentary, paragraphs on the principle and the resident set;
  cheshm.ai article, paragraph on how it works).
* The routing weights are renormalised over the chosen experts
  (norm_topk_prob): the 80B config sets it, and the 35B config defaulting it
  to false made greedy output diverge until a fix matched mlx-lm (alphalab.site
  field test, section on the 35B correctness fix, and its FAQ item 6).
* The model is a hybrid MoE with high sparsity plus shared experts (cheshm.ai
  article, paragraph on the code base); the expert MLP form (SwiGLU) and the
  sigmoid gate on the shared expert are not printed on the pages and are the
  plain reading taken here.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Callable, Dict, List, NamedTuple, Optional, Tuple

import numpy as np

from . import quant

_U64 = 2.0 ** -53


# ------------------------------------------------------------------ router ---

def router_logits(x: np.ndarray, w_r: np.ndarray, rho: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 logits l[t,e] = fp32_rne( sum_h x[t,h] * W_r[h,e] + rho[e] ), the sum taken exactly.

    x [T][H] float64 holding bf16 values; W_r [H][E] fp32; rho [E] fp32 or None.
    Each product x*W_r is exact in float64 (8 + 24 significant bits). The
    float64 BLAS sum is within gamma_(H+1) * sum|terms| of the exact sum; when
    that interval rounds to one fp32 value it is the answer, otherwise the sum
    is redone in exact rational arithmetic and rounded once.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    W = np.asarray(w_r, dtype=np.float32).astype(np.float64)
    T, H = x.shape
    r = np.zeros(W.shape[1]) if rho is None else np.asarray(rho, dtype=np.float32).astype(np.float64)
    l64 = x @ W + r
    mag = np.abs(x) @ np.abs(W) + np.abs(r)
    bound = 4.0 * (H + 2) * _U64 * mag
    lo = (l64 - bound).astype(np.float32)
    hi = (l64 + bound).astype(np.float32)
    out = lo.copy()
    amb = np.argwhere(lo != hi)
    for t, e in amb:
        terms = [Fraction(float(x[t, h])) * Fraction(float(W[h, e])) for h in range(H)]
        out[t, e] = quant.fp32_round_exact(sum(terms, Fraction(float(r[e]))))
    return out


def route_abs_mass(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """sum_h |x[t,h] * W_r[h,e]|, used for the near-tie allowance between fp32 and exact logits."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return np.abs(x) @ np.abs(np.asarray(w_r, dtype=np.float32).astype(np.float64))


class Route(NamedTuple):
    idx: np.ndarray      # int32 [T][k], selection order: logit descending, index ascending on ties
    w: np.ndarray        # float64 [T][k] routing weights
    logits: np.ndarray   # float32 [T][E]


def topk_order(logits_row: np.ndarray, k: int) -> np.ndarray:
    """First k experts of the order (logit descending, expert index ascending); NaN sorts last."""
    l = np.asarray(logits_row, dtype=np.float64)
    key = np.where(np.isnan(l), -np.inf, l)
    e = np.arange(l.shape[0])
    order = np.lexsort((e, -key))
    return order[:k].astype(np.int32)


def route_weights(logits_row: np.ndarray, sel: np.ndarray, norm_topk: int = 1) -> np.ndarray:
    """Routing weights of the selected experts, float64.

    norm_topk = 1: softmax over the full row followed by renormalisation over
    the selection, which equals exp(l_e - m) / sum_{e' in S} exp(l_e' - m).
    norm_topk = 0: the plain softmax probabilities of the selected experts.
    """
    l = np.asarray(logits_row, dtype=np.float64)
    if norm_topk:
        ls = l[sel]
        z = np.exp(ls - ls.max())
        return z / z.sum()
    z = np.exp(l - l.max())
    return z[sel] / z.sum()


def route(x: np.ndarray, w_r: np.ndarray, rho: Optional[np.ndarray], k: int, norm_topk: int = 1) -> Route:
    logits = router_logits(x, w_r, rho)
    T = logits.shape[0]
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        idx[t] = topk_order(logits[t], k)
        w[t] = route_weights(logits[t], idx[t], norm_topk)
    return Route(idx, w, logits)


# ----------------------------------------------------------------- experts ---

def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


class DenseExpert(NamedTuple):
    """Dequantised expert weights, float64."""
    gate: np.ndarray   # [I][H]
    up: np.ndarray     # [I][H]
    down: np.ndarray   # [H][I]


def dense_expert(e: quant.Expert) -> DenseExpert:
    return DenseExpert(quant.dequantize(e.gate), quant.dequantize(e.up), quant.dequantize(e.down))


def expert_ffn(x: np.ndarray, d: DenseExpert) -> np.ndarray:
    """y = W_down ( silu(W_gate x) * (W_up x) ) for each row of x [T][H]."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    g = x @ d.gate.T
    u = x @ d.up.T
    return (silu(g) * u) @ d.down.T


class LayerWeights(NamedTuple):
    w_r: np.ndarray                  # fp32 [H][E]
    rho: Optional[np.ndarray]        # fp32 [E] or None
    g_s: np.ndarray                  # fp32 [H]
    shared: DenseExpert
    expert: Callable[[int], DenseExpert]   # e -> dequantised routed expert


class LayerResult(NamedTuple):
    out: np.ndarray      # float64 [T][H]
    route: Route
    gamma: np.ndarray    # float64 [T], sigmoid(x . g_s)


def layer_forward(x: np.ndarray, lw: LayerWeights, k: int, norm_topk: int = 1,
                  sel: Optional[np.ndarray] = None) -> LayerResult:
    """out[t] = sum_{j<k} w[t,j] * y_{idx[t,j]}(x_t) + sigmoid(x_t . g_s) * y_shared(x_t).

    Tokens are grouped by expert so each used expert is applied once to all of
    its tokens; every output row is still the plain definition. ``sel`` [T][k]
    replaces the top-k selection (used only to re-evaluate a token whose
    selection legitimately differs at a near-tie); the weights are still the
    definition's, computed from the exact logits over that selection.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    T, H = x.shape
    rt = route(x, lw.w_r, lw.rho, k, norm_topk)
    if sel is not None:
        sel = np.asarray(sel, dtype=np.int32).reshape(T, k)
        w = np.stack([route_weights(rt.logits[t], sel[t], norm_topk) for t in range(T)])
        rt = Route(sel.copy(), w, rt.logits)
    gamma = sigmoid(x @ np.asarray(lw.g_s, dtype=np.float32).astype(np.float64))
    contrib = np.zeros((T, k, H))
    for e in np.unique(rt.idx):
        tt, jj = np.nonzero(rt.idx == e)
        y = expert_ffn(x[tt], lw.expert(int(e)))
        contrib[tt, jj] = y * rt.w[tt, jj][:, None]
    out = contrib.sum(axis=1) + gamma[:, None] * expert_ffn(x, lw.shared)
    return LayerResult(out, rt, gamma)


class StackResult(NamedTuple):
    r_final: np.ndarray          # float64 [T][H]
    delta: np.ndarray            # r_final - r0
    routes: List[Route]          # per layer


def stack_forward(x0: np.ndarray, layers: List[LayerWeights], k: int, norm_topk: int = 1,
                  sels: Optional[List[np.ndarray]] = None) -> StackResult:
    """Residual stack without attention or norms: r0 = x0; x_l = bf16(r_l); r_{l+1} = r_l + out_l(x_l).

    ``sels`` (per layer, [T][k]) replaces the top-k selections, as in layer_forward.
    The returned routes keep the oracle's own logits for every layer.
    """
    r = np.atleast_2d(np.asarray(x0, dtype=np.float64)).copy()
    r0 = r.copy()
    routes = []
    for l, lw in enumerate(layers):
        xl = quant.bf16_rne_from_f64(r)
        res = layer_forward(xl, lw, k, norm_topk, None if sels is None else sels[l])
        r = r + res.out
        routes.append(res.route)
    return StackResult(r, r - r0, routes)


# --------------------------------------------------------- prefill buckets ---

class Buckets(NamedTuple):
    count: np.ndarray    # int32 [E]
    offset: np.ndarray   # int32 [E+1], exclusive prefix sum of count
    perm: np.ndarray     # int32 [T*k] pair ids p = t*k + j, grouped by expert, ascending p inside a group


def bucket_pairs(idx: np.ndarray, n_experts: int) -> Buckets:
    """Counting sort of the (token, slot) pairs of a batch by their expert."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    count = np.bincount(flat, minlength=n_experts).astype(np.int32)
    offset = np.zeros(n_experts + 1, dtype=np.int32)
    offset[1:] = np.cumsum(count)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    return Buckets(count, offset, perm)


# ------------------------------------------------------------------ errors ---

def rel_l2_per_token(y: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """||y_t - ref_t||_2 / ||ref_t||_2 for each token row."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return num / np.where(den == 0, 1.0, den)
