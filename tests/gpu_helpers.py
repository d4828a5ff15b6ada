"""Shared plumbing of the GPU parity tests: device buffers, model loading, and
the comparison rules against the oracle.

Matching rules:
* top-k selections are bit-exact, except where the oracle's exactly rounded
  logits of the two differing experts lie within
  eps = eps_rel * sum_h |x_h * W_r[h, e]| of each other (an fp32-vs-exact
  near-tie); such tokens are re-evaluated by the oracle with the GPU's
  selection and counted. eps_rel is 2^-16 for the decode router (fp64
  accumulation, one fp32 rounding) and prefill_eps_rel(H) for the batched
  router (3H exact bf16 products, each summed with at most one fp32 rounding);
* outputs: per-token relative L2 error <= 2e-3 against the float64 oracle.
"""
from __future__ import annotations

import numpy as np

import routed_expert_int4_router_amd as moe
from routed_expert_int4_router_amd import loader
import synth
from oracle import moe as omoe
from oracle import quant

REL_L2_TOL = 2e-3


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return torch


def dev_bf16(bits: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def dev_f32(shape):
    torch = torch_cuda()
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def build(cfg: synth.Config, storage=moe.STORE_DEVICE):
    return loader.load_model(cfg, synth.SynthWeights(cfg), storage=storage)


DECODE_EPS_REL = 2.0 ** -16


def prefill_eps_rel(hidden: int) -> float:
    """Bound on |fp32 MFMA logit - exact| / sum|x w| for the batched router:
    3 * hidden exact products (three bf16 parts per fp32 weight) accumulated
    in fp32, one rounding of at most 2^-24 relative each, plus the bias add."""
    return (3 * hidden + 2) * 2.0 ** -24


def selection_ok(gpu_sel, oracle_logits, x_row, w_r, k, eps_rel=DECODE_EPS_REL, extra=None):
    """True when gpu_sel equals the oracle's top-k, or differs only at near-ties.
    extra[e] (optional) widens expert e's tie margin by an absolute amount."""
    want = omoe.topk_order(oracle_logits, k)
    if np.array_equal(np.asarray(gpu_sel), want):
        return True, 0
    mass = omoe.route_abs_mass(x_row[None, :], w_r)[0]
    eps = eps_rel * mass
    if extra is not None:
        eps = eps + extra
    l = oracle_logits.astype(np.float64)
    for a, b in zip(want, gpu_sel):
        if a != b and abs(l[a] - l[b]) > eps[a] + eps[b]:
            return False, 1
    return True, 1


def recast_slack(r, w_r, layer):
    """Logit slack from the bf16 recast x_l = bf16(r_l) between stack layers.
    The GPU's fp32 residual is taken to agree with the oracle's fp64 one to
    within layer * 2^-20 * rms(r) + 2^-24 |r_h| per element (a few fp32 roundings
    per layer; the measured deltas agree to ~1e-6). An element whose oracle
    value lies that close to a bf16 rounding boundary may round to the other
    neighbour on the GPU, moving logit e by up to ulp_h * |w_r[h, e]|; the slack
    of e sums that over such elements. w_r is [H][E + 1] or [H][E]."""
    r = np.asarray(r, dtype=np.float64)
    xv = quant.bf16_rne_from_f64(r)
    ax = np.abs(xv)
    expo = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    ulp = np.where(ax > 0, 2.0 ** (expo - 7), 2.0 ** -133)
    delta = layer * 2.0 ** -20 * np.sqrt(np.mean(r * r)) + 2.0 ** -24 * np.abs(r)
    to_boundary = np.abs(ulp / 2 - np.abs(r - xv))
    near = to_boundary <= delta
    w = np.abs(np.asarray(w_r, dtype=np.float64))
    return (ulp * near) @ w


def check_layer(cfg, om, layer, x_bits, gpu_out, gpu_idx, tokens, eps_rel=DECODE_EPS_REL, lw=None):
    """Compare GPU outputs/selections of one layer with the oracle on the sampled tokens
    (lw overrides the oracle's weights of that layer)."""
    lw = om.layer(layer) if lw is None else lw
    x = quant.f64_from_bf16_bits(x_bits[tokens])
    res = omoe.layer_forward(x, lw, cfg.top_k, cfg.norm_topk)
    ties = 0
    sel = res.route.idx.copy()
    for i, t in enumerate(tokens):
        ok, tie = selection_ok(gpu_idx[t], res.route.logits[i], x[i], lw.w_r, cfg.top_k, eps_rel)
        assert ok, f"token {t}: GPU selection {list(gpu_idx[t])} vs oracle {list(res.route.idx[i])}"
        if tie:
            ties += 1
            sel[i] = gpu_idx[t]
    if ties:
        res = omoe.layer_forward(x, lw, cfg.top_k, cfg.norm_topk, sel=sel)
    err = omoe.rel_l2_per_token(gpu_out[tokens], res.out)
    return float(err.max()), ties


def check_routing_only(cfg, layer, x_bits, gpu_idx, eps_rel=DECODE_EPS_REL):
    """Top-k of every token against the oracle's exactly rounded logits (no expert math)."""
    w_r = synth.router_weight(cfg.seed, layer, cfg.hidden, cfg.n_experts)
    rho = synth.router_bias(cfg, layer)
    x = quant.f64_from_bf16_bits(x_bits)
    logits = omoe.router_logits(x, w_r, rho)
    ties = 0
    for t in range(x.shape[0]):
        ok, tie = selection_ok(gpu_idx[t], logits[t], x[t], w_r, cfg.top_k, eps_rel)
        assert ok, f"token {t}: selection {list(gpu_idx[t])} vs {list(omoe.topk_order(logits[t], cfg.top_k))}"
        ties += tie
    return ties


def check_stack(cfg, om, x0_bits, gpu_out, gpu_idx, tokens):
    """Stack parity on sampled tokens: the oracle follows the GPU's selections
    (each checked to be the oracle top-k up to near-ties); compares
    delta = r_L - r_0 per token."""
    L, k = cfg.n_layers, cfg.top_k
    x0 = quant.f64_from_bf16_bits(x0_bits[tokens])
    sels = [np.stack([gpu_idx[t * L + l] for t in tokens]) for l in range(L)]
    layers = om.layers()
    st = omoe.stack_forward(x0, layers, k, cfg.norm_topk, sels=sels)
    # validate every GPU selection against the oracle's logits at the oracle's own x_l
    ties = 0
    r = x0.copy()
    for l, lw in enumerate(layers):
        xl = quant.bf16_rne_from_f64(r)
        logits = st.routes[l].logits
        for i, t in enumerate(tokens):
            extra = recast_slack(r[i], lw.w_r, l) if l > 0 else None
            ok, tie = selection_ok(sels[l][i], logits[i], xl[i], lw.w_r, k, extra=extra)
            assert ok, f"token {t} layer {l}: selection {list(sels[l][i])} vs {list(omoe.topk_order(logits[i], k))}"
            ties += tie
        r = r + omoe.layer_forward(xl, lw, k, cfg.norm_topk, sel=sels[l]).out
    delta_gpu = gpu_out[tokens].astype(np.float64) - x0
    err = omoe.rel_l2_per_token(delta_gpu, st.delta)
    return float(err.max()), ties
