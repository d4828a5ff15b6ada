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

from typing import NamedTuple

import numpy as np

import routed_expert_int4_router_amd as moe
from routed_expert_int4_router_amd import loader
import synth
from oracle import moe as omoe
from oracle import quant

REL_L2_TOL = 2e-3

_T0 = None


def log(msg: str) -> None:
    """Progress line of a long GPU test, flushed to stderr and appended to
    gpurun_out/gpu_test_progress.log at the repository root: pytest captures
    stderr, and the file shows a slow step is alive either way."""
    import os
    import sys
    import time
    global _T0
    if _T0 is None:
        _T0 = time.time()
    line = f"[{time.time() - _T0:8.1f}s] {msg}"
    print(line, file=sys.stderr, flush=True)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    try:
        os.makedirs(os.path.join(root, "gpurun_out"), exist_ok=True)
        with open(os.path.join(root, "gpurun_out", "gpu_test_progress.log"), "a") as f:
            f.write(line + "\n")
    except OSError:
        pass


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
    big = cfg.n_layers * cfg.n_experts >= 4096
    if big:
        log(f"loading {cfg.name}: {cfg.n_layers} layers x {cfg.n_experts} experts")
    prog = (lambda l: log(f"  {cfg.name}: layer {l + 1} of {cfg.n_layers} filled") if l % 8 == 7 else None) \
        if big else None
    m = loader.load_model(cfg, synth.SynthWeights(cfg), storage=storage, progress=prog)
    if big:
        log(f"loaded {cfg.name}")
    return m


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


class Replay(NamedTuple):
    x: np.ndarray        # uint16 [L][T][H]: bf16 input of every layer
    idx: np.ndarray      # int32 [L][T][k]: the selection of every (layer, token)
    out: np.ndarray      # float32 [L][len(keep)][H]: layer outputs of the kept tokens
    r_final: np.ndarray  # float32 [T][H]: r_L


def replay_layers(model, cfg, x0_bits, keep=()):
    """Run a resident stack one layer at a time through moe_layer_decode, with
    the fp32 residual r_{l+1} = r_l + out_l and the recast x_{l+1} = bf16(r_{l+1})
    done by torch (IEEE fp32 add, round to nearest even): the same operations
    the stack's own epilogue performs, so r_L must equal moe_stack_decode's
    output bit for bit. Gives each layer's actual input, selection and output."""
    torch = torch_cuda()
    L, T, H = cfg.n_layers, x0_bits.shape[0], cfg.hidden
    x = dev_bf16(x0_bits)
    r = x.view(torch.bfloat16).float()
    xs = np.empty((L, T, H), np.uint16)
    idxs = np.empty((L, T, cfg.top_k), np.int32)
    outs = np.empty((L, len(keep), H), np.float32)
    keep_t = torch.as_tensor(list(keep), dtype=torch.long, device="cuda")
    out = dev_f32((T, H))
    for l in range(L):
        if l % 8 == 0:
            log(f"replay: layer {l} of {L}")
        model.layer_decode(l, x, out)
        idx, _ = model.debug_routing()   # synchronises the device
        xs[l] = x.cpu().numpy().view(np.uint16)
        idxs[l] = idx
        if len(keep):
            outs[l] = out[keep_t].cpu().numpy()
        r = r + out
        x = r.to(torch.bfloat16).view(torch.int16).contiguous()
    return Replay(xs, idxs, outs, r.cpu().numpy())


def check_layers_local(cfg, om, rep, keep=(), eps_rel=DECODE_EPS_REL):
    """Layer-local parity of a stack at its actual layer inputs: every
    (layer, token) selection against the oracle's exactly rounded logits of
    that layer's GPU input x_l (no slack beyond the fp32 router's), and the
    outputs of the kept tokens against the oracle's layer at the same x_l.
    Returns (max rel L2 over kept tokens and layers, near-ties)."""
    ties = 0
    worst = 0.0
    for l in range(cfg.n_layers):
        if l % 8 == 0:
            log(f"layer-local oracle checks: layer {l} of {cfg.n_layers}")
        w_r = synth.router_weight(cfg.seed, l, cfg.hidden, cfg.n_experts)
        rho = synth.router_bias(cfg, l)
        x = quant.f64_from_bf16_bits(rep.x[l])
        logits = omoe.router_logits(x, w_r, rho)
        for t in range(x.shape[0]):
            ok, tie = selection_ok(rep.idx[l, t], logits[t], x[t], w_r, cfg.top_k, eps_rel)
            assert ok, (f"layer {l} token {t}: selection {list(rep.idx[l, t])} vs "
                        f"{list(omoe.topk_order(logits[t], cfg.top_k))}")
            ties += tie
        if len(keep):
            err, _ = check_layer(cfg, om, l, rep.x[l], _scatter(rep.out[l], keep, rep.x.shape[1]),
                                 rep.idx[l], list(keep), eps_rel)
            worst = max(worst, err)
    return worst, ties


def _scatter(rows, keep, T):
    full = np.zeros((T, rows.shape[1]), np.float32)
    full[list(keep)] = rows
    return full


def check_stack(cfg, om, x0_bits, gpu_out, gpu_idx, tokens):
    """End-to-end stack parity on sampled tokens: the oracle runs the whole
    stack in fp64 from x0 (r0 = x0, x_l = bf16(r_l)), taking at each layer the
    GPU's selection (each one is checked against the oracle at the GPU's own
    layer input by check_layers_local), and delta = r_L - r_0 is compared per
    token. The oracle's x_l can differ from the GPU's in an element whose
    residual lies within rounding of a bf16 boundary; its effect on delta is
    part of the measured error."""
    L, k = cfg.n_layers, cfg.top_k
    x0 = quant.f64_from_bf16_bits(x0_bits[tokens])
    sels = [np.stack([gpu_idx[t * L + l] for t in tokens]) for l in range(L)]
    st = omoe.stack_forward(x0, om.layers(), k, cfg.norm_topk, sels=sels)
    delta_gpu = gpu_out[tokens].astype(np.float64) - x0
    err = omoe.rel_l2_per_token(delta_gpu, st.delta)
    return float(err.max())
