"""GPU parity of the batched (prefill) path: router GEMM, top-k, bucketing of
(token, slot) pairs by expert, grouped MFMA GEMMs and combine, against the
fp64 oracle through the C ABI. moe_layer_forward takes this path when
n_tok >= 8 and the layer is int4 with H % 256 == 0."""
import numpy as np
import pytest

import routed_expert_int4_router_amd as moe
import synth
from oracle.model import OracleModel

import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _forward(model, cfg, xb):
    torch = gh.torch_cuda()
    x = gh.dev_bf16(xb)
    out = gh.dev_f32((xb.shape[0], cfg.hidden))
    model.layer_forward(0, x, out)
    torch.cuda.synchronize()
    idx, w = model.debug_routing()
    return out.cpu().numpy(), idx, w


def _takes_prefill(cfg, n):
    return n >= 8 and cfg.hidden % 256 == 0 and cfg.bits == 4


# Shapes chosen to hit the tile edges: several 64-row tiles per expert with a
# ragged last tile, experts that receive no token, a shared-expert tile count
# that is not a multiple of anything, K = H from 256 to 2048 and I from 64.
PREFILL_CASES = [
    (dict(), 37),
    (dict(n_experts=4, top_k=2, hidden=512, inter=256, shared_inter=256), 200),
    (dict(n_experts=100, top_k=7, hidden=1024, inter=64, shared_inter=64, norm_topk=0), 131),
    (dict(n_experts=33, top_k=5, hidden=256, inter=64, shared_inter=64, bias="normal"), 65),
    (dict(n_experts=8, top_k=8, hidden=256, inter=128, shared_inter=128), 129),
    (dict(n_experts=64, top_k=4, hidden=2048, inter=512, shared_inter=512, bias="normal"), 64),
]


@pytest.mark.parametrize("variant,n_tok", PREFILL_CASES)
def test_prefill_small_parity(variant, n_tok):
    cfg = synth.get_config("tiny", **variant)
    assert _takes_prefill(cfg, n_tok)
    model = gh.build(cfg)
    xb = synth.tokens(cfg.seed + 11, n_tok, cfg.hidden)
    out, idx, w = _forward(model, cfg, xb)
    assert idx.shape == (n_tok, cfg.top_k)
    assert np.all(np.isfinite(out))
    err, ties = gh.check_layer(cfg, OracleModel(cfg), 0, xb, out, idx, list(range(n_tok)),
                               eps_rel=gh.prefill_eps_rel(cfg.hidden))
    print(f"{variant} T={n_tok}: max rel L2 {err:.3e}, near-ties {ties}")
    assert err <= gh.REL_L2_TOL
    model.close()


# Batches just above the batched path's threshold (8 tokens): nearly every
# touched expert holds one or two rows of a 64-row tile; up to the full 80B
# layer shape.
SMALL_BATCH_CASES = [
    (dict(), 8),
    (dict(n_experts=64, top_k=8, hidden=2048, inter=512, shared_inter=512, bias="normal"), 9),
    (dict(n_experts=512, top_k=10, hidden=2048, inter=512, shared_inter=512), 13),
]


@pytest.mark.parametrize("variant,n_tok", SMALL_BATCH_CASES)
def test_prefill_small_batches_at_the_threshold(variant, n_tok):
    cfg = synth.get_config("tiny", **variant)
    assert _takes_prefill(cfg, n_tok)
    model = gh.build(cfg)
    xb = synth.tokens(cfg.seed + 21, n_tok, cfg.hidden)
    out, idx, w = _forward(model, cfg, xb)
    assert np.all(np.isfinite(out))
    err, ties = gh.check_layer(cfg, OracleModel(cfg), 0, xb, out, idx, list(range(n_tok)),
                               eps_rel=gh.prefill_eps_rel(cfg.hidden))
    print(f"{variant} T={n_tok}: max rel L2 {err:.3e}, near-ties {ties}")
    assert err <= gh.REL_L2_TOL
    model.close()


def test_prefill_run_to_run_bit_identical_and_matches_decode_routing():
    cfg = synth.get_config("tiny", n_experts=32, top_k=4, hidden=512, inter=128, shared_inter=128)
    model = gh.build(cfg)
    xb = synth.tokens(cfg.seed + 5, 96, cfg.hidden)
    a, ia, wa = _forward(model, cfg, xb)
    b, ib, wb = _forward(model, cfg, xb)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(ia, ib) and np.array_equal(wa.view(np.uint32), wb.view(np.uint32))
    # the decode path on the same tokens: same selections up to near-ties, outputs close
    torch = gh.torch_cuda()
    x = gh.dev_bf16(xb)
    out = gh.dev_f32((96, cfg.hidden))
    model.layer_decode(0, x, out)
    torch.cuda.synchronize()
    idec, _ = model.debug_routing()
    same = np.all(idec == ia, axis=1)
    assert same.mean() > 0.9
    d = out.cpu().numpy()[same].astype(np.float64)
    p = a[same].astype(np.float64)
    rel = np.linalg.norm(d - p, axis=1) / np.maximum(np.linalg.norm(d, axis=1), 1e-30)
    assert rel.max() <= 2 * gh.REL_L2_TOL
    model.close()


def test_prefill_all_tokens_to_same_experts():
    """A router bias that sends every token to experts 0..k-1: each of them gets
    all T rows (many tiles), every other expert none."""
    cfg = synth.get_config("tiny", n_experts=24, top_k=3, hidden=256, inter=128, shared_inter=128)
    model = gh.build(cfg)
    om = OracleModel(cfg)
    lw = om.layer(0)
    bias = np.zeros(cfg.n_experts, np.float32)
    bias[:cfg.top_k] = np.float32(1000.0) - np.arange(cfg.top_k, dtype=np.float32)
    weights = synth.SynthWeights(cfg)
    wg, wu, wd = weights.shared(0)
    shared_rec = moe.pack(cfg, wg, wu, wd, inter=cfg.shared_inter)
    model.set_layer(0, weights.router(0), bias, shared_rec, weights.shared_gate(0))
    n_tok = 300
    xb = synth.tokens(cfg.seed + 3, n_tok, cfg.hidden)
    out, idx, _ = _forward(model, cfg, xb)
    assert np.all(np.sort(idx, axis=1) == np.arange(cfg.top_k)[None, :])
    err, ties = gh.check_layer(cfg, om, 0, xb, out, idx, list(range(n_tok)),
                               eps_rel=gh.prefill_eps_rel(cfg.hidden), lw=lw._replace(rho=bias))
    print(f"skewed routing: max rel L2 {err:.3e}")
    assert err <= gh.REL_L2_TOL
    model.close()


def test_prefill_workspace_regrows_and_shrinks():
    """Batches of growing then shrinking size reuse/regrow the workspace; each
    result equals a fresh model's."""
    cfg = synth.get_config("tiny", n_experts=16, top_k=4, hidden=256, inter=128, shared_inter=128)
    model = gh.build(cfg)
    fresh = {}
    for n in (16, 200, 40):
        xb = synth.tokens(cfg.seed + n, n, cfg.hidden)
        out, idx, _ = _forward(model, cfg, xb)
        m2 = gh.build(cfg)
        ref, ridx, _ = _forward(m2, cfg, xb)
        m2.close()
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32)), n
        assert np.array_equal(idx, ridx)
        fresh[n] = out
    model.close()


def test_prefill80b_full_size_every_token():
    """2048-token batch of the 80B-shaped layer in the benchmark's launch
    configuration: every token's routing and output against the oracle (which
    groups the 20,480 pairs by expert and dequantises each touched expert once)."""
    cfg = synth.get_config("prefill80b")
    model = gh.build(cfg)
    xb = synth.tokens(cfg.seed, cfg.n_tokens, cfg.hidden)
    out, idx, w = _forward(model, cfg, xb)
    model.close()
    assert idx.shape == (cfg.n_tokens, cfg.top_k)
    assert np.all(np.isfinite(out))
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-5)
    gh.log("prefill80b: oracle on all tokens")
    err, ties = gh.check_layer(cfg, OracleModel(cfg), 0, xb, out, idx, list(range(cfg.n_tokens)),
                               eps_rel=gh.prefill_eps_rel(cfg.hidden))
    print(f"prefill80b: all {cfg.n_tokens} tokens, max rel L2 {err:.3e}, near-ties {ties}")
    assert err <= gh.REL_L2_TOL


RANGE_CASES = [(17, "all"), (17, "half"), (17, "one"), (12, "half"), (12, "one"),
               (-8, "all"), (-8, "half"), (-8, "one"), (-16, "all"), (-16, "half"), (-16, "one")]


@pytest.mark.parametrize("shift,which", RANGE_CASES)
def test_prefill_scaled_activations_use_the_range_scales(shift, which):
    """x scaled by 2^shift (exact in bf16) on every token, on every second
    token, or on one token. The fp16 copies of x and h take power-of-two
    scales in either direction: large activations (2^17: max |x| >= 65504)
    are scaled down, small ones (2^-8, 2^-16: h near or below fp16's
    subnormal range) scaled up. Where the scaled tokens share 64-row tiles
    with unscaled ones, h of the two kinds differs by 2^16 to 2^34 in one
    tile, and the small rows keep a range factor of their own."""
    cfg = synth.get_config("tiny", n_experts=8, top_k=2, hidden=256, inter=128, shared_inter=128)
    n_tok = 48
    assert _takes_prefill(cfg, n_tok)
    model = gh.build(cfg)
    xb = synth.tokens(cfg.seed + 21, n_tok, cfg.hidden)
    rows = {"all": slice(None), "half": slice(0, n_tok, 2), "one": slice(5, 6)}[which]
    x = synth.bf16_bits_to_f32(xb)
    x[rows] *= np.float32(2.0 ** shift)
    xb = synth.f32_to_bf16_bits(x)
    out, idx, w = _forward(model, cfg, xb)
    assert np.all(np.isfinite(out))
    err, ties = gh.check_layer(cfg, OracleModel(cfg), 0, xb, out, idx, list(range(n_tok)),
                               eps_rel=gh.prefill_eps_rel(cfg.hidden))
    print(f"shift {shift} on {which}: max rel L2 {err:.3e}, near-ties {ties}")
    assert err <= gh.REL_L2_TOL
    model.close()


@pytest.mark.parametrize("shift,which", [(17, "half"), (17, "one"), (-16, "half"), (-16, "one")])
def test_prefill_small_tiles_scaled_activations(shift, which):
    """Experts that get at most four tokens take the dot-product path of the
    gate/up kernel (H a multiple of 512): 12 tokens over 64 experts, top-4, so
    nearly every tile holds one to three rows. Scaled and unscaled tokens then
    share such tiles, whose h rows keep range factors of their own."""
    cfg = synth.get_config("tiny", n_experts=64, top_k=4, hidden=512, inter=128, shared_inter=128)
    n_tok = 12
    assert _takes_prefill(cfg, n_tok)
    model = gh.build(cfg)
    xb = synth.tokens(cfg.seed + 31, n_tok, cfg.hidden)
    rows = {"half": slice(0, n_tok, 2), "one": slice(3, 4)}[which]
    x = synth.bf16_bits_to_f32(xb)
    x[rows] *= np.float32(2.0 ** shift)
    xb = synth.f32_to_bf16_bits(x)
    out, idx, w = _forward(model, cfg, xb)
    assert np.all(np.isfinite(out))
    err, ties = gh.check_layer(cfg, OracleModel(cfg), 0, xb, out, idx, list(range(n_tok)),
                               eps_rel=gh.prefill_eps_rel(cfg.hidden))
    print(f"small tiles, shift {shift} on {which}: max rel L2 {err:.3e}, near-ties {ties}")
    assert err <= gh.REL_L2_TOL
    model.close()


@pytest.mark.parametrize("shift", [-16, 17])
def test_decode_scaled_activations(shift):
    """The decode kernels (exact products of codes and activations, fp32
    sums) on the same scaled tokens: one token at a time, each within the
    bound."""
    cfg = synth.get_config("tiny", n_experts=8, top_k=2, hidden=256, inter=128, shared_inter=128)
    n_tok = 6
    model = gh.build(cfg)
    xb = synth.tokens(cfg.seed + 21, n_tok, cfg.hidden)
    x = synth.bf16_bits_to_f32(xb) * np.float32(2.0 ** shift)
    xb = synth.f32_to_bf16_bits(x)
    torch = gh.torch_cuda()
    xd = gh.dev_bf16(xb)
    out = gh.dev_f32((n_tok, cfg.hidden))
    model.layer_decode(0, xd, out)
    torch.cuda.synchronize()
    idx, _ = model.debug_routing()
    err, ties = gh.check_layer(cfg, OracleModel(cfg), 0, xb, out.cpu().numpy(), idx, list(range(n_tok)))
    print(f"decode shift {shift}: max rel L2 {err:.3e}, near-ties {ties}")
    assert err <= gh.REL_L2_TOL
    model.close()
