"""Edge cases of the decode and batched paths through the C ABI: empty
batches, an all-zero input (every logit equal, every expert product zero),
the widest routing the ABI takes (1024 experts, top-16), a single expert, and
the widest code rows (hidden 4096 / inter 4096 for int4, inter 2048 for int8)."""
import numpy as np
import pytest

import synth
from oracle.model import OracleModel

import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _run(model, cfg, xb, mode):
    torch = gh.torch_cuda()
    x = gh.dev_bf16(xb)
    out = gh.dev_f32((xb.shape[0], cfg.hidden))
    getattr(model, mode)(0, x, out)
    torch.cuda.synchronize()
    idx, w = model.debug_routing()
    return out.cpu().numpy(), idx, w


def _takes_prefill(cfg, n):
    return n >= 8 and cfg.hidden % 256 == 0 and cfg.bits == 4


def test_empty_batch_is_a_no_op():
    torch = gh.torch_cuda()
    cfg = synth.get_config("tiny", n_layers=2)
    model = gh.build(cfg)
    xb = synth.tokens(cfg.seed, 1, cfg.hidden)
    x = gh.dev_bf16(xb)
    model.layer_decode(0, x, gh.dev_f32((1, cfg.hidden)))
    torch.cuda.synchronize()
    assert model.debug_routing()[0].shape[0] == 1
    for call in (lambda o: model.layer_decode(0, x, o, n_tok=0),
                 lambda o: model.layer_forward(0, x, o, n_tok=0),
                 lambda o: model.stack_decode(x, o, n_tok=0)):
        out = gh.dev_f32((1, cfg.hidden))
        call(out)
        torch.cuda.synchronize()
        assert torch.isnan(out).all(), "an empty call wrote its output"
        assert model.debug_routing()[0].shape[0] == 0
    # NULL pointers are accepted with no tokens
    empty = torch.empty((0, cfg.hidden), dtype=torch.int16, device="cuda")
    model.layer_decode(0, empty, torch.empty((0, cfg.hidden), device="cuda"))
    model.close()


@pytest.mark.parametrize("variant,n_tok,mode", [
    (dict(n_experts=33, top_k=5), 7, "layer_decode"),
    (dict(n_experts=33, top_k=5, norm_topk=0, bits=8), 7, "layer_decode"),
    (dict(n_experts=33, top_k=5, hidden=256), 64, "layer_forward"),
    (dict(n_experts=33, top_k=5, hidden=256, norm_topk=0), 64, "layer_forward"),
])
def test_zero_input_gives_index_order_and_exact_zero(variant, n_tok, mode):
    """x = 0 with no router bias: all logits are exactly 0, so the selection is
    experts 0..k-1 (index order breaks ties), each weight is 1/k (renormalised)
    or 1/E, and every product of a zero input is zero, so the output is exactly 0."""
    cfg = synth.get_config("tiny", bias="none", **variant)
    if mode == "layer_forward":
        assert _takes_prefill(cfg, n_tok)
    model = gh.build(cfg)
    out, idx, w = _run(model, cfg, np.zeros((n_tok, cfg.hidden), np.uint16), mode)
    k, E = cfg.top_k, cfg.n_experts
    assert np.array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (n_tok, 1)))
    want = 1.0 / (k if cfg.norm_topk else E)
    assert np.allclose(w, want, rtol=2 ** -22, atol=0)
    assert np.all(out == 0.0)
    model.close()


@pytest.mark.parametrize("variant,n_tok,mode", [
    # widest routing: 1024 experts, top-16 (every lane ranks 16 logits)
    (dict(n_experts=1024, top_k=16, hidden=256, inter=64, shared_inter=64), 9, "layer_decode"),
    (dict(n_experts=1024, top_k=16, hidden=256, inter=64, shared_inter=64, bias="normal"), 300, "layer_forward"),
    # a single routed expert: its weight is 1 under either normalisation
    (dict(n_experts=1, top_k=1, hidden=256, inter=64, shared_inter=64), 5, "layer_decode"),
    (dict(n_experts=1, top_k=1, hidden=256, inter=64, shared_inter=64, norm_topk=0), 40, "layer_forward"),
    # widest code rows: hidden and inter at 4096 (int4), the unfused decode kernels and
    # the batched kernels at 64 groups along K
    (dict(n_experts=4, top_k=2, hidden=4096, inter=4096, shared_inter=4096), 3, "layer_decode"),
    (dict(n_experts=4, top_k=2, hidden=4096, inter=4096, shared_inter=4096), 16, "layer_forward"),
    # smallest hidden with the widest int4 inter: 384 partial rows in the fused decode
    (dict(n_experts=4, top_k=2, hidden=64, inter=4096, shared_inter=4096), 3, "layer_decode"),
    # widest int8 rows: inter 2048 with (k + 1) * inter near the limit
    (dict(n_experts=8, top_k=6, hidden=2048, inter=2048, shared_inter=2048, bits=8), 3, "layer_decode"),
])
def test_extreme_shapes_parity(variant, n_tok, mode):
    cfg = synth.get_config("tiny", **variant)
    if mode == "layer_forward":
        assert _takes_prefill(cfg, n_tok)
    model = gh.build(cfg)
    xb = synth.tokens(cfg.seed + 5, n_tok, cfg.hidden)
    print(f"{variant} T={n_tok} {mode}", flush=True)
    out, idx, w = _run(model, cfg, xb, mode)
    model.close()
    assert idx.shape == (n_tok, cfg.top_k)
    assert np.all(np.isfinite(out))
    if cfg.n_experts == 1:
        assert np.all(idx == 0)
        if cfg.norm_topk:
            assert np.all(w == 1.0)
    eps = gh.prefill_eps_rel(cfg.hidden) if mode == "layer_forward" else gh.DECODE_EPS_REL
    err, ties = gh.check_layer(cfg, OracleModel(cfg), 0, xb, out, idx, list(range(n_tok)), eps_rel=eps)
    print(f"  max rel L2 {err:.3e}, near-ties {ties}")
    assert err <= gh.REL_L2_TOL
