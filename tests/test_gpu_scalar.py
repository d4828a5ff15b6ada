"""The plainly written ("scalar") kernels against the fast ones on identical
inputs: the decode expert kernel (route, gate/up + SwiGLU, partial down rows)
and the batched path's two grouped GEMMs must give the same output bits, and
so the same routing, for int4 and int8, several shapes, a stack, and the
80B-shaped layer at full size."""
import numpy as np
import pytest

import routed_expert_int4_router_amd as moe
import synth

import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _both(cfg, xb, call):
    torch = gh.torch_cuda()
    model = gh.build(cfg)
    res = []
    for kernels in (moe.KERNELS_FAST, moe.KERNELS_SCALAR):
        model.set_kernels(kernels)
        x = gh.dev_bf16(xb)
        out = gh.dev_f32((xb.shape[0], cfg.hidden))
        getattr(model, call)(x, out) if call == "stack_decode" else getattr(model, call)(0, x, out)
        torch.cuda.synchronize()
        idx, w = model.debug_routing()
        res.append((out.cpu().numpy(), idx, w))
    model.close()
    return res


@pytest.mark.parametrize("variant,n_tok", [
    (dict(), 5),
    (dict(bits=8), 5),
    (dict(hidden=512, inter=256, shared_inter=256, n_experts=100, top_k=7, norm_topk=0), 4),
    (dict(hidden=1024, inter=64, shared_inter=64, n_experts=33, top_k=5, bits=8), 4),
    (dict(hidden=64, inter=64, shared_inter=64, n_experts=3, top_k=3), 3),
    (dict(hidden=2048, inter=512, shared_inter=512, n_experts=512, top_k=10), 3),
])
def test_scalar_decode_bit_identical(variant, n_tok):
    cfg = synth.get_config("tiny", **variant)
    xb = synth.tokens(cfg.seed + 5, n_tok, cfg.hidden)
    (fo, fi, fw), (so, si, sw) = _both(cfg, xb, "layer_decode")
    assert np.array_equal(fi, si)
    assert np.array_equal(fw.view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(fo.view(np.uint32), so.view(np.uint32)), f"max diff {np.abs(fo - so).max()}"


def test_scalar_stack_bit_identical():
    cfg = synth.get_config("stack35b_int8", n_layers=3)
    xb = synth.tokens(cfg.seed, 3, cfg.hidden)
    (fo, fi, _), (so, si, _) = _both(cfg, xb, "stack_decode")
    assert np.array_equal(fi, si)
    assert np.array_equal(fo.view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("variant,n_tok,scale", [
    (dict(n_experts=4, top_k=2, hidden=512, inter=256, shared_inter=256), 200, 0),
    (dict(n_experts=33, top_k=5, hidden=256, inter=64, shared_inter=64, bias="normal"), 65, 0),
    (dict(n_experts=8, top_k=2, hidden=256, inter=128, shared_inter=128), 48, -16),   # rows with own range factors
    (dict(n_experts=512, top_k=10, hidden=2048, inter=512, shared_inter=512, bias="normal"), 256, 0),
    (dict(n_experts=64, top_k=4, hidden=512, inter=128, shared_inter=128), 12, 17),   # small tiles, mixed rows
])
def test_scalar_grouped_gemms_bit_identical(variant, n_tok, scale):
    cfg = synth.get_config("tiny", **variant)
    xb = synth.tokens(cfg.seed + 9, n_tok, cfg.hidden)
    if scale:
        x = synth.bf16_bits_to_f32(xb)
        x[0::2] *= np.float32(2.0 ** scale)
        xb = synth.f32_to_bf16_bits(x)
    (fo, fi, _), (so, si, _) = _both(cfg, xb, "layer_forward")
    assert np.array_equal(fi, si)
    assert np.array_equal(fo.view(np.uint32), so.view(np.uint32)), f"max diff {np.abs(fo - so).max()}"
