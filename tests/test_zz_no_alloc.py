"""moe_layer_forward_noalloc, the batched path with its workspace in a static
device array, against moe_layer_forward through the C ABI: bit-identical
outputs on two calls in a row (the second with fewer tokens, so it must not
depend on what the first left in the shared array), a call with no tokens,
and the size limit."""
import numpy as np
import pytest

import routed_expert_int4_router_amd as moe
import synth

import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _both(model, cfg, xb):
    torch = gh.torch_cuda()
    x = gh.dev_bf16(xb)
    ref = gh.dev_f32((xb.shape[0], cfg.hidden))
    got = gh.dev_f32((xb.shape[0], cfg.hidden))
    model.layer_forward(0, x, ref)
    model.layer_forward_noalloc(0, x, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("variant,sizes", [
    (dict(n_experts=16, top_k=4, hidden=256, inter=128, shared_inter=128), (200, 37)),
    (dict(n_experts=512, top_k=10, hidden=2048, inter=512, shared_inter=512, bias="normal"), (600, 64)),
])
def test_noalloc_equals_layer_forward_on_two_calls(variant, sizes):
    cfg = synth.get_config("tiny", **variant)
    model = gh.build(cfg)
    for i, n in enumerate(sizes):
        xb = synth.tokens(cfg.seed + 40 + i, n, cfg.hidden)
        ref, got = _both(model, cfg, xb)
        assert np.all(np.isfinite(got))
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), f"call {i} ({n} tokens) differs"
    model.close()


def test_noalloc_empty_and_over_the_limit():
    torch = gh.torch_cuda()
    cfg = synth.get_config("prefill80b")
    model = gh.build(cfg)
    x = gh.dev_bf16(synth.tokens(cfg.seed, 1, cfg.hidden))
    out = gh.dev_f32((1, cfg.hidden))
    model.layer_forward_noalloc(0, x, out, n_tok=0)
    torch.cuda.synchronize()
    assert torch.isnan(out).all(), "an empty call wrote its output"
    big = torch.zeros((4096, cfg.hidden), dtype=torch.int16, device="cuda")
    big_out = torch.empty((4096, cfg.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        model.layer_forward_noalloc(0, big, big_out)
    assert e.value.status == moe.MOE_EINVAL and "at most" in str(e.value)
    model.close()
