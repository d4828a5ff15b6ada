"""Repeated calls on the same device buffers. moe_layer_decode captures a call
of at least 64 tokens into a HIP graph keyed by (layer, n_tok, x, out) and
replays it on later calls with the same buffers, so every replay must read
what the buffers hold at that moment; the batched path of moe_layer_forward
launches eagerly and keeps a workspace that grows with the batch. Between
calls the test does ordinary eager work (copies, fills, synchronisations) and
checks each call against the fp64 oracle, and a repeat of earlier input bit
for bit against the first run of that input."""
import numpy as np
import pytest

import synth
from oracle.model import OracleModel

import gpu_helpers as gh

pytestmark = pytest.mark.gpu

CFG = dict(n_experts=32, top_k=4, hidden=512, inter=128, shared_inter=128)


def _fill(torch, x, bits):
    x.copy_(torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda())


def _call(model, mode, x, out):
    if mode == "decode":
        model.layer_decode(0, x, out)
    else:
        model.layer_forward(0, x, out)


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_replays_see_new_inputs(mode):
    torch = gh.torch_cuda()
    cfg = synth.get_config("tiny", **CFG)
    n = 96
    assert n >= 8  # the batched path for "prefill"
    model = gh.build(cfg)
    om = OracleModel(cfg)
    inputs = [synth.tokens(cfg.seed + 40 + i, n, cfg.hidden) for i in range(3)]
    x = torch.empty((n, cfg.hidden), dtype=torch.int16, device="cuda")
    out = gh.dev_f32((n, cfg.hidden))
    first = {}
    for step, which in enumerate([0, 1, 0, 2, 1]):
        _fill(torch, x, inputs[which])
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        _call(model, mode, x, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        idx, _ = model.debug_routing()
        assert np.all(np.isfinite(got)), f"step {step}"
        err, ties = gh.check_layer(cfg, om, 0, inputs[which], got, idx, list(range(n)),
                                   eps_rel=gh.prefill_eps_rel(cfg.hidden) if mode == "prefill" else gh.DECODE_EPS_REL)
        print(f"{mode} step {step} input {which}: max rel L2 {err:.3e}, near-ties {ties}")
        assert err <= gh.REL_L2_TOL, f"step {step}"
        if which in first:
            assert np.array_equal(got.view(np.uint32), first[which].view(np.uint32)), f"step {step}"
        else:
            first[which] = got
    model.close()


def test_prefill_after_the_workspace_grows():
    """A larger batch reallocates the batched path's workspace; a later
    smaller batch with the first buffers runs in the grown one."""
    torch = gh.torch_cuda()
    cfg = synth.get_config("tiny", **CFG)
    model = gh.build(cfg)
    om = OracleModel(cfg)
    small = synth.tokens(cfg.seed + 50, 64, cfg.hidden)
    large = synth.tokens(cfg.seed + 51, 300, cfg.hidden)
    xs = gh.dev_bf16(small)
    outs = gh.dev_f32((64, cfg.hidden))
    xl = gh.dev_bf16(large)
    outl = gh.dev_f32((300, cfg.hidden))
    for step, (x, out, bits) in enumerate([(xs, outs, small), (xl, outl, large), (xs, outs, small)]):
        out.fill_(float("nan"))
        model.layer_forward(0, x, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        idx, _ = model.debug_routing()
        n = bits.shape[0]
        toks = list(range(0, n, max(1, n // 48)))
        err, ties = gh.check_layer(cfg, om, 0, bits, got, idx, toks, eps_rel=gh.prefill_eps_rel(cfg.hidden))
        print(f"step {step} T={n}: max rel L2 {err:.3e}, near-ties {ties}")
        assert np.all(np.isfinite(got)) and err <= gh.REL_L2_TOL, f"step {step}"
    model.close()
