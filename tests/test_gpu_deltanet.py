"""GPU parity of the Gated DeltaNet decode step against the fp64 oracle
(oracle/deltanet.py) through the C ABI: every token's output at every layer,
and the recurrent state and conv history after the last token, for a tiny
shape and the 80B shape (16 key / 32 value heads of 128); sequences split over
several calls (eager and graph-replayed) must equal one call bit for bit."""
import numpy as np
import pytest

import routed_expert_int4_router_amd as moe
import synth
from oracle import deltanet as gdn
from oracle import moe as omoe

import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _setup(cfg):
    net = moe.GatedDeltaNet(cfg.n_layers, cfg.n_k, cfg.n_v, cfg.d_k, cfg.d_v)
    params = [synth.gdn_params(cfg, l) for l in range(cfg.n_layers)]
    for l, p in enumerate(params):
        net.set_layer(l, *p)
    return net, params


def _inputs(cfg, n_tok):
    """Per layer inputs, and the device tensors laid out [token][layer][...]."""
    torch = gh.torch_cuda()
    per = [synth.gdn_inputs(cfg, l, n_tok) for l in range(cfg.n_layers)]
    dev = []
    for i in range(4):
        arr = np.stack([per[l][i] for l in range(cfg.n_layers)], axis=1)   # [T][L][...]
        dev.append(torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda())
    return per, dev


def _oracle(cfg, params, per, l):
    sh = gdn.Shape(cfg.n_k, cfg.n_v, cfg.d_k, cfg.d_v)
    f = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)  # noqa: E731
    qkv, z, a, b = per[l]
    return gdn.run(sh, gdn.Params(*params[l]), f(qkv), f(z), f(a), f(b))


def _decode(net, cfg, dev, t0, t1, out):
    L = cfg.n_layers
    net.decode(0, L, dev[0][t0:t1], dev[1][t0:t1], dev[2][t0:t1], dev[3][t0:t1], out[t0:t1])


@pytest.mark.parametrize("name,n_tok,splits", [
    ("gdn_tiny", 16, [16]),
    ("gdn_tiny", 16, [3, 1, 12]),
    ("gdn80b", 12, [12]),
])
def test_deltanet_parity(name, n_tok, splits):
    cfg = synth.get_gdn_config(name, n_layers=2)
    torch = gh.torch_cuda()
    net, params = _setup(cfg)
    per, dev = _inputs(cfg, n_tok)
    out = torch.full((n_tok, cfg.n_layers, cfg.n_v * cfg.d_v), float("nan"), device="cuda")
    t = 0
    for n in splits:
        _decode(net, cfg, dev, t, t + n, out)
        t += n
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for l in range(cfg.n_layers):
        ref, st = _oracle(cfg, params, per, l)
        err = omoe.rel_l2_per_token(got[:, l, :], ref.reshape(n_tok, -1))
        worst = max(worst, float(err.max()))
        s, w = net.read_state(l)
        # GPU state is [n_v][d_v][d_k]; the oracle's is [n_v][d_k][d_v]
        serr = np.linalg.norm(s.transpose(0, 2, 1) - st.s) / np.linalg.norm(st.s)
        assert serr <= 1e-4, (l, serr)
        assert np.array_equal(w.astype(np.float64), st.window), "conv history differs"
    print(f"{name} splits {splits}: max rel L2 {worst:.3e}")
    assert worst <= gh.REL_L2_TOL
    net.close()


def test_deltanet_split_calls_bit_identical_and_reset():
    cfg = synth.get_gdn_config("gdn80b", n_layers=3)
    torch = gh.torch_cuda()
    net, _ = _setup(cfg)
    n_tok = 20
    _, dev = _inputs(cfg, n_tok)
    outs = []
    for splits in ([20], [7, 13], [1, 18, 1]):
        net.reset()
        out = torch.zeros((n_tok, cfg.n_layers, cfg.n_v * cfg.d_v), device="cuda")
        t = 0
        for n in splits:
            _decode(net, cfg, dev, t, t + n, out)
            t += n
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))
    # layers that have taken different numbers of tokens cannot share a call
    x = dev
    net.decode(0, 1, *[x[i][:1, :1].contiguous() for i in range(4)],
               torch.zeros((1, 1, cfg.n_v * cfg.d_v), device="cuda"))
    with pytest.raises(moe.MoeError) as e:
        net.decode(0, 2, x[0][:1], x[1][:1], x[2][:1], x[3][:1], torch.zeros((1, 2, cfg.n_v * cfg.d_v), device="cuda"))
    assert e.value.status == moe.MOE_ESTATE
    net.close()


def test_deltanet_full_size_as_benchmarked():
    """The 80B shape as the benchmark runs it: 36 layers, 256 tokens in one
    call (a replayed graph). Every layer's every token against the oracle,
    and every layer's final state and conv history. Bound 1e-4 relative L2:
    the step is fp32 throughout and the recurrence is contracting (alpha <= 1;
    I - beta k k^T with |k| = 1, beta in (0, 1)), so rounding does not grow
    with the token count beyond a few 1e-7 per step (measured: ~6e-7 on 16
    tokens)."""
    cfg = synth.get_gdn_config("gdn80b")
    torch = gh.torch_cuda()
    gh.log("deltanet full size: 36 layers x 256 tokens in one call")
    net, params = _setup(cfg)
    per, dev = _inputs(cfg, cfg.n_tokens)
    out = torch.full((cfg.n_tokens, cfg.n_layers, cfg.n_v * cfg.d_v), float("nan"), device="cuda")
    _decode(net, cfg, dev, 0, cfg.n_tokens, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = worst_s = 0.0
    for l in range(cfg.n_layers):
        ref, st = _oracle(cfg, params, per, l)
        err = omoe.rel_l2_per_token(got[:, l, :], ref.reshape(cfg.n_tokens, -1))
        worst = max(worst, float(err.max()))
        s, w = net.read_state(l)
        worst_s = max(worst_s, float(np.linalg.norm(s.transpose(0, 2, 1) - st.s) / np.linalg.norm(st.s)))
        assert np.array_equal(w.astype(np.float64), st.window), f"layer {l}: conv history differs"
        if l % 6 == 5:
            gh.log(f"  layers 0..{l}: max rel L2 {worst:.3e}, state {worst_s:.3e}")
    assert worst <= 1e-4 and worst_s <= 1e-4, (worst, worst_s)
    net.close()
