"""GPU parity of the gated GQA decode attention step against the fp64 oracle
(oracle/attention.py) through the C ABI: every token's output at every layer
and every cache row the step writes, for small shapes that span several
32-position spans with a ragged tail, and on sampled tokens of the 80B shape at
its full 8192-position context in the configuration the benchmark times.

Tolerance: the kernels carry q and the softmax weights as fp16 hi + lo pairs
into fp32 MFMA accumulation, so scores and weighted sums hold about fp32
accuracy (relative error a few 1e-7 per sum of 8192 terms); the one place the
two sides may differ by more is the fp16 rounding of a new K value whose fp32
and fp64 values fall on either side of a rounding boundary (one fp16 ulp,
2^-11 relative, in that element); near zero, where fp16 spacing falls below
the fp32 rotation's own error (a few 1e-8 times the row's scale, from the fp32
sine and cosine of the reduced angle), the bound is 2^-21 absolute instead.
The bars: per-(token, layer) relative L2 error <= 1e-4; written V rows
bit-exact (fp16 of a bf16 input); written K rows within max(one fp16 ulp,
2^-21), on at most 1% of the values."""
import numpy as np
import pytest

import routed_expert_int4_router_amd as moe
import synth
from oracle import attention as att
from oracle import moe as omoe

import gpu_helpers as gh

pytestmark = pytest.mark.gpu

TOL = 1e-4
K_ABS = 2.0 ** -21


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


class Case:
    """A decode run: the GPU handle with the context cached, the device inputs,
    and the oracle's caches, which the oracle steps token by token."""

    def __init__(self, cfg, max_pos=None, n_tok=None):
        torch = gh.torch_cuda()
        self.cfg = cfg
        self.n_tok = cfg.n_tokens if n_tok is None else n_tok
        self.max_pos = cfg.context + self.n_tok if max_pos is None else max_pos
        L = cfg.n_layers
        self.net = moe.GatedAttention(L, cfg.n_q, cfg.n_kv, cfg.d, cfg.rot, self.max_pos)
        self.params = [synth.attn_params(cfg, l) for l in range(L)]
        self.K, self.V = [], []
        for l in range(L):
            self.net.set_layer(l, *self.params[l])
            k16, v16 = synth.attn_cache(cfg, l, cfg.context)
            if cfg.context:
                self.net.write_cache(l, 0, k16, v16)
            K = np.zeros((cfg.n_kv, self.max_pos, cfg.d))
            V = np.zeros((cfg.n_kv, self.max_pos, cfg.d))
            K[:, :cfg.context] = k16.view(np.float16).astype(np.float64)
            V[:, :cfg.context] = v16.view(np.float16).astype(np.float64)
            self.K.append(K)
            self.V.append(V)
        self.per = [synth.attn_inputs(cfg, l, self.n_tok) for l in range(L)]
        self.dev = []
        for i in range(4):
            arr = np.stack([self.per[l][i] for l in range(L)], axis=1)  # [T][L][...]
            self.dev.append(torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda())
        self.out = torch.full((self.n_tok, L, cfg.n_q * cfg.d), float("nan"), device="cuda")

    def decode(self, splits):
        t = 0
        for n in splits:
            d = self.dev
            self.net.decode(0, self.cfg.n_layers, self.cfg.context + t, d[0][t:t + n], d[1][t:t + n],
                            d[2][t:t + n], d[3][t:t + n], self.out[t:t + n])
            t += n
        assert t == self.n_tok
        gh.torch_cuda().cuda.synchronize()
        return self.out.cpu().numpy()

    def oracle(self, l, t, attend=True):
        """Oracle step of token t at layer l (in token order per layer): writes
        the cache row; returns out [n_q * d] (or None when attend is False)."""
        c = self.cfg
        sh = att.Shape(c.n_q, c.n_kv, c.d, c.rot)
        p = att.Params(*[np.asarray(w, np.float64) for w in self.params[l]])
        q, g, k, v = (_f64(x[t]) for x in self.per[l])
        pos = c.context + t
        q, g = q.reshape(c.n_q, c.d), g.reshape(c.n_q, c.d)
        k, v = k.reshape(c.n_kv, c.d), v.reshape(c.n_kv, c.d)
        if attend:
            return att.step(sh, p, pos, self.K[l], self.V[l], q, g, k, v).reshape(-1)
        self.K[l][:, pos] = att.fp16(att.rope(att.rms(k) * p.wk, pos, c.rot))
        self.V[l][:, pos] = att.fp16(v)
        return None

    def check_cache(self, l):
        c = self.cfg
        k16, v16 = self.net.read_cache(l, c.context, self.n_tok)
        kg = k16.view(np.float16).astype(np.float64)
        vg = v16.view(np.float16).astype(np.float64)
        ko = self.K[l][:, c.context:c.context + self.n_tok]
        vo = self.V[l][:, c.context:c.context + self.n_tok]
        assert np.array_equal(vg, vo), f"layer {l}: written V rows differ"
        diff = kg != ko
        if diff.any():
            bound = np.maximum(np.spacing(np.abs(ko).astype(np.float16)).astype(np.float64), K_ABS)
            over = np.abs(kg - ko) / bound
            assert over.max() <= 1.0, f"layer {l}: K differs by {over.max():.2f} x the bound"
            assert diff.mean() <= 0.01, f"layer {l}: {diff.mean():.3%} of K values differ"
        # the context below the new rows is untouched
        if c.context:
            k0, v0 = self.net.read_cache(l, 0, c.context)
            ke, ve = synth.attn_cache(c, l, c.context)
            assert np.array_equal(k0, ke) and np.array_equal(v0, ve), f"layer {l}: context rows changed"


@pytest.mark.parametrize("name,over,splits", [
    ("attn_tiny", {}, [9]),                                     # 18 steps: one replayed graph
    ("attn_tiny", {}, [3, 1, 5]),                               # eager calls
    ("attn_tiny", {"context": 0, "n_tokens": 40}, [40]),        # from an empty cache across two spans
    ("attn_tiny", {"context": 31, "n_tokens": 3}, [3]),         # a span boundary at position 32
    ("attn_tiny", {"n_q": 2, "n_kv": 2, "d": 128, "rot": 128}, [9]),   # one head per group, full rotation
    ("attn_tiny", {"n_q": 32, "n_kv": 2, "d": 256, "rot": 64}, [9]),   # 16 heads per group
    ("attn80b", {"n_layers": 2, "context": 1000, "n_tokens": 8}, [8]),
])
def test_attention_parity(name, over, splits):
    cfg = synth.get_attn_config(name, **over)
    gh.log(f"attention parity {name} {over} splits {splits}")
    case = Case(cfg)
    got = case.decode(splits)
    worst = 0.0
    for l in range(cfg.n_layers):
        ref = np.stack([case.oracle(l, t) for t in range(case.n_tok)])
        err = omoe.rel_l2_per_token(got[:, l, :], ref)
        worst = max(worst, float(err.max()))
        case.check_cache(l)
    gh.log(f"  max rel L2 {worst:.3e}")
    assert worst <= TOL
    case.net.close()


def test_attention_full_size_sampled():
    """The 80B shape as the benchmark runs it: 12 layers, 8192 cached
    positions, 64 tokens in one call (a replayed graph). Every written cache
    row is checked; outputs on sampled tokens (first, second, middle, last)."""
    cfg = synth.get_attn_config("attn80b")
    gh.log("attention full size: 12 layers x 64 tokens over 8192 positions")
    case = Case(cfg)
    got = case.decode([cfg.n_tokens])
    sample = {0, 1, cfg.n_tokens // 2, cfg.n_tokens - 1}
    worst = 0.0
    for l in range(cfg.n_layers):
        for t in range(cfg.n_tokens):
            ref = case.oracle(l, t, attend=t in sample)
            if ref is not None:
                err = omoe.rel_l2_per_token(got[t, l][None], ref[None])
                worst = max(worst, float(err.max()))
        case.check_cache(l)
    gh.log(f"  max rel L2 {worst:.3e}")
    assert worst <= TOL
    assert np.isfinite(got).all()
    case.net.close()


def test_attention_split_calls_bit_identical():
    cfg = synth.get_attn_config("attn_tiny", context=20, n_tokens=30)
    outs = []
    for splits in ([30], [7, 23], [1, 28, 1]):
        case = Case(cfg)
        outs.append(case.decode(splits))
        case.net.close()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))


def test_attention_last_position_and_errors():
    """Decoding into the last position of a cache whose capacity is not a
    multiple of 32, then the range and state errors."""
    torch = gh.torch_cuda()
    cfg = synth.get_attn_config("attn_tiny", context=45, n_tokens=2)
    case = Case(cfg, max_pos=47)
    got = case.decode([2])
    for l in range(cfg.n_layers):
        ref = np.stack([case.oracle(l, t) for t in range(2)])
        assert omoe.rel_l2_per_token(got[:, l, :], ref).max() <= TOL
        case.check_cache(l)
    d = case.dev
    with pytest.raises(moe.MoeError) as e:   # position 47 is past the capacity
        case.net.decode(0, 1, 47, d[0][:1], d[1][:1], d[2][:1], d[3][:1], case.out[:1])
    assert e.value.status == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError) as e:
        case.net.decode(1, 2, 0, d[0][:1], d[1][:1], d[2][:1], d[3][:1], case.out[:1])
    assert e.value.status == moe.MOE_EINVAL
    case.net.close()
    fresh = moe.GatedAttention(2, cfg.n_q, cfg.n_kv, cfg.d, cfg.rot, 64)
    with pytest.raises(moe.MoeError) as e:    # no norm weights set
        fresh.decode(0, 1, 0, d[0][:1], d[1][:1], d[2][:1], d[3][:1], torch.zeros_like(case.out[:1]))
    assert e.value.status == moe.MOE_ESTATE
    fresh.close()
