"""Pins of the Gated DeltaNet oracle (oracle/deltanet.py) against what the
pages and the mathematics fix: the pages' state size, the delta rule's
defining retrieval property, its special cases, an independent matrix form of
the update, a brute-force causal convolution, and the gated norm's
invariances. CPU only."""
import json
import os

import numpy as np

from oracle import deltanet as gdn
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, n):
    x = rng.standard_normal(n)
    return x / np.linalg.norm(x)


def test_state_size_is_the_pages_72_mib():
    """alphalab.site field test, section explaining MoE expert streaming: the
    36 DeltaNet layers hold a fixed ~72 MiB state; the 80B linear-attention
    shape (32 value heads, 128 x 128 fp32 per head) gives exactly that."""
    g = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["deltanet_state"]
    cfg = synth.get_gdn_config("gdn80b")
    sh = gdn.Shape(cfg.n_k, cfg.n_v, cfg.d_k, cfg.d_v)
    assert cfg.n_layers == g["layers"] == 36
    assert cfg.n_layers * sh.state_bytes() == g["mib"] * 2 ** 20


def test_delta_rule_stores_v_at_k():
    """With no decay (alpha = 1), full write strength (beta = 1) and a unit key,
    the updated state maps k to v exactly: S'^T k = v (the delta rule replaces
    the value stored at k)."""
    rng = np.random.default_rng(1)
    s = rng.standard_normal((32, 24))
    k = _unit(rng, 32)
    v = rng.standard_normal(24)
    s2, o = gdn.delta_rule(s, k, k, v, 1.0, 1.0)
    assert np.allclose(s2.T @ k, v, rtol=0, atol=1e-12)
    assert np.allclose(o, v, rtol=0, atol=1e-12)
    # other keys orthogonal to k read what they read before
    w = rng.standard_normal(32)
    w -= (w @ k) * k
    assert np.allclose(s2.T @ w, s.T @ w, atol=1e-12)


def test_delta_rule_special_cases():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((16, 8))
    q, k, v = rng.standard_normal(16), _unit(rng, 16), rng.standard_normal(8)
    # beta = 0: pure decay
    s2, o = gdn.delta_rule(s, q, k, v, 0.25, 0.0)
    assert np.array_equal(s2, 0.25 * s)
    assert np.allclose(o, 0.25 * (s.T @ q))
    # alpha = 0: the state forgets everything and holds beta * k v^T
    s2, o = gdn.delta_rule(s, q, k, v, 0.0, 0.5)
    assert np.allclose(s2, 0.5 * np.outer(k, v), atol=1e-15)
    assert np.allclose(o, 0.5 * (k @ q) * v)


def test_delta_rule_matches_its_matrix_form():
    """Independent form of the same update: S' = alpha (I - beta k k^T) S + beta k v^T."""
    rng = np.random.default_rng(3)
    for _ in range(5):
        s = rng.standard_normal((20, 12))
        q, k, v = rng.standard_normal(20), rng.standard_normal(20), rng.standard_normal(12)
        alpha, beta = rng.uniform(), rng.uniform()
        ref = alpha * (np.eye(20) - beta * np.outer(k, k)) @ s + beta * np.outer(k, v)
        s2, o = gdn.delta_rule(s, q, k, v, alpha, beta)
        assert np.allclose(s2, ref, rtol=1e-12, atol=1e-12)
        assert np.allclose(o, ref.T @ q, rtol=1e-12, atol=1e-12)


def test_conv_matches_brute_force_over_the_history():
    rng = np.random.default_rng(4)
    C, T = 6, 9
    w = rng.standard_normal((C, 4))
    xs = rng.standard_normal((T, C))
    window = np.zeros((C, 3))
    for t in range(T):
        y, window = gdn.conv_step(window, xs[t], w)
        acc = np.zeros(C)
        for j in range(4):                      # tap j sees x(t - 3 + j), zero before t = 0
            s = t - 3 + j
            if s >= 0:
                acc += w[:, j] * xs[s]
        assert np.allclose(y, acc / (1 + np.exp(-acc)), rtol=1e-14, atol=1e-14)


def test_gated_rmsnorm_invariances():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((3, 64))
    z = rng.standard_normal((3, 64))
    w = rng.standard_normal(64)
    a = gdn.gated_rmsnorm(o, z, w)
    b = gdn.gated_rmsnorm(37.0 * o, z, w)
    assert np.allclose(a, b, rtol=1e-6)      # scale invariant (up to the 1e-6 epsilon)
    assert np.array_equal(gdn.gated_rmsnorm(o, np.zeros_like(z), w), np.zeros_like(o))
    r = a / (w * z / (1 + np.exp(-z)))       # unit rms before the gate
    assert np.allclose(np.sqrt(np.mean(r * r, axis=1)), 1.0, rtol=1e-6)


def test_layer_step_shapes_and_zero_inputs():
    cfg = synth.get_gdn_config("gdn_tiny")
    sh = gdn.Shape(cfg.n_k, cfg.n_v, cfg.d_k, cfg.d_v)
    conv_w, a_log, dt_bias, norm_w = synth.gdn_params(cfg, 0)
    p = gdn.Params(conv_w, a_log, dt_bias, norm_w)
    st = gdn.zero_state(sh)
    zero = np.zeros
    out, st2 = gdn.layer_step(sh, p, st, zero(sh.channels), zero(sh.n_v * sh.d_v), zero(sh.n_v), zero(sh.n_v))
    assert out.shape == (sh.n_v, sh.d_v)
    assert not out.any() and not st2.s.any()     # silu(0) = 0 everywhere
    qkv, z, a, b = synth.gdn_inputs(cfg, 0, 5)
    f = synth.bf16_bits_to_f32
    outs, st3 = gdn.run(sh, p, f(qkv).astype(np.float64), f(z).astype(np.float64), f(a).astype(np.float64),
                        f(b).astype(np.float64))
    assert outs.shape == (5, sh.n_v, sh.d_v) and np.all(np.isfinite(outs))
    # the window holds the last three inputs
    assert np.array_equal(st3.window, f(qkv)[2:5].T.astype(np.float64))
