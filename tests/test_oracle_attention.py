"""Pins of the gated attention oracle (oracle/attention.py) against what the
pages and the mathematics fix: the pages' KV-cache sizes, rotary embedding's
defining properties, softmax attention's special cases, and the GQA grouping.
CPU only."""
import json
import os

import numpy as np

from oracle import attention as att
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_kv_sizes_are_the_pages_figures():
    """alphalab.site field test, section explaining MoE expert streaming: 12
    attention layers, 24 KiB per token in the fp16 budget, >= 48 KiB as fp32,
    384 MiB at 8K, 1.5 GiB at 32K, 12 GiB at 262,144 positions."""
    g = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["attention_kv"]
    cfg = synth.get_attn_config("attn80b")
    sh = att.Shape(cfg.n_q, cfg.n_kv, cfg.d, cfg.rot)
    assert cfg.n_layers == g["layers"]
    assert cfg.n_layers * sh.kv_bytes_per_token(2) == g["fp16_budget_kib_per_token"] * 1024
    per_tok32 = cfg.n_layers * sh.kv_bytes_per_token(4)
    assert per_tok32 == g["stored_fp32_kib_per_token"] * 1024
    assert 8192 * per_tok32 == g["mib_at_8k"] * 2 ** 20
    assert 32768 * per_tok32 == g["gib_at_32k"] * 2 ** 30
    assert 262144 * per_tok32 == g["gib_at_262144"] * 2 ** 30
    assert cfg.context == 8192


def test_rope_properties():
    rng = np.random.default_rng(1)
    d, rot = 32, 16
    x = rng.standard_normal((3, d))
    assert np.array_equal(att.rope(x, 0, rot), x)                     # position 0: identity
    y = att.rope(x, 123, rot)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1))   # a rotation
    assert np.array_equal(y[:, rot:], x[:, rot:])                     # unrotated dims untouched
    # scores depend on the relative position only
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    a = att.rope(q, 50, rot) @ att.rope(k, 20, rot)
    b = att.rope(q, 1030, rot) @ att.rope(k, 1000, rot)
    assert np.isclose(a, b, rtol=1e-9)
    # the pair (i, i + rot/2) turns by p * theta^(-2i/rot): i = 0 turns by p radians
    e = np.zeros(d)
    e[0] = 1.0
    r = att.rope(e, 3, rot)
    assert np.isclose(r[0], np.cos(3.0)) and np.isclose(r[rot // 2], np.sin(3.0))


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    d = 16
    q = rng.standard_normal(d)
    V = rng.standard_normal((5, d))
    assert np.allclose(att.attend(q, rng.standard_normal((1, d)), V[:1]), V[0])        # one position
    K = np.tile(rng.standard_normal(d), (5, 1))
    assert np.allclose(att.attend(q, K, V), V.mean(axis=0))                            # equal scores
    # brute force softmax
    K = rng.standard_normal((5, d))
    s = np.array([q @ K[j] / np.sqrt(d) for j in range(5)])
    w = np.exp(s) / np.exp(s).sum()
    assert np.allclose(att.attend(q, K, V), sum(w[j] * V[j] for j in range(5)))


def test_step_groups_and_cache():
    cfg = synth.get_attn_config("attn_tiny")
    sh = att.Shape(cfg.n_q, cfg.n_kv, cfg.d, cfg.rot)
    p = att.Params(*synth.attn_params(cfg, 0))
    kc, vc = synth.attn_cache(cfg, 0, cfg.context)
    K = np.zeros((cfg.n_kv, cfg.context + 1, cfg.d))
    V = np.zeros_like(K)
    K[:, :cfg.context] = kc.view(np.float16)
    V[:, :cfg.context] = vc.view(np.float16)
    q, gate, k, v = [synth.bf16_bits_to_f32(a[0]).astype(np.float64) for a in synth.attn_inputs(cfg, 0, 1)]
    q = q.reshape(cfg.n_q, cfg.d)
    gate = gate.reshape(cfg.n_q, cfg.d)
    k = k.reshape(cfg.n_kv, cfg.d)
    v = v.reshape(cfg.n_kv, cfg.d)
    out = att.step(sh, p, cfg.context, K, V, q, gate, k, v)
    assert out.shape == (cfg.n_q, cfg.d)
    # the new row is the fp16 of the normed, rotated k and of v
    assert np.array_equal(V[:, cfg.context], att.fp16(v))
    assert np.array_equal(K[:, cfg.context], att.fp16(att.rope(att.rms(k) * p.wk, cfg.context, cfg.rot)))
    # two query heads of one group with the same q and gate give the same output
    q2 = q.copy()
    q2[1] = q2[0]
    gate2 = gate.copy()
    gate2[1] = gate2[0]
    K2, V2 = K.copy(), V.copy()
    out2 = att.step(sh, p, cfg.context, K2, V2, q2, gate2, k, v)
    assert np.array_equal(out2[0], out2[1])
    # a zero gate halves the attention output
    out3 = att.step(sh, p, cfg.context, K.copy(), V.copy(), q, np.zeros_like(gate), k, v)
    o = att.attend(att.rope(att.rms(q[0]) * p.wq, cfg.context, cfg.rot), K[0, :cfg.context + 1], V[0, :cfg.context + 1])
    assert np.allclose(out3[0], 0.5 * o)
