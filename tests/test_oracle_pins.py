"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: a figure a
page prints (tests/golden/pages_figures.json), a hand-worked example
(tests/golden/quant_hand_examples.json), a closed form, exact rational
arithmetic, a brute-force twin on tiny inputs, or a special case that reduces
to a textbook routine.
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import synth
from oracle import moe, pool, quant
from oracle.model import OracleModel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------ sizes, offsets

def test_record_sizes_closed_form():
    # 3 matrices of H*I codes at b bits + 3 * (H*I/64) (scale, bias) fp16 pairs
    assert quant.record_bytes(2048, 512, 4) == 1_769_472
    assert quant.record_bytes(2048, 512, 8) == 3_342_336
    assert quant.record_bytes(256, 128, 4) == 55_296
    assert quant.record_stride(2048, 512, 4) == 1_769_472 == 432 * 4096
    assert quant.record_stride(2048, 512, 8) == 3_342_336 == 816 * 4096
    assert quant.record_stride(256, 128, 4) == 57_344 == 14 * 4096
    lay = quant.record_layout(2048, 512, 4)
    assert lay.end == 1_769_472
    assert lay.up_codes == 512 * 2048 // 2


def test_zero_hit_fetch_matches_printed_figure():
    g = _golden("pages_figures.json")
    fetch = g["zero_hit_fetch"]
    layers = g["layers_80b"]["value"]
    k = g["routing"]["80b"]["top_k"]
    assert layers * k == fetch["experts_per_token"]
    total = fetch["experts_per_token"] * quant.record_bytes(2048, 512, 4)
    # the page prints "about 810 MiB"; the int4 record makes it exactly 810.0 MiB
    assert total == 849_346_560
    assert total / 2 ** 20 == pytest.approx(fetch["logical_mib"], abs=0.5)


def test_container_sizes_consistent_with_printed_totals():
    g = _golden("pages_figures.json")
    rec4 = quant.record_bytes(2048, 512, 4)
    rec8 = quant.record_bytes(2048, 512, 8)
    routed_80b = 48 * 512 * rec4
    manifest = g["manifest_80b"]["gb"] * 1e9
    # routed records must fit inside the printed manifest, the rest being the dense core
    assert routed_80b < manifest
    assert manifest - routed_80b == pytest.approx(1.35e9, rel=0.01)
    assert g["manifest_80b"]["gb"] * 1e9 / 2 ** 30 == pytest.approx(g["manifest_80b"]["gib"], abs=0.01)
    # 35B: 40 layers x 256 experts; printed disk sizes (GB, 2 digits) cover records + dense core
    routed_35b_4 = 40 * 256 * rec4
    routed_35b_8 = 40 * 256 * rec8
    dense_35b_4 = g["dense_core_4bit"]["35b_gb"] * 1e9
    assert (routed_35b_4 + dense_35b_4) / 2 ** 30 == pytest.approx(g["disk"]["35b_int4_gb"], abs=0.5)
    assert routed_35b_8 / 2 ** 30 < g["disk"]["35b_int8_gb"] < (routed_35b_8 + 2 * 2 * dense_35b_4) / 2 ** 30
    assert (routed_80b / 2 ** 30) < g["disk"]["80b_int4_gb"] < manifest / 2 ** 30 + 0.5


def test_blob_offsets_64bit():
    stride = quant.record_stride(2048, 512, 4)
    base = 4096
    for gid in [0, 1, 511, 512, 2427, 2428, 24_575]:
        assert quant.blob_offset(base, gid, stride) == base + gid * stride
    last = quant.blob_offset(0, 24_575, stride)
    assert last > 2 ** 32
    assert last + stride == 43_486_543_872


# -------------------------------------------------------------- rounding

def _fp16_exact_rne(v: float) -> np.float16:
    """Textbook round-to-nearest-even onto the fp16 grid, in exact rationals."""
    fr = Fraction(v)
    if fr == 0:
        return np.float16(0.0) if math.copysign(1, v) > 0 else np.float16(-0.0)
    a = abs(fr)
    e = math.floor(math.log2(a)) if a >= Fraction(1, 2 ** 14) else -14
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    n = a / ulp
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * ulp
    if val > 65504:
        return np.float16(np.inf if v > 0 else -np.inf)
    return np.float16(float(val) if v > 0 else -float(val))


def test_fp16_rounding_is_rne():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(2000).astype(np.float32) * 0.05)
    vals += list((rng.standard_normal(500) * 1e-6).astype(np.float32))       # subnormal fp16 range
    # exact ties halfway between fp16 neighbours
    for m in [1025, 1027, 2047, 1500]:
        vals.append(np.float32((m + 0.5) * 2.0 ** -10))
        vals.append(np.float32((m + 0.5) * 2.0 ** -24))
    for v in vals:
        got = quant.fp16_rne(np.float32(v))
        want = _fp16_exact_rne(float(v))
        assert got.view(np.uint16) == want.view(np.uint16), v


def test_bf16_rounding_from_f64():
    rng = np.random.default_rng(2)
    vals = list(rng.standard_normal(3000) * 3.0) + [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),
                                                    1.0 + 2 ** -8 + 2 ** -40, 0.0, 2.0 ** -130]
    got = quant.bf16_rne_from_f64(np.array(vals))
    for v, g in zip(vals, got):
        fr = Fraction(v)
        if fr == 0:
            assert g == 0
            continue
        a = abs(fr)
        e = max(math.floor(math.log2(a)), -126)
        while Fraction(2) ** e > a and e > -126:
            e -= 1
        ulp = Fraction(2) ** (e - 7)
        n = a / ulp
        fl = math.floor(n)
        rem = n - fl
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
            fl += 1
        want = float(fl * ulp) * (1 if v > 0 else -1)
        assert g == want, v
    # ties go to even
    assert quant.bf16_rne_from_f64(1.0 + 2 ** -8) == 1.0
    assert quant.bf16_rne_from_f64(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6


# --------------------------------------------------------- quantisation

def _hand_groups():
    a = (-1 + 0.25 * (np.arange(64) % 16)).astype(np.float32)
    b = np.full(64, 0.5, dtype=np.float32)
    c = np.zeros(64, dtype=np.float32)
    c[:5] = [0, 1.875, 0.0625, 0.1875, 0.3125]
    d = (0.125 * (np.arange(64) % 16)).astype(np.float32)
    d[np.arange(64) % 16 == 0] = -0.0
    return [a, b, c, d]


def test_quant_hand_examples():
    ex = _golden("quant_hand_examples.json")["examples"]
    assert len(ex) == len(_hand_groups())
    for w, e in zip(_hand_groups(), ex):
        m = quant.quantize(w[None, :], 4)
        assert int(m.s.view(np.uint16)[0, 0]) == int(e["scale_fp16_bits"], 16), e["name"]
        assert int(m.c.view(np.uint16)[0, 0]) == int(e["bias_fp16_bits"], 16), e["name"]
        assert quant.encode_codes(m.q, 4).tobytes().hex() == e["code_bytes_hex"], e["name"]


def test_quant_grid_invariants_and_error_bound():
    rng = np.random.default_rng(3)
    for bits in (4, 8):
        w = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
        w[3, :64] = 0.125          # a degenerate group
        m = quant.quantize(w, bits)
        qmax = (1 << bits) - 1
        assert m.q.min() >= 0 and m.q.max() <= qmax
        wh = quant.dequantize(m)
        g = w.reshape(32, 4, 64).astype(np.float64)
        s = m.s.astype(np.float64)[..., None]
        c = m.c.astype(np.float64)[..., None]
        lo = g.min(axis=2, keepdims=True)
        hi = g.max(axis=2, keepdims=True)
        bound = s / 2 + np.abs(lo - c) + np.abs(hi - lo - qmax * s) + 2 ** -20 * np.abs(g).max()
        err = np.abs(wh.reshape(32, 4, 64) - g)
        assert np.all(err <= bound)
        assert np.all(wh[3, :64] == float(np.float16(0.125)))


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(4)
    H, I = 256, 128
    for bits in (4, 8):
        wg, wu, wd = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in [(I, H), (I, H), (H, I)]]
        ex = quant.quantize_expert(wg, wu, wd, bits)
        rec = quant.pack_record(ex, bits)
        assert rec.shape[0] == quant.record_stride(H, I, bits)
        assert not rec[quant.record_bytes(H, I, bits):].any()
        back = quant.unpack_record(rec, H, I, bits)
        for a, b in zip(ex, back):
            assert np.array_equal(a.q, b.q)
            assert np.array_equal(a.s.view(np.uint16), b.s.view(np.uint16))
            assert np.array_equal(a.c.view(np.uint16), b.c.view(np.uint16))


def test_quantize_rejects_bad_input():
    with pytest.raises(ValueError):
        quant.quantize(np.full((1, 64), np.nan, dtype=np.float32), 4)
    with pytest.raises(ValueError):
        quant.quantize(np.zeros((1, 60), dtype=np.float32), 4)
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 0] = 1e6            # range/15 overflows fp16
    with pytest.raises(ValueError):
        quant.quantize(w, 4)


# ---------------------------------------------------------------- router

def test_router_logits_exact_rounding():
    rng = np.random.default_rng(5)
    H, E, T = 64, 12, 4
    xb = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    x = quant.f64_from_bf16_bits(xb)
    W = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    rho = rng.standard_normal(E).astype(np.float32)
    got = moe.router_logits(x, W, rho)
    for t in range(T):
        for e in range(E):
            exact = sum((Fraction(float(x[t, h])) * Fraction(float(W[h, e])) for h in range(H)), Fraction(float(rho[e])))
            assert got[t, e] == quant.fp32_round_exact(exact)


def test_router_logits_near_tie_branch():
    # a sum that sits exactly halfway between two fp32 neighbours: the float64 interval is ambiguous
    H = 3
    x = np.array([[1.0, 1.0, 1.0]])
    one_plus = np.float32(1.0)
    W = np.array([[1.0], [2.0 ** -24], [2.0 ** -60]], dtype=np.float32)
    got = moe.router_logits(x, W)
    # exact 1 + 2^-24 + 2^-60 is just above the tie 1 + 2^-24: rounds up to 1 + 2^-23
    assert got[0, 0] == np.float32(1.0 + 2 ** -23)
    W2 = np.array([[1.0], [2.0 ** -24], [0.0]], dtype=np.float32)
    assert moe.router_logits(x, W2)[0, 0] == one_plus           # exact tie -> even (1.0)


def test_topk_matches_brute_force_sort():
    rng = np.random.default_rng(6)
    for trial in range(200):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(1, E + 1))
        l = rng.integers(-3, 4, size=E).astype(np.float32) * np.float32(0.5)   # many exact ties
        want = [e for _, e in sorted((-float(l[e]), e) for e in range(E))][:k]
        assert list(moe.topk_order(l, k)) == want
    assert list(moe.topk_order(np.zeros(16, np.float32), 4)) == [0, 1, 2, 3]
    l = np.array([0.5, np.nan, 2.0, np.nan, 2.0], dtype=np.float32)
    assert list(moe.topk_order(l, 5)) == [2, 4, 0, 1, 3]


def test_route_weights_identities():
    rng = np.random.default_rng(7)
    l = rng.standard_normal(64).astype(np.float32)
    sel = moe.topk_order(l, 10)
    w = moe.route_weights(l, sel, 1)
    assert w.sum() == pytest.approx(1.0, abs=1e-15)
    full = scipy.special.softmax(l.astype(np.float64))
    assert np.allclose(w, full[sel] / full[sel].sum(), rtol=1e-14, atol=0)
    assert np.allclose(moe.route_weights(l, sel, 0), full[sel], rtol=1e-14, atol=0)
    all_sel = moe.topk_order(l, 64)
    assert np.allclose(moe.route_weights(l, all_sel, 1), full[all_sel], rtol=1e-14, atol=0)
    assert np.all(np.diff(l[sel].astype(np.float64)) <= 0)


# ---------------------------------------------------------------- experts

def _loops_ffn(x, gate, up, down):
    """Pure-Python triple loop of W_down (silu(W_gate x) * (W_up x))."""
    I, H = len(gate), len(gate[0])
    h = []
    for i in range(I):
        g = sum(gate[i][j] * x[j] for j in range(H))
        u = sum(up[i][j] * x[j] for j in range(H))
        h.append(g / (1.0 + math.exp(-g)) * u)
    return [sum(down[o][i] * h[i] for i in range(I)) for o in range(H)]


def _tiny_dense(rng, H=64, I=64, bits=4, scale=0.3):
    ws = [(rng.standard_normal(s) * scale).astype(np.float32) for s in [(I, H), (I, H), (H, I)]]
    ex = quant.quantize_expert(*ws, bits)
    return moe.dense_expert(ex)


def test_expert_ffn_matches_python_loops():
    rng = np.random.default_rng(8)
    d = _tiny_dense(rng)
    x = quant.f64_from_bf16_bits(synth.f32_to_bf16_bits(rng.standard_normal(64).astype(np.float32)))
    want = np.array(_loops_ffn(list(x), d.gate.tolist(), d.up.tolist(), d.down.tolist()))
    got = moe.expert_ffn(x, d)[0]
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def _layer_weights(rng, H, E, I, bits=4, zero_shared=False, gs=None):
    experts = [_tiny_dense(rng, H, I, bits) for _ in range(E)]
    shared = _tiny_dense(rng, H, I, bits)
    if zero_shared:
        z = np.zeros_like
        shared = moe.DenseExpert(z(shared.gate), z(shared.up), z(shared.down))
    w_r = (rng.standard_normal((H, E)) * 0.2).astype(np.float32)
    g_s = np.zeros(H, np.float32) if gs is None else gs
    return moe.LayerWeights(w_r, None, g_s, shared, lambda e: experts[e]), experts, shared


def test_one_hot_router_reproduces_single_expert():
    rng = np.random.default_rng(9)
    H, E, I = 64, 6, 64
    lw, experts, _ = _layer_weights(rng, H, E, I, zero_shared=True)
    x = quant.f64_from_bf16_bits(synth.f32_to_bf16_bits(rng.standard_normal((3, H)).astype(np.float32)))
    res = moe.layer_forward(x, lw, k=1)
    assert np.all(res.route.w == 1.0)
    for t in range(3):
        d = experts[int(res.route.idx[t, 0])]
        want = np.array(_loops_ffn(list(x[t]), d.gate.tolist(), d.up.tolist(), d.down.tolist()))
        assert np.max(np.abs(res.out[t] - want)) <= 1e-12 * np.max(np.abs(want))


def test_layer_matches_loops_two_experts_plus_shared():
    rng = np.random.default_rng(10)
    H, E, I = 64, 5, 64
    gs = (rng.standard_normal(H) * 0.1).astype(np.float32)
    lw, experts, shared = _layer_weights(rng, H, E, I, gs=gs)
    x = quant.f64_from_bf16_bits(synth.f32_to_bf16_bits(rng.standard_normal((2, H)).astype(np.float32)))
    res = moe.layer_forward(x, lw, k=2)
    for t in range(2):
        l = [float(v) for v in res.route.logits[t]]
        order = sorted(range(E), key=lambda e: (-l[e], e))[:2]
        z = [math.exp(l[e] - l[order[0]]) for e in order]
        ws = [v / sum(z) for v in z]
        gamma = 1.0 / (1.0 + math.exp(-sum(float(x[t, h]) * float(gs[h]) for h in range(H))))
        want = np.zeros(H)
        for e, w in zip(order, ws):
            d = experts[e]
            want += w * np.array(_loops_ffn(list(x[t]), d.gate.tolist(), d.up.tolist(), d.down.tolist()))
        want += gamma * np.array(_loops_ffn(list(x[t]), shared.gate.tolist(), shared.up.tolist(), shared.down.tolist()))
        assert list(res.route.idx[t]) == order
        assert np.max(np.abs(res.out[t] - want)) <= 1e-12 * np.max(np.abs(want))


def test_shared_gate_zero_is_one_half():
    rng = np.random.default_rng(11)
    H, E, I = 64, 4, 64
    lw, _, _ = _layer_weights(rng, H, E, I)
    x = rng.standard_normal((3, H))
    assert np.all(moe.layer_forward(x, lw, k=2).gamma == 0.5)


def test_zero_experts_give_zero_output_and_zero_stack_delta():
    H, E, I = 64, 4, 64
    zero = quant.quantize_expert(np.zeros((I, H), np.float32), np.zeros((I, H), np.float32),
                                 np.zeros((H, I), np.float32), 4)
    assert not zero.gate.s.view(np.uint16).any() and not zero.gate.c.view(np.uint16).any()
    d = moe.dense_expert(zero)
    rng = np.random.default_rng(12)
    lw = moe.LayerWeights((rng.standard_normal((H, E)) * 0.2).astype(np.float32), None,
                          np.ones(H, np.float32), d, lambda e: d)
    x = quant.f64_from_bf16_bits(synth.f32_to_bf16_bits(rng.standard_normal((4, H)).astype(np.float32)))
    assert np.all(moe.layer_forward(x, lw, k=2).out == 0)
    st = moe.stack_forward(x, [lw, lw, lw], k=2)
    assert np.all(st.delta == 0)


def test_stack_single_layer_equals_layer_and_recast():
    rng = np.random.default_rng(13)
    H, E, I = 64, 4, 64
    lw, _, _ = _layer_weights(rng, H, E, I)
    x = quant.f64_from_bf16_bits(synth.f32_to_bf16_bits(rng.standard_normal((3, H)).astype(np.float32)))
    st = moe.stack_forward(x, [lw], k=2)
    out = moe.layer_forward(x, lw, k=2).out
    assert np.array_equal(st.r_final, x + out)
    assert np.allclose(st.delta, out, rtol=0, atol=1e-14 * np.abs(out).max())
    # two layers: the second layer sees bf16(r1)
    st2 = moe.stack_forward(x, [lw, lw], k=2)
    r1 = x + moe.layer_forward(x, lw, k=2).out
    r2 = r1 + moe.layer_forward(quant.bf16_rne_from_f64(r1), lw, k=2).out
    assert np.allclose(st2.r_final, r2, rtol=0, atol=1e-15)


def test_batch_equals_single_tokens():
    rng = np.random.default_rng(14)
    H, E, I = 64, 8, 64
    lw, _, _ = _layer_weights(rng, H, E, I)
    x = quant.f64_from_bf16_bits(synth.f32_to_bf16_bits(rng.standard_normal((6, H)).astype(np.float32)))
    full = moe.layer_forward(x, lw, k=3).out
    for t in range(6):
        assert np.allclose(moe.layer_forward(x[t:t + 1], lw, k=3).out[0], full[t], rtol=1e-13, atol=1e-16)


def test_bucket_pairs_brute_force():
    rng = np.random.default_rng(15)
    T, k, E = 37, 3, 11
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    b = moe.bucket_pairs(idx, E)
    pairs = [(int(idx[t, j]), t * k + j) for t in range(T) for j in range(k)]
    pairs.sort()
    assert list(b.perm) == [p for _, p in pairs]
    for e in range(E):
        assert b.count[e] == sum(1 for ee, _ in pairs if ee == e)
        assert all(idx.reshape(-1)[p] == e for p in b.perm[b.offset[e]:b.offset[e + 1]])
    assert b.offset[-1] == T * k


# ------------------------------------------------------------------- pool

def test_pool_sim_matches_naive_twin():
    rng = np.random.default_rng(16)
    for trial in range(12):
        E = int(rng.integers(4, 24))
        k = int(rng.integers(1, min(E, 5) + 1))
        L = int(rng.integers(1, 4))
        slots = int(rng.integers(k, E * L + 2))
        a, b = pool.PoolSim(slots, 100), pool.PoolSimNaive(slots, 100)
        p = rng.random(E) ** 3
        p /= p.sum()
        for t in range(60):
            for l in range(L):
                sel = rng.choice(E, size=k, replace=False, p=p)
                a.step(l * E + sel)
                b.step(l * E + sel)
        assert a.trace_hit == b.trace_hit
        assert a.trace_victim == b.trace_victim
        assert a.trace_slot == b.trace_slot


def test_pool_capacity_covers_everything():
    rng = np.random.default_rng(17)
    sim = pool.PoolSim(1000, 10)
    seen = set()
    for t in range(50):
        gids = rng.choice(200, size=5, replace=False)
        seen.update(int(g) for g in gids)
        sim.step(gids)
    st = sim.stats()
    assert st.misses == len(seen) and st.evictions == 0
    assert st.hits + st.misses == st.accesses == 250


def test_pool_cold_token_480_misses_810_mib():
    g = _golden("pages_figures.json")
    rec = quant.record_bytes(2048, 512, 4)
    slots = (2 * 2 ** 30) // quant.record_stride(2048, 512, 4)
    assert slots == 1213
    sim = pool.PoolSim(slots, rec)
    rng = np.random.default_rng(18)
    for l in range(48):
        sim.step(l * 512 + rng.choice(512, size=10, replace=False))
    st = sim.stats()
    assert st.misses == g["zero_hit_fetch"]["experts_per_token"] and st.hits == 0
    assert st.requested_bytes / 2 ** 20 == pytest.approx(g["zero_hit_fetch"]["logical_mib"], abs=0.5)


def test_pool_step_never_evicts_its_own_experts():
    sim = pool.PoolSim(3, 1)
    sim.step([0, 1, 2])
    sim.step([0, 3, 4])       # 3 evicts one of {1,2}; 4 must not evict 3 or 0
    assert 0 in sim.where and 3 in sim.where and 4 in sim.where


def test_zipf_hit_rate_is_plausible():
    """Routing-only proxy of the pooled 48-layer workload lands in the pages' 43-70% band.

    The proxy routes each token's own activations at every layer (the residual
    update is small next to x), with the real router matrices and Zipf bias.
    """
    g = _golden("pages_figures.json")["hit_rate"]
    cfg = synth.get_config("pool80b")
    T = 160
    x = quant.f64_from_bf16_bits(synth.tokens(cfg.seed, T, cfg.hidden))
    idx = np.empty((T, cfg.n_layers, cfg.top_k), dtype=np.int64)
    for l in range(cfg.n_layers):
        W = synth.router_weight(cfg.seed, l, cfg.hidden, cfg.n_experts).astype(np.float64)
        rho = synth.router_bias(cfg, l).astype(np.float64)
        lg = x @ W + rho
        idx[:, l] = np.argsort(-lg, axis=1, kind="stable")[:, :cfg.top_k]
    sim = pool.PoolSim(cfg.pool_budget // quant.record_stride(cfg.hidden, cfg.inter, cfg.bits), 1)
    warm = 32
    for t in range(T):
        if t == warm:
            h0, a0 = sim.hits, sim.accesses
        for l in range(cfg.n_layers):
            sim.step(l * cfg.n_experts + idx[t, l])
    rate = (sim.hits - h0) / (sim.accesses - a0)
    assert g["low"] <= rate <= g["high"], rate
