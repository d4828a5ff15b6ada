"""Host-side checks of libmoe through its C ABI (no GPU needed).

The library loads and exports what include/moe.h declares; the C++ packer is
bit-exact with the oracle's independent packer; the C++ pool policy replays a
trace exactly like the oracle's simulator; invalid arguments fail with the
documented status before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import routed_expert_int4_router_amd as moe
import synth
from oracle import pool as opool
from oracle import quant

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert declared == set(moe.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def _cfg(name, **kw):
    return moe.config_of(synth.get_config(name, **kw))


@pytest.mark.parametrize("name", ["tiny", "decode80b", "stack35b_int8", "stack35b_int4", "pool80b"])
def test_record_geometry_matches_oracle(name):
    c = synth.get_config(name)
    assert moe.expert_bytes(_cfg(name)) == quant.record_bytes(c.hidden, c.inter, c.bits)
    assert moe.expert_stride(_cfg(name)) == quant.record_stride(c.hidden, c.inter, c.bits)


def test_blob_offset_64bit():
    stride = quant.record_stride(2048, 512, 4)
    for gid in [0, 7, 2427, 2428, 24_575]:
        assert moe.blob_offset(123, gid, stride) == quant.blob_offset(123, gid, stride)
    assert moe.blob_offset(0, 24_575, stride) > 2 ** 32


def _oracle_record(wg, wu, wd, bits):
    return quant.pack_record(quant.quantize_expert(wg, wu, wd, bits), bits)


@pytest.mark.parametrize("bits", [4, 8])
def test_packer_bit_exact_random_tiny(bits):
    cfg = _cfg("tiny", bits=bits)
    rng = np.random.default_rng(20 + bits)
    n, H, I = 5, cfg.hidden, cfg.inter
    wg = (rng.standard_normal((n, I, H)) * 0.02).astype(np.float32)
    wu = (rng.standard_normal((n, I, H)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((n, H, I)) * 1.5).astype(np.float32)
    # edge groups: degenerate, exact ties, -0 minimum, tiny range (fp16 subnormal scale)
    wg[0, 0, :64] = 0.375
    wg[0, 1, :64] = 0.0
    wg[0, 1, 5] = 1.875
    wg[0, 1, 6] = 0.0625
    wg[0, 1, 7] = 0.1875
    wg[0, 2, :64] = np.float32(-0.0)
    wg[0, 2, 3] = 0.5
    wu[1, 0, :64] = (rng.standard_normal(64) * 1e-6).astype(np.float32)
    wu[1, 1, :64] = (rng.standard_normal(64) * 1e-9).astype(np.float32)
    got = moe.pack(cfg, wg, wu, wd)
    stride = moe.expert_stride(cfg)
    for e in range(n):
        want = _oracle_record(wg[e], wu[e], wd[e], bits)
        assert np.array_equal(got[e * stride:(e + 1) * stride], want), f"expert {e}"


@pytest.mark.parametrize("name", ["decode80b", "stack35b_int8"])
def test_packer_bit_exact_full_size(name):
    c = synth.get_config(name)
    cfg = moe.config_of(c)
    for layer, e in [(0, 0), (0, 311)]:
        wg, wu, wd = synth.expert_weights(c.seed, layer, e, c.hidden, c.inter)
        got = moe.pack(cfg, wg, wu, wd)
        assert np.array_equal(got, _oracle_record(wg, wu, wd, c.bits))


def test_unpack_round_trip_matches_oracle_codes():
    c = synth.get_config("tiny")
    cfg = moe.config_of(c)
    wg, wu, wd = synth.expert_weights(0, 0, 3, c.hidden, c.inter)
    rec = moe.pack(cfg, wg, wu, wd)
    q, sc = moe.unpack(cfg, rec)
    ex = quant.unpack_record(rec, c.hidden, c.inter, c.bits)
    n = c.hidden * c.inter
    assert np.array_equal(q[:n], ex.gate.q.reshape(-1))
    assert np.array_equal(q[n:2 * n], ex.up.q.reshape(-1))
    assert np.array_equal(q[2 * n:], ex.down.q.reshape(-1))
    g = n // 64
    assert np.array_equal(sc[0:2 * g:2], ex.gate.s.reshape(-1).view(np.uint16))
    assert np.array_equal(sc[1:2 * g:2], ex.gate.c.reshape(-1).view(np.uint16))


def test_pack_hand_examples():
    cfg = _cfg("tiny")
    H, I = cfg.hidden, cfg.inter
    wg = np.zeros((I, H), np.float32)
    wg[0, :64] = -1 + 0.25 * (np.arange(64) % 16)
    rec = moe.pack(cfg, wg, np.zeros((I, H), np.float32), np.zeros((H, I), np.float32))
    assert rec[:32].tobytes().hex() == "1032547698badcfe" * 4
    lay = quant.record_layout(H, I, 4)
    assert rec[lay.gate_sc:lay.gate_sc + 4].tobytes().hex() == "0034" + "00bc"


def test_pack_rejects_bad_input():
    cfg = _cfg("tiny")
    H, I = cfg.hidden, cfg.inter
    z = np.zeros((I, H), np.float32)
    zd = np.zeros((H, I), np.float32)
    bad = z.copy()
    bad[3, 7] = np.nan
    with pytest.raises(moe.MoeError) as ei:
        moe.pack(cfg, bad, z, zd)
    assert ei.value.status == moe.MOE_EINVAL
    big = z.copy()
    big[0, 0] = 1e6
    with pytest.raises(moe.MoeError):
        moe.pack(cfg, big, z, zd)
    with pytest.raises(moe.MoeError):
        moe.pack(cfg, z, z, zd, out=np.zeros(10, np.uint8))
    bad_cfg = moe.make_config(256, 16, 2, 128, bits=3)
    with pytest.raises(moe.MoeError):
        moe.pack(bad_cfg, z, z, zd)


@pytest.mark.parametrize("kw,msg", [
    (dict(bits=3), "bits"), (dict(group=32), "group"), (dict(hidden=300), "hidden"),
    (dict(top_k=17, n_experts=32), "top_k"), (dict(top_k=5, n_experts=4), "top_k"),
    (dict(inter=96), "inter"), (dict(shared_inter=256), "shared_inter"), (dict(n_layers=0), "n_layers"),
    (dict(norm_topk=2), "norm_topk"),
])
def test_model_create_validates_before_hip(kw, msg):
    base = dict(hidden=256, n_experts=16, top_k=2, inter=128, shared_inter=128, bits=4, group=64, n_layers=1,
                norm_topk=1)
    base.update(kw)
    cfg = moe.Config(*[base[n] for n, _ in moe.Config._fields_])
    h = ctypes.c_void_p()
    st = moe.lib().moe_model_create(ctypes.byref(cfg), 0, ctypes.byref(h))
    assert st == moe.MOE_EINVAL
    assert msg in moe.last_error()
    assert moe.expert_bytes(cfg) == 0 or msg in ("top_k", "n_layers", "norm_topk")


def test_null_and_dead_handles():
    L = moe.lib()
    assert L.moe_layer_forward(None, 0, None, 1, None, None) == moe.MOE_EINVAL
    assert L.moe_stack_decode(None, None, None, 1, None, None) == moe.MOE_EINVAL
    fake = ctypes.c_void_p(0x1234)
    assert L.moe_layer_decode(fake, 0, None, 1, None, None) == moe.MOE_ESTATE
    assert L.moe_pool_reset(fake) == moe.MOE_ESTATE
    h = ctypes.c_void_p()
    assert L.moe_pool_create(None, 1 << 30, ctypes.byref(h)) == moe.MOE_EINVAL
    L.moe_model_destroy(None)
    L.moe_pool_destroy(None)
    L.moe_model_destroy(fake)       # not a live handle: ignored


def test_pool_policy_matches_oracle_simulator():
    rng = np.random.default_rng(30)
    for trial in range(8):
        E = int(rng.integers(8, 64))
        k = int(rng.integers(1, 9))
        L = int(rng.integers(1, 4))
        slots = int(rng.integers(k, E * L))
        p = rng.random(E) ** 4
        p /= p.sum()
        steps = []
        for t in range(80):
            for l in range(L):
                steps.append(l * E + rng.choice(E, size=k, replace=False, p=p))
        gids = np.array(steps, dtype=np.int64)
        hit, victim = moe.pool_simulate(slots, gids)
        sim = opool.PoolSim(slots, 1)
        for s in gids:
            sim.step(s)
        assert list(hit) == sim.trace_hit
        assert list(victim) == sim.trace_victim


def test_pool_simulate_rejects_bad_args():
    with pytest.raises(moe.MoeError):
        moe.pool_simulate(2, np.zeros((1, 3), np.int64) + np.arange(3))
    with pytest.raises(moe.MoeError):
        moe.pool_simulate(4, np.array([[1, 1]], np.int64))
