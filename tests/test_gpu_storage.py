"""The pool's storage-backed miss path: routed experts read from a blob file
(one pread of the record at gid * stride into pinned staging, then the
host->device copy into the slot), with the page cache bypassed (O_DIRECT)
where the filesystem allows it, or buffered. Outputs must equal the
all-resident stack's bit for bit and the pool's trace the oracle simulator's."""
import os

import numpy as np
import pytest

import routed_expert_int4_router_amd as moe
from routed_expert_int4_router_amd import loader
import synth
from oracle import pool as opool

import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def stack3(tmp_path_factory):
    """A 3-layer 80B-shaped stack: its blob file (2.7 GB) and its resident twin's outputs."""
    torch = gh.torch_cuda()
    cfg = synth.get_config("pool80b", n_layers=3)
    path = str(tmp_path_factory.mktemp("blob") / "experts.qblob")
    n_tok = 12
    xb = synth.tokens(cfg.seed, n_tok, cfg.hidden)
    res = gh.build(cfg)
    x = gh.dev_bf16(xb)
    out = gh.dev_f32((n_tok, cfg.hidden))
    res.stack_decode(x, out)
    torch.cuda.synchronize()
    idx, _ = res.debug_routing()
    ref = out.cpu().numpy()
    res.close()
    gh.log(f"writing the blob file {path}")
    m = loader.load_model(cfg, synth.SynthWeights(cfg), storage=moe.STORE_FILE, blob_path=path)
    m.close()
    assert os.path.getsize(path) == cfg.n_layers * cfg.n_experts * moe.expert_stride(cfg)
    yield cfg, path, xb, ref, idx
    os.remove(path)


@pytest.mark.parametrize("slots,direct", [(10, True), (37, True), (37, False)])
def test_file_pool_bit_identical_to_resident_and_trace_matches_oracle(stack3, slots, direct):
    cfg, path, xb, ref, idx_res = stack3
    torch = gh.torch_cuda()
    model = moe.Model(cfg, moe.STORE_FILE)
    loader.fill_dense(model, synth.SynthWeights(cfg))
    model.open_blob(path, 0, direct)
    pool = moe.Pool(model, slots * moe.expert_stride(cfg))
    n = xb.shape[0]
    x = gh.dev_bf16(xb)
    out = gh.dev_f32((n, cfg.hidden))
    model.stack_decode(x, out, pool=pool)
    torch.cuda.synchronize()
    idx, _ = model.debug_routing()
    assert np.array_equal(idx, idx_res)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), "file pool != resident"
    sim = opool.replay(slots, moe.expert_bytes(cfg), idx, cfg.n_experts, cfg.n_layers)
    hit, victim = pool.trace()
    assert np.array_equal(hit, np.asarray(sim.trace_hit, np.uint8))
    assert np.array_equal(victim, np.asarray(sim.trace_victim, np.int64))
    st = pool.stats()
    assert st["misses"] == sim.misses and st["hits"] == sim.hits
    assert st["storage_reads"] == sim.misses
    per_read = moe.expert_stride(cfg) if st["direct_io"] else moe.expert_bytes(cfg)
    assert st["storage_bytes"] == sim.misses * per_read
    if not direct:
        assert st["direct_io"] == 0
    print(f"slots {slots}, direct asked {direct}: O_DIRECT in effect {st['direct_io']}, "
          f"{st['storage_reads']} reads, {st['hits']} hits of {st['accesses']}")
    pool.close()
    model.close()


def test_open_blob_errors(stack3, tmp_path):
    cfg, path, *_ = stack3
    model = moe.Model(cfg, moe.STORE_FILE)
    with pytest.raises(moe.MoeError) as e:
        model.open_blob(str(tmp_path / "missing.qblob"))
    assert e.value.status == moe.MOE_EINVAL
    short = tmp_path / "short.qblob"
    short.write_bytes(b"\0" * 4096)
    with pytest.raises(moe.MoeError) as e:
        model.open_blob(str(short))
    assert e.value.status == moe.MOE_EINVAL and "holds 4096 bytes" in str(e.value)
    with pytest.raises(moe.MoeError) as e:
        moe.Pool(model, 64 * moe.expert_stride(cfg))
    assert e.value.status == moe.MOE_ESTATE      # no blob opened yet
    model.close()
    dev = moe.Model(cfg, moe.STORE_DEVICE)
    with pytest.raises(moe.MoeError) as e:
        dev.open_blob(path)
    assert e.value.status == moe.MOE_ESTATE
    dev.close()
