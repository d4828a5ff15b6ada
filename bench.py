#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Workloads (synthetic, seeded, weights ~N(0, 0.02) packed to int4/int8 g64):
  decode80b      80B-shaped single layer (H 2048, 512 experts, top-10, I 512,
                 int4), batch-1 decode of 1024 tokens one after another; the
                 default, and the configuration the headline metric is quoted on
  stack35b_int8  35B-shaped 40-layer stack (256 experts, top-8), int8, 512 tokens
  stack35b_int4  the same stack in int4
  prefill80b     80B-shaped layer, one 2048-token batch (grouped GEMM path)
  pool80b        80B-shaped 48-layer stack, experts in pinned host memory,
                 2 GiB HBM pool, 1024 tokens (host-link bound)
  resident80b    the same 48-layer stack with every expert in HBM
  gdn80b         the Gated DeltaNet decode step beside the MoE: 36 layers of
                 16 key / 32 value heads of 128, 256 tokens one at a time
  attn80b        the gated GQA attention decode step beside the MoE: 12 layers
                 of 16 query / 2 KV heads of 256 over an fp16 KV cache holding
                 8192 positions, 64 tokens one at a time

A step is one pass of the workload's tokens through the whole path (router,
top-k, expert GEMV/GEMM, combine, stack glue, pool). W untimed steps, then K
timed steps bracketed by device synchronisation; value = tokens / second.
A second, instrumented pass of the same steps hands every kernel launch a
hipEvent pair that the launch fills with the kernel's own begin/end
timestamps; the dominant kernel's average duration and its algorithmic bytes
(or flops) give the roofline entry. The CPU oracle is timed
on a bounded sample of the same workload, single-threaded.

The default run (decode80b) also measures the batched path on prefill80b (a
2048-token batch of the same layer shape) and reports its grouped GEMMs
against the fp16 matrix-core peak under extra.prefill, so one run carries
both halves of the headline metric.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

# the oracle leg runs single-threaded; BLAS reads these at import time
for _v in ("OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "OMP_NUM_THREADS"):
    os.environ[_v] = "1"

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 (and bf16) MFMA, TFLOP/s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------- algorithmic bytes ---

def decode_kernel_bytes(cfg, stack: bool) -> dict:
    """Bytes of the method each decode kernel moves per launch (one token, one
    layer), and the scratch it moves on top: {kernel: (algorithmic, scratch)}.

    Algorithmic bytes are what the step itself must read or write: the router
    rows, the k + 1 expert records, x, the logits, out (and for a stack the
    residual and the bf16 recast). Scratch is the fused path's partial rows,
    fp32 [(k + 1) * I / 32][H], written by the expert kernel and read back by
    reduce: an artefact of splitting the down projection over blocks, so it is
    reported beside the roofline, never in it.
    """
    H, I, E, k, b = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.bits
    codes = I * H * b // 8          # one matrix
    sc = I * H // 64 * 4
    rec = 3 * (codes + sc)
    logits = (E + 1) * 4
    parts = (k + 1) * (I // 32) * H * 4
    glue = (H * 4 + H * 2) if stack else 0     # residual read + bf16 recast write
    return {
        "router": ((E + 1) * H * 4 + E * 4 + H * 2 + logits, 0),
        "expert": ((k + 1) * rec + H * 2 + logits, parts),
        "reduce": (H * 4 + glue, parts),
        "gateup": ((k + 1) * 2 * (codes + sc) + H * 2 + logits, (k + 1) * I * 4),
        "down": ((k + 1) * (codes + sc) + (k + 1) * 4 + H * 4 + glue, (k + 1) * I * 4),
    }


def step_bytes_per_token(cfg) -> int:
    """Whole-step algorithmic bytes per token-layer: W_r + g_s + (k+1) records + x + out."""
    H, I, E, k, b = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.bits
    rec = 3 * H * I * b // 8 + 3 * (H * I // 64) * 4
    return H * E * 4 + (k + 1) * rec + H * 4 + H * 2 + H * 4


def prefill_flops(cfg, n_tok: int) -> dict:
    H, I, k = cfg.hidden, cfg.inter, cfg.top_k
    pairs = n_tok * k + n_tok          # routed pairs + shared expert rows
    return {"prefill_gateup": 2 * pairs * H * 2 * I, "prefill_down": 2 * pairs * I * H}


# ----------------------------------------------------------------- oracle ---

def cpu_baseline(cfg, xb, budget_s: float) -> dict:
    """The oracle as it stands, single thread, on the first tokens of the workload."""
    from oracle import moe as omoe
    from oracle import quant
    from oracle.model import OracleModel
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    om = OracleModel(cfg)
    t0 = time.perf_counter()
    done = 0
    if cfg.n_layers == 1:
        lw = om.layer(0)
        while done < xb.shape[0] and time.perf_counter() - t0 < budget_s:
            x = quant.f64_from_bf16_bits(xb[done:done + 1])
            omoe.layer_forward(x, lw, cfg.top_k, cfg.norm_topk)
            done += 1
        unit_tokens = done
        sample = f"first {done} of {xb.shape[0]} tokens, one layer, experts dequantised from oracle-packed records"
    else:
        layers = om.layers()
        while done < xb.shape[0] and time.perf_counter() - t0 < budget_s:
            x = quant.f64_from_bf16_bits(xb[done:done + 1])
            omoe.stack_forward(x, layers, cfg.top_k, cfg.norm_topk)
            done += 1
        unit_tokens = done
        sample = f"first {done} of {xb.shape[0]} tokens through all {cfg.n_layers} layers"
    dt = time.perf_counter() - t0
    return {"value": unit_tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle", "sample": sample,
            "seconds": round(dt, 2), "cpu_model": cpu_model(), "host_cores": os.cpu_count()}


def cpu_model() -> str:
    """The host CPU's model name (lscpu's, from /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ traffic ---

def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when missing or taken on a different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    # the hash covers every source the kernel is built from, in the listed order
    h = hashlib.sha256()
    for name in kv.get("source", "").split():
        src = os.path.join(ROOT, "routed_expert_int4_router_amd", "csrc", name)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    if not kv.get("source") or kv.get("source_sha256_16") != h.hexdigest()[:16]:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, nbytes: int) -> None:
    """One plain device-to-device copy of nbytes: the known-size reference that
    scales rocprofv3's FETCH_SIZE / WRITE_SIZE to bytes."""
    if nbytes <= 0:
        return
    n = nbytes // 4
    src_t = torch.ones(n, dtype=torch.float32, device="cuda")
    dst_t = torch.empty_like(src_t)
    torch.cuda.synchronize()
    dst_t.copy_(src_t)
    torch.cuda.synchronize()
    log(f"copy calibration: {4 * n} bytes")
    del src_t, dst_t


def link_probe(torch, chunk: int, n: int = 512) -> float:
    """Host->device rate of pinned hipMemcpyAsync copies of one expert record
    (the pool's miss unit), back to back on one stream after a warm-up: the
    link's practical peak for that transfer size."""
    slots = 16
    src = torch.empty(chunk * slots, dtype=torch.uint8).pin_memory()
    dst = torch.empty(chunk * slots, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()

    def burst(count):
        with torch.cuda.stream(s):
            for i in range(count):
                j = (i % slots) * chunk
                dst[j:j + chunk].copy_(src[j:j + chunk], non_blocking=True)
        s.synchronize()

    burst(2 * slots)
    t0 = time.perf_counter()
    burst(n)
    dt = time.perf_counter() - t0
    return round(n * chunk / dt / 1e9, 2)


# -------------------------------------------------------------------- main ---

def kernel_pass(model, step, n_prof, torch) -> dict:
    """Per-kernel launch count and total ms over n_prof instrumented steps."""
    model.profile_enable(True)
    for _ in range(n_prof):
        step()
    torch.cuda.synchronize()
    prof = model.profile_read()
    model.profile_enable(False)
    return {k: v for k, v in prof.items() if v[0] > 0}


def kernel_table(prof: dict) -> dict:
    total = max(1e-9, sum(p[1] for p in prof.values()))
    return {k: {"launches": v[0], "avg_us": round(1000.0 * v[1] / v[0], 3), "share": round(v[1] / total, 3)}
            for k, v in prof.items()}


def gemm_roofline(cfg, T, prof) -> tuple:
    """Roofline of the grouped GEMMs (fp16 matrix cores) from the kernel pass:
    the dominant one, and both, each as algorithmic flops / average duration."""
    fl = prefill_flops(cfg, T)
    gemms = {k: v for k, v in prof.items() if k in fl}
    if not gemms:
        return None, {}
    per = {}
    for k, v in gemms.items():
        avg_s = v[1] / v[0] / 1000.0
        ach = fl[k] / avg_s / 1e12
        per[k] = {"flops_per_launch": fl[k], "avg_us": round(avg_s * 1e6, 3), "achieved_TFLOPs": round(ach, 1),
                  "frac": round(ach / FP16_MFMA_PEAK_TFLOPS, 4)}
    both_s = sum(gemms[k][1] / gemms[k][0] / 1000.0 for k in gemms)
    both = sum(fl[k] for k in gemms) / both_s / 1e12
    per["both"] = {"avg_us": round(both_s * 1e6, 3), "achieved_TFLOPs": round(both, 1),
                   "frac": round(both / FP16_MFMA_PEAK_TFLOPS, 4)}
    dom = max(gemms, key=lambda k: gemms[k][1])
    ach = per[dom]["achieved_TFLOPs"]
    roof = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": per[dom]["frac"], "traffic": measured_traffic(dom, cfg.name),
            "flops_per_launch": fl[dom], "avg_launch_us": per[dom]["avg_us"]}
    return roof, per


def measure(cfg, args, torch, moe, loader, synth, steps: int, warmup: int, kernels: bool) -> dict:
    """Load the workload, run warmup + timed steps, then the instrumented pass."""
    T = cfg.n_tokens
    log(f"workload {cfg.name}: {cfg.description}")
    t0 = time.perf_counter()

    def prog(layer):
        if cfg.n_layers >= 8 and layer % 8 == 7:
            log(f"filled {layer + 1} of {cfg.n_layers} layers ({time.perf_counter() - t0:.0f}s)")

    storage = moe.STORE_HOST if cfg.pool_budget else moe.STORE_DEVICE
    blob_path = None
    if cfg.pool_budget and args.storage == "file":
        storage = moe.STORE_FILE
        blob_path = os.path.join(args.blob_dir, f"{cfg.name}.qblob")
        size = cfg.n_layers * cfg.n_experts * moe.expert_stride(cfg)
        if args.keep_blob and os.path.exists(blob_path) and os.path.getsize(blob_path) == size:
            log(f"reusing the blob file {blob_path}")
            model = moe.Model(cfg, moe.STORE_FILE)
            loader.fill_dense(model, synth.SynthWeights(cfg))
            with open(blob_path, "rb") as f:   # cold start, as after writing it
                os.posix_fadvise(f.fileno(), 0, 0, os.POSIX_FADV_DONTNEED)
            model.open_blob(blob_path, 0, not args.buffered)
        else:
            log(f"writing the blob file {blob_path} ({size} bytes)")
            model = loader.load_model(cfg, synth.SynthWeights(cfg), storage=storage, blob_path=blob_path,
                                      direct=not args.buffered, progress=prog)
    else:
        model = loader.load_model(cfg, synth.SynthWeights(cfg), storage=storage, progress=prog)
    log(f"model loaded in {time.perf_counter() - t0:.1f}s")
    pool = moe.Pool(model, cfg.pool_budget) if cfg.pool_budget else None
    xb = synth.tokens(cfg.seed, T, cfg.hidden)
    x = torch.from_numpy(xb.view(np.int16)).cuda()
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    prefill = cfg.name.startswith("prefill")

    if prefill:
        def step():
            model.layer_forward(0, x, out, stream=stream)
    elif cfg.n_layers == 1:
        def step():
            model.layer_decode(0, x, out, stream=stream)
    else:
        def step():
            if pool is not None:
                pool.reset()
            model.stack_decode(x, out, pool=pool, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({warmup} steps)")
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"timed {steps} steps in {elapsed:.3f}s")
    res = {"tok_s": steps * T / elapsed, "ms_step": 1000.0 * elapsed / steps, "xb": xb, "extra": {},
           "roofline": None}
    extra = res["extra"]
    if pool is not None:
        st = pool.stats()  # counts of the last timed step (the pool is reset at every step)
        extra["pool"] = {**st, "hit_rate": round(st["hits"] / max(1, st["accesses"]), 4),
                         "h2d_GBps": round(st["h2d_bytes"] / (elapsed / steps) / 1e9, 2),
                         "storage_GBps": round(st["storage_bytes"] / (elapsed / steps) / 1e9, 2),
                         "link_probe_GBps": link_probe(torch, moe.expert_bytes(cfg))}
    copy_calibration(torch, args.copy_calibration)
    if kernels:
        n_prof = max(1, min(steps, 5 if cfg.n_layers == 1 else 1))
        prof = kernel_pass(model, step, n_prof, torch)
        extra["kernels"] = kernel_table(prof)
        log(f"kernel pass: {extra['kernels']}")
        if "expert_miss" in prof:
            # a pooled layer runs its hit and shared experts (one launch, during
            # the miss copies) and its missed experts (a second launch): the
            # expert kernel's per-layer figure is the two together
            prof = dict(prof)
            n, ms = prof.pop("expert")
            prof["expert"] = (n, ms + prof.pop("expert_miss")[1])
        if prefill:
            res["roofline"], extra["gemms"] = gemm_roofline(cfg, T, prof)
        else:
            by = decode_kernel_bytes(cfg, stack=cfg.n_layers > 1)
            cands = {k: v for k, v in prof.items() if k in by}
            dom = max(cands, key=lambda k: cands[k][1])
            avg_s = cands[dom][1] / cands[dom][0] / 1000.0
            alg, scratch = by[dom]
            ach = alg / avg_s / 1e9
            res["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                               "traffic": measured_traffic(dom, cfg.name),
                               "bytes_per_launch": alg, "scratch_bytes_per_launch": scratch,
                               "avg_launch_us": round(avg_s * 1e6, 3)}
            per_tok = step_bytes_per_token(cfg) * cfg.n_layers
            extra["whole_step"] = {"bytes_per_token": per_tok,
                                   "GBps": round(per_tok * res["tok_s"] / 1e9, 1),
                                   "frac_of_hbm_peak": round(per_tok * res["tok_s"] / 1e9 / HBM_PEAK_GBS, 4)}
    if pool is not None:
        pool.close()
    model.close()
    if blob_path and not args.keep_blob:
        os.remove(blob_path)
    return res


def gdn_step_bytes(cfg) -> int:
    """Algorithmic bytes of one DeltaNet step kernel (one token, one layer):
    the fp32 state read and written, the conv history read and written, the
    conv weights, the bf16 inputs (qkv, z, a, b), the fp32 output and the
    per-head parameters."""
    C, Z = cfg.channels, cfg.n_v * cfg.d_v
    state = cfg.n_v * cfg.d_k * cfg.d_v * 4
    return 2 * state + 2 * C * 3 * 4 + C * 4 * 4 + C * 2 + Z * 2 + 2 * cfg.n_v * 2 + Z * 4 + 2 * cfg.n_v * 4 + cfg.d_v * 4


def measure_gdn(cfg, args, torch, moe, synth, steps: int, warmup: int, kernels: bool) -> dict:
    """Gated DeltaNet decode: each step takes the workload's tokens one after
    another through all its layers (token-major), the state carried on."""
    log(f"workload {cfg.name}: {cfg.description}")
    net = moe.GatedDeltaNet(cfg.n_layers, cfg.n_k, cfg.n_v, cfg.d_k, cfg.d_v)
    for l in range(cfg.n_layers):
        net.set_layer(l, *synth.gdn_params(cfg, l))
    T, L = cfg.n_tokens, cfg.n_layers
    per = [synth.gdn_inputs(cfg, l, T) for l in range(L)]
    dev = [torch.from_numpy(np.ascontiguousarray(np.stack([per[l][i] for l in range(L)], axis=1)).view(np.int16))
           .cuda() for i in range(4)]
    out = torch.empty((T, L, cfg.n_v * cfg.d_v), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        net.decode(0, L, dev[0], dev[1], dev[2], dev[3], out, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"timed {steps} steps in {elapsed:.3f}s")
    copy_calibration(torch, args.copy_calibration)
    res = {"tok_s": steps * T / elapsed, "ms_step": 1000.0 * elapsed / steps, "extra": {}, "roofline": None,
           "inputs": per}
    per_launch = gdn_step_bytes(cfg)
    res["extra"]["whole_step"] = {"bytes_per_token": per_launch * L,
                                  "GBps": round(per_launch * L * res["tok_s"] / 1e9, 1),
                                  "frac_of_hbm_peak": round(per_launch * L * res["tok_s"] / 1e9 / HBM_PEAK_GBS, 4)}
    if kernels:
        net.profile(True)
        step()
        torch.cuda.synchronize()
        ms, n = net.profile(False)
        avg_s = ms / n / 1000.0
        ach = per_launch / avg_s / 1e9
        res["extra"]["kernels"] = {"gdn_step": {"launches": n, "avg_us": round(avg_s * 1e6, 3), "share": 1.0}}
        res["roofline"] = {"bound": "hbm", "kernel": "gdn_step", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic("gdn_step", cfg.name),
                           "bytes_per_launch": per_launch, "avg_launch_us": round(avg_s * 1e6, 3)}
        log(f"kernel pass: {res['extra']['kernels']}")
    net.close()
    return res


def cpu_baseline_gdn(cfg, per, budget_s: float) -> dict:
    """The oracle as it stands, single thread: the first tokens through all layers."""
    from oracle import deltanet as ognd
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    import synth
    sh = ognd.Shape(cfg.n_k, cfg.n_v, cfg.d_k, cfg.d_v)
    params = [ognd.Params(*synth.gdn_params(cfg, l)) for l in range(cfg.n_layers)]
    states = [ognd.zero_state(sh) for _ in range(cfg.n_layers)]
    f = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)  # noqa: E731
    t0 = time.perf_counter()
    done = 0
    while done < cfg.n_tokens and time.perf_counter() - t0 < budget_s:
        for l in range(cfg.n_layers):
            qkv, z, a, b = per[l]
            _, states[l] = ognd.layer_step(sh, params[l], states[l], f(qkv[done]), f(z[done]), f(a[done]), f(b[done]))
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {cfg.n_tokens} tokens through all {cfg.n_layers} layers",
            "seconds": round(dt, 2), "cpu_model": cpu_model(), "host_cores": os.cpu_count()}


def attn_split_bytes(cfg) -> tuple:
    """(algorithmic, scratch) bytes of one attention partials kernel, averaged
    over the workload's tokens: the cached K and V read (fp16, positions 0..p),
    the new K/V row written, the bf16 q of every head and the k, v inputs, the
    norm weights; scratch = the softmax partials written for the merge (one
    set per 128 positions)."""
    kv_row = 2 * cfg.n_kv * cfg.d * 2
    avg_pos = cfg.context + (cfg.n_tokens - 1) / 2.0 + 1.0
    inputs = cfg.n_q * cfg.d * 2 + 2 * cfg.n_kv * cfg.d * 2 + 2 * cfg.d * 4
    algo = avg_pos * kv_row + kv_row + inputs
    blocks = np.mean([(cfg.context + t) // 128 + 1 for t in range(cfg.n_tokens)])
    scratch = blocks * cfg.n_q * (cfg.d + 2) * 4
    return algo, scratch


def measure_attn(cfg, args, torch, moe, synth, steps: int, warmup: int, kernels: bool) -> dict:
    """Gated attention decode: each step takes the workload's tokens one after
    another through all its layers (token-major) at positions context,
    context + 1, ...; every step rewrites the same rows, so steps are equal."""
    log(f"workload {cfg.name}: {cfg.description}")
    T, L = cfg.n_tokens, cfg.n_layers
    net = moe.GatedAttention(L, cfg.n_q, cfg.n_kv, cfg.d, cfg.rot, cfg.context + T)
    for l in range(L):
        net.set_layer(l, *synth.attn_params(cfg, l))
        net.write_cache(l, 0, *synth.attn_cache(cfg, l, cfg.context))
    per = [synth.attn_inputs(cfg, l, T) for l in range(L)]
    dev = [torch.from_numpy(np.ascontiguousarray(np.stack([per[l][i] for l in range(L)], axis=1)).view(np.int16))
           .cuda() for i in range(4)]
    out = torch.empty((T, L, cfg.n_q * cfg.d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        net.decode(0, L, cfg.context, dev[0], dev[1], dev[2], dev[3], out, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"timed {steps} steps in {elapsed:.3f}s")
    copy_calibration(torch, args.copy_calibration)
    res = {"tok_s": steps * T / elapsed, "ms_step": 1000.0 * elapsed / steps, "extra": {}, "roofline": None,
           "inputs": per}
    algo, scratch = attn_split_bytes(cfg)
    res["extra"]["whole_step"] = {"bytes_per_token": round(algo * L),
                                  "GBps": round(algo * L * res["tok_s"] / 1e9, 1),
                                  "frac_of_hbm_peak": round(algo * L * res["tok_s"] / 1e9 / HBM_PEAK_GBS, 4)}
    if kernels:
        net.profile(True)
        step()
        torch.cuda.synchronize()
        ms_s, ms_c, n = net.profile(False)
        avg_s, avg_c = ms_s / n / 1000.0, ms_c / n / 1000.0
        ach = algo / avg_s / 1e9
        tot = ms_s + ms_c
        res["extra"]["kernels"] = {
            "attn_split": {"launches": n, "avg_us": round(avg_s * 1e6, 3), "share": round(ms_s / tot, 4),
                           "scratch_bytes_per_launch": round(scratch)},
            "attn_combine": {"launches": n, "avg_us": round(avg_c * 1e6, 3), "share": round(ms_c / tot, 4)}}
        res["roofline"] = {"bound": "hbm", "kernel": "attn_split", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic("attn_split", cfg.name),
                           "bytes_per_launch": round(algo), "avg_launch_us": round(avg_s * 1e6, 3)}
        log(f"kernel pass: {res['extra']['kernels']}")
    net.close()
    return res


def cpu_baseline_attn(cfg, per, budget_s: float) -> dict:
    """The oracle as it stands, single thread: the first tokens through all layers."""
    from oracle import attention as oatt
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    import synth
    sh = oatt.Shape(cfg.n_q, cfg.n_kv, cfg.d, cfg.rot)
    L, P = cfg.n_layers, cfg.context + cfg.n_tokens
    params, caches = [], []
    for l in range(L):
        params.append(oatt.Params(*[np.asarray(w, np.float64) for w in synth.attn_params(cfg, l)]))
        k16, v16 = synth.attn_cache(cfg, l, cfg.context)
        K = np.zeros((cfg.n_kv, P, cfg.d))
        V = np.zeros((cfg.n_kv, P, cfg.d))
        K[:, :cfg.context] = k16.view(np.float16)
        V[:, :cfg.context] = v16.view(np.float16)
        caches.append((K, V))
    f = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)  # noqa: E731
    t0 = time.perf_counter()
    done = 0
    while done < cfg.n_tokens and time.perf_counter() - t0 < budget_s:
        for l in range(L):
            q, g, k, v = (f(x[done]) for x in per[l])
            oatt.step(sh, params[l], cfg.context + done, *caches[l], q.reshape(cfg.n_q, cfg.d),
                      g.reshape(cfg.n_q, cfg.d), k.reshape(cfg.n_kv, cfg.d), v.reshape(cfg.n_kv, cfg.d))
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {cfg.n_tokens} tokens through all {L} layers",
            "seconds": round(dt, 2), "cpu_model": cpu_model(), "host_cores": os.cpu_count()}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 20 for one layer, 3 for resident stacks, 2 for the pooled stack)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default: 3 for one layer, else 1)")
    ap.add_argument("--workload", default="decode80b")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-pass", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill80b measurement that the default decode80b run adds under extra.prefill")
    ap.add_argument("--pool-gb", type=float, default=None,
                    help="HBM pool budget in GiB for the pooled workload (default: the workload's 2 GiB)")
    ap.add_argument("--storage", choices=("host", "file"), default="host",
                    help="pooled workload: misses come from the pinned host blob (default) or from a blob file "
                         "read with pread (O_DIRECT unless --buffered)")
    ap.add_argument("--blob-dir", default=os.environ.get("TMPDIR", "/tmp"),
                    help="directory for the blob file of --storage file (deleted afterwards)")
    ap.add_argument("--buffered", action="store_true", help="--storage file: read through the page cache")
    ap.add_argument("--keep-blob", action="store_true",
                    help="--storage file: keep the blob file afterwards, and reuse one of the right size "
                         "(evicted from the page cache first) instead of writing it again")
    ap.add_argument("--tokens", type=int, default=None,
                    help="tokens per step instead of the workload's own count (for sweeps of the slow "
                         "storage-backed path; the reported config says so)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after the timed steps, copy BYTES of device memory once with a plain copy "
                         "kernel (a known-size reference for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU mode",
              file=sys.stderr)
        return 2

    import torch
    import routed_expert_int4_router_amd as moe
    from routed_expert_int4_router_amd import loader
    import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.workload in synth.GDN_CONFIGS:
        gcfg = synth.get_gdn_config(args.workload)
        if args.tokens is not None:
            gcfg = gcfg.replace(n_tokens=args.tokens)
        steps = args.steps if args.steps is not None else 5
        warmup = args.warmup if args.warmup is not None else 1
        r = measure_gdn(gcfg, args, torch, moe, synth, steps, warmup, not args.no_kernel_pass)
        cpu = None
        if not args.no_cpu_baseline:
            log("timing the CPU oracle on a bounded sample")
            cpu = cpu_baseline_gdn(gcfg, r["inputs"], args.cpu_seconds)
            log(f"oracle: {cpu}")
        print(json.dumps({
            "metric": "MoE decode tok/s & % HBM roofline (80B-shape, bs=1); prefill % MFMA peak",
            "value": round(r["tok_s"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": round(r["ms_step"], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": gcfg.name, "layers": gcfg.n_layers, "key_heads": gcfg.n_k, "value_heads": gcfg.n_v,
                       "d_k": gcfg.d_k, "d_v": gcfg.d_v, "tokens_per_step": gcfg.n_tokens, "batch": 1},
            "roofline": r["roofline"], "cpu_baseline": cpu, "extra": r["extra"]}), flush=True)
        return 0
    if args.workload in synth.ATTN_CONFIGS:
        acfg = synth.get_attn_config(args.workload)
        if args.tokens is not None:
            acfg = acfg.replace(n_tokens=args.tokens)
        steps = args.steps if args.steps is not None else 10
        warmup = args.warmup if args.warmup is not None else 2
        r = measure_attn(acfg, args, torch, moe, synth, steps, warmup, not args.no_kernel_pass)
        cpu = None
        if not args.no_cpu_baseline:
            log("timing the CPU oracle on a bounded sample")
            cpu = cpu_baseline_attn(acfg, r["inputs"], args.cpu_seconds)
            log(f"oracle: {cpu}")
        print(json.dumps({
            "metric": "MoE decode tok/s & % HBM roofline (80B-shape, bs=1); prefill % MFMA peak",
            "value": round(r["tok_s"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": round(r["ms_step"], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16", "data": "synthetic",
            "config": {"workload": acfg.name, "layers": acfg.n_layers, "query_heads": acfg.n_q,
                       "kv_heads": acfg.n_kv, "head_dim": acfg.d, "rot_dim": acfg.rot, "context": acfg.context,
                       "tokens_per_step": acfg.n_tokens, "batch": 1},
            "roofline": r["roofline"], "cpu_baseline": cpu, "extra": r["extra"]}), flush=True)
        return 0
    cfg = synth.get_config(args.workload)
    if args.pool_gb is not None:
        if not cfg.pool_budget:
            print(f"--pool-gb applies to a pooled workload; {cfg.name} keeps every expert resident", file=sys.stderr)
            return 2
        cfg = cfg.replace(pool_budget=int(args.pool_gb * (1 << 30)))
    if args.tokens is not None:
        cfg = cfg.replace(n_tokens=args.tokens)
    if args.steps is None:
        args.steps = 20 if cfg.n_layers == 1 else (2 if cfg.pool_budget else 3)
    if args.warmup is None:
        args.warmup = 3 if cfg.n_layers == 1 else 1
    r = measure(cfg, args, torch, moe, loader, synth, args.steps, args.warmup, not args.no_kernel_pass)
    extra = r["extra"]
    prefill = cfg.name.startswith("prefill")

    if cfg.name == "decode80b" and not args.no_prefill:
        pcfg = synth.get_config("prefill80b")
        p = measure(pcfg, args, torch, moe, loader, synth, max(args.steps // 2, 1), args.warmup,
                    not args.no_kernel_pass)
        extra["prefill"] = {"workload": pcfg.name, "value": round(p["tok_s"], 1), "unit": "tokens/s",
                            "ms_per_step": round(p["ms_step"], 4), "dtype": "fp16",
                            "tokens_per_step": pcfg.n_tokens, "roofline": p["roofline"],
                            "gemms": p["extra"].get("gemms"), "kernels": p["extra"].get("kernels")}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg, r["xb"], args.cpu_seconds)
        log(f"oracle: {cpu}")

    # the arithmetic the path computes in: the decode kernels work in fp32 on
    # exact integer codes; the batched path's grouped GEMMs run fp16 MFMA
    dtype = "fp16" if prefill else "f32"
    T = cfg.n_tokens
    line = {
        "metric": "MoE decode tok/s & % HBM roofline (80B-shape, bs=1); prefill % MFMA peak",
        "value": round(r["tok_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "hidden": cfg.hidden, "experts": cfg.n_experts, "top_k": cfg.top_k,
                   "inter": cfg.inter, "bits": cfg.bits, "group": cfg.group, "layers": cfg.n_layers,
                   "tokens_per_step": T, "batch": T if prefill else 1,
                   "pool_budget": cfg.pool_budget,
                   "expert_storage": (args.storage + ("-buffered" if args.buffered else "")) if cfg.pool_budget
                   else "hbm"},
        "roofline": r["roofline"],
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
