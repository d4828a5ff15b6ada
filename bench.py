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

A step is one pass of the workload's tokens through the whole path (router,
top-k, expert GEMV/GEMM, combine, stack glue, pool). W untimed steps, then K
timed steps bracketed by device synchronisation; value = tokens / second.
A second, instrumented pass of the same steps hands every kernel launch a
hipEvent pair that the launch fills with the kernel's own begin/end
timestamps; the dominant kernel's average duration and its algorithmic bytes
(or flops) give the roofline entry. The CPU oracle is timed
on a bounded sample of the same workload, single-threaded.
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
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------- algorithmic bytes ---

def decode_kernel_bytes(cfg, stack: bool) -> dict:
    """Bytes each decode kernel must move per launch (one token, one layer).

    Fused path (expert + reduce): the expert kernel reads the k + 1 records
    (gate, up, down codes and scales), x and the logits, and writes one fp32
    partial row of H per (slot, I slice); reduce reads those rows and writes
    out (a stack also reads the residual and writes the bf16 recast).
    Two-kernel path (gateup + down, for shapes the fused kernel does not take).
    """
    H, I, E, k, b = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.bits
    codes = I * H * b // 8          # one matrix
    sc = I * H // 64 * 4
    router = (E + 1) * H * 4 + E * 4 + H * 2 + (E + 1) * 4
    parts = (k + 1) * (I // 32) * H * 4
    expert = (k + 1) * 3 * (codes + sc) + H * 2 + (E + 1) * 4 + parts
    reduce = parts + H * 4
    gateup = (k + 1) * 2 * (codes + sc) + H * 2 + (E + 1) * 4 + (k + 1) * I * 4
    down = (k + 1) * (codes + sc) + (k + 1) * I * 4 + (k + 1) * 4 + H * 4
    if stack:
        reduce += H * 4 + H * 2     # residual read + bf16 recast write
        down += H * 4 + H * 2
    return {"router": router, "expert": expert, "reduce": reduce, "gateup": gateup, "down": down,
            "topk": (E + 1) * 4 + 2 * k * 4}


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
            "seconds": round(dt, 2)}


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
    ap.add_argument("--pool-gb", type=float, default=None,
                    help="HBM pool budget in GiB for the pooled workload (default: the workload's 2 GiB)")
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
    cfg = synth.get_config(args.workload)
    if args.pool_gb is not None:
        if not cfg.pool_budget:
            print(f"--pool-gb applies to a pooled workload; {cfg.name} keeps every expert resident", file=sys.stderr)
            return 2
        cfg = cfg.replace(pool_budget=int(args.pool_gb * (1 << 30)))
    T = cfg.n_tokens
    if args.steps is None:
        args.steps = 20 if cfg.n_layers == 1 else (2 if cfg.pool_budget else 3)
    if args.warmup is None:
        args.warmup = 3 if cfg.n_layers == 1 else 1
    log(f"workload {cfg.name}: {cfg.description}")
    t0 = time.perf_counter()
    storage = moe.STORE_HOST if cfg.pool_budget else moe.STORE_DEVICE
    model = loader.load_model(cfg, synth.SynthWeights(cfg), storage=storage)
    log(f"model loaded in {time.perf_counter() - t0:.1f}s")
    pool = moe.Pool(model, cfg.pool_budget) if cfg.pool_budget else None
    xb = synth.tokens(cfg.seed, T, cfg.hidden)
    x = torch.from_numpy(xb.view(np.int16)).cuda()
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    if cfg.name.startswith("prefill"):
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

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {elapsed:.3f}s")
    tok_s = args.steps * T / elapsed
    ms_step = 1000.0 * elapsed / args.steps

    extra = {}
    if pool is not None:
        st = pool.stats()  # counts of the last timed step (the pool is reset at every step)
        extra["pool"] = {**st, "hit_rate": round(st["hits"] / max(1, st["accesses"]), 4),
                         "h2d_GBps": round(st["h2d_bytes"] / (elapsed / args.steps) / 1e9, 2),
                         "link_probe_GBps": link_probe(torch, moe.expert_bytes(cfg))}
    if args.copy_calibration > 0:
        n = args.copy_calibration // 4
        src_t = torch.ones(n, dtype=torch.float32, device="cuda")
        dst_t = torch.empty_like(src_t)
        torch.cuda.synchronize()
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        log(f"copy calibration: {4 * n} bytes")
        del src_t, dst_t
    roofline = None
    if not args.no_kernel_pass:
        n_prof = max(1, min(args.steps, 5 if cfg.n_layers == 1 else 1))
        model.profile_enable(True)
        for i in range(n_prof):
            step()
        torch.cuda.synchronize()
        prof = model.profile_read()
        model.profile_enable(False)
        prof = {k: v for k, v in prof.items() if v[0] > 0}
        extra["kernels"] = {k: {"launches": v[0], "avg_us": round(1000.0 * v[1] / v[0], 3),
                                "share": round(v[1] / max(1e-9, sum(p[1] for p in prof.values())), 3)}
                            for k, v in prof.items()}
        log(f"kernel pass: {extra['kernels']}")
        if cfg.name.startswith("prefill"):
            fl = prefill_flops(cfg, T)
            gemms = {k: v for k, v in prof.items() if k in fl}
            if gemms:
                dom = max(gemms, key=lambda k: gemms[k][1])
                avg_s = gemms[dom][1] / gemms[dom][0] / 1000.0
                ach = fl[dom] / avg_s / 1e12
                roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2),
                            "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(ach / BF16_MFMA_PEAK_TFLOPS, 4),
                            "traffic": measured_traffic(dom, cfg.name)}
        else:
            by = decode_kernel_bytes(cfg, stack=cfg.n_layers > 1)
            cands = {k: v for k, v in prof.items() if k in by}
            dom = max(cands, key=lambda k: cands[k][1])
            avg_s = cands[dom][1] / cands[dom][0] / 1000.0
            ach = by[dom] / avg_s / 1e9
            roofline = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(dom, cfg.name),
                        "bytes_per_launch": by[dom], "avg_launch_us": round(avg_s * 1e6, 3)}
            per_tok = step_bytes_per_token(cfg) * cfg.n_layers
            extra["whole_step"] = {"bytes_per_token": per_tok,
                                   "GBps": round(per_tok * tok_s / 1e9, 1),
                                   "frac_of_hbm_peak": round(per_tok * tok_s / 1e9 / HBM_PEAK_GBS, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg, xb, args.cpu_seconds)
        log(f"oracle: {cpu}")

    dtype = "bf16" if cfg.name.startswith("prefill") else "f32"
    line = {
        "metric": "MoE decode tok/s & % HBM roofline (80B-shape, bs=1); prefill % MFMA peak",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "hidden": cfg.hidden, "experts": cfg.n_experts, "top_k": cfg.top_k,
                   "inter": cfg.inter, "bits": cfg.bits, "group": cfg.group, "layers": cfg.n_layers,
                   "tokens_per_step": T, "batch": T if cfg.name.startswith("prefill") else 1,
                   "pool_budget": cfg.pool_budget},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
