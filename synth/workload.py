"""Workload shapes and seeded random inputs.

Shapes follow the Qwen3-Next-80B-A3B and Qwen3.6-35B-A3B families as the pages
describe them: each layer routes a token to 10 of 512 experts (80B) or 8 of
256 (35B) (cheshm.ai news article on Swiftlet, paragraph on how it works), and
the 80B model has 48 layers (Swiftlet field test at alphalab.site, section
explaining MoE expert streaming). Hidden size 2048, expert intermediate 512,
group size 64 and the value distributions are the workload recipe of this
project; the pages do not print them.

Every tensor has its own numpy SeedSequence built from
``[seed, layer, expert_or_slot, tensor_id]`` so any single expert can be
regenerated on its own (the oracle recomputes only what it samples).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

# tensor ids inside a SeedSequence key
_GATE, _UP, _DOWN = 0, 1, 2
_ROUTER, _SHARED_GATE, _BIAS, _PERM = 3, 4, 5, 6
_TOKENS = 7
_LAYER_SLOT = 1 << 20   # "expert" field used for per-layer, non-expert tensors
_TOKEN_SLOT = 1 << 21   # "layer" field used for token streams

WEIGHT_STD = 0.02       # router and shared-gate weights; expert weights by default
# Expert weight std of the layer stacks. With no normalisation between layers
# the residual r_{l+1} = r_l + out_l grows, and an expert's output is
# quadratic in its input (SwiGLU), so at 0.02 the 48-layer 80B-shaped stack
# runs away after ~32 layers (rms 2 -> inf by layer 44) and the 40-layer
# 35B-shaped one nearly so. An expert's output scales as std^3, and 0.014
# keeps every stack's residual within a few per cent of unit rms.
STACK_EXPERT_STD = 0.014
ZIPF_S = 1.1            # popularity exponent of the pooled-stack workload


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    bits: int
    group: int
    n_layers: int
    n_tokens: int
    seed: int = 0
    bias: str = "none"            # "none" | "normal" | "zipf"
    zipf_lambda: float = 0.0
    pool_budget: Optional[int] = None   # bytes of HBM expert pool, None = all resident
    norm_topk: int = 1
    expert_std: float = WEIGHT_STD       # std of the routed and shared expert weights
    description: str = ""

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


GiB = 1 << 30

CONFIGS: Dict[str, Config] = {
    "tiny": Config(
        "tiny", hidden=256, n_experts=16, top_k=2, inter=128, shared_inter=128, bits=4, group=64,
        n_layers=1, n_tokens=8, seed=0,
        description="tiny MoE layer: H 256, 16 experts, top-2, I 128, int4 g64, 8 tokens"),
    "decode80b": Config(
        "decode80b", hidden=2048, n_experts=512, top_k=10, inter=512, shared_inter=512, bits=4, group=64,
        n_layers=1, n_tokens=1024, seed=0,
        description="80B-shaped single MoE layer, batch-1 decode, 1024 sequential tokens, all experts in HBM"),
    "stack35b_int8": Config(
        "stack35b_int8", hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512, bits=8, group=64,
        n_layers=40, n_tokens=512, seed=0, expert_std=STACK_EXPERT_STD,
        description="35B-shaped 40-layer MoE stack, int8, batch-1 decode, 512 tokens, all experts in HBM"),
    "stack35b_int4": Config(
        "stack35b_int4", hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512, bits=4, group=64,
        n_layers=40, n_tokens=512, seed=0, expert_std=STACK_EXPERT_STD,
        description="35B-shaped 40-layer MoE stack, int4, batch-1 decode, 512 tokens, all experts in HBM"),
    "prefill80b": Config(
        "prefill80b", hidden=2048, n_experts=512, top_k=10, inter=512, shared_inter=512, bits=4, group=64,
        n_layers=1, n_tokens=2048, seed=0, bias="normal",
        description="80B-shaped MoE layer, 2048-token batched prefill, router bias ~N(0,1) per expert"),
    "pool80b": Config(
        "pool80b", hidden=2048, n_experts=512, top_k=10, inter=512, shared_inter=512, bits=4, group=64,
        n_layers=48, n_tokens=1024, seed=0, bias="zipf", zipf_lambda=0.6, pool_budget=2 * GiB,
        expert_std=STACK_EXPERT_STD,
        description="80B-shaped 48-layer stack decode, experts in pinned host memory, 2 GiB HBM pool"),
    "resident80b": Config(
        "resident80b", hidden=2048, n_experts=512, top_k=10, inter=512, shared_inter=512, bits=4, group=64,
        n_layers=48, n_tokens=1024, seed=0, bias="zipf", zipf_lambda=0.6, pool_budget=None,
        expert_std=STACK_EXPERT_STD,
        description="80B-shaped 48-layer stack decode with every expert resident in HBM"),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _normal(shape, *key: int, std: float = WEIGHT_STD) -> np.ndarray:
    n = int(np.prod(shape))
    a = _rng(*key).standard_normal(n, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a.reshape(shape)


def expert_weights(seed: int, layer: int, expert: int, hidden: int, inter: int, std: float = WEIGHT_STD
                   ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """fp32 gate [inter][hidden], up [inter][hidden], down [hidden][inter], each ~N(0, std)."""
    wg = _normal((inter, hidden), seed, layer, expert, _GATE, std=std)
    wu = _normal((inter, hidden), seed, layer, expert, _UP, std=std)
    wd = _normal((hidden, inter), seed, layer, expert, _DOWN, std=std)
    return wg, wu, wd


def shared_expert_weights(seed: int, layer: int, n_experts: int, hidden: int, shared_inter: int,
                          std: float = WEIGHT_STD):
    """The shared expert is drawn as expert index ``n_experts`` of its layer."""
    return expert_weights(seed, layer, n_experts, hidden, shared_inter, std)


def router_weight(seed: int, layer: int, hidden: int, n_experts: int) -> np.ndarray:
    """fp32 W_r [hidden][n_experts] ~N(0, 0.02)."""
    return _normal((hidden, n_experts), seed, layer, _LAYER_SLOT, _ROUTER)


def shared_gate(seed: int, layer: int, hidden: int) -> np.ndarray:
    """fp32 g_s [hidden] ~N(0, 0.02): the shared expert's sigmoid gate vector."""
    return _normal((hidden,), seed, layer, _LAYER_SLOT, _SHARED_GATE)


def router_bias(cfg: Config, layer: int) -> Optional[np.ndarray]:
    """Per-expert fp32 bias added to the router logits, or None.

    "normal": rho[e] ~ N(0, 1) (skews the prefill bucket sizes).
    "zipf":   rho[e] = -lambda * s * ln(rank(e)), rank a seeded permutation of 1..E,
              so exp(rho) follows a Zipf(s) popularity law when lambda = 1.
    """
    E = cfg.n_experts
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal":
        return _normal((E,), cfg.seed, layer, _LAYER_SLOT, _BIAS, std=1.0)
    if cfg.bias == "zipf":
        rank = _rng(cfg.seed, layer, _LAYER_SLOT, _PERM).permutation(E).astype(np.float64) + 1.0
        return (-cfg.zipf_lambda * ZIPF_S * np.log(rank)).astype(np.float32)
    raise ValueError(f"unknown bias kind {cfg.bias!r}")


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def tokens(seed: int, n_tokens: int, hidden: int, stream: int = 0) -> np.ndarray:
    """bf16 activations ~N(0,1) as uint16 bit patterns, shape [n_tokens][hidden].

    Row t depends only on (seed, stream, t), so a prefix of a longer stream is
    the same tokens.
    """
    out = np.empty((n_tokens, hidden), dtype=np.uint16)
    for t in range(n_tokens):
        row = _rng(seed, _TOKEN_SLOT, stream, _TOKENS, t).standard_normal(hidden, dtype=np.float32)
        out[t] = f32_to_bf16_bits(row)
    return out


class SynthWeights:
    """The seeded fp32 weights of a config, in the shape a model loader asks for them."""

    def __init__(self, cfg: Config):
        self.cfg = cfg

    def expert(self, layer: int, e: int):
        c = self.cfg
        return expert_weights(c.seed, layer, e, c.hidden, c.inter, c.expert_std)

    def shared(self, layer: int):
        c = self.cfg
        return shared_expert_weights(c.seed, layer, c.n_experts, c.hidden, c.shared_inter, c.expert_std)

    def router(self, layer: int) -> np.ndarray:
        c = self.cfg
        return router_weight(c.seed, layer, c.hidden, c.n_experts)

    def bias(self, layer: int) -> Optional[np.ndarray]:
        return router_bias(self.cfg, layer)

    def shared_gate(self, layer: int) -> np.ndarray:
        c = self.cfg
        return shared_gate(c.seed, layer, c.hidden)


# ------------------------------------------------------------ DeltaNet step ---
# Seeded inputs of the Gated DeltaNet decode step (the linear-attention layers
# beside the MoE). Shapes follow the Qwen3-Next-80B linear-attention layer: 16
# key heads and 32 value heads of dimension 128, a 4-tap causal convolution;
# the distributions are this project's recipe.

_GDN_CONV, _GDN_ALOG, _GDN_DT, _GDN_NORM, _GDN_QKV, _GDN_Z, _GDN_A, _GDN_B = 20, 21, 22, 23, 24, 25, 26, 27


@dataclasses.dataclass(frozen=True)
class GdnConfig:
    name: str
    n_k: int
    n_v: int
    d_k: int
    d_v: int
    n_layers: int
    n_tokens: int
    seed: int = 0
    description: str = ""

    @property
    def channels(self) -> int:
        return 2 * self.n_k * self.d_k + self.n_v * self.d_v

    def replace(self, **kw) -> "GdnConfig":
        return dataclasses.replace(self, **kw)


GDN_CONFIGS: Dict[str, GdnConfig] = {
    "gdn_tiny": GdnConfig("gdn_tiny", n_k=2, n_v=4, d_k=32, d_v=32, n_layers=2, n_tokens=16,
                          description="tiny Gated DeltaNet: 2 key / 4 value heads of 32, 2 layers"),
    "gdn80b": GdnConfig("gdn80b", n_k=16, n_v=32, d_k=128, d_v=128, n_layers=36, n_tokens=256,
                        description="80B-shaped Gated DeltaNet decode: 36 layers, 16 key / 32 value heads of 128, "
                                    "256 tokens one at a time"),
}


def get_gdn_config(name: str, **overrides) -> GdnConfig:
    cfg = GDN_CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


def gdn_params(cfg: GdnConfig, layer: int):
    """fp32 (conv_w [C][4] ~ N(0, 0.3), A_log = ln U(1, 16) [n_v], dt_bias ~ N(0, 1) [n_v],
    norm_w ~ 1 + N(0, 0.1) [d_v])."""
    conv_w = _normal((cfg.channels, 4), cfg.seed, layer, _LAYER_SLOT, _GDN_CONV, std=0.3)
    a_log = np.log(_rng(cfg.seed, layer, _LAYER_SLOT, _GDN_ALOG).uniform(1.0, 16.0, cfg.n_v)).astype(np.float32)
    dt_bias = _normal((cfg.n_v,), cfg.seed, layer, _LAYER_SLOT, _GDN_DT, std=1.0)
    norm_w = (np.float32(1.0) + _normal((cfg.d_v,), cfg.seed, layer, _LAYER_SLOT, _GDN_NORM, std=0.1))
    return conv_w, a_log, dt_bias, norm_w.astype(np.float32)


def gdn_inputs(cfg: GdnConfig, layer: int, n_tokens: int):
    """bf16 bit patterns ~ N(0, 1): qkv [T][C], z [T][n_v * d_v], a [T][n_v], b [T][n_v]."""
    def bits(shape, tid):
        return f32_to_bf16_bits(_normal(shape, cfg.seed, layer, _TOKEN_SLOT, tid, std=1.0))
    return (bits((n_tokens, cfg.channels), _GDN_QKV), bits((n_tokens, cfg.n_v * cfg.d_v), _GDN_Z),
            bits((n_tokens, cfg.n_v), _GDN_A), bits((n_tokens, cfg.n_v), _GDN_B))


# ------------------------------------------------------ gated attention step ---
# Seeded inputs of the gated GQA decode step (the full-attention layers). Shapes
# follow the Qwen3-Next-80B attention layer: 16 query heads, 2 KV heads of
# dimension 256, the first quarter of each head rotated; the cache is filled
# with `context` synthetic positions before the decoded tokens.

_ATT_WQ, _ATT_WK, _ATT_KC, _ATT_VC, _ATT_Q, _ATT_G, _ATT_K, _ATT_V = 30, 31, 32, 33, 34, 35, 36, 37


@dataclasses.dataclass(frozen=True)
class AttnConfig:
    name: str
    n_q: int
    n_kv: int
    d: int
    rot: int
    n_layers: int
    context: int      # positions already in the cache
    n_tokens: int     # tokens decoded after them
    seed: int = 0
    description: str = ""

    def replace(self, **kw) -> "AttnConfig":
        return dataclasses.replace(self, **kw)


ATTN_CONFIGS: Dict[str, AttnConfig] = {
    "attn_tiny": AttnConfig("attn_tiny", n_q=4, n_kv=2, d=64, rot=16, n_layers=2, context=37, n_tokens=9,
                            description="tiny gated GQA decode: 4 query / 2 KV heads of 64, 2 layers"),
    "attn80b": AttnConfig("attn80b", n_q=16, n_kv=2, d=256, rot=64, n_layers=12, context=8192, n_tokens=64,
                          description="80B-shaped gated GQA decode: 12 layers, 16 query / 2 KV heads of 256, "
                                      "8192 cached positions, 64 tokens one at a time"),
}


def get_attn_config(name: str, **overrides) -> AttnConfig:
    cfg = ATTN_CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


def attn_params(cfg: AttnConfig, layer: int):
    """fp32 q and k norm weights [d] ~ 1 + N(0, 0.1)."""
    wq = np.float32(1.0) + _normal((cfg.d,), cfg.seed, layer, _LAYER_SLOT, _ATT_WQ, std=0.1)
    wk = np.float32(1.0) + _normal((cfg.d,), cfg.seed, layer, _LAYER_SLOT, _ATT_WK, std=0.1)
    return wq.astype(np.float32), wk.astype(np.float32)


def attn_cache(cfg: AttnConfig, layer: int, n_pos: int):
    """fp16 bit patterns of the cached positions: K ~ N(0, 1) and V ~ N(0, 1), [n_kv][n_pos][d] each."""
    k = _normal((cfg.n_kv, n_pos, cfg.d), cfg.seed, layer, _LAYER_SLOT, _ATT_KC, std=1.0).astype(np.float16)
    v = _normal((cfg.n_kv, n_pos, cfg.d), cfg.seed, layer, _LAYER_SLOT, _ATT_VC, std=1.0).astype(np.float16)
    return k.view(np.uint16), v.view(np.uint16)


def attn_inputs(cfg: AttnConfig, layer: int, n_tokens: int):
    """bf16 bit patterns ~ N(0, 1): q and gate [T][n_q * d], k and v [T][n_kv * d]."""
    def bits(shape, tid):
        return f32_to_bf16_bits(_normal(shape, cfg.seed, layer, _TOKEN_SLOT, tid, std=1.0))
    return (bits((n_tokens, cfg.n_q * cfg.d), _ATT_Q), bits((n_tokens, cfg.n_q * cfg.d), _ATT_G),
            bits((n_tokens, cfg.n_kv * cfg.d), _ATT_K), bits((n_tokens, cfg.n_kv * cfg.d), _ATT_V))
