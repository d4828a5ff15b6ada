"""Oracle-side assembly of layer weights from the seeded synthetic inputs.

Test infrastructure only; see the package docstring. Every expert goes
through the oracle's own packer and back (quantise -> record bytes -> unpack
-> dequantise in float64), so what the oracle computes with is exactly what a
packed record holds.
"""
from __future__ import annotations

from functools import lru_cache
from typing import Dict, List, Optional

import numpy as np

import synth
from . import moe, quant


def expert_record(cfg: synth.Config, layer: int, e: int) -> np.ndarray:
    """Oracle-packed record bytes (padded to the stride) of routed expert e, or of the shared expert (e == E)."""
    inter = cfg.shared_inter if e == cfg.n_experts else cfg.inter
    wg, wu, wd = synth.expert_weights(cfg.seed, layer, e, cfg.hidden, inter, cfg.expert_std)
    return quant.pack_record(quant.quantize_expert(wg, wu, wd, cfg.bits), cfg.bits)


class OracleModel:
    """Lazily dequantised weights of a config; experts are cached per (layer, e)."""

    def __init__(self, cfg: synth.Config, cache_limit: int = 4096):
        self.cfg = cfg
        self._cache: Dict[tuple, moe.DenseExpert] = {}
        self._cache_limit = cache_limit

    def dense(self, layer: int, e: int) -> moe.DenseExpert:
        key = (layer, e)
        d = self._cache.get(key)
        if d is None:
            cfg = self.cfg
            inter = cfg.shared_inter if e == cfg.n_experts else cfg.inter
            rec = expert_record(cfg, layer, e)
            d = moe.dense_expert(quant.unpack_record(rec, cfg.hidden, inter, cfg.bits))
            if len(self._cache) >= self._cache_limit:
                self._cache.pop(next(iter(self._cache)))
            self._cache[key] = d
        return d

    def layer(self, layer: int) -> moe.LayerWeights:
        cfg = self.cfg
        return moe.LayerWeights(
            w_r=synth.router_weight(cfg.seed, layer, cfg.hidden, cfg.n_experts),
            rho=synth.router_bias(cfg, layer),
            g_s=synth.shared_gate(cfg.seed, layer, cfg.hidden),
            shared=self.dense(layer, cfg.n_experts),
            expert=lambda e, _l=layer: self.dense(_l, e),
        )

    def layers(self) -> List[moe.LayerWeights]:
        return [self.layer(l) for l in range(self.cfg.n_layers)]
