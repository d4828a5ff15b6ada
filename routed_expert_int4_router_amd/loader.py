"""Load fp32 weights into a libmoe model: quantise + pack (moe_pack) and upload.

``weights`` is any object with
    expert(layer, e)   -> (w_gate [I][H], w_up [I][H], w_down [H][I]) fp32
    shared(layer)      -> the same for the shared expert
    router(layer)      -> W_r [H][E] fp32
    bias(layer)        -> [E] fp32 or None
    shared_gate(layer) -> [H] fp32
Experts are produced by a thread pool and packed in chunks, so host memory
stays bounded (a chunk of fp32 weights, not the whole model). For a
host-storage model the records are packed straight into the pinned blob.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

from . import _lib


def load_model(cfg, weights, storage: int = _lib.STORE_DEVICE, threads: int = 16, chunk: int = 64,
               layers: Optional[range] = None) -> _lib.Model:
    c = _lib.config_of(cfg)
    model = _lib.Model(c, storage)
    try:
        fill_model(model, weights, threads=threads, chunk=chunk, layers=layers)
    except Exception:
        model.close()
        raise
    return model


def fill_model(model: _lib.Model, weights, threads: int = 16, chunk: int = 64, layers: Optional[range] = None):
    c = model.cfg
    H, I, E = c.hidden, c.inter, c.n_experts
    stride = _lib.expert_stride(c)
    blob = model.host_blob() if model.storage == _lib.STORE_HOST else None
    layers = range(c.n_layers) if layers is None else layers
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        for layer in layers:
            wg_s, wu_s, wd_s = weights.shared(layer)
            shared_rec = _lib.pack(c, wg_s, wu_s, wd_s, inter=c.shared_inter)
            model.set_layer(layer, weights.router(layer), weights.bias(layer), shared_rec, weights.shared_gate(layer))
            for e0 in range(0, E, chunk):
                n = min(chunk, E - e0)
                wg = np.empty((n, I, H), np.float32)
                wu = np.empty((n, I, H), np.float32)
                wd = np.empty((n, H, I), np.float32)

                def gen(i, _e0=e0, _layer=layer):
                    a, b, d = weights.expert(_layer, _e0 + i)
                    wg[i], wu[i], wd[i] = a, b, d

                list(ex.map(gen, range(n)))
                gid = layer * E + e0
                if blob is not None:
                    _lib.pack(c, wg, wu, wd, out=blob[gid * stride:(gid + n) * stride])
                else:
                    model.set_experts(gid, _lib.pack(c, wg, wu, wd))
    return model
