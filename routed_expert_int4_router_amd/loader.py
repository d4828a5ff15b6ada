"""Load fp32 weights into a libmoe model: quantise + pack (moe_pack) and upload.

``weights`` is any object with
    expert(layer, e)   -> (w_gate [I][H], w_up [I][H], w_down [H][I]) fp32
    shared(layer)      -> the same for the shared expert
    router(layer)      -> W_r [H][E] fp32
    bias(layer)        -> [E] fp32 or None
    shared_gate(layer) -> [H] fp32
Experts are produced by a thread pool and packed in chunks, so host memory
stays bounded (a chunk of fp32 weights, not the whole model). For a
host-storage model the records are packed straight into the pinned blob; for
a file-backed model they are written, in gid order at the stride, into a
blob file that the model then reads its misses from.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

from . import _lib


def load_model(cfg, weights, storage: int = _lib.STORE_DEVICE, threads: int = 16, chunk: int = 64,
               layers: Optional[range] = None, blob_path: Optional[str] = None, direct: bool = True,
               progress=None) -> _lib.Model:
    """A model filled from ``weights``. A file-backed model (STORE_FILE) needs
    ``blob_path``: the records are written there (replacing the file) and the
    model opens it, with O_DIRECT when ``direct`` and the filesystem allow.
    ``progress(layer)``, if given, is called after each layer is filled."""
    c = _lib.config_of(cfg)
    if storage == _lib.STORE_FILE and not blob_path:
        raise ValueError("a file-backed model needs blob_path")
    model = _lib.Model(c, storage)
    try:
        if storage == _lib.STORE_FILE:
            with open(blob_path, "wb") as f:
                fill_model(model, weights, threads=threads, chunk=chunk, layers=layers, blob_file=f,
                           progress=progress)
                # on storage and out of the page cache: the first read of every
                # record comes from the device, buffered or not
                f.flush()
                os.fsync(f.fileno())
                if hasattr(os, "posix_fadvise"):
                    os.posix_fadvise(f.fileno(), 0, 0, os.POSIX_FADV_DONTNEED)
            model.open_blob(blob_path, 0, direct)
        else:
            fill_model(model, weights, threads=threads, chunk=chunk, layers=layers, progress=progress)
    except Exception:
        model.close()
        raise
    return model


def fill_dense(model: _lib.Model, weights, layers: Optional[range] = None):
    """Upload only the resident dense part of each layer: router, bias, shared
    expert and shared gate (for a file-backed model whose blob file exists)."""
    c = model.cfg
    for layer in (range(c.n_layers) if layers is None else layers):
        wg_s, wu_s, wd_s = weights.shared(layer)
        shared_rec = _lib.pack(c, wg_s, wu_s, wd_s, inter=c.shared_inter)
        model.set_layer(layer, weights.router(layer), weights.bias(layer), shared_rec, weights.shared_gate(layer))
    return model


def fill_model(model: _lib.Model, weights, threads: int = 16, chunk: int = 64, layers: Optional[range] = None,
               blob_file=None, progress=None):
    """Upload the dense weights and pack the experts: into the pinned blob
    (host storage), into a writable binary ``blob_file`` at gid * stride (file
    storage), or into HBM (device storage)."""
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
                elif blob_file is not None:
                    blob_file.seek(gid * stride)
                    blob_file.write(_lib.pack(c, wg, wu, wd).tobytes())
                else:
                    model.set_experts(gid, _lib.pack(c, wg, wu, wd))
            if progress is not None:
                progress(layer)
    return model
