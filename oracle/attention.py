"""Gated grouped-query attention decode step with a KV cache (oracle). Test
infrastructure only; see the package docstring.

Pages: 12 of the 80B model's 48 layers are full-attention layers, the only
ones with a growing K/V cache; the pinned architecture config budgets it at
24 KiB per token in fp16, while the current runtime stores it as fp32, at
least 48 KiB per token: about 384 MiB at 8K context, 1.5 GiB at 32K and
12 GiB at the native 262,144 (alphalab.site field test, section explaining
MoE expert streaming); the model pairs linear attention with gated attention
(cheshm.ai article, paragraph on the code base).

The pages print no formula. Reading taken: the decode form of the
Qwen3-Next gated attention layer, with the cache in the fp16 format the
budget names. For the token at position p, per query head h of KV group
h // (n_q / n_kv), on the projected inputs q, gate [n_q][d], k, v [n_kv][d]:
  norms     q_h = rms(q_h) * wq, k_g = rms(k_g) * wk   (rms(x) = x / sqrt(mean(x^2) + 1e-6))
  rope      the first r dims rotated by position: pairs (i, i + r/2), angle
            p * theta^(-2i/r), theta = 1e7; the other d - r dims unchanged
  cache     K[p] = fp16(k_g), V[p] = fp16(v_g)  (round to nearest even)
  attend    s_j = q_h . K[j] / sqrt(d) for j <= p; w = softmax(s); o = sum_j w_j V[j]
  gate      out_h = o * sigmoid(gate_h)
KV bytes per token and layer: 2 * n_kv * d * 2 (fp16); with 2 KV heads of 256
that is 2 KiB, and 12 layers hold 24 KiB per token, the pages' budget.
"""
from __future__ import annotations

from typing import NamedTuple

import numpy as np

THETA = 1.0e7
EPS = 1e-6


class Shape(NamedTuple):
    n_q: int
    n_kv: int
    d: int
    rot: int     # rotated dims (even, <= d)

    def kv_bytes_per_token(self, bytes_per_value: int = 2) -> int:
        return 2 * self.n_kv * self.d * bytes_per_value


class Params(NamedTuple):
    wq: np.ndarray   # [d] q norm weight
    wk: np.ndarray   # [d] k norm weight


def rms(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS)


def rope(x: np.ndarray, p: int, rot: int) -> np.ndarray:
    """Rotate the first `rot` dims of each row of x by position p (pairs i, i + rot/2)."""
    x = np.asarray(x, dtype=np.float64).copy()
    half = rot // 2
    i = np.arange(half, dtype=np.float64)
    ang = p * THETA ** (-2.0 * i / rot)
    c, s = np.cos(ang), np.sin(ang)
    x1 = x[..., :half].copy()
    x2 = x[..., half:rot].copy()
    x[..., :half] = x1 * c - x2 * s
    x[..., half:rot] = x2 * c + x1 * s
    return x


def fp16(x) -> np.ndarray:
    """The cache format: fp16, round to nearest even."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """softmax(q . K^T / sqrt(d)) . V for one query row over rows K, V [n][d]."""
    s = K @ q / np.sqrt(q.shape[-1])
    w = np.exp(s - s.max())
    return (w / w.sum()) @ V


def step(sh: Shape, p: Params, pos: int, K: np.ndarray, V: np.ndarray, q, gate, k, v):
    """One token at position pos. K, V: fp16-valued float64 caches [n_kv][>pos][d]
    (positions < pos filled); row pos is written here. q, gate [n_q][d], k, v
    [n_kv][d] (float64 holding bf16 inputs). Returns out [n_q][d]."""
    qn = rope(rms(q) * p.wq, pos, sh.rot)
    kn = rope(rms(k) * p.wk, pos, sh.rot)
    K[:, pos] = fp16(kn)
    V[:, pos] = fp16(v)
    g = sh.n_q // sh.n_kv
    out = np.empty((sh.n_q, sh.d))
    for h in range(sh.n_q):
        o = attend(qn[h], K[h // g, :pos + 1], V[h // g, :pos + 1])
        out[h] = o / (1.0 + np.exp(-np.asarray(gate[h], np.float64)))
    return out
