"""Gated DeltaNet decode step (oracle). Test infrastructure only; see the
package docstring.

Pages: 36 of the 80B model's 48 layers are DeltaNet layers, whose recurrent
state has a fixed size, about 72 MiB over those layers, while only the 12
full-attention layers keep a growing KV cache (alphalab.site field test,
section explaining MoE expert streaming); the architecture is a hybrid of
linear attention (Gated DeltaNet) and gated attention with a sparse MoE
(cheshm.ai article, paragraph on the code base).

The pages print no formula. Reading taken: the gated delta rule as published
(Yang, Kautz and Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with
Delta Rule", 2024), in the decode form of the Qwen3-Next linear-attention
layer, one token at a time, per value head h with key head h // (Hv / Hk):

  conv      y_c = silu(sum_{j<4} w[c, j] * x_c(t - 3 + j)) over the q, k, v
            channels (a depthwise causal convolution, inputs before the first
            token are 0)
  norms     q = q / sqrt(|q|^2 + 1e-6) / sqrt(d_k),  k = k / sqrt(|k|^2 + 1e-6)
  gates     alpha = exp(-exp(A_log[h]) * softplus(a[h] + dt_bias[h])),
            beta = sigmoid(b[h])
  state     S <- alpha * S;  u = beta * (v - S^T k);  S <- S + k u^T
            (S is [d_k][d_v]); o = S^T q
  output    out = o / sqrt(mean(o^2) + 1e-6) * w_norm * silu(z)

State bytes: Hv * d_k * d_v * 4 per layer; with the Qwen3-Next-80B shape
(32 value heads, 16 key heads, d_k = d_v = 128) that is 2 MiB, and 36 layers
hold exactly 72 MiB, the pages' figure.
"""
from __future__ import annotations

from typing import NamedTuple

import numpy as np

CONV_K = 4
EPS_L2 = 1e-6
EPS_NORM = 1e-6


class Shape(NamedTuple):
    n_k: int     # key (and query) heads
    n_v: int     # value heads
    d_k: int
    d_v: int

    @property
    def channels(self) -> int:
        """Convolution channels: q and k (n_k * d_k each), then v (n_v * d_v)."""
        return 2 * self.n_k * self.d_k + self.n_v * self.d_v

    def state_bytes(self) -> int:
        """fp32 recurrent state of one layer."""
        return self.n_v * self.d_k * self.d_v * 4


class Params(NamedTuple):
    conv_w: np.ndarray   # [C][4]
    a_log: np.ndarray    # [n_v]
    dt_bias: np.ndarray  # [n_v]
    norm_w: np.ndarray   # [d_v]


class State(NamedTuple):
    s: np.ndarray        # float64 [n_v][d_k][d_v]
    window: np.ndarray   # float64 [C][3]: the last three conv inputs, oldest first


def zero_state(sh: Shape) -> State:
    return State(np.zeros((sh.n_v, sh.d_k, sh.d_v)), np.zeros((sh.channels, CONV_K - 1)))


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def softplus(z):
    z = np.asarray(z, dtype=np.float64)
    return np.log1p(np.exp(-np.abs(z))) + np.maximum(z, 0.0)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def conv_step(window: np.ndarray, x: np.ndarray, w: np.ndarray):
    """One causal depthwise convolution step with SiLU: returns (y, new window)."""
    full = np.concatenate([window, x[:, None]], axis=1)       # x(t-3) .. x(t)
    y = silu(np.sum(full * np.asarray(w, dtype=np.float64), axis=1))
    return y, full[:, 1:]


def l2norm(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS_L2)


def delta_rule(s: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: float, beta: float):
    """One head: decay, delta-rule write of v at key k, read at q. s [d_k][d_v]."""
    s = alpha * s
    u = beta * (v - s.T @ k)
    s = s + np.outer(k, u)
    return s, s.T @ q


def gated_rmsnorm(o: np.ndarray, z: np.ndarray, w: np.ndarray) -> np.ndarray:
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + EPS_NORM)
    return o / rms * np.asarray(w, dtype=np.float64) * silu(z)


def layer_step(sh: Shape, p: Params, st: State, qkv: np.ndarray, z: np.ndarray, a: np.ndarray, b: np.ndarray):
    """One token through one layer. qkv [C], z [n_v * d_v], a and b [n_v]
    (float64 holding the bf16 inputs). Returns (out [n_v][d_v], new State)."""
    y, window = conv_step(st.window, np.asarray(qkv, dtype=np.float64), p.conv_w)
    nq = sh.n_k * sh.d_k
    q = l2norm(y[:nq].reshape(sh.n_k, sh.d_k)) / np.sqrt(sh.d_k)
    k = l2norm(y[nq:2 * nq].reshape(sh.n_k, sh.d_k))
    v = y[2 * nq:].reshape(sh.n_v, sh.d_v)
    alpha = np.exp(-np.exp(np.asarray(p.a_log, np.float64)) * softplus(np.asarray(a, np.float64) + p.dt_bias))
    beta = sigmoid(b)
    rep = sh.n_v // sh.n_k
    s_new = np.empty_like(st.s)
    o = np.empty((sh.n_v, sh.d_v))
    for h in range(sh.n_v):
        s_new[h], o[h] = delta_rule(st.s[h], q[h // rep], k[h // rep], v[h], alpha[h], beta[h])
    out = gated_rmsnorm(o, np.asarray(z, np.float64).reshape(sh.n_v, sh.d_v), p.norm_w)
    return out, State(s_new, window)


def run(sh: Shape, p: Params, qkv: np.ndarray, z: np.ndarray, a: np.ndarray, b: np.ndarray, st: State = None):
    """Tokens one after another from `st` (zero state by default): outputs [T][n_v][d_v] and the final state."""
    st = zero_state(sh) if st is None else st
    outs = []
    for t in range(qkv.shape[0]):
        o, st = layer_step(sh, p, st, qkv[t], z[t], a[t], b[t])
        outs.append(o)
    return np.stack(outs), st
