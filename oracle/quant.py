"""Affine group quantisation, packed expert records and blob addressing (oracle).

Test infrastructure only; see the package docstring.

Pages: the experts are repacked into a .qpack container as blobs at a fixed
stride, so fetching expert i is one read of expertSize bytes at
blobBase + i * expertStride with no index hops (paotong.dev commentary,
paragraph on the fetch path; cheshm.ai article, paragraph on how it works).
The weights use MLX-style int4/int8 group quantisation and the kernels use
64-bit byte offsets for GB-sized files (cheshm.ai article, paragraph on the
code base). The pages do not print the grid, so this module takes the plain
reading: per group of 64 consecutive input-dimension weights, bias = the
group minimum and scale = range / (2^bits - 1), both stored as fp16, codes
unsigned, every rounding to nearest with ties to even, and the codes computed
from the already-rounded scale and bias.

Record layout (both packers are written from this description):
  gate codes [I][H], up codes [I][H]   row-major;
  down codes [I*bits/128][H][16 bytes]: row n of the down matrix [H][I] is cut
      into 16-byte tiles (32 int4 / 16 int8 codes) and tile t of every row
      comes before tile t+1 of any row (so one I-slice of the whole matrix is
      contiguous);
      in a row or tile, int4 element k sits in byte k>>1, even k in the low
      nibble; int8: one unsigned byte per element;
  gate (s,c) [I][H/64][2], up (s,c) [I][H/64][2]  fp16, row-major;
  down (s,c) [I/64][H][2]  fp16, group-major;
  zero bytes up to the stride, stride = round_up(record bytes, 4096).
"""
from __future__ import annotations

from fractions import Fraction
from typing import NamedTuple, Tuple

import numpy as np

GROUP = 64
STRIDE_ALIGN = 4096


# ---------------------------------------------------------------- rounding ---

def fp16_rne(a) -> np.ndarray:
    """Round fp32/fp64 values to fp16, nearest with ties to even (numpy's cast)."""
    return np.asarray(a).astype(np.float16)


def bf16_rne_from_f64(a) -> np.ndarray:
    """Round float64 values directly (once) to the nearest bf16, ties to even.

    Returns the values as float64. bf16 keeps 8 significant bits: write
    a = m * 2^e with 0.5 <= |m| < 1, round m * 256 to an integer (np.rint is
    ties-to-even and m * 256 is exact), scale back. Magnitudes below the bf16
    normal range are rounded on the subnormal grid of spacing 2^-133.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    e = np.maximum(e, -125)            # below bf16's normal range: fixed grid 2^-133
    r = np.ldexp(np.rint(np.ldexp(a, 8 - e)), e - 8)
    big = np.abs(r) >= np.ldexp(1.0, 128)
    return np.where(big, np.copysign(np.inf, a), r)


def f64_from_bf16_bits(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp32_round_exact(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32, ties to even (finite range)."""
    f = np.float32(float(fr))
    best, best_err = None, None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - fr)
        if best is None or err < best_err or (
                err == best_err and (int(np.float32(cand).view(np.uint32)) & 1) == 0):
            best, best_err = cand, err
    return np.float32(best)


# ----------------------------------------------------------------- sizing ---

def record_bytes(hidden: int, inter: int, bits: int) -> int:
    """Packed bytes of one expert: 3 code matrices plus fp16 (s,c) per 64-group."""
    codes = 3 * hidden * inter * bits // 8
    scales = 3 * (hidden * inter // GROUP) * 4
    return codes + scales


def record_stride(hidden: int, inter: int, bits: int) -> int:
    n = record_bytes(hidden, inter, bits)
    return (n + STRIDE_ALIGN - 1) // STRIDE_ALIGN * STRIDE_ALIGN


def blob_offset(base: int, gid: int, stride: int) -> int:
    """Byte offset of global expert ``gid`` (= layer * E + e): base + gid * stride.

    Python integers, so the value is exact beyond 2^32 (the 48-layer 80B blob
    is about 43.5 GB).
    """
    return int(base) + int(gid) * int(stride)


class RecordLayout(NamedTuple):
    gate_codes: int
    up_codes: int
    down_codes: int
    gate_sc: int
    up_sc: int
    down_sc: int
    end: int


def record_layout(hidden: int, inter: int, bits: int) -> RecordLayout:
    cgu = inter * hidden * bits // 8
    cd = hidden * inter * bits // 8
    sgu = inter * (hidden // GROUP) * 4
    sd = hidden * (inter // GROUP) * 4
    o = [0, cgu, 2 * cgu, 2 * cgu + cd, 2 * cgu + cd + sgu, 2 * cgu + cd + 2 * sgu]
    return RecordLayout(*o, 2 * cgu + cd + 2 * sgu + sd)


# ----------------------------------------------------------- quantisation ---

class QMatrix(NamedTuple):
    q: np.ndarray   # uint8 [N][K] codes in 0..2^bits-1
    s: np.ndarray   # float16 [N][K/64]
    c: np.ndarray   # float16 [N][K/64]


def quantize(w: np.ndarray, bits: int) -> QMatrix:
    """Affine min/max quantisation of an fp32 matrix [N][K] in groups of 64 along K.

    Per row n and group j (columns 64j..64j+63), all arithmetic in IEEE fp32:
      lo, hi = min, max of the group
      s = fp16(fl32(fl32(hi - lo) / (2^bits - 1)))      c = fp16(lo)   (a -0 minimum becomes +0)
      q_i = clamp(rne(fl32(fl32(w_i - c) / s)), 0, 2^bits - 1), and q_i = 0 when s == 0.
    Non-finite weights, or a scale or bias that overflows fp16, raise ValueError.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % GROUP:
        raise ValueError("expects [N][K] with K a multiple of 64")
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    N, K = w.shape
    g = w.reshape(N, K // GROUP, GROUP)
    lo = g.min(axis=2) + np.float32(0)     # a -0 minimum is stored as +0
    hi = g.max(axis=2)
    qmax = np.float32((1 << bits) - 1)
    with np.errstate(over="ignore"):
        s16 = fp16_rne((hi - lo) / qmax)
        c16 = fp16_rne(lo)
    if not (np.all(np.isfinite(s16)) and np.all(np.isfinite(c16))):
        raise ValueError("group scale or bias overflows fp16")
    sf = s16.astype(np.float32)[..., None]
    cf = c16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g - cf) / sf
    q = np.clip(np.rint(t), 0, qmax)
    q = np.where(sf == 0, np.float32(0), q)
    return QMatrix(q.reshape(N, K).astype(np.uint8), s16, c16)


def dequantize(m: QMatrix) -> np.ndarray:
    """W_hat = s * q + c per group, in float64 (exact: s, c are fp16 and q has <= 8 bits)."""
    N, K = m.q.shape
    s = np.repeat(m.s.astype(np.float64), GROUP, axis=1)
    c = np.repeat(m.c.astype(np.float64), GROUP, axis=1)
    return s * m.q.astype(np.float64) + c


def encode_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Row-major code bytes; int4 puts even elements in the low nibble."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    if bits == 8:
        return q.reshape(-1).copy()
    lo = q[:, 0::2]
    hi = q[:, 1::2]
    return (lo | (hi << 4)).astype(np.uint8).reshape(-1)


def decode_codes(b: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    if bits == 8:
        return b[: rows * cols].reshape(rows, cols).copy()
    b = b[: rows * cols // 2].reshape(rows, cols // 2)
    q = np.empty((rows, cols), dtype=np.uint8)
    q[:, 0::2] = b & 0x0F
    q[:, 1::2] = b >> 4
    return q


def _sc_bytes(m: QMatrix) -> np.ndarray:
    N, G = m.s.shape
    sc = np.empty((N, G, 2), dtype=np.float16)
    sc[:, :, 0] = m.s
    sc[:, :, 1] = m.c
    return sc.reshape(-1).view(np.uint8)


def _sc_from_bytes(b: np.ndarray, rows: int, groups: int) -> Tuple[np.ndarray, np.ndarray]:
    sc = np.ascontiguousarray(b[: rows * groups * 4]).view(np.float16).reshape(rows, groups, 2)
    return sc[:, :, 0].copy(), sc[:, :, 1].copy()


TILE = 16  # bytes of a down-matrix tile


def tile_rows(b: np.ndarray, rows: int) -> np.ndarray:
    """Row-major bytes [rows][row_bytes] -> [row_bytes/16][rows][16]."""
    b = np.asarray(b, dtype=np.uint8).reshape(rows, -1, TILE)
    return np.ascontiguousarray(b.transpose(1, 0, 2)).reshape(-1)


def untile_rows(b: np.ndarray, rows: int, row_bytes: int) -> np.ndarray:
    """Inverse of tile_rows."""
    b = np.asarray(b, dtype=np.uint8)[: rows * row_bytes].reshape(row_bytes // TILE, rows, TILE)
    return np.ascontiguousarray(b.transpose(1, 0, 2)).reshape(-1)


def _sc_bytes_group_major(m: QMatrix) -> np.ndarray:
    N, G = m.s.shape
    sc = np.empty((G, N, 2), dtype=np.float16)
    sc[:, :, 0] = m.s.T
    sc[:, :, 1] = m.c.T
    return sc.reshape(-1).view(np.uint8)


def _sc_from_bytes_group_major(b: np.ndarray, rows: int, groups: int) -> Tuple[np.ndarray, np.ndarray]:
    sc = np.ascontiguousarray(b[: rows * groups * 4]).view(np.float16).reshape(groups, rows, 2)
    return sc[:, :, 0].T.copy(), sc[:, :, 1].T.copy()


class Expert(NamedTuple):
    gate: QMatrix   # [I][H]
    up: QMatrix     # [I][H]
    down: QMatrix   # [H][I]


def quantize_expert(wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, bits: int) -> Expert:
    return Expert(quantize(wg, bits), quantize(wu, bits), quantize(wd, bits))


def pack_record(e: Expert, bits: int, pad_to_stride: bool = True) -> np.ndarray:
    """Serialise one quantised expert into its record bytes (uint8)."""
    I, H = e.gate.q.shape
    lay = record_layout(H, I, bits)
    n = record_stride(H, I, bits) if pad_to_stride else lay.end
    out = np.zeros(n, dtype=np.uint8)
    out[lay.gate_codes:lay.up_codes] = encode_codes(e.gate.q, bits)
    out[lay.up_codes:lay.down_codes] = encode_codes(e.up.q, bits)
    out[lay.down_codes:lay.gate_sc] = tile_rows(encode_codes(e.down.q, bits), H)
    out[lay.gate_sc:lay.up_sc] = _sc_bytes(e.gate)
    out[lay.up_sc:lay.down_sc] = _sc_bytes(e.up)
    out[lay.down_sc:lay.end] = _sc_bytes_group_major(e.down)
    return out


def unpack_record(rec: np.ndarray, hidden: int, inter: int, bits: int) -> Expert:
    rec = np.asarray(rec, dtype=np.uint8)
    lay = record_layout(hidden, inter, bits)
    H, I = hidden, inter
    gq = decode_codes(rec[lay.gate_codes:lay.up_codes], I, H, bits)
    uq = decode_codes(rec[lay.up_codes:lay.down_codes], I, H, bits)
    dq = decode_codes(untile_rows(rec[lay.down_codes:lay.gate_sc], H, I * bits // 8), H, I, bits)
    gs, gc = _sc_from_bytes(rec[lay.gate_sc:lay.up_sc], I, H // GROUP)
    us, uc = _sc_from_bytes(rec[lay.up_sc:lay.down_sc], I, H // GROUP)
    ds, dc = _sc_from_bytes_group_major(rec[lay.down_sc:lay.end], H, I // GROUP)
    return Expert(QMatrix(gq, gs, gc), QMatrix(uq, us, uc), QMatrix(dq, ds, dc))


def pack_blob(experts, bits: int) -> np.ndarray:
    """Records of ``experts`` (a list of Expert) one after another at the fixed stride."""
    recs = [pack_record(e, bits) for e in experts]
    return np.concatenate(recs) if recs else np.zeros(0, dtype=np.uint8)
