// Gated grouped-query attention decode step with an fp16 KV cache, for gfx950:
// the full-attention layers beside the routed MoE (12 of the 80B model's 48).
//
// Pages: those layers are the only ones with a growing K/V cache, budgeted at
// 24 KiB per token in fp16 (alphalab.site field test, section explaining MoE
// expert streaming); the model pairs linear attention with gated attention
// (cheshm.ai article, paragraph on the code base). The pages print no
// formula; the step is the decode form of the Qwen3-Next gated attention
// layer: per-head RMS norms of q and k, rotary embedding of the first `rot`
// dims (pairs (i, i + rot/2), angle p * 1e7^(-2i/rot), the angle in fp64), the
// new K/V row stored in fp16, softmax attention of each query head over its KV
// group's cached rows, and the sigmoid output gate.
//
// Per step (token, layer), bound by reading the cache (2 * d * 2 bytes per
// cached position and KV group):
// - prep: the G query rows of each KV group normed, rotated, scaled by
//   1 / sqrt(d) and split into fp16 hi + lo (the MFMA operand, in a scratch
//   buffer), and the new K/V row normed, rotated, rounded to fp16 and written
//   into the cache. A call's first step runs it as a kernel of its own; every
//   later step's prep rides in the previous step's merge kernel (its inputs
//   are all given up front), so it costs no launch.
// - partials: a block of four waves per (KV group, 128 positions); each wave
//   loads the q operand, the K rows and V columns of its 32 positions straight
//   into MFMA operand registers, 16 bytes per load, and contracts them on
//   v_mfma_f32_16x16x32_f16: scores S[j][h] = K[j] . q_h, then
//   O[d][h] = sum_j V[j][d] P[h][j]. The G heads sharing one KV group make
//   this a real contraction (8 heads per group at the 80B shape): on the
//   vector ALU it would take 8 fp32 FMAs per cached byte. q and the softmax
//   weights P ride as fp16 hi + lo pairs (two MFMAs each), so scores and
//   weighted sums keep close to fp32 accuracy. The four waves merge their
//   softmax partials (max, sum of exp, weighted sum of V) in LDS and the block
//   writes one set.
// - merge: per query head, the blocks' partials folded with a running max,
//   times sigmoid(gate); plus the next step's prep.
//
// Cache layout: K [n_kv][max_pos][d] (a position's row contiguous, as the
// score contracts over d); V in tiles of 32 positions, [n_kv][span][d][32] (a
// dim's 32 positions contiguous, as the weighted sum contracts over
// positions, and a span's tile one contiguous 16 KiB at d = 256).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "common.h"
#include "dpp.h"
#include "launch.h"
#include "moe.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kSpan = 32;                   // positions per wave of the partials kernel
constexpr int kWaves = 4;                   // waves per block of the partials kernel
constexpr int kBlockPos = kSpan * kWaves;   // positions per block
constexpr int kCombineDims = 16;            // merge kernel: dims per block
constexpr int kCombineGroups = 16;          // merge kernel: groups of partials per block
constexpr int kPrepThreads = 256;           // prep: one thread per dim (head_dim <= 256)
static_assert(kCombineDims * kCombineGroups == kPrepThreads, "the merge kernel's blocks run the prep");

__device__ __forceinline__ float bfv(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

struct AttnLayer {
  const float* wq;  // [d] q norm weight
  const float* wk;  // [d] k norm weight
  uint16_t* kc;     // [n_kv][max_pos][d] fp16
  uint16_t* vt;     // [n_kv][n_spans][d][32] fp16
};

struct AttnIo {
  const uint16_t* q;     // [n_q][d] bf16
  const uint16_t* gate;  // [n_q][d]
  const uint16_t* k;     // [n_kv][d]
  const uint16_t* v;     // [n_kv][d]
  float* out;            // [n_q][d]
};

struct AttnShape {
  const double* freq;  // [d]: rotation frequency of each dim, 0 past rot
  int n_kv, max_pos, n_spans, rot;
};

struct AttnWork {
  float* ml;       // [n_kv][max_split][G][2]: max, sum of exp
  float* o;        // [n_kv][max_split][G][d]
  _Float16* qop;   // [n_q][2][d]: prepared q, hi then lo
  int max_split;   // blocks of the partials kernel per KV group at full capacity
};

struct AttnStep {  // one (token, layer) step: its layer, inputs, position
  AttnLayer L;
  AttnIo io;
  int pos;
};

// Rotation of dim d of a normed row in LDS: pairs (i, i + rot/2).
__device__ __forceinline__ float rotated(const float* row, int d, int rot, float cs, float sn) {
  const int half = rot / 2;
  if (d < half) return row[d] * cs - row[d + half] * sn;
  if (d < rot) return row[d] * cs + row[d - half] * sn;
  return row[d];
}

// Prep of one row of a step by a block of kPrepThreads threads (thread = dim):
// row < n_q is query head `row`; row = n_q + g is KV group g's new K/V row.
// The angle: pos * freq in fp64, reduced to [-pi, pi] in fp64, then sin and
// cos in fp32 of the reduced angle split into hi + lo (a first-order
// correction for lo). Every load is unconditional, at an in-range address.
template <int D, int G>
__device__ void prep_row(const AttnShape& S, const AttnStep& st, const AttnWork& W, int row, float* s_row,
                         float* s_red) {
  const int n_q = S.n_kv * G, t = threadIdx.x;
  const bool isq = row < n_q;
  const int g = isq ? row / G : row - n_q;
  const int d = t < D ? t : D - 1;
  const uint16_t* src = isq ? st.io.q + (size_t)row * D : st.io.k + (size_t)g * D;
  const float x = t < D ? bfv(src[d]) : 0.f;
  const float w = (isq ? st.L.wq : st.L.wk)[d];
  const float vv = bfv(st.io.v[(size_t)g * D + d]);
  float cs = 1.f, sn = 0.f;
  if (d < S.rot) {
    const double ang = (double)st.pos * S.freq[d];
    const double turns = rint(ang * 0.15915494309189535);        // 1 / (2 pi)
    double red = fma(-turns, 6.283185307179586, ang);             // 2 pi, high part
    red = fma(-turns, 2.4492935982947064e-16, red);               // 2 pi - high part
    const float hi = (float)red, lo = (float)(red - (double)hi);  // red = hi + lo
    float sh, ch;
    sincosf(hi, &sh, &ch);
    sn = fmaf(ch, lo, sh);   // sin(hi + lo), |lo| < 2^-22
    cs = fmaf(-sh, lo, ch);
  }
  const float ss = dpp::wave_sum(x * x);
  if ((t & 63) == 0) s_red[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kPrepThreads / 64; ++i) tot += s_red[i];
  const float inv = 1.0f / sqrtf(tot / (float)D + 1e-6f);
  if (t < D) s_row[t] = x * inv * w;
  __syncthreads();
  if (t < D) {
    const float y = rotated(s_row, t, S.rot, cs, sn);
    if (isq) {
      const float yq = y * (1.0f / sqrtf((float)D));
      const _Float16 h = (_Float16)yq;
      W.qop[(size_t)row * 2 * D + t] = h;
      W.qop[(size_t)row * 2 * D + D + t] = (_Float16)(yq - (float)h);
    } else {
      st.L.kc[((size_t)g * S.max_pos + st.pos) * D + t] = f2h(y);
      st.L.vt[(((size_t)g * S.n_spans + st.pos / kSpan) * D + t) * kSpan + st.pos % kSpan] = f2h(vv);
    }
  }
  __syncthreads();  // s_row and s_red are reused
}

// A call's first step: block b < n_q + n_kv preps row b.
template <int D, int G>
__global__ void __launch_bounds__(kPrepThreads) attn_prep_kernel(AttnShape S, AttnStep st, AttnWork W) {
  __shared__ float s_row[D];
  __shared__ float s_red[kPrepThreads / 64];
  prep_row<D, G>(S, st, W, blockIdx.x, s_row, s_red);
}

// LDS of the partials kernel: first the KV group's q operand, G rows of hi
// and lo (2 D fp16 + 32 of padding, so consecutive heads' rows start 16 banks
// apart), then, once every wave is past its MFMAs, the waves' scaled weighted
// sums, rows of D + 16 floats (the same purpose).
template <int D>
constexpr int q_pitch() {
  return 2 * D + 32;
}
template <int D, int G>
constexpr size_t lds_bytes() {
  constexpr size_t q = (size_t)G * q_pitch<D>() * 2, o = (size_t)kWaves * G * (D + 16) * 4;
  return q > o ? q : o;
}

// Block barrier that waits for this wave's LDS accesses only (lgkmcnt(0);
// vmcnt and expcnt at their maximum), so global loads stay in flight across
// it; the compiler may not move memory accesses across it either.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Block (KV group g = blockIdx.x % n_kv, positions [b0, b0 + 128), b0 = 128 *
// (blockIdx.x / n_kv)); wave w takes positions [j0, j0 + 32), j0 = b0 + 32 w,
// and is live when j0 <= pos. Position pos (this step's) is in the cache.
//
// MFMA 16x16x32 operand map (lane = r + 16 * gq, r < 16, gq < 4): A supplies
// row r, B column r, each 8 consecutive k-values of the lane's group gq; C
// gives lane rows 4 * gq + i (i < 4) of column r. Which k-values a group's 8
// slots stand for is free as long as A and B agree, so:
// - scores, C = S[j][h]: row r of tile t is position j0 + 8 * (r / 4) + 4 * t
//   + r % 4, so that C lane (r, gq) holds head r at positions j0 + 8 * gq +
//   e (e = 4 t + i < 8); k-slots of step s are dims 32 s + 8 gq + [0, 8);
// - weighted sums, C = O[d][h], tile n covers dims 16 n + [0, 16); k-slots are
//   positions j0 + 8 gq + [0, 8): A is 16 contiguous bytes of the V tile row
//   of dim 16 n + r, B the lane's own 8 weights of head r.
template <int D, int G>
__global__ void __launch_bounds__(64 * kWaves) attn_split_kernel(AttnLayer L, AttnWork W, AttnShape S, int pos) {
  static_assert(D % 64 == 0 && D <= 256 && G <= 16, "shape");
  constexpr int NS = D / 32;   // score k-steps
  constexpr int NT = D / 16;   // weighted-sum tiles
  constexpr int OP = D + 16;   // LDS row pitch of the merge, floats
  constexpr int QP = q_pitch<D>();
  extern __shared__ __align__(16) float s_o[];   // [kWaves][G][OP], after the MFMAs
  _Float16* s_q = reinterpret_cast<_Float16*>(s_o);   // [G][QP]: hi [D], lo [D]
  __shared__ float s_ml[kWaves * G * 2];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, gq = lane >> 4;
  const int g = blockIdx.x % S.n_kv, blk = blockIdx.x / S.n_kv;
  const int j0 = blk * kBlockPos + kSpan * w;
  const bool live = j0 <= pos;                  // wave-uniform
  const bool mine = live && pos < j0 + kSpan;   // this wave's span holds pos

  // 1. loads, every one unconditional at an in-range address: the group's q
  //    operand (8 KiB at the 80B shape, shared by the block: 16 bytes per
  //    thread per round), the K rows (rows past pos read row pos), the V tile
  //    (a wave past pos reads its own tile, in range as n_spans covers whole
  //    blocks, and uses none of it)
  constexpr int QCH = G * D / 4;                         // 16-byte chunks of the q operand
  constexpr int QR = (QCH + 64 * kWaves - 1) / (64 * kWaves);
  const _Float16* qsrc = W.qop + (size_t)g * G * 2 * D;
  uint4 qv[QR];
#pragma unroll
  for (int u = 0; u < QR; ++u)
    qv[u] = *reinterpret_cast<const uint4*>(qsrc + 8 * (size_t)min(tid + 64 * kWaves * u, QCH - 1));
  uint4 ka[2][NS], va[NT];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int p = min(j0 + 8 * (r >> 2) + 4 * t + (r & 3), pos);
    const uint16_t* row = L.kc + ((size_t)g * S.max_pos + p) * D + 8 * gq;
#pragma unroll
    for (int s = 0; s < NS; ++s) ka[t][s] = *reinterpret_cast<const uint4*>(row + 32 * s);
  }
  const uint16_t* tile = L.vt + ((size_t)g * S.n_spans + j0 / kSpan) * D * kSpan;
#pragma unroll
  for (int n = 0; n < NT; ++n) va[n] = *reinterpret_cast<const uint4*>(tile + (16 * n + r) * kSpan + 8 * gq);

  // the q operand to LDS (its loads came first, so waiting for them leaves
  // the cache loads in flight), then column r's operand (columns r >= G read
  // row G - 1, then zero)
#pragma unroll
  for (int u = 0; u < QR; ++u) {
    const int idx = tid + 64 * kWaves * u;
    if (idx < QCH) *reinterpret_cast<uint4*>(s_q + (idx / (D / 4)) * QP + 8 * (idx % (D / 4))) = qv[u];
  }
  lds_barrier();
  f16x8 bh[NS], bl[NS];
  {
    const _Float16* qrow = s_q + min(r, G - 1) * QP + 8 * gq;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bh[s] = *reinterpret_cast<const f16x8*>(qrow + 32 * s);
      bl[s] = *reinterpret_cast<const f16x8*>(qrow + D + 32 * s);
    }
  }

  float m = -INFINITY, l = 0.f;
  f32x4 o[NT];
  if (live) {
    if (r >= G) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        bh[s] = f16x8{};
        bl[s] = f16x8{};
      }
    }
    if (mine) {
      // V slots past pos may hold anything (a stale inf would poison 0 * v):
      // the lane's slots e > pos - (j0 + 8 gq) are zeroed, per dword
      const int e_last = pos - (j0 + 8 * gq);
      uint32_t keep[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) keep[q] = (2 * q <= e_last ? 0xFFFFu : 0u) | (2 * q + 1 <= e_last ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int n = 0; n < NT; ++n) va[n] = make_uint4(va[n].x & keep[0], va[n].y & keep[1], va[n].z & keep[2],
                                                      va[n].w & keep[3]);
    }
    // 2. scores S[j][h] = K[j] . q_h (q as hi + lo)
    f32x4 sc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f16x8 a = __builtin_bit_cast(f16x8, ka[t][s]);
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh[s], sc[t], 0, 0, 0);
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl[s], sc[t], 0, 0, 0);
      }
    // 3. softmax partials of head r over the span: lane (r, gq) holds
    //    positions j0 + 8 gq + e, e = 4 t + i; positions past pos are masked
    float sv[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * t + i;
        sv[e] = j0 + 8 * gq + e <= pos ? sc[t][i] : -INFINITY;
      }
    m = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) m = fmaxf(m, sv[e]);
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));  // finite: position j0 is live
    f16x8 ph, pl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = expf(sv[e] - m);
      const _Float16 hi = (_Float16)p;
      ph[e] = hi;
      pl[e] = (_Float16)(p - (float)hi);
      l += p;
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (r >= G) {
      ph = f16x8{};
      pl = f16x8{};
    }
    // 4. weighted sums O[d][h] = sum_j V[j][d] P[h][j]
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const f16x8 a = __builtin_bit_cast(f16x8, va[n]);
      o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ph, o[n], 0, 0, 0);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pl, o[n], 0, 0, 0);
    }
  }

  // 5. merge of the four waves: each scales its sums by exp(m_w - M), the
  //    block sums them; a wave with no live position (m = -inf) adds nothing
  //    (its rows zero; the LDS holding the q operand is free once every
  //    wave is past the first barrier below)
  if (lane < G) {
    s_ml[(w * G + lane) * 2] = m;
    s_ml[(w * G + lane) * 2 + 1] = l;
  }
  __syncthreads();
  if (r < G) {
    float M = s_ml[r * 2];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) M = fmaxf(M, s_ml[(v * G + r) * 2]);
    float* row = s_o + ((size_t)w * G + r) * OP + 4 * gq;
    if (live) {
      const float f = expf(m - M);
#pragma unroll
      for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(row + 16 * n) = o[n] * f;
    } else {
#pragma unroll
      for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(row + 16 * n) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __syncthreads();
  const size_t part = ((size_t)g * W.max_split + blk) * G;
  for (int idx = tid; idx < G * D / 4; idx += 64 * kWaves) {
    const int h = idx * 4 / D, d = idx * 4 % D;
    f32x4 acc = *reinterpret_cast<const f32x4*>(s_o + (size_t)h * OP + d);
#pragma unroll
    for (int v = 1; v < kWaves; ++v) acc += *reinterpret_cast<const f32x4*>(s_o + ((size_t)v * G + h) * OP + d);
    *reinterpret_cast<f32x4*>(W.o + (part + h) * D + d) = acc;
  }
  if (tid < G) {
    float M = s_ml[tid * 2];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) M = fmaxf(M, s_ml[(v * G + tid) * 2]);
    float Ls = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float mv = s_ml[(v * G + tid) * 2];
      if (mv != -INFINITY) Ls = fmaf(s_ml[(v * G + tid) * 2 + 1], expf(mv - M), Ls);
    }
    W.ml[(part + tid) * 2] = M;
    W.ml[(part + tid) * 2 + 1] = Ls;
  }
}

// Block (query head hq, 16 dims), 256 threads = 16 groups of partials x 16
// dims. Each thread folds its partials eight at a time (loads issued
// together; one rescale of its running sums per batch), the groups' sums are
// scaled to the block's max and added through LDS, then out = o / l *
// sigmoid(gate). With has_next, blocks b < n_q + n_kv then prep row b of the
// next step.
template <int D, int G>
__global__ void __launch_bounds__(kPrepThreads) attn_combine_kernel(AttnIo io, AttnWork W, int n_split, AttnShape S,
                                                                    AttnStep next, int has_next) {
  constexpr int B = 8;  // partials per batch
  __shared__ float s_m[kCombineGroups][kCombineDims], s_l[kCombineGroups][kCombineDims],
      s_o[kCombineGroups][kCombineDims];
  __shared__ float s_row[D];
  __shared__ float s_red[kPrepThreads / 64];
  constexpr int PH = D / kCombineDims;
  const int hq = blockIdx.x / PH, d0 = (blockIdx.x % PH) * kCombineDims;
  const int g = hq / G, h = hq % G;
  const int dl = threadIdx.x % kCombineDims, grp = threadIdx.x / kCombineDims, d = d0 + dl;
  float M = -INFINITY, l = 0.f, o = 0.f;
  for (int s0 = grp; s0 < n_split; s0 += B * kCombineGroups) {
    float ms[B], ls[B], os[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      // partials past the last are read at the last one's address (no branch
      // around the loads) and marked empty: max -inf, weight exp(-inf) = 0
      const int s = s0 + u * kCombineGroups;
      const size_t part = ((size_t)g * W.max_split + min(s, n_split - 1)) * G + h;
      ms[u] = W.ml[part * 2];
      ls[u] = W.ml[part * 2 + 1];
      os[u] = W.o[part * D + d];
      if (s >= n_split) ms[u] = -INFINITY;
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < B; ++u) Mb = fmaxf(Mb, ms[u]);   // finite: s0 < n_split
    const float a = expf(M - Mb);
    l *= a;
    o *= a;
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const float b = expf(ms[u] - Mb);
      l = fmaf(ls[u], b, l);
      o = fmaf(os[u], b, o);
    }
    M = Mb;
  }
  s_m[grp][dl] = M;
  __syncthreads();
  float Mt = s_m[0][dl];
#pragma unroll
  for (int q = 1; q < kCombineGroups; ++q) Mt = fmaxf(Mt, s_m[q][dl]);   // finite: split 0 exists
  const float f = expf(M - Mt);   // 0 for a group with no partials
  s_l[grp][dl] = l * f;
  s_o[grp][dl] = o * f;
  __syncthreads();
  if (grp == 0) {
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int q = 0; q < kCombineGroups; ++q) {
      lt += s_l[q][dl];
      ot += s_o[q][dl];
    }
    const float gt = bfv(io.gate[(size_t)hq * D + d]);
    io.out[(size_t)hq * D + d] = ot / lt / (1.0f + expf(-gt));
  }
  if (has_next && (int)blockIdx.x < S.n_kv * G + S.n_kv) prep_row<D, G>(S, next, W, blockIdx.x, s_row, s_red);
}

struct AttnGraph {
  int layer0, n_layers, n_tok, pos0;
  const void* q;
  const void* gate;
  const void* k;
  const void* v;
  void* out;
  hipGraphExec_t exec;
  hipEvent_t done;
  uint64_t stamp;
};

}  // namespace
}  // namespace moe

using namespace moe;

struct moe_attn {
  moe_attn_config cfg{};
  int n_spans = 0;         // 32-position V tiles per KV group (a multiple of 4)
  float* norms = nullptr;  // [L][2][d]: q norm weight, k norm weight
  double* freq = nullptr;  // [d]: 1e7^(-2i/rot) for dims i and i + rot/2, 0 past rot
  uint16_t* kc = nullptr;  // [L][n_kv][max_pos][d]
  uint16_t* vt = nullptr;  // [L][n_kv][n_spans][d][32]
  AttnWork work{};
  std::vector<uint8_t> set;
  std::vector<AttnGraph> graphs;
  hipStream_t cap_stream = nullptr;
  uint64_t clock = 0;
  bool prof = false;  // time every launch (graphs bypassed)
  std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_split, prof_combine;
};

namespace {

std::mutex g_attn_mu;
std::set<const moe_attn*> g_attn_live;

moe_status attn_check(const moe_attn* a, const char* fn) {
  if (!a) return fail(MOE_EINVAL, std::string(fn) + ": handle is NULL");
  std::lock_guard<std::mutex> l(g_attn_mu);
  if (!g_attn_live.count(a)) return fail(MOE_ESTATE, std::string(fn) + ": not a live attention handle");
  return MOE_OK;
}

std::string attn_config_error(const moe_attn_config* c) {
  if (!c) return "config is NULL";
  if (c->n_layers < 1 || c->n_layers > 4096) return "n_layers must be in [1, 4096]";
  if (c->n_kv_heads < 1 || c->n_kv_heads > 256 || c->n_q_heads < c->n_kv_heads || c->n_q_heads % c->n_kv_heads)
    return "n_q_heads must be a positive multiple of n_kv_heads (n_kv_heads <= 256)";
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return "n_q_heads / n_kv_heads must be 1, 2, 4, 8 or 16";
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return "head_dim must be 64, 128 or 256";
  if (c->rot_dim < 0 || c->rot_dim > c->head_dim || c->rot_dim % 2) return "rot_dim must be even and <= head_dim";
  if (c->max_pos < 1 || c->max_pos > (1 << 20)) return "max_pos must be in [1, 2^20]";
  return "";
}

void record(moe_attn* a, std::vector<std::pair<hipEvent_t, hipEvent_t>>& into) {
  if (!a->prof) return;
  LaunchEvents ev{};
  if (hipEventCreate(&ev.start) != hipSuccess) return;
  if (hipEventCreate(&ev.stop) != hipSuccess) {
    hipEventDestroy(ev.start);
    return;
  }
  launch_events() = ev;
  into.emplace_back(ev.start, ev.stop);
}

AttnLayer layer_args(moe_attn* a, int layer) {
  const size_t D = a->cfg.head_dim, KV = a->cfg.n_kv_heads;
  const float* w = a->norms + (size_t)layer * 2 * D;
  return AttnLayer{w, w + D, a->kc + (size_t)layer * KV * a->cfg.max_pos * D,
                   a->vt + (size_t)layer * KV * a->n_spans * D * kSpan};
}

AttnShape shape_of(const moe_attn* a) {
  return AttnShape{a->freq, a->cfg.n_kv_heads, a->cfg.max_pos, a->n_spans, a->cfg.rot_dim};
}

// One call's steps in order: the first step's prep, then per step the
// partials kernel and the merge kernel (which also preps the next step).
template <int D, int G>
hipError_t launch_steps_dg(moe_attn* a, const std::vector<AttnStep>& steps, hipStream_t s) {
  constexpr size_t lds = lds_bytes<D, G>();
  static std::once_flag attr_once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(attr_once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_split_kernel<D, G>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  if (attr_err != hipSuccess) return attr_err;
  const AttnShape S = shape_of(a);
  const int n_q = a->cfg.n_q_heads, n_kv = a->cfg.n_kv_heads;
  launch(attn_prep_kernel<D, G>, dim3(n_q + n_kv), dim3(kPrepThreads), 0, s, S, steps[0], a->work);
  for (size_t i = 0; i < steps.size(); ++i) {
    const AttnStep& st = steps[i];
    const int n_split = st.pos / kBlockPos + 1;
    const bool has_next = i + 1 < steps.size();
    record(a, a->prof_split);
    launch(attn_split_kernel<D, G>, dim3(n_kv * n_split), dim3(64 * kWaves), (uint32_t)lds, s, st.L, a->work, S,
           st.pos);
    record(a, a->prof_combine);
    launch(attn_combine_kernel<D, G>, dim3(n_q * (D / kCombineDims)), dim3(kPrepThreads), 0, s, st.io, a->work,
           n_split, S, has_next ? steps[i + 1] : st, has_next ? 1 : 0);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_steps_d(moe_attn* a, const std::vector<AttnStep>& steps, hipStream_t s) {
  switch (a->cfg.n_q_heads / a->cfg.n_kv_heads) {
    case 1: return launch_steps_dg<D, 1>(a, steps, s);
    case 2: return launch_steps_dg<D, 2>(a, steps, s);
    case 4: return launch_steps_dg<D, 4>(a, steps, s);
    case 8: return launch_steps_dg<D, 8>(a, steps, s);
    default: return launch_steps_dg<D, 16>(a, steps, s);
  }
}

hipError_t launch_steps(moe_attn* a, const std::vector<AttnStep>& steps, hipStream_t s) {
  switch (a->cfg.head_dim) {
    case 64: return launch_steps_d<64>(a, steps, s);
    case 128: return launch_steps_d<128>(a, steps, s);
    default: return launch_steps_d<256>(a, steps, s);
  }
}

double drain(std::vector<std::pair<hipEvent_t, hipEvent_t>>& ev, uint64_t* n) {
  double ms = 0.0;
  for (auto& pr : ev) {
    float t = 0.f;
    if (hipEventSynchronize(pr.second) == hipSuccess && hipEventElapsedTime(&t, pr.first, pr.second) == hipSuccess) {
      ms += t;
      if (n) ++*n;
    }
    hipEventDestroy(pr.first);
    hipEventDestroy(pr.second);
  }
  ev.clear();
  return ms;
}

// Host-side access to positions [p0, p0 + n) of one KV group's V tiles: the
// spans covering them are copied out whole, edited or read, and (for a write)
// copied back.
hipError_t v_tiles(uint16_t* vt_group, size_t D, int p0, int n, uint16_t* v, bool write) {
  const int s0 = p0 / kSpan, s1 = (p0 + n - 1) / kSpan;
  const size_t tile = D * kSpan, count = (size_t)(s1 - s0 + 1) * tile;
  std::vector<uint16_t> buf(count);
  hipError_t e = hipMemcpy(buf.data(), vt_group + (size_t)s0 * tile, count * 2, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  for (int i = 0; i < n; ++i) {
    const int p = p0 + i;
    uint16_t* col = buf.data() + (size_t)(p / kSpan - s0) * tile + p % kSpan;
    for (size_t d = 0; d < D; ++d) {
      if (write) col[d * kSpan] = v[(size_t)i * D + d];
      else v[(size_t)i * D + d] = col[d * kSpan];
    }
  }
  if (!write) return hipSuccess;
  return hipMemcpy(vt_group + (size_t)s0 * tile, buf.data(), count * 2, hipMemcpyHostToDevice);
}

}  // namespace

extern "C" {

moe_status moe_attn_create(const moe_attn_config* cfg, moe_attn** out) {
  clear_error();
  if (!out) return fail(MOE_EINVAL, "moe_attn_create: out is NULL");
  *out = nullptr;
  const std::string why = attn_config_error(cfg);
  if (!why.empty()) return fail(MOE_EINVAL, "moe_attn_create: " + why);
  moe_attn* a = new moe_attn();
  a->cfg = *cfg;
  a->n_spans = (cfg->max_pos + kBlockPos - 1) / kBlockPos * kWaves;
  const size_t L = cfg->n_layers, D = cfg->head_dim, KV = cfg->n_kv_heads, P = cfg->max_pos;
  const size_t G = (size_t)(cfg->n_q_heads / cfg->n_kv_heads);
  a->work.max_split = a->n_spans / kWaves;
  a->set.assign(L, 0);
  const size_t kbytes = L * KV * P * D * 2, vbytes = L * KV * (size_t)a->n_spans * D * kSpan * 2;
  // rotation frequencies in fp64, as the definition takes them: dims i and
  // i + rot/2 turn by pos * 1e7^(-2i/rot)
  std::vector<double> freq(D, 0.0);
  for (int i = 0; i < cfg->rot_dim / 2; ++i)
    freq[(size_t)i] = freq[(size_t)i + cfg->rot_dim / 2] = std::pow(1.0e7, -2.0 * i / cfg->rot_dim);
  bool ok = hipMalloc(&a->norms, L * 2 * D * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&a->freq, D * sizeof(double)) == hipSuccess;
  ok = ok && hipMemcpy(a->freq, freq.data(), D * sizeof(double), hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipMalloc(&a->kc, kbytes) == hipSuccess;
  ok = ok && hipMalloc(&a->vt, vbytes) == hipSuccess;
  ok = ok && hipMalloc(&a->work.ml, KV * a->work.max_split * G * 2 * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&a->work.o, KV * a->work.max_split * G * D * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&a->work.qop, (size_t)cfg->n_q_heads * 2 * D * sizeof(_Float16)) == hipSuccess;
  ok = ok && hipMemset(a->kc, 0, kbytes) == hipSuccess && hipMemset(a->vt, 0, vbytes) == hipSuccess;
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  {
    std::lock_guard<std::mutex> l(g_attn_mu);
    g_attn_live.insert(a);
  }
  if (!ok) {
    moe_attn_destroy(a);
    return fail(MOE_ENOMEM, "moe_attn_create: allocation failed");
  }
  *out = a;
  return MOE_OK;
}

moe_status moe_attn_set_layer(moe_attn* a, int32_t layer, const float* q_norm_w, const float* k_norm_w) {
  clear_error();
  moe_status st = attn_check(a, "moe_attn_set_layer");
  if (st) return st;
  if (layer < 0 || layer >= a->cfg.n_layers) return fail(MOE_EINVAL, "moe_attn_set_layer: layer out of range");
  if (!q_norm_w || !k_norm_w) return fail(MOE_EINVAL, "moe_attn_set_layer: NULL pointer");
  const size_t D = a->cfg.head_dim;
  std::vector<float> w(2 * D);
  std::memcpy(w.data(), q_norm_w, D * sizeof(float));
  std::memcpy(w.data() + D, k_norm_w, D * sizeof(float));
  const hipError_t e =
      hipMemcpy(a->norms + (size_t)layer * 2 * D, w.data(), w.size() * sizeof(float), hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(MOE_EHIP, std::string("moe_attn_set_layer: ") + hipGetErrorString(e));
  a->set[(size_t)layer] = 1;
  return MOE_OK;
}

moe_status moe_attn_write_cache(moe_attn* a, int32_t layer, int32_t first_pos, int32_t n, const uint16_t* k,
                                const uint16_t* v) {
  clear_error();
  moe_status st = attn_check(a, "moe_attn_write_cache");
  if (st) return st;
  if (layer < 0 || layer >= a->cfg.n_layers) return fail(MOE_EINVAL, "moe_attn_write_cache: layer out of range");
  if (first_pos < 0 || n < 0 || (int64_t)first_pos + n > a->cfg.max_pos)
    return fail(MOE_EINVAL, "moe_attn_write_cache: positions outside [0, max_pos)");
  if (n == 0) return MOE_OK;
  if (!k || !v) return fail(MOE_EINVAL, "moe_attn_write_cache: NULL pointer");
  if (hipDeviceSynchronize() != hipSuccess) return fail(MOE_EHIP, "moe_attn_write_cache: sync");
  const size_t D = a->cfg.head_dim, KV = a->cfg.n_kv_heads, P = a->cfg.max_pos;
  const AttnLayer L = layer_args(a, layer);
  for (size_t g = 0; g < KV; ++g) {
    std::vector<uint16_t> vg(v + g * n * D, v + (g + 1) * n * D);
    if (hipMemcpy(L.kc + (g * P + first_pos) * D, k + g * n * D, (size_t)n * D * 2, hipMemcpyHostToDevice) !=
            hipSuccess ||
        v_tiles(L.vt + g * a->n_spans * D * kSpan, D, first_pos, n, vg.data(), true) != hipSuccess)
      return fail(MOE_EHIP, "moe_attn_write_cache: upload");
  }
  return MOE_OK;
}

moe_status moe_attn_read_cache(moe_attn* a, int32_t layer, int32_t first_pos, int32_t n, uint16_t* k, uint16_t* v) {
  clear_error();
  moe_status st = attn_check(a, "moe_attn_read_cache");
  if (st) return st;
  if (layer < 0 || layer >= a->cfg.n_layers) return fail(MOE_EINVAL, "moe_attn_read_cache: layer out of range");
  if (first_pos < 0 || n < 0 || (int64_t)first_pos + n > a->cfg.max_pos)
    return fail(MOE_EINVAL, "moe_attn_read_cache: positions outside [0, max_pos)");
  if (n == 0) return MOE_OK;
  if (hipDeviceSynchronize() != hipSuccess) return fail(MOE_EHIP, "moe_attn_read_cache: sync");
  const size_t D = a->cfg.head_dim, KV = a->cfg.n_kv_heads, P = a->cfg.max_pos;
  const AttnLayer L = layer_args(a, layer);
  for (size_t g = 0; g < KV; ++g) {
    if (k && hipMemcpy(k + g * n * D, L.kc + (g * P + first_pos) * D, (size_t)n * D * 2, hipMemcpyDeviceToHost) !=
                 hipSuccess)
      return fail(MOE_EHIP, "moe_attn_read_cache: copy");
    if (v && v_tiles(L.vt + g * a->n_spans * D * kSpan, D, first_pos, n, v + g * n * D, false) != hipSuccess)
      return fail(MOE_EHIP, "moe_attn_read_cache: copy");
  }
  return MOE_OK;
}

moe_status moe_attn_decode(moe_attn* a, int32_t first_layer, int32_t n_layers, int32_t pos0, const uint16_t* q,
                           const uint16_t* gate, const uint16_t* k, const uint16_t* v, int32_t n_tok, float* out,
                           void* stream) {
  clear_error();
  moe_status st = attn_check(a, "moe_attn_decode");
  if (st) return st;
  if (first_layer < 0 || n_layers < 1 || (int64_t)first_layer + n_layers > a->cfg.n_layers)
    return fail(MOE_EINVAL, "moe_attn_decode: layer range outside [0, n_layers)");
  if (n_tok < 0 || pos0 < 0 || (int64_t)pos0 + n_tok > a->cfg.max_pos)
    return fail(MOE_EINVAL, "moe_attn_decode: positions outside [0, max_pos)");
  if (n_tok == 0) return MOE_OK;
  if (!q || !gate || !k || !v || !out) return fail(MOE_EINVAL, "moe_attn_decode: NULL pointer");
  for (int l = first_layer; l < first_layer + n_layers; ++l)
    if (!a->set[(size_t)l]) return fail(MOE_ESTATE, "moe_attn_decode: moe_attn_set_layer was not called for a layer");
  const size_t D = a->cfg.head_dim, QD = (size_t)a->cfg.n_q_heads * D, KD = (size_t)a->cfg.n_kv_heads * D;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<AttnStep> steps;
  steps.reserve((size_t)n_tok * n_layers);
  for (int t = 0; t < n_tok; ++t)
    for (int l = first_layer; l < first_layer + n_layers; ++l) {
      const size_t r = (size_t)t * n_layers + (l - first_layer);
      steps.push_back(AttnStep{layer_args(a, l), AttnIo{q + r * QD, gate + r * QD, k + r * KD, v + r * KD, out + r * QD},
                               pos0 + t});
    }
  auto enqueue = [&](hipStream_t qs) -> moe_status {
    const hipError_t e = launch_steps(a, steps, qs);
    if (e != hipSuccess) return fail(MOE_EHIP, std::string("moe_attn_decode: launch: ") + hipGetErrorString(e));
    return MOE_OK;
  };
  if ((int64_t)n_tok * n_layers < 16 || a->prof) return enqueue(s);
  AttnGraph* hit = nullptr;
  for (auto& e : a->graphs)
    if (e.layer0 == first_layer && e.n_layers == n_layers && e.n_tok == n_tok && e.pos0 == pos0 && e.q == q &&
        e.gate == gate && e.k == k && e.v == v && e.out == out)
      hit = &e;
  if (!hit) {
    if (!a->cap_stream && hipStreamCreateWithFlags(&a->cap_stream, hipStreamNonBlocking) != hipSuccess)
      return fail(MOE_EHIP, "moe_attn_decode: capture stream");
    if (hipStreamBeginCapture(a->cap_stream, hipStreamCaptureModeThreadLocal) != hipSuccess)
      return fail(MOE_EHIP, "moe_attn_decode: capture begin");
    st = enqueue(a->cap_stream);
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(a->cap_stream, &graph);
    if (st) {
      if (graph) hipGraphDestroy(graph);
      return st;
    }
    if (e != hipSuccess) return fail(MOE_EHIP, "moe_attn_decode: capture end");
    AttnGraph ent{first_layer, n_layers, n_tok, pos0, q, gate, k, v, out, nullptr, nullptr, 0};
    const hipError_t ei = hipGraphInstantiate(&ent.exec, graph, nullptr, nullptr, 0);
    hipGraphDestroy(graph);
    if (ei != hipSuccess) return fail(MOE_EHIP, "moe_attn_decode: graph instantiate");
    if (hipEventCreateWithFlags(&ent.done, hipEventDisableTiming) != hipSuccess) {
      hipGraphExecDestroy(ent.exec);
      return fail(MOE_EHIP, "moe_attn_decode: graph event");
    }
    if (a->graphs.size() >= 8) {
      auto lru = std::min_element(a->graphs.begin(), a->graphs.end(),
                                  [](const AttnGraph& x, const AttnGraph& y) { return x.stamp < y.stamp; });
      hipEventSynchronize(lru->done);  // its last launch may still run
      hipGraphExecDestroy(lru->exec);
      hipEventDestroy(lru->done);
      a->graphs.erase(lru);
    }
    a->graphs.push_back(ent);
    hit = &a->graphs.back();
  }
  hit->stamp = ++a->clock;
  if (hipGraphLaunch(hit->exec, s) != hipSuccess) return fail(MOE_EHIP, "moe_attn_decode: graph launch");
  if (hipEventRecord(hit->done, s) != hipSuccess) return fail(MOE_EHIP, "moe_attn_decode: graph event record");
  return MOE_OK;
}

moe_status moe_attn_profile(moe_attn* a, int32_t enable, double* split_ms, double* combine_ms, uint64_t* launches) {
  clear_error();
  moe_status st = attn_check(a, "moe_attn_profile");
  if (st) return st;
  if (enable != 0 && enable != 1) return fail(MOE_EINVAL, "moe_attn_profile: enable must be 0 or 1");
  uint64_t n = 0;
  const double ms_s = drain(a->prof_split, &n);
  const double ms_c = drain(a->prof_combine, nullptr);
  if (split_ms) *split_ms = ms_s;
  if (combine_ms) *combine_ms = ms_c;
  if (launches) *launches = n;
  a->prof = enable != 0;
  return MOE_OK;
}

void moe_attn_destroy(moe_attn* a) {
  {
    std::lock_guard<std::mutex> l(g_attn_mu);
    if (!a || !g_attn_live.count(a)) return;
    g_attn_live.erase(a);
  }
  hipDeviceSynchronize();
  drain(a->prof_split, nullptr);
  drain(a->prof_combine, nullptr);
  for (auto& e : a->graphs) {
    hipGraphExecDestroy(e.exec);
    hipEventDestroy(e.done);
  }
  if (a->cap_stream) hipStreamDestroy(a->cap_stream);
  hipFree(a->norms);
  hipFree(a->freq);
  hipFree(a->kc);
  hipFree(a->vt);
  hipFree(a->work.ml);
  hipFree(a->work.o);
  hipFree(a->work.qop);
  delete a;
}

}  // extern "C"
