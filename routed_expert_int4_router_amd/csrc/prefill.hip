// Batched (prefill) path of the routed MoE step for gfx950.
//
// The pages' runtime has no batched prefill: long prompts run token by token
// (alphalab.site field test, FAQ item 4, and the method section on prompt
// length). Here a batch of T tokens takes the layer in nine launches:
//   xprep       per token: a power-of-two scale 2^e that brings max |x| / 2^e
//               into [2^14, 2^15) and that fp16 copy, k-permuted for the GEMM
//   router      logits [T][E+1] = x . W_r^T with bf16 MFMA on an exact
//               three-way bf16 split of the fp32 router rows, fp32 accumulate
//               (batches of at most 64 tokens: one wave per fp32 router row,
//               fp64 accumulation)
//   route       top-k + weights + shared gate per token (one wave each)
//   bucket x3   stable counting sort of the T*k (token, slot) pairs by expert
//               (per-chunk counts, scan + tile list, scatter), deterministic
//   gateup      grouped GEMM per (expert, 64-row tile, 64-column tile):
//               int4 codes -> fp16 weights s * q + c (one rounding), fp16
//               MFMA with fp32 accumulate, the token scale and SwiGLU in the
//               epilogue, h stored in fp16 under power-of-two range scales
//               (one per (tile, 64-group), plus a factor of its own for a row
//               far below the tile's largest) and per-group sums
//   down        grouped GEMM on h (fp16 MFMA, codes as fp16 16 + q), the range
//               scales and router weight applied to the fp32 partial sums,
//               one fp32 row per (token, slot) and per token
//   combine     out[t] = sum_j y[t,j] + y_shared[t] in fixed order
// Pages for the method itself: top-k routing, resident router and shared
// expert, int4/int8 group quantisation (cheshm.ai news article, paragraphs on
// how it works and on the code base).
#include "prefill.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "decode_math.h"
#include "dpp.h"
#include "launch.h"
#include "topk.h"

namespace moe {

hipError_t launch_route(const Geometry& g, const float* logits, int ld_logits, int n_tok, int32_t* route_idx,
                        float* route_w, float* route_gamma, int32_t* host_route, hipStream_t s);

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BM = 64;        // tile rows (tokens or pairs)
constexpr int CHUNK = 512;    // pairs per bucketing chunk

using Workspace = PrefillWorkspace;

// bf16f, f16f and the activation-pair helpers (x_chunk, code_pairs4,
// pairs_term) come from decode_math.h.

// Reorder the 8 bf16 of a 16-byte chunk (0,1,...,7) -> (0,4,1,5,2,6,3,7): the
// k-order in which the nibble conversion below emits the codes of a dword.
__device__ __forceinline__ uint4 perm8(uint4 v) {
  uint4 o;
  o.x = (v.x & 0xFFFFu) | (v.z << 16);                 // 0, 4
  o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);             // 1, 5
  o.z = (v.y & 0xFFFFu) | (v.w << 16);                 // 2, 6
  o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);             // 3, 7
  return o;
}

// Nibble-to-fp16 constants, kept opaque to the compiler (an empty asm
// "changes" them) so that (x & mask) | (magic & ~mask) stays one v_bfi_b32
// instead of being folded into an and plus an or. Set once per kernel.
struct NibConst {
  uint32_t mask16, magic16;      // 16 + q: nibble at bits 6..9 of each half, fp16 16.0 = 0x4C00
  uint32_t mask1024, magic1024;  // 1024 + q: nibble at bits 0..3 of each half, fp16 1024.0 = 0x6400
};
__device__ __forceinline__ NibConst nib_const() {
  NibConst k{0x03C003C0u, 0x4C004C00u, 0x000F000Fu, 0x64006400u};
  asm volatile("" : "+s"(k.mask16), "+v"(k.magic16), "+s"(k.mask1024), "+v"(k.magic1024));
  return k;
}
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t x, uint32_t y) { return (x & mask) | (y & ~mask); }

// 8 int4 codes of a dword -> fp16 values 16 + q in the order (0,4,1,5,2,6,3,7).
__device__ __forceinline__ f16x8 nib_to_f16(uint32_t w, const NibConst& k) {
  uint32_t d[4];
  d[0] = bfi(k.mask16, w << 6, k.magic16);
  d[1] = bfi(k.mask16, w << 2, k.magic16);
  d[2] = bfi(k.mask16, w >> 2, k.magic16);
  d[3] = bfi(k.mask16, w >> 6, k.magic16);
  return __builtin_bit_cast(f16x8, *reinterpret_cast<uint4*>(d));
}

// 8 int4 codes of a dword -> fp16 weights s * q + c (q exact, one fused
// rounding) in the same order; s2 = (s, s), c2 = (c, c). The codes enter as
// 1024 + q (no shift for the first pair), then q = v - 1024 exactly.
__device__ __forceinline__ f16x8 nib_dequant_f16(uint32_t w, f16x2 s2, f16x2 c2, const NibConst& k) {
  uint32_t d[4];
  d[0] = bfi(k.mask1024, w, k.magic1024);
  d[1] = bfi(k.mask1024, w >> 4, k.magic1024);
  d[2] = bfi(k.mask1024, w >> 8, k.magic1024);
  d[3] = bfi(k.mask1024, w >> 12, k.magic1024);
  const f16x2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  f16x8 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 q = __builtin_bit_cast(f16x2, d[i]) - k1024;
    const f16x2 r = __builtin_elementwise_fma(q, s2, c2);
    o[2 * i] = r[0];
    o[2 * i + 1] = r[1];
  }
  return o;
}

// ------------------------------------------------------------------ xprep ---
// One wave per token: the scale 2^e, e of either sign, that brings max |x| /
// 2^e into [2^14, 2^15) (e = 0 for an all-zero token), and x / 2^e in fp16
// with every 8-chunk in the order (0,4,1,5,2,6,3,7), the order in which
// nib_to_f16 emits the codes of a dword. Both small and large activations
// then use fp16's full precision: a bf16 value x / 2^e is exact in fp16 down
// to 2^-14, i.e. for every element above max |x| * 2^-29. The grouped GEMM
// streams that copy into LDS unchanged. NC = 16-byte chunks per lane (H /
// 512, at least 1).
template <int NC>
__global__ void __launch_bounds__(256) xprep_kernel(const uint16_t* __restrict__ x, int T, int H, float* xscale,
                                                    uint16_t* xp) {
  const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;  // whole waves
  const int nch = H / 8;
  const uint4* p = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  uint4 v[NC];
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + 64 * c;
    v[c] = p[min(ch, nch - 1)];
    const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16f(w[i] & 0xFFFFu)), fabsf(bf16f(w[i] >> 16))));
  }
  amax = __uint_as_float(dpp::wave_max_u32(__float_as_uint(amax)));  // non-negative floats order as integers
  int ex = 0;
  if (amax > 0.f) {
    int x2;
    (void)frexpf(amax, &x2);  // 2^(x2-1) <= amax < 2^x2
    ex = x2 - 15;
  }
  if (lane == 0) xscale[t] = ldexpf(1.f, ex);
  uint4* q = reinterpret_cast<uint4*>(xp + (size_t)t * H);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)ldexpf(bf16f(w[i] & 0xFFFFu), -ex));
        const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)ldexpf(bf16f(w[i] >> 16), -ex));
        o[i] = lo | (hi << 16);
      }
      q[ch] = perm8(make_uint4(o[0], o[1], o[2], o[3]));
    }
  }
}

// ------------------------------------------------------- router (MFMA) ---
// Block barrier that waits for this wave's LDS accesses only (lgkmcnt(0);
// vmcnt and expcnt at their maximum), so global loads stay in flight across
// it; the compiler may not move memory accesses across it either.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// logits[t][e] = sum_h x[t][h] * w[e][h] (+ bias[e] for e < E), rows e <= E of
// the fp32 router matrix (row E = shared gate). Each fp32 weight enters as
// the three bf16 of its exact split (hi + mid + lo, prepared once per layer
// when the layer is set), so every bf16 x fp32 product is taken exactly as
// three bf16 x bf16 MFMA products; accumulation is fp32. Block: 128 tokens x
// 64 rows, 8 waves of 32 x 32 (32x32x16 MFMA), waves 0-3 on tokens 0-63 and
// 4-7 on 64-127 of the same rows; all waves stage x, waves 0-3 also the
// three planes' rows (read from L2 once per 128 tokens). The operands of K
// step k + 1 are loaded into registers while step k runs on the matrix
// cores. 144 blocks for T = 2048, E = 512: one per CU at most.
__global__ void __launch_bounds__(512) router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ ws,
                                                          const float* __restrict__ bias, int T, int H, int E,
                                                          float* logits) {
  __shared__ __align__(16) uint16_t sa[128][72];
  __shared__ __align__(16) uint16_t sb[3][64][72];
  const int t0 = blockIdx.x * 128, e0 = blockIdx.y * 64;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int wm = (wv >> 2) * 64 + ((wv & 3) >> 1) * 32, wn = (wv & 1) * 32;
  const bool wload = wv < 4;  // waves 0-3 also stage the 64 router rows
  const int R = E + 1;
  f32x16 acc = {};
  const int lr = threadIdx.x >> 2, lq = threadIdx.x & 3;  // staging: row, 16-element quarter
  const int ta = min(t0 + lr, T - 1), eb = min(e0 + (lr & 63), R - 1);
  const u32x4* ga = reinterpret_cast<const u32x4*>(x + (size_t)ta * H + 16 * lq);
  const u32x4* gb0 = reinterpret_cast<const u32x4*>(ws + ((size_t)0 * R + eb) * H + 16 * lq);
  const u32x4* gb1 = reinterpret_cast<const u32x4*>(ws + ((size_t)1 * R + eb) * H + 16 * lq);
  const u32x4* gb2 = reinterpret_cast<const u32x4*>(ws + ((size_t)2 * R + eb) * H + 16 * lq);
  u32x4 a0 = ga[0], a1 = ga[1];
  u32x4 b00 = gb0[0], b01 = gb0[1], b10 = gb1[0], b11 = gb1[1], b20 = gb2[0], b21 = gb2[1];
  for (int k0 = 0; k0 < H; k0 += 64) {
    lds_barrier();  // every wave is done reading the previous step from LDS
    *reinterpret_cast<u32x4*>(&sa[lr][16 * lq]) = a0;
    *reinterpret_cast<u32x4*>(&sa[lr][16 * lq + 8]) = a1;
    if (wload) {
      *reinterpret_cast<u32x4*>(&sb[0][lr][16 * lq]) = b00;
      *reinterpret_cast<u32x4*>(&sb[0][lr][16 * lq + 8]) = b01;
      *reinterpret_cast<u32x4*>(&sb[1][lr][16 * lq]) = b10;
      *reinterpret_cast<u32x4*>(&sb[1][lr][16 * lq + 8]) = b11;
      *reinterpret_cast<u32x4*>(&sb[2][lr][16 * lq]) = b20;
      *reinterpret_cast<u32x4*>(&sb[2][lr][16 * lq + 8]) = b21;
    }
    // next step's operands (the last step reloads itself: every load issues)
    const int kn = min(k0 + 64, H - 64) / 8;
    a0 = ga[kn];
    a1 = ga[kn + 1];
    if (wload) {
      b00 = gb0[kn];
      b01 = gb0[kn + 1];
      b10 = gb1[kn];
      b11 = gb1[kn + 1];
      b20 = gb2[kn];
      b21 = gb2[kn + 1];
    }
    lds_barrier();  // the step is in LDS; the next step's loads are in flight
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kk = 16 * s + 8 * (lane >> 5);
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sa[wm + (lane & 31)][kk]);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&sb[p][wn + (lane & 31)][kk]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
      }
    }
  }
  const int n = e0 + wn + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = t0 + wm + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
    if (m < T && n < R) logits[(size_t)m * R + n] = acc[r] + ((n < E && bias) ? bias[n] : 0.f);
  }
}

// Router for small batches (T <= kRouterRowsMaxT): a block of 8 waves
// covers 4 router rows; wave w keeps row 4 b + (w % 4) in registers and takes
// the tokens t = w / 4, w / 4 + 2, ..., loading U tokens' x at once so the
// loads' latency overlaps (U = 4, or 2 where H = 4096 leaves fewer
// registers). Products of a bf16 and an fp32 are exact in fp64;
// the fp64 sum is rounded once to fp32 (as the decode router does). For a few
// tokens this beats the MFMA GEMM, whose blocks each walk all of K for up to
// 128 tokens: measured on the 80B-shaped layer, 8 tokens 7.4 us against 27.9,
// 16 tokens 10.7 against 28.9, 64 tokens 26.5 against 30.8, 256 tokens 85.9
// against 33.9 (~0.4 us per token against a flat ~30 us).
constexpr int kRouterRowsMaxT = 64;

template <int NIT, int U>
__global__ void __launch_bounds__(512) router_rows_kernel(const float* __restrict__ wr, const float* __restrict__ bias,
                                                           const uint16_t* __restrict__ x, int T, int H, int E,
                                                           float* logits) {
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (wv & 3);
  if (row > E) return;  // whole waves; no block-wide sync below
  const int n4 = H / 4;
  const float4* w4 = reinterpret_cast<const float4*>(wr + (size_t)row * H);
  float4 w[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int i = lane + 64 * it;
    w[it] = i < n4 ? w4[min(i, n4 - 1)] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const double b = (row < E && bias) ? (double)bias[row] : 0.0;
  for (int t0 = wv >> 2; t0 < T; t0 += 2 * U) {  // U tokens per round: t0, t0 + 2, ...
    uint2 xv[U][NIT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint2* x4 = reinterpret_cast<const uint2*>(x + (size_t)min(t0 + 2 * u, T - 1) * H);
#pragma unroll
      for (int it = 0; it < NIT; ++it) xv[u][it] = x4[min(lane + 64 * it, n4 - 1)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      double acc = 0.0;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        // lanes past H / 4 hold zero weights, so their (clamped) x adds nothing
        acc += (double)bf16f(xv[u][it].x & 0xFFFFu) * (double)w[it].x;
        acc += (double)bf16f(xv[u][it].x >> 16) * (double)w[it].y;
        acc += (double)bf16f(xv[u][it].y & 0xFFFFu) * (double)w[it].z;
        acc += (double)bf16f(xv[u][it].y >> 16) * (double)w[it].w;
      }
      acc = dpp::wave_sum(acc);
      const int t = t0 + 2 * u;
      if (lane == 0 && t < T) logits[(size_t)t * (E + 1) + row] = (float)(acc + b);
    }
  }
}

// ------------------------------------------------------------- bucketing ---
__global__ void __launch_bounds__(CHUNK) bucket_count_kernel(const int32_t* __restrict__ idx, int P, int E, int32_t* cnt) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += CHUNK) hist[e] = 0;
  __syncthreads();
  const int p = blockIdx.x * CHUNK + threadIdx.x;
  if (p < P) atomicAdd(&hist[idx[p]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += CHUNK) cnt[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block: per-expert totals, per-chunk offsets and the tile list (routed
// experts, then the shared expert over all T tokens; each tile carries its
// expert, first row within the expert, first row in the bucketed order and
// row count).
__global__ void __launch_bounds__(1024) bucket_scan_kernel(const int32_t* __restrict__ cnt, int nchunk, int E, int T,
                                                           int32_t* __restrict__ chunk_off,
                                                           int32_t* __restrict__ tiles, int max_tiles) {
  __shared__ int32_t s_tot[1024], s_tiles[1024];
  __shared__ int32_t s_base, s_tbase;
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E) {
#pragma unroll 8
    for (int c = 0; c < nchunk; ++c) tot += cnt[(size_t)c * E + e];
  }
  const int ntile = (tot + BM - 1) / BM;
  // block-wide exclusive scans (sequential over waves, DPP within a wave)
  const uint32_t inc_t = dpp::wave_prefix_u32((uint32_t)tot);
  const uint32_t inc_n = dpp::wave_prefix_u32((uint32_t)ntile);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 63) {
    s_tot[wv] = (int)inc_t;
    s_tiles[wv] = (int)inc_n;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0, b = 0;
    for (int w = 0; w < 16; ++w) {
      const int ta = s_tot[w], tb = s_tiles[w];
      s_tot[w] = a;
      s_tiles[w] = b;
      a += ta;
      b += tb;
    }
    s_base = a;
    s_tbase = b;
  }
  __syncthreads();
  const int off = s_tot[wv] + (int)inc_t - tot;
  const int toff = s_tiles[wv] + (int)inc_n - ntile;
  if (e < E) {
    int run = off;
#pragma unroll 8
    for (int c = 0; c < nchunk; ++c) {
      chunk_off[(size_t)c * E + e] = run;
      run += cnt[(size_t)c * E + e];
    }
    for (int i = 0; i < ntile; ++i)
      *reinterpret_cast<int4*>(tiles + 4 + 4 * (toff + i)) =
          make_int4(e, i * BM, off + i * BM, min(tot - i * BM, BM));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int nsh = (T + BM - 1) / BM;
    for (int i = 0; i < nsh; ++i)
      *reinterpret_cast<int4*>(tiles + 4 + 4 * (s_tbase + i)) =
          make_int4(E, i * BM, s_base + i * BM, min(T - i * BM, BM));
    tiles[0] = min(s_tbase + nsh, max_tiles);
  }
}

// Stable scatter: a pair's position is its chunk's offset for its expert plus
// the number of earlier pairs of the same expert in the chunk, counted as
// the same-expert lanes below it in its wave (64 uniform readlane compares)
// plus the same-expert pairs of the earlier waves (per-wave histograms in
// LDS, [CHUNK / 64][E]).
__global__ void __launch_bounds__(CHUNK) bucket_scatter_kernel(const int32_t* __restrict__ idx,
                                                               const float* __restrict__ route_w, int P, int E,
                                                               const int32_t* __restrict__ chunk_off, int32_t* perm,
                                                               float* wperm) {
  extern __shared__ int32_t s_hist[];
  const int p = blockIdx.x * CHUNK + threadIdx.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = p < P ? idx[p] : -1;
  for (int i = threadIdx.x; i < (CHUNK / 64) * E; i += CHUNK) s_hist[i] = 0;
  int rank = 0;
  for (int j = 0; j < 64; ++j) rank += (j < lane && __builtin_amdgcn_readlane(e, j) == e) ? 1 : 0;
  __syncthreads();
  if (e >= 0) atomicAdd(&s_hist[wv * E + e], 1);
  __syncthreads();
  if (p >= P) return;
  for (int w = 0; w < wv; ++w) rank += s_hist[w * E + e];
  const int pos = chunk_off[(size_t)blockIdx.x * E + e] + rank;
  perm[pos] = p;
  wperm[pos] = route_w[p];
}

// ------------------------------------------------- shared GEMM arithmetic ---
// Element-wise steps of the grouped GEMMs' epilogues, used by the fast kernels
// and by their plainly written variants alike.

// h = silu(gate) * up with the hardware exp2 and reciprocal.
__device__ __forceinline__ float silu_mul(float gt, float up) {
  return gt * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gt)) * up;
}

// Natural exponent n of a row whose largest |h| is rmax (max |h| / 2^n in
// [2^14, 2^15)), biased by 256 so exponents order as unsigned integers; 0 for
// no value (a padding row, or a row of zeros).
__device__ __forceinline__ uint32_t row_exp_biased(float rmax, bool live) {
  if (!live || !(rmax > 0.f)) return 0u;
  int x2;
  (void)frexpf(rmax, &x2);  // 2^(x2-1) <= rmax < 2^x2
  return (uint32_t)(x2 - 15 + 256);
}

// A row's exponent given the tile-group's largest T: T for a row within 2^12
// of it (its maximum stays >= 4 under 2^T, so only values below 2^-16 of it
// leave fp16's normal range), else its own (at most 126 below T).
__device__ __forceinline__ int row_exp(uint32_t nb, int T) {
  if (nb && (int)nb - 256 < T - 12) return max((int)nb - 256, T - 126);
  return T;
}

// 16 consecutive columns of a row as fp16 h / 2^er, each 8-chunk in
// nib_to_f16 order (0,4,1,5,2,6,3,7) in pk, and the sum of the values the
// down GEMM multiplies (2^er * fp16) in column order.
__device__ __forceinline__ float pack16(const float* hv, int er, uint32_t (&pk)[8]) {
  float sum = 0.f;
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) {
    const _Float16 hq = (_Float16)ldexpf(hv[cc], -er);
    sum += ldexpf((float)hq, er);
    const uint32_t b = __builtin_bit_cast(uint16_t, hq);
    const int ch = cc >> 3, p = cc & 7;
    const int w = 4 * ch + (p & 3);  // dword of the pair (p, p + 4)
    if (p < 4) pk[w] = b;
    else pk[w] |= b << 16;
  }
  return sum;
}

// ------------------------------------------------------- grouped GEMM 1 ---
// Block = (tile, 64 columns of I), 4 waves, two blocks per CU: 64 rows of one
// expert (sorted pairs, or tokens for the shared expert) x 64 gate + 64 up
// columns. Waves 0,1 compute gate columns [32w, 32w + 32), waves 2,3 the
// same up columns; each wave is 64 x 32 (two 32x32x16 MFMA tiles). K runs
// over the 64-groups of H. The two blocks of a CU are not tied by a common
// barrier, so one block's VALU work (code conversion, group scaling)
// overlaps the other's MFMAs on the same SIMD.
//
// Operands reach LDS by direct global->LDS DMA (no registers): the A rows
// (the k-permuted x of the tile's tokens; rows past the tile's end are not
// fetched) one group (8 KB) at a time, GU_PF groups ahead, into a GU_NA-stage
// ring; the code rows and (s, c) words a quad of 4 groups at a time (one
// 128-byte line per code row, 16 bytes of scales per row), one quad ahead,
// into 2-stage rings. Few, full-line requests matter: with partial-line code
// requests the L2 request rate, not its bandwidth, limited the kernel. A tile
// of at most 32 rows runs a copy of the K loop without each wave's lower
// 32-row MFMA tile. Every wave issues the same
// DMAs in the same order, so fixed "all but the newest n" waits plus one
// barrier per group make a group's stages visible to every wave.
//
// Per group: the lane's 32 codes become fp16 weights s * q + c (packed fp16
// FMA, one rounding) and acc += A . w on the matrix cores, A = x / 2^e_t in
// fp16; the token scale 2^e_t multiplies the rows in the epilogue. The
// conversion of a group does not depend on any MFMA result, so it overlaps
// the previous group's MFMAs. The epilogue computes h = silu(gate) * up in
// fp32 and stores it in fp16 under power-of-two range scales chosen from the
// tile's values, in either direction, so small and large activations keep
// fp16's 11 significant bits.
struct GemmArgs {
  const uint16_t* x;          // [T][H]
  const uint16_t* xp;         // [T][H] fp16 x / xscale, 8-chunks in nib_to_f16 order
  const float* xscale;        // [T]
  const uint8_t* experts;     // routed records of the layer
  const uint8_t* shared;      // shared record
  uint64_t stride;
  uint64_t gate_codes, up_codes, down_codes, gate_sc, up_sc, down_sc;
  const int32_t* perm;        // [T*k]
  const float* wperm;         // [T*k] router weight at each sorted position
  const int32_t* tiles;       // count at [0], then (expert, row0, base, rows) per tile from [4]
  const float* route_w;       // [T*k]
  const float* route_gamma;   // [T]
  uint16_t* h16;
  float* hscale;              // [tiles][I/64] 2^T per (tile, group), negative when rows carry own factors
  float* hrowf;               // [T*k + T][I/64] per-row factor 2^(e_row - T) (1 for most rows)
  float* hsum;
  float* y;
  int T, H, I, E, k;
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 4, 0, 0);
}

// LDS rows of 128 bytes hold their eight 16-byte chunks permuted: chunk c of
// row r sits in slot c ^ swz(r). A 16-byte read by 16 lanes of 16
// consecutive rows then touches 16 different 16-byte bank groups (the
// group of slot s of row r is 8 (r & 1) + s modulo 16), so it runs
// without bank conflicts.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Tile of a block. The 8 XCDs take blocks round-robin (block b runs on XCD
// b % 8). XCD x gets an equal share of the shared expert's tiles (all full,
// the tile list's last nsh entries) first, then a contiguous range of the
// routed tiles, each tile as NT consecutive blocks: the column tiles of one
// row tile, and neighbouring row tiles of one expert, share that XCD's L2,
// and no XCD gets more than its share of the long tiles. The grid is sized
// for the worst case (the tile count is known only on the device); a block
// with nothing to do gets -1.
__device__ __forceinline__ int xcd_tile(int ntile, int nsh, int NT, int& nt) {
  const int nr = ntile - nsh;
  const int psh = (nsh + 7) / 8, pr = (nr + 7) / 8;
  const int x = (int)(blockIdx.x % 8), i = (int)(blockIdx.x / 8);
  const int nsx = min(max(nsh - x * psh, 0), psh), nrx = min(max(nr - x * pr, 0), pr);
  if (i < nsx * NT) {
    nt = i % NT;
    return nr + x * psh + i / NT;
  }
  const int j = i - nsx * NT;
  if (j >= nrx * NT) return -1;
  nt = j % NT;
  return x * pr + j / NT;
}

// Blocks per XCD that xcd_tile may ask for: shared tiles ceil(nsh / 8), routed
// at most ceil((max_tiles - nsh) / 8).
int xcd_grid(int max_tiles, int nsh, int NT) { return 8 * ((nsh + 7) / 8 + (max_tiles - nsh + 7) / 8) * NT; }

constexpr int GU_BN = 64;                     // I columns per block
constexpr int GU_NA = 4;                      // A ring stages (one group each)
constexpr int GU_PF = GU_NA - 1;              // A prefetch distance in groups
constexpr int A_STAGE = BM * 64 * 2;          // 64 rows x 64 bf16 (8 KB)
constexpr int BQ_STAGE = 2 * GU_BN * 128;     // 128 code rows x 4 groups (16 KB)
constexpr int SQ_STAGE = 2 * GU_BN * 16;      // 128 rows x 4 (s, c) words (2 KB)

size_t gateup_lds_bytes() { return (size_t)GU_NA * A_STAGE + 2 * (size_t)BQ_STAGE + 2 * (size_t)SQ_STAGE; }

// Per-lane DMA sources (group / quad 0).
struct GateUpSources {
  const uint16_t* a[2];  // A (instruction t): row 8 (2w + t) + lane / 8, chunk (lane % 8) ^ (row % 8); +64 g
  bool a_live[2];        // the row exists (lane 0 always fetches, keeping the DMA issued)
  const uint8_t* b[4];   // code rows, instruction t: row 32w + 8t + lane / 8, chunk (lane % 8) ^ (row % 8); +128 Q
  const uint8_t* s;      // scale words of row 32w + lane (lanes < 32); +16 Q
};

// Operands of one K group for one lane, read one group ahead of their use.
struct GroupFrag {
  f16x8 a0[4], a1[4];   // A rows mrow and 32 + mrow for the 4 MFMA steps
  uint4 codes;          // 32 codes of column brow (k half hh)
  uint32_t sc;          // (s, c) of column brow: fp16 bits, s low
  f16x8 b[4];           // the codes as fp16 weights, for the 4 MFMA steps
};

// Step for group g = 4Q + J: issue (for J == 0) the next quad's code rows and
// scale words, then A(g + PF); then read group g's operands from LDS. The
// restrict qualifiers tell the compiler that the stages read are not the
// ones written, so it adds no wait of its own between DMAs and LDS reads;
// the caller's vmcnt wait + barrier orders them.
template <int J, bool FULL>
__device__ __forceinline__ void gateup_fetch(const uint8_t* __restrict__ rdA, const uint8_t* __restrict__ rdB,
                                             const uint8_t* __restrict__ rdS, uint8_t* __restrict__ wrA,
                                             uint8_t* __restrict__ wrB, uint8_t* __restrict__ wrS,
                                             const GateUpSources& src, int qn, int gn, int wv, int lane, int brow,
                                             int hh, int mrow, GroupFrag& f) {
  if constexpr (J == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) dma16(src.b[t] + 128 * qn, wrB + (4 * wv + t) * 1024);
    if (lane < 32) dma16(src.s + 16 * qn, wrS + wv * 512);
  }
  if (src.a_live[0]) dma16(src.a[0] + 64 * gn, wrA + (2 * wv) * 1024);
  if (src.a_live[1]) dma16(src.a[1] + 64 * gn, wrA + (2 * wv + 1) * 1024);
  const int slot = (2 * J + hh) ^ swz(brow);
  f.codes = *reinterpret_cast<const uint4*>(rdB + brow * 128 + slot * 16);
  f.sc = *reinterpret_cast<const uint32_t*>(rdS + brow * 16 + J * 4);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int off = ((4 * hh + st) ^ swz(mrow)) * 16;  // swz(32 + mrow) == swz(mrow)
    f.a0[st] = *reinterpret_cast<const f16x8*>(rdA + mrow * 128 + off);
    if constexpr (FULL) f.a1[st] = *reinterpret_cast<const f16x8*>(rdA + (32 + mrow) * 128 + off);
  }
}

// The group's weights w = s * q + c in fp16.
__device__ __forceinline__ void gateup_dequant(GroupFrag& f, const NibConst& k) {
  const f16x2 s2 = __builtin_bit_cast(f16x2, (f.sc & 0xFFFFu) * 0x00010001u);
  const f16x2 c2 = __builtin_bit_cast(f16x2, (f.sc >> 16) * 0x00010001u);
  f.b[0] = nib_dequant_f16(f.codes.x, s2, c2, k);
  f.b[1] = nib_dequant_f16(f.codes.y, s2, c2, k);
  f.b[2] = nib_dequant_f16(f.codes.z, s2, c2, k);
  f.b[3] = nib_dequant_f16(f.codes.w, s2, c2, k);
}

// acc += A . w for one group (weights converted beforehand); rows 32..63
// only when the tile has them (FULL).
template <bool FULL>
__device__ __forceinline__ void gateup_mfma(const GroupFrag& f, f32x16& acc0, f32x16& acc1) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a0[st], f.b[st], acc0, 0, 0, 0);
    if constexpr (FULL) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a1[st], f.b[st], acc1, 0, 0, 0);
  }
}

// The K loop of a gate/up block, instantiated for tiles of more than 32 rows
// (FULL) and for the rest, so neither copy branches inside the loop.
template <bool FULL>
__device__ __forceinline__ void gateup_loop(uint8_t* sA, uint8_t* sB, uint8_t* sS, const GateUpSources& src, int G,
                                            int NQ, int wv, int lane, int brow, int hh, int mrow, f32x16& acc0,
                                            f32x16& acc1) {
  GroupFrag fa, fb;
  // Step g (wait, barrier, DMAs, LDS -> registers) runs one group ahead of
  // compute g. Per step a wave issues A(g + 3) (2 DMAs), preceded at a quad's
  // first group by the next quad's codes and scales (5 DMAs). Waiting for
  // A(g) leaves the DMAs of steps g-2 and g-1 in flight: 4 when neither
  // starts a quad (J = 0, 3), 9 otherwise; the codes and scales of quad Q
  // were issued before A(4Q) and so are covered at J = 0. lgkmcnt(0) makes
  // this wave's reads of the stages about to be overwritten complete.
  static_assert(GU_PF == 3, "wait counts below are written for PF = 3");
#define GU_STEP(Q, J, WAIT, F)                                                                                   \
  {                                                                                                              \
    const int g = 4 * (Q) + (J);                                                                                 \
    __builtin_amdgcn_s_waitcnt(0x0070 | (WAIT));                                                                 \
    __builtin_amdgcn_s_barrier();                                                                                \
    gateup_fetch<J, FULL>(sA + (g % GU_NA) * A_STAGE, sB + ((Q) & 1) * BQ_STAGE, sS + ((Q) & 1) * SQ_STAGE,      \
                          sA + ((g + GU_PF) % GU_NA) * A_STAGE, sB + (((Q) + 1) & 1) * BQ_STAGE,                 \
                          sS + (((Q) + 1) & 1) * SQ_STAGE, src, min((Q) + 1, NQ - 1), min(g + GU_PF, G - 1), wv, \
                          lane, brow, hh, mrow, F);                                                              \
  }
  // The weights of group g + 1 are converted right after the MFMAs of group
  // g are issued, so the conversion runs while those MFMAs execute.
  const NibConst nk = nib_const();
  GU_STEP(0, 0, 4, fa)
  gateup_dequant(fa, nk);
  for (int Q = 0; Q < NQ; ++Q) {
    GU_STEP(Q, 1, 9, fb)
    gateup_mfma<FULL>(fa, acc0, acc1);
    gateup_dequant(fb, nk);
    GU_STEP(Q, 2, 9, fa)
    gateup_mfma<FULL>(fb, acc0, acc1);
    gateup_dequant(fa, nk);
    GU_STEP(Q, 3, 4, fb)
    gateup_mfma<FULL>(fa, acc0, acc1);
    gateup_dequant(fb, nk);
    if (Q + 1 < NQ) GU_STEP(Q + 1, 0, 4, fa)
    gateup_mfma<FULL>(fb, acc0, acc1);
    if (Q + 1 < NQ) gateup_dequant(fa, nk);
  }
#undef GU_STEP
}

// The tile's h rows (sg: [64][GU_BN + 1] fp32, after SwiGLU) under their
// fp16 range scales into h16, with the per-row group sums, the per-row
// factors and the tile-group scale; all 256 threads of the block.
__device__ __forceinline__ void gateup_store_h(const GemmArgs& a, const float* sg, int nrow, int tile, int nt,
                                               int base, int n0, int tid, int wv, int lane) {
  constexpr int SGS = GU_BN + 1;
  // fp16 range scales. Row m (4 threads, 16 columns each) has the natural
  // exponent n_m: max |h_m| / 2^n_m in [2^14, 2^15). The tile-group scale is
  // 2^T with T = the largest n_m over the tile's rows. A row within 2^12 of
  // the tile's largest stores h / 2^T (its maximum stays >= 4, so only values
  // below 2^-16 of it leave fp16's normal range); a smaller row stores
  // h / 2^n_m and the factor 2^(n_m - T) that the down GEMM applies to its
  // partial sums. hscale = 2^T, negated when any row of the tile-group has
  // its own factor.
  const int m = tid >> 2, qq = tid & 3;
  float hv[16];
  float rmax = 0.f;
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) {
    hv[cc] = sg[m * SGS + 16 * qq + cc];
    rmax = fmaxf(rmax, fabsf(hv[cc]));
  }
  rmax = fmaxf(rmax, __uint_as_float(dpp::mov<dpp::kQuadXor1, 0xF>(0u, __float_as_uint(rmax))));
  rmax = fmaxf(rmax, __uint_as_float(dpp::mov<dpp::kQuadXor2, 0xF>(0u, __float_as_uint(rmax))));
  const uint32_t nb = row_exp_biased(rmax, m < nrow);
  __shared__ uint32_t s_tmax[4];
  {
    const uint32_t wm = dpp::wave_max_u32(nb);
    if (lane == 0) s_tmax[wv] = wm;
  }
  __syncthreads();
  const uint32_t tb = max(max(s_tmax[0], s_tmax[1]), max(s_tmax[2], s_tmax[3]));
  const int T = tb ? (int)tb - 256 : 0;
  const int er = row_exp(nb, T);  // this row's exponent
  const bool own = m < nrow && er != T;
  // h / 2^er in fp16 and the group sum of the values the down GEMM
  // multiplies: this thread's 16 columns, then the row's four quarters
  // combined as (q0 + q1) + (q2 + q3)
  uint32_t pk[8];
  float sum = pack16(hv, er, pk);
  sum += __uint_as_float(dpp::mov<dpp::kQuadXor1, 0xF>(0u, __float_as_uint(sum)));
  sum += __uint_as_float(dpp::mov<dpp::kQuadXor2, 0xF>(0u, __float_as_uint(sum)));
  const int GI = a.I / 64;
  if (m < nrow) {
    uint16_t* dst = a.h16 + (size_t)(base + m) * a.I + n0 + 16 * qq;
    *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    *reinterpret_cast<uint4*>(dst + 8) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    if (qq == 0) {
      a.hsum[(size_t)(base + m) * GI + nt] = sum;
      a.hrowf[(size_t)(base + m) * GI + nt] = ldexpf(1.f, er - T);
    }
  }
  const uint64_t any_own = __ballot(own);
  __shared__ uint32_t s_own[4];
  if (lane == 0) s_own[wv] = any_own != 0;
  __syncthreads();
  if (tid == 0) {
    const float sc = ldexpf(1.f, T);
    a.hscale[(size_t)tile * GI + nt] = (s_own[0] | s_own[1] | s_own[2] | s_own[3]) ? -sc : sc;
  }
}

// ------------------------------------------------ gate/up, small tiles ---
// A tile of at most kSmallRows rows (an expert that got a handful of tokens)
// skips the matrix cores: converting a group's weights to fp16 for a 32-row
// MFMA tile costs the same whatever the tile holds, and these tiles are a
// large share of the weight bytes but a small share of the flops. The block
// streams its 64 gate + 64 up code rows once and multiplies them on the
// dot-product unit as the decode kernel does: codes as the exact bf16 values
// 128 + q, activations as their own bf16 values re-paired to match, two
// products per v_dot2, fp32 sums (s * sum((128 + q) x) + (c - 128 s) * sum(x)
// per 32-code chunk). Wave w takes I columns [16w, 16w + 16) of the block, of
// gate and of up; a lane (rsub = lane / 16, c0 = lane % 16) takes row
// 4p + rsub of pass p (gate for p < 4, up after) at the chunks c0 + 16i; the
// 16 lanes of a row are summed by DPP. h = silu(gate) * up then takes the
// same range-scale epilogue as the MFMA tiles. The tiles' tokens' activations
// are staged once per block in LDS, already paired, with their chunk sums.
constexpr int kSmallRows = 4;

// The small-tile path covers H a multiple of 512 up to 2048: one to four chunk
// positions per lane, every code load issued before the first product.
__host__ __device__ constexpr bool small_tiles_ok(int H) { return H % 512 == 0 && H <= 2048; }

template <int NP>
__device__ __forceinline__ void gateup_small(const GemmArgs& a, uint8_t* smem, int tile, int nt, int e, int r0,
                                             int base, int nrow, const uint8_t* rec) {
  constexpr int H = 512 * NP;   // hidden size of this instance
  constexpr int NCH = H / 32;   // 32-code chunks per row
  constexpr int G = H / 64;     // quantisation groups per row
  constexpr int SGS = GU_BN + 1;
  static_assert(kSmallRows * NCH * 68 + BM * SGS * 4 <= GU_NA * A_STAGE + 2 * BQ_STAGE + 2 * SQ_STAGE,
                "small-tile staging must fit the block's LDS");
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n0 = nt * GU_BN;
  uint32_t* xp = reinterpret_cast<uint32_t*>(smem);                        // [kSmallRows][NCH][16] pairs
  float* xsm = reinterpret_cast<float*>(smem + kSmallRows * NCH * 64);     // [kSmallRows][NCH] chunk sums
  float* sg = xsm + kSmallRows * NCH;                                      // [64][SGS] h
  const int rsub = lane >> 4, c0 = lane & 15;
  // this lane's row r = 4 (p & 3) + rsub of pass p, at the chunks c0 + 16 it
  const size_t row0 = (size_t)(n0 + 16 * wv + rsub);
  const uint8_t* gcode = rec + a.gate_codes + row0 * (H / 2) + 16 * c0;
  const uint8_t* ucode = rec + a.up_codes + row0 * (H / 2) + 16 * c0;
  const uint8_t* gsc = rec + a.gate_sc + row0 * G * 4 + 4 * (c0 >> 1);
  const uint8_t* usc = rec + a.up_sc + row0 * G * 4 + 4 * (c0 >> 1);
  auto load = [&](int it, uint4 (&cd)[8], uint32_t (&sc)[8]) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const size_t r = (size_t)(4 * (p & 3));
      cd[p] = *reinterpret_cast<const uint4*>((p < 4 ? gcode : ucode) + r * (H / 2) + 256 * it);
      sc[p] = *reinterpret_cast<const uint32_t*>((p < 4 ? gsc : usc) + r * G * 4 + 32 * it);
    }
  };
  uint4 cdA[8];
  uint32_t scA[8];
  load(0, cdA, scA);
  // the tokens' activations, paired, and their chunk sums
  for (int q = tid; q < nrow * NCH; q += 256) {
    const int m = q / NCH, c = q % NCH;
    const int tok = e < a.E ? a.perm[base + m] / a.k : r0 + m;
    const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)tok * H + 32 * c);
    uint32_t xr[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 v = src[u];
      xr[4 * u] = v.x, xr[4 * u + 1] = v.y, xr[4 * u + 2] = v.z, xr[4 * u + 3] = v.w;
    }
    const XChunk<4> xc = x_chunk<4>(xr);
    uint4* d = reinterpret_cast<uint4*>(xp + (size_t)(m * NCH + c) * 16);
#pragma unroll
    for (int u = 0; u < 4; ++u) d[u] = make_uint4(xc.p[4 * u], xc.p[4 * u + 1], xc.p[4 * u + 2], xc.p[4 * u + 3]);
    xsm[m * NCH + c] = xc.s;
  }
  __syncthreads();
  float acc[8][kSmallRows];
#pragma unroll
  for (int p = 0; p < 8; ++p)
#pragma unroll
    for (int m = 0; m < kSmallRows; ++m) acc[p][m] = 0.f;
#pragma unroll
  for (int it = 0; it < NP; ++it) {
    uint4 cdB[8];
    uint32_t scB[8];
    if (it + 1 < NP) load(it + 1, cdB, scB);
    const int c = c0 + 16 * it;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t q[4][16];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) code_pairs4(cdA[4 * half + pp], q[pp]);
#pragma unroll
      for (int m = 0; m < kSmallRows; ++m) {
        if (m < nrow) {  // uniform
          uint32_t xv[16];
          const uint4* xs4 = reinterpret_cast<const uint4*>(xp + (size_t)(m * NCH + c) * 16);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint4 v = xs4[u];
            xv[4 * u] = v.x, xv[4 * u + 1] = v.y, xv[4 * u + 2] = v.z, xv[4 * u + 3] = v.w;
          }
          const float xs = xsm[m * NCH + c];
#pragma unroll
          for (int pp = 0; pp < 4; ++pp)
            acc[4 * half + pp][m] += pairs_term(q[pp], scA[4 * half + pp], xv, xs);
        }
      }
    }
    if (it + 1 < NP) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        cdA[p] = cdB[p];
        scA[p] = scB[p];
      }
    }
  }
  // row totals in lane c0 = 15 of each row's 16 lanes; h to LDS (rows past
  // the tile's end as zeros)
#pragma unroll
  for (int m = 0; m < kSmallRows; ++m) {
#pragma unroll
    for (int p = 0; p < 8; ++p) acc[p][m] = dpp::group_sum<16>(acc[p][m]);
  }
  if (c0 == 15) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int nl = 16 * wv + 4 * p + rsub;
#pragma unroll
      for (int m = 0; m < kSmallRows; ++m) sg[m * SGS + nl] = m < nrow ? silu_mul(acc[p][m], acc[p + 4][m]) : 0.f;
    }
  }
  for (int q = tid; q < (BM - kSmallRows) * GU_BN; q += 256)
    sg[(kSmallRows + q / GU_BN) * SGS + q % GU_BN] = 0.f;
  __syncthreads();
  gateup_store_h(a, sg, nrow, tile, nt, base, n0, tid, wv, lane);
}

__global__ void __launch_bounds__(256, 2) gemm_gateup_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int32_t s_tok[BM];
  __shared__ float s_xs[BM];  // token scale of each row
  const int G = a.H / 64, NQ = G / 4, NT = (a.I + GU_BN - 1) / GU_BN;
  int nt = 0;
  const int tile = xcd_tile(a.tiles[0], (a.T + BM - 1) / BM, NT, nt);
  if (tile < 0) return;
  const int4 td = *reinterpret_cast<const int4*>(a.tiles + 4 + 4 * tile);
  const int e = td.x, r0 = td.y, base = td.z;
  const int nrow = td.w;  // rows of this tile (>= 1)
  const int n0 = nt * GU_BN;
  const uint8_t* rec = e < a.E ? a.experts + (uint64_t)e * a.stride : a.shared;
  if (small_tiles_ok(a.H) && __builtin_amdgcn_readfirstlane(nrow) <= kSmallRows) {
    switch (a.H / 512) {
      case 1: gateup_small<1>(a, smem, tile, nt, e, r0, base, nrow, rec); break;
      case 2: gateup_small<2>(a, smem, tile, nt, e, r0, base, nrow, rec); break;
      case 3: gateup_small<3>(a, smem, tile, nt, e, r0, base, nrow, rec); break;
      default: gateup_small<4>(a, smem, tile, nt, e, r0, base, nrow, rec); break;
    }
    return;
  }
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  uint8_t* sA = smem;                                       // [NA][64 rows][8 slots of 16 B]
  uint8_t* sB = sA + GU_NA * A_STAGE;                       // [2][128 rows][8 slots of 16 B] (4 groups)
  uint8_t* sS = sB + 2 * BQ_STAGE;                          // [2][128 rows][4 words]

  GateUpSources src;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 32 * wv + 8 * t + (lane >> 3), chunk = (lane & 7) ^ swz(row);
    const int n = min(n0 + (row & (GU_BN - 1)), a.I - 1);
    src.b[t] = rec + (row < GU_BN ? a.gate_codes : a.up_codes) + (size_t)n * (a.H / 2) + 16 * chunk;
  }
  {
    const int row = 32 * wv + (lane & 31);
    const int n = min(n0 + (row & (GU_BN - 1)), a.I - 1);
    src.s = rec + (row < GU_BN ? a.gate_sc : a.up_sc) + (size_t)n * G * 4;
  }
  // quad 0 of codes and scales first: they do not depend on the tile's tokens
#pragma unroll
  for (int t = 0; t < 4; ++t) dma16(src.b[t], sB + (4 * wv + t) * 1024);
  if (lane < 32) dma16(src.s, sS + wv * 512);

  // A tile of at most 32 rows leaves the second 32-row MFMA tile of every
  // wave out (its accumulator stays zero and is never stored).
  const bool full = __builtin_amdgcn_readfirstlane(nrow) > 32;
  int tok = -1;
  if (tid < BM) {
    if (tid < nrow) tok = e < a.E ? a.perm[base + tid] / a.k : r0 + tid;
    s_tok[tid] = tok;
  }
  __syncthreads();
  // the token scales are needed only in the epilogue: loaded beside the
  // first A DMAs
  const float xs = tok >= 0 ? a.xscale[tok] : 1.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 8 * (2 * wv + t) + (lane >> 3), chunk = (lane & 7) ^ swz(row);
    src.a[t] = a.xp + (size_t)max(s_tok[row], 0) * a.H + 8 * chunk;
    src.a_live[t] = s_tok[row] >= 0 || lane == 0;
  }
  for (int g = 0; g < GU_PF; ++g) {
    const int gc = min(g, G - 1);
    if (src.a_live[0]) dma16(src.a[0] + 64 * gc, sA + g * A_STAGE + (2 * wv) * 1024);
    if (src.a_live[1]) dma16(src.a[1] + 64 * gc, sA + g * A_STAGE + (2 * wv + 1) * 1024);
  }

  const int mat = wv >> 1;
  const int nl = 32 * (wv & 1) + (lane & 31);  // column within the block
  const int brow = GU_BN * mat + nl;           // code / scale row within the block
  const int hh = lane >> 5;
  const int mrow = lane & 31;
  f32x16 acc0 = {}, acc1 = {};
  if (full)
    gateup_loop<true>(sA, sB, sS, src, G, NQ, wv, lane, brow, hh, mrow, acc0, acc1);
  else
    gateup_loop<false>(sA, sB, sS, src, G, NQ, wv, lane, brow, hh, mrow, acc0, acc1);
  // Epilogue. Gate and up tiles go through LDS (the rings are idle once no
  // DMA is in flight) so that all four waves share the SwiGLU arithmetic.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (tid < BM) s_xs[tid] = xs;
  __syncthreads();
  constexpr int SGS = GU_BN + 1;  // padded row stride (floats)
  static_assert(BM * SGS * 4 <= GU_NA * A_STAGE, "gate tile must fit the A ring");
  static_assert(BM * SGS * 4 <= 2 * BQ_STAGE, "up tile must fit the code ring");
  float* sg = reinterpret_cast<float*>(sA);  // [64][SGS]: gate, then h
  float* su = reinterpret_cast<float*>(sB);  // [64][SGS]: up
  {
    float* dst = mat == 0 ? sg : su;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = (r >> 2) * 8 + hh * 4 + (r & 3);
      dst[m * SGS + nl] = acc0[r] * s_xs[m];  // powers of two: exact
      dst[(32 + m) * SGS + nl] = acc1[r] * s_xs[32 + m];
    }
  }
  __syncthreads();
  {
    // h = silu(gate) * up, thread (tid / 64 + 4 j, tid % 64); hardware exp2
    // and reciprocal
    const int c = tid & 63;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int m = (tid >> 6) + 4 * j;
      const float gt = sg[m * SGS + c];
      sg[m * SGS + c] = silu_mul(gt, su[m * SGS + c]);
    }
  }
  __syncthreads();
  gateup_store_h(a, sg, nrow, tile, nt, base, n0, tid, wv, lane);
}

// ------------------------------------------------------- grouped GEMM 2 ---
// Block = (tile, 256 output columns of H), 4 waves, two blocks per CU: 64
// rows of one expert x 256 columns; wave w computes columns [64w, 64w + 64)
// as 2 x 2 tiles of 32x32x16 fp16 MFMA. A = h / 2^e in fp16 (2^e the
// (tile, group) scale from the gate/up kernel, folded into the group's
// weight scale), B = the codes as fp16 16 + q, K over the 64-groups of I. A
// tile where some rows carry their own range factor (rows far below the
// tile's largest) runs a copy of the K loop that multiplies those rows'
// partial sums by their factors before the group scale.
// Operands move by global->LDS DMA into DN_NS-stage rings, DN_PF groups
// ahead, 5 DMAs per wave per group (h 2, codes 2, scales 1); the affine term
// uses the per-group sums of h written by the gate/up kernel. Output:
// y[pair][n] = weight * acc (one fp32 row per (token, slot), the shared
// expert's rows after them).
constexpr int DN_BN = 256;                 // H columns per block
constexpr int DN_NS = 3;                   // ring stages
constexpr int DN_PF = DN_NS - 1;           // prefetch distance in groups
constexpr int DA_STAGE = BM * 64 * 2;      // 64 rows x 64 fp16
constexpr int DB_STAGE = DN_BN * 32;       // 256 code rows x 64 int4
constexpr int DS_STAGE = DN_BN * 4;        // 256 (s, c) words

size_t down_lds_bytes(int GI) { return (size_t)DN_NS * (DA_STAGE + DB_STAGE + DS_STAGE) + (size_t)2 * 256 * GI; }

struct DownSources {
  const uint16_t* h[2];   // A (instruction t): row 8 (2w + t) + lane / 8, chunk (lane % 8) ^ (row % 8)
  bool live[2];
  const uint8_t* b[2];    // code rows: instruction t covers rows 64w + 32t + lane / 2, tile half lane % 2
  const uint8_t* s;       // scale word of row 64w + lane
  size_t bq, sq;          // bytes from one I group to the next: codes (2 tiles of H rows), scales (H words)
};

// DMAs of group gn into the free stages; the restrict qualifiers keep the
// compiler from ordering them against this group's LDS reads (the caller's
// wait + barrier does).
__device__ __forceinline__ void down_issue(uint8_t* __restrict__ wrH, uint8_t* __restrict__ wrB,
                                           uint8_t* __restrict__ wrS, const DownSources& src, int gn, int wv) {
  dma16(src.b[0] + (size_t)gn * src.bq, wrB + (2 * wv) * 1024);
  dma16(src.b[1] + (size_t)gn * src.bq, wrB + (2 * wv + 1) * 1024);
  dma4(src.s + (size_t)gn * src.sq, wrS + wv * 256);
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (src.live[t]) dma16(src.h[t] + 64 * gn, wrH + (2 * wv + t) * 1024);
}

// One group: acc += s * 2^e * A . (16 + q); for an odd group also the affine
// term of the pair (g - 1, g) (lanes of k-half hh take group g-1+hh). Rows
// 32..63 only for a tile that has them (FULL).
template <bool FULL, bool MIXED>
__device__ __forceinline__ void down_group(const uint8_t* __restrict__ rdH, const uint8_t* __restrict__ rdB,
                                           const uint8_t* __restrict__ rdS, const float* __restrict__ sHs,
                                           const float* __restrict__ sRf, float hscale, uint8_t* __restrict__ wrH,
                                           uint8_t* __restrict__ wrB,
                                           uint8_t* __restrict__ wrS, const DownSources& src, int gn, int g,
                                           int wv, int brow, int hh, int mrow, float (&cprev)[2],
                                           f32x16 (&acc)[4], const NibConst& nk) {
  down_issue(wrH, wrB, wrS, src, gn, wv);
  f16x8 ah[2][4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int off = ((4 * hh + st) ^ swz(mrow)) * 16;  // swz(32 + mrow) == swz(mrow)
    ah[0][st] = *reinterpret_cast<const f16x8*>(rdH + mrow * 128 + off);
    if constexpr (FULL) ah[1][st] = *reinterpret_cast<const f16x8*>(rdH + (32 + mrow) * 128 + off);
  }
  float cval[2];
#pragma unroll
  for (int nn = 0; nn < 2; ++nn) {
    const int crow = brow + 32 * nn;  // 32-byte rows: tile half t sits in half t ^ ((row >> 3) & 1)
    const uint4 cw = *reinterpret_cast<const uint4*>(rdB + crow * 32 + (hh ^ ((crow >> 3) & 1)) * 16);
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(rdS + (brow + 32 * nn) * 4);
    const f16x8 b[4] = {nib_to_f16(cw.x, nk), nib_to_f16(cw.y, nk), nib_to_f16(cw.z, nk), nib_to_f16(cw.w, nk)};
    f32x16 p0 = {}, p1 = {};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[0][st], b[st], p0, 0, 0, 0);
      if constexpr (FULL) p1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[1][st], b[st], p1, 0, 0, 0);
    }
    if constexpr (MIXED) {
      // rows with their own range scale: 2^(e_row - T) on their partial sums
      // (exact); lane rows (r / 4) * 8 + 4 hh + r % 4 are four runs of four
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 f0 = *reinterpret_cast<const float4*>(sRf + g * 64 + 8 * i + 4 * hh);
        p0[4 * i] *= f0.x;
        p0[4 * i + 1] *= f0.y;
        p0[4 * i + 2] *= f0.z;
        p0[4 * i + 3] *= f0.w;
        if constexpr (FULL) {
          const float4 f1 = *reinterpret_cast<const float4*>(sRf + g * 64 + 32 + 8 * i + 4 * hh);
          p1[4 * i] *= f1.x;
          p1[4 * i + 1] *= f1.y;
          p1[4 * i + 2] *= f1.z;
          p1[4 * i + 3] *= f1.w;
        }
      }
    }
    const float sv = f16f(sw & 0xFFFFu);
    const float svh = sv * hscale;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[2 * nn][r] = fmaf(svh, p0[r], acc[2 * nn][r]);
    if constexpr (FULL) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[2 * nn + 1][r] = fmaf(svh, p1[r], acc[2 * nn + 1][r]);
    }
    cval[nn] = fmaf(-16.0f, sv, f16f(sw >> 16));
  }
  if (g & 1) {
    const int gx = g - 1 + hh;
    const float x0 = sHs[gx * 64 + mrow], x1 = sHs[gx * 64 + 32 + mrow];
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const float cp = hh ? cval[nn] : cprev[nn];
      acc[2 * nn] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, cp, acc[2 * nn], 0, 0, 0);
      if constexpr (FULL) acc[2 * nn + 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, cp, acc[2 * nn + 1], 0, 0, 0);
    }
  } else {
    cprev[0] = cval[0];
    cprev[1] = cval[1];
  }
}

// The K loop of a down block, instantiated for tiles of more than 32 rows
// (FULL) and for the rest, so neither copy branches inside the loop.
template <bool FULL, bool MIXED>
__device__ __forceinline__ void down_loop(uint8_t* sH, uint8_t* sB, uint8_t* sS, const float* sHs, const float* sRf,
                                          const float* s_hscale, const DownSources& src, int GI, int wv, int brow,
                                          int hh, int mrow, float (&cprev)[2], f32x16 (&acc)[4], const NibConst& nk) {
  // Waits (PF = 2): step 0 needs A(0), after which only A(1) (2 DMAs) was
  // issued; step g >= 1 needs group g, issued one step (5 DMAs) earlier.
  static_assert(DN_PF == 2, "wait counts below are written for PF = 2");
  for (int g = 0; g < GI; ++g) {
    if (g == 0)
      __builtin_amdgcn_s_waitcnt(0x0070 | 2);
    else
      __builtin_amdgcn_s_waitcnt(0x0070 | 5);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // no LDS read moves above the barrier
    const int rd = g % DN_NS, wr = (g + DN_PF) % DN_NS;
    down_group<FULL, MIXED>(sH + rd * DA_STAGE, sB + rd * DB_STAGE, sS + rd * DS_STAGE, sHs, sRf, s_hscale[g],
                     sH + wr * DA_STAGE, sB + wr * DB_STAGE, sS + wr * DS_STAGE, src, min(g + DN_PF, GI - 1), g, wv,
                     brow, hh, mrow, cprev, acc, nk);
  }
}

__global__ void __launch_bounds__(256, 2) gemm_down_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int32_t s_dst[BM];
  __shared__ float s_w[BM];
  const int GI = a.I / 64, NT = a.H / DN_BN;
  int nt = 0;
  const int tile = xcd_tile(a.tiles[0], (a.T + BM - 1) / BM, NT, nt);
  if (tile < 0) return;
  const int4 td = *reinterpret_cast<const int4*>(a.tiles + 4 + 4 * tile);
  const int e = td.x, r0 = td.y, base = td.z;
  const int nrow = td.w;  // rows of this tile (>= 1)
  const int n0 = nt * DN_BN;
  const uint8_t* rec = e < a.E ? a.experts + (uint64_t)e * a.stride : a.shared;
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  __shared__ float s_hscale[64];
  uint8_t* sH = smem;                                               // [NS][64][8 slots of 16 B]
  uint8_t* sB = sH + DN_NS * DA_STAGE;                              // [NS][256 rows][32 B]
  uint8_t* sS = sB + DN_NS * DB_STAGE;                              // [NS][256 rows] words
  float* sHs = reinterpret_cast<float*>(sS + DN_NS * DS_STAGE);     // [GI][64 rows] group sums of h
  float* sRf = sHs + 64 * GI;                                       // [GI][64 rows] row factors

  DownSources src;
  // down codes are stored in 16-byte tiles [I/32][H][16 B] (group g = tiles
  // 2g, 2g + 1) and the (s, c) words group-major [I/64][H]
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int q = (2 * wv + t) * 64 + lane, row = q >> 1;
    src.b[t] = rec + a.down_codes + ((size_t)((q & 1) ^ ((row >> 3) & 1)) * a.H + n0 + row) * 16;
  }
  src.s = rec + a.down_sc + (size_t)(n0 + 64 * wv + lane) * 4;
  src.bq = (size_t)2 * a.H * 16;
  src.sq = (size_t)a.H * 4;
  for (int g = 0; g < DN_PF; ++g) {
    const int gc = min(g, GI - 1);
    dma16(src.b[0] + (size_t)gc * src.bq, sB + g * DB_STAGE + (2 * wv) * 1024);
    dma16(src.b[1] + (size_t)gc * src.bq, sB + g * DB_STAGE + (2 * wv + 1) * 1024);
    dma4(src.s + (size_t)gc * src.sq, sS + g * DS_STAGE + wv * 256);
  }
  // destination rows, router weights and the h scales: independent loads,
  // in flight together with the h DMAs below
  int dst = -1;
  float w = 0.f, hs = 1.f;
  if (tid < nrow) {
    if (e < a.E) {
      dst = a.perm[base + tid];
      w = a.wperm[base + tid];
    } else {
      dst = a.T * a.k + r0 + tid;
      w = a.route_gamma[r0 + tid];
    }
  }
  if (tid < GI) hs = a.hscale[(size_t)tile * GI + tid];
  // A tile of at most 32 rows leaves the second 32-row MFMA tile of every
  // wave out (its accumulators stay zero and are never stored).
  const bool full = __builtin_amdgcn_readfirstlane(nrow) > 32;
  // h group sums and row factors: instruction g loads group g of the 64 rows
  {
    const size_t hrow = (size_t)base + min(lane, nrow - 1);
    for (int g = wv; g < GI; g += 4) {
      dma4(a.hsum + hrow * GI + g, reinterpret_cast<uint8_t*>(sHs) + g * 256);
      dma4(a.hrowf + hrow * GI + g, reinterpret_cast<uint8_t*>(sRf) + g * 256);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 8 * (2 * wv + t) + (lane >> 3), chunk = (lane & 7) ^ swz(row);
    const size_t hrow = (size_t)base + min(row, nrow - 1);
    src.h[t] = a.h16 + hrow * a.I + 8 * chunk;
    src.live[t] = row < nrow || lane == 0;
  }
  for (int g = 0; g < DN_PF; ++g) {
    const int gc = min(g, GI - 1);
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (src.live[t]) dma16(src.h[t] + 64 * gc, sH + g * DA_STAGE + (2 * wv + t) * 1024);
  }
  if (tid < BM) {
    s_dst[tid] = dst;
    s_w[tid] = w;
  }
  // tile-group scales 2^T; a negative entry marks a group where some rows
  // carry their own factor, and the block then runs the loop that applies them
  __shared__ uint32_t s_mixed;
  if (tid < GI) s_hscale[tid] = fabsf(hs);
  if (wv == 0) {
    const uint64_t b = __ballot(tid < GI && hs < 0.f);
    if (lane == 0) s_mixed = b != 0;
  }
  __syncthreads();
  const bool mixed = __builtin_amdgcn_readfirstlane(s_mixed) != 0;
  const int nl = 64 * wv + (lane & 31);  // first column of this lane (second: + 32)
  const int brow = nl;
  const int hh = lane >> 5;
  const int mrow = lane & 31;
  f32x16 acc[4] = {};
  float cprev[2] = {0.f, 0.f};
  const NibConst nk = nib_const();
  if (mixed) {
    if (full)
      down_loop<true, true>(sH, sB, sS, sHs, sRf, s_hscale, src, GI, wv, brow, hh, mrow, cprev, acc, nk);
    else
      down_loop<false, true>(sH, sB, sS, sHs, sRf, s_hscale, src, GI, wv, brow, hh, mrow, cprev, acc, nk);
  } else {
    if (full)
      down_loop<true, false>(sH, sB, sS, sHs, sRf, s_hscale, src, GI, wv, brow, hh, mrow, cprev, acc, nk);
    else
      down_loop<false, false>(sH, sB, sS, sHs, sRf, s_hscale, src, GI, wv, brow, hh, mrow, cprev, acc, nk);
  }
  if (GI & 1) {  // odd group count: the last group's affine term, paired with zeros
    const float x0 = hh ? 0.f : sHs[(GI - 1) * 64 + mrow], x1 = hh ? 0.f : sHs[(GI - 1) * 64 + 32 + mrow];
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const float cp = hh ? 0.f : cprev[nn];
      acc[2 * nn] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, cp, acc[2 * nn], 0, 0, 0);
      acc[2 * nn + 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, cp, acc[2 * nn + 1], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no DMA in flight at exit
  // Epilogue: the tile's y rows. Each wave stages its 64 x 64 results in LDS,
  // 32 columns at a time, and writes every destination row as a 128-byte run
  // of 16-byte stores (scattered 4-byte stores had made this phase a third of
  // the block's life). The rings are free once every wave has left the loop.
  __syncthreads();
  constexpr int YS = 40;  // staged row stride in floats: rows m and m + 4 fall in opposite bank halves
  static_assert(4 * BM * YS * 4 <= DN_NS * (DA_STAGE + DB_STAGE + DS_STAGE), "y staging must fit the rings");
  float* sy = reinterpret_cast<float*>(smem) + wv * (BM * YS);
#pragma unroll
  for (int nn = 0; nn < 2; ++nn) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m0 = (r >> 2) * 8 + hh * 4 + (r & 3);
      sy[m0 * YS + mrow] = s_w[m0] * acc[2 * nn][r];
      sy[(32 + m0) * YS + mrow] = s_w[32 + m0] * acc[2 * nn + 1][r];
    }
    // a wave's LDS operations complete in issue order: the reads below see
    // the writes above, and the next pass's writes follow these reads
    const int c4 = lane & 7;
    float* ydst = a.y + n0 + 64 * wv + 32 * nn + 4 * c4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = 8 * i + (lane >> 3);
      const float4 v = *reinterpret_cast<const float4*>(sy + m * YS + 4 * c4);
      const int dst = s_dst[m];
      if (dst >= 0) *reinterpret_cast<float4*>(ydst + (size_t)dst * a.H) = v;
    }
  }
}

// ------------------------------------------- plain (scalar) GEMM variants ---
// The two grouped GEMMs written plainly: one wave per block, no LDS rings, no
// DMA, no prefetch, every operand read from global memory right before the
// MFMA that uses it, the fast block's four waves done one after another. For
// every output tile they issue the fast kernels' MFMAs with the same operands
// in the same K order and repeat the epilogues' arithmetic (the shared
// helpers above), so their results equal the fast kernels' bit for bit.
// Rows past a tile's end hold zeros here and stale values in the fast
// kernels; neither is ever stored or folded into a kept value. Block b takes
// tile b / NT, column block b % NT.

// 8 fp16 of a stored row (the k-permuted fp16 x of a token, or a bucketed row
// of h): chunk c of 64-group g.
__device__ __forceinline__ f16x8 ld_frag(const uint16_t* rowp, int g, int c) {
  return *reinterpret_cast<const f16x8*>(rowp + 64 * g + 8 * c);
}

// A small tile (at most kSmallRows rows) as the fast small-tile path computes
// it: thread = column of the block; each row's 16 lane partials (a lane's
// chunks c0, c0 + 16, ... in order) summed pairwise like the lanes' DPP
// reduction; rows past the tile's end as zeros.
template <int NP>
__device__ void gateup_small_plain(const GemmArgs& a, float (*sg)[GU_BN + 1], int e, int r0, int base, int nrow,
                                   const uint8_t* rec, int n0) {
  constexpr int H = 512 * NP, G = H / 64;
  const int nl = threadIdx.x;
  const int n = n0 + nl;
  for (int m = 0; m < BM; ++m) {
    if (m >= nrow) {
      sg[m][nl] = 0.f;
      continue;
    }
    const int tok = e < a.E ? a.perm[base + m] / a.k : r0 + m;
    float tot[2];
    for (int mat = 0; mat < 2; ++mat) {
      const uint8_t* crow = rec + (mat == 0 ? a.gate_codes : a.up_codes) + (size_t)n * (H / 2);
      const uint8_t* srow = rec + (mat == 0 ? a.gate_sc : a.up_sc) + (size_t)n * G * 4;
      float part[16];
      for (int c0 = 0; c0 < 16; ++c0) {
        float acc = 0.f;
        for (int it = 0; it < NP; ++it) {
          const int c = c0 + 16 * it;
          uint32_t xr[16];
          for (int u = 0; u < 16; ++u)
            xr[u] = (uint32_t)a.x[(size_t)tok * H + 32 * c + 2 * u] | ((uint32_t)a.x[(size_t)tok * H + 32 * c + 2 * u + 1] << 16);
          const XChunk<4> xc = x_chunk<4>(xr);
          uint32_t q[16];
          code_pairs4(*reinterpret_cast<const uint4*>(crow + 16 * c), q);
          acc += pairs_term(q, *reinterpret_cast<const uint32_t*>(srow + 4 * (c >> 1)), xc.p, xc.s);
        }
        part[c0] = acc;
      }
      for (int w = 1; w < 16; w *= 2)
        for (int i = 0; i < 16; i += 2 * w) part[i] = part[i] + part[i + w];
      tot[mat] = part[0];
    }
    sg[m][nl] = silu_mul(tot[0], tot[1]);
  }
}

__global__ void __launch_bounds__(64) gemm_gateup_plain_kernel(GemmArgs a) {
  __shared__ float sg[BM][GU_BN + 1], su[BM][GU_BN + 1];
  __shared__ float s_xs[BM];
  __shared__ int32_t s_tok[BM];
  __shared__ uint32_t s_nb[BM];
  const int G = a.H / 64, NT = (a.I + GU_BN - 1) / GU_BN;
  const int tile = (int)blockIdx.x / NT, nt = (int)blockIdx.x % NT;
  if (tile >= a.tiles[0]) return;
  const int4 td = *reinterpret_cast<const int4*>(a.tiles + 4 + 4 * tile);
  const int e = td.x, r0 = td.y, base = td.z, nrow = td.w;
  const int n0 = nt * GU_BN;
  const uint8_t* rec = e < a.E ? a.experts + (uint64_t)e * a.stride : a.shared;
  const int lane = threadIdx.x, hh = lane >> 5, mrow = lane & 31;
  {
    const int tok = lane < nrow ? (e < a.E ? a.perm[base + lane] / a.k : r0 + lane) : -1;
    s_tok[lane] = tok;
    s_xs[lane] = tok >= 0 ? a.xscale[tok] : 1.f;
  }
  __syncthreads();
  if (small_tiles_ok(a.H) && nrow <= kSmallRows) {
    switch (a.H / 512) {
      case 1: gateup_small_plain<1>(a, sg, e, r0, base, nrow, rec, n0); break;
      case 2: gateup_small_plain<2>(a, sg, e, r0, base, nrow, rec, n0); break;
      case 3: gateup_small_plain<3>(a, sg, e, r0, base, nrow, rec, n0); break;
      default: gateup_small_plain<4>(a, sg, e, r0, base, nrow, rec, n0); break;
    }
  } else {
    const int tok0 = s_tok[mrow], tok1 = s_tok[32 + mrow];
    const NibConst nk = nib_const();
    for (int wv = 0; wv < 4; ++wv) {
      const int mat = wv >> 1, nl = 32 * (wv & 1) + mrow;
      const int n = min(n0 + nl, a.I - 1);
      const uint8_t* crow = rec + (mat == 0 ? a.gate_codes : a.up_codes) + (size_t)n * (a.H / 2);
      const uint8_t* srow = rec + (mat == 0 ? a.gate_sc : a.up_sc) + (size_t)n * G * 4;
      f32x16 acc0 = {}, acc1 = {};
      for (int g = 0; g < G; ++g) {
        GroupFrag f;
        f.codes = *reinterpret_cast<const uint4*>(crow + 32 * g + 16 * hh);
        f.sc = *reinterpret_cast<const uint32_t*>(srow + 4 * g);
        for (int st = 0; st < 4; ++st) {
          f.a0[st] = tok0 >= 0 ? ld_frag(a.xp + (size_t)tok0 * a.H, g, 4 * hh + st) : f16x8{};
          f.a1[st] = tok1 >= 0 ? ld_frag(a.xp + (size_t)tok1 * a.H, g, 4 * hh + st) : f16x8{};
        }
        gateup_dequant(f, nk);
        gateup_mfma<true>(f, acc0, acc1);
      }
      float(*dst)[GU_BN + 1] = mat == 0 ? sg : su;
      for (int r = 0; r < 16; ++r) {
        const int m = (r >> 2) * 8 + hh * 4 + (r & 3);
        dst[m][nl] = acc0[r] * s_xs[m];
        dst[32 + m][nl] = acc1[r] * s_xs[32 + m];
      }
    }
    __syncthreads();
    for (int m = 0; m < BM; ++m) sg[m][lane] = silu_mul(sg[m][lane], su[m][lane]);
    __syncthreads();
  }
  __syncthreads();
  // thread = row m
  const int m = lane;
  float rmax = 0.f;
  for (int c = 0; c < GU_BN; ++c) rmax = fmaxf(rmax, fabsf(sg[m][c]));
  s_nb[m] = row_exp_biased(rmax, m < nrow);
  __syncthreads();
  uint32_t tb = 0;
  for (int q = 0; q < BM; ++q) tb = max(tb, s_nb[q]);
  const int T = tb ? (int)tb - 256 : 0;
  const int er = row_exp(s_nb[m], T);
  const int GI = a.I / 64;
  float part[4];
  for (int qq = 0; qq < 4; ++qq) {
    uint32_t pk[8];
    part[qq] = pack16(&sg[m][16 * qq], er, pk);
    if (m < nrow) {
      uint16_t* hd = a.h16 + (size_t)(base + m) * a.I + n0 + 16 * qq;
      *reinterpret_cast<uint4*>(hd) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      *reinterpret_cast<uint4*>(hd + 8) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    }
  }
  if (m < nrow) {
    a.hsum[(size_t)(base + m) * GI + nt] = (part[0] + part[1]) + (part[2] + part[3]);
    a.hrowf[(size_t)(base + m) * GI + nt] = ldexpf(1.f, er - T);
  }
  const bool own = __ballot(m < nrow && er != T) != 0;
  if (lane == 0) {
    const float sc = ldexpf(1.f, T);
    a.hscale[(size_t)tile * GI + nt] = own ? -sc : sc;
  }
}

__global__ void __launch_bounds__(64) gemm_down_plain_kernel(GemmArgs a) {
  const int GI = a.I / 64, NT = a.H / DN_BN;
  const int tile = (int)blockIdx.x / NT, nt = (int)blockIdx.x % NT;
  if (tile >= a.tiles[0]) return;
  const int4 td = *reinterpret_cast<const int4*>(a.tiles + 4 + 4 * tile);
  const int e = td.x, r0 = td.y, base = td.z, nrow = td.w;
  const int n0 = nt * DN_BN;
  const uint8_t* rec = e < a.E ? a.experts + (uint64_t)e * a.stride : a.shared;
  const int lane = threadIdx.x, hh = lane >> 5, mrow = lane & 31;
  // the bucketed rows the fast kernel stages (rows past the end repeat the last)
  const size_t ra = (size_t)base + min(mrow, nrow - 1), rb = (size_t)base + min(32 + mrow, nrow - 1);
  const uint16_t* h0 = a.h16 + ra * a.I;
  const uint16_t* h1 = a.h16 + rb * a.I;
  const NibConst nk = nib_const();
  for (int wv = 0; wv < 4; ++wv) {
    const int brow = 64 * wv + mrow;
    f32x16 acc[4] = {};
    float cprev[2] = {0.f, 0.f};
    for (int g = 0; g < GI; ++g) {
      const float hscale = fabsf(a.hscale[(size_t)tile * GI + g]);
      f16x8 ah[2][4];
      for (int st = 0; st < 4; ++st) {
        ah[0][st] = ld_frag(h0, g, 4 * hh + st);
        ah[1][st] = ld_frag(h1, g, 4 * hh + st);
      }
      float cval[2];
      for (int nn = 0; nn < 2; ++nn) {
        const int n = n0 + brow + 32 * nn;
        const uint4 cw = *reinterpret_cast<const uint4*>(rec + a.down_codes + ((size_t)(2 * g + hh) * a.H + n) * 16);
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(rec + a.down_sc + ((size_t)g * a.H + n) * 4);
        const f16x8 b[4] = {nib_to_f16(cw.x, nk), nib_to_f16(cw.y, nk), nib_to_f16(cw.z, nk), nib_to_f16(cw.w, nk)};
        f32x16 p0 = {}, p1 = {};
        for (int st = 0; st < 4; ++st) {
          p0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[0][st], b[st], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[1][st], b[st], p1, 0, 0, 0);
        }
        // row factors (1 for every row of a tile-group without own factors)
        for (int r = 0; r < 16; ++r) {
          const int m = (r >> 2) * 8 + hh * 4 + (r & 3);
          p0[r] *= a.hrowf[((size_t)base + min(m, nrow - 1)) * GI + g];
          p1[r] *= a.hrowf[((size_t)base + min(32 + m, nrow - 1)) * GI + g];
        }
        const float sv = f16f(sw & 0xFFFFu);
        const float svh = sv * hscale;
        for (int r = 0; r < 16; ++r) acc[2 * nn][r] = fmaf(svh, p0[r], acc[2 * nn][r]);
        for (int r = 0; r < 16; ++r) acc[2 * nn + 1][r] = fmaf(svh, p1[r], acc[2 * nn + 1][r]);
        cval[nn] = fmaf(-16.0f, sv, f16f(sw >> 16));
      }
      if (g & 1) {
        const int gx = g - 1 + hh;
        const float x0 = a.hsum[ra * GI + gx], x1 = a.hsum[rb * GI + gx];
        for (int nn = 0; nn < 2; ++nn) {
          const float cp = hh ? cval[nn] : cprev[nn];
          acc[2 * nn] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, cp, acc[2 * nn], 0, 0, 0);
          acc[2 * nn + 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, cp, acc[2 * nn + 1], 0, 0, 0);
        }
      } else {
        cprev[0] = cval[0];
        cprev[1] = cval[1];
      }
    }
    if (GI & 1) {
      const float x0 = hh ? 0.f : a.hsum[ra * GI + GI - 1], x1 = hh ? 0.f : a.hsum[rb * GI + GI - 1];
      for (int nn = 0; nn < 2; ++nn) {
        const float cp = hh ? 0.f : cprev[nn];
        acc[2 * nn] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, cp, acc[2 * nn], 0, 0, 0);
        acc[2 * nn + 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, cp, acc[2 * nn + 1], 0, 0, 0);
      }
    }
    for (int nn = 0; nn < 2; ++nn) {
      const int n = n0 + brow + 32 * nn;
      for (int r = 0; r < 16; ++r) {
        for (int half = 0; half < 2; ++half) {
          const int m = (r >> 2) * 8 + hh * 4 + (r & 3) + 32 * half;
          if (m >= nrow) continue;
          const size_t dst = e < a.E ? (size_t)a.perm[base + m] : (size_t)a.T * a.k + r0 + m;
          const float w = e < a.E ? a.wperm[base + m] : a.route_gamma[r0 + m];
          a.y[dst * a.H + n] = w * acc[2 * nn + half][r];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ combine ---
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y, int T, int k, int H, float* out) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;  // one float4 of one token
  const size_t per = (size_t)H / 4;
  if (q >= (size_t)T * per) return;
  const size_t t = q / per, c = q % per;
  const float4* y4 = reinterpret_cast<const float4*>(y);
  float4 s = y4[(t * k) * per + c];
  for (int j = 1; j < k; ++j) {
    const float4 v = y4[(t * k + j) * per + c];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  const float4 v = y4[((size_t)T * k + t) * per + c];
  s.x += v.x;
  s.y += v.y;
  s.z += v.z;
  s.w += v.w;
  reinterpret_cast<float4*>(out)[q] = s;
}

template <class T>
bool grow(T*& p, size_t n) {
  hipFree(p);
  p = nullptr;
  return hipMalloc(&p, (n ? n : 1) * sizeof(T)) == hipSuccess;
}

Workspace* ws_of(void* p) { return static_cast<Workspace*>(p); }

int max_tiles_for(const moe_config& c, int T) {
  const size_t P = (size_t)T * c.top_k;
  return (int)((P + BM - 1) / BM) + c.n_experts + (T + BM - 1) / BM;
}

// The workspace arrays of a batch of up to T tokens, in one block: element
// counts and sizes, each array starting on a 256-byte boundary.
struct Placement {
  size_t off[16];
  size_t total;
};
Placement placement(const moe_config& c, int T) {
  const size_t E = c.n_experts, k = c.top_k, H = c.hidden, I = c.inter;
  const size_t P = (size_t)T * k, rows = P + T;
  const size_t nchunk = (P + CHUNK - 1) / CHUNK;
  const size_t mt = (size_t)max_tiles_for(c, T);
  const size_t bytes[16] = {
      (size_t)T * (E + 1) * 4,  // logits
      (size_t)T * 4,            // xscale
      (size_t)T * H * 2,        // xp
      nchunk * E * 4,           // cnt
      nchunk * E * 4,           // chunk_off
      P * 4,                    // perm
      P * 4,                    // wperm
      (4 + 4 * mt) * 4,         // tiles
      rows * I * 2,             // h16
      mt * (I / 64) * 4,        // hscale
      rows * (I / 64) * 4,      // hrowf
      rows * (I / 64) * 4,      // hsum
      rows * H * 4,             // y
      P * 4,                    // route_idx
      P * 4,                    // route_w
      (size_t)T * 4,            // route_gamma
  };
  Placement p{};
  size_t o = 0;
  for (int i = 0; i < 16; ++i) {
    p.off[i] = o;
    o += (bytes[i] + 255) / 256 * 256;
  }
  p.total = o;
  return p;
}

GemmArgs gemm_args(const Workspace* w, const PrefillArgs& pa) {
  GemmArgs ga{};
  ga.x = pa.x;
  ga.xscale = w->xscale;
  ga.xp = w->xp;
  ga.experts = pa.experts;
  ga.shared = pa.shared;
  ga.stride = pa.stride;
  ga.gate_codes = pa.geo.gate_codes;
  ga.up_codes = pa.geo.up_codes;
  ga.down_codes = pa.geo.down_codes;
  ga.gate_sc = pa.geo.gate_sc;
  ga.up_sc = pa.geo.up_sc;
  ga.down_sc = pa.geo.down_sc;
  ga.perm = w->perm;
  ga.wperm = w->wperm;
  ga.tiles = w->tiles;
  ga.route_w = pa.route_w;
  ga.route_gamma = pa.route_gamma;
  ga.h16 = w->h16;
  ga.hscale = w->hscale;
  ga.hrowf = w->hrowf;
  ga.hsum = w->hsum;
  ga.y = w->y;
  ga.T = pa.n_tok;
  ga.H = pa.cfg.hidden;
  ga.I = pa.cfg.inter;
  ga.E = pa.cfg.n_experts;
  ga.k = pa.cfg.top_k;
  return ga;
}

int n_chunks(const PrefillArgs& pa) { return (pa.n_tok * pa.cfg.top_k + CHUNK - 1) / CHUNK; }

}  // namespace

bool prefill_supported(const moe_config& cfg) {
  // the gate/up block loads the scale words 4 groups (16 bytes) at a time: H % 256 == 0
  return cfg.bits == 4 && cfg.hidden % 256 == 0 && cfg.inter % 64 == 0 && cfg.hidden / 64 <= 64 &&
         cfg.inter / 64 <= 64 && cfg.n_experts <= 1024 && cfg.top_k <= kTopkMax;
}

void prefill_free(void* ws) {
  if (!ws) return;
  Workspace* w = ws_of(ws);
  hipFree(w->logits);
  hipFree(w->xscale);
  hipFree(w->xp);
  hipFree(w->cnt);
  hipFree(w->chunk_off);
  hipFree(w->perm);
  hipFree(w->wperm);
  hipFree(w->tiles);
  hipFree(w->h16);
  hipFree(w->hscale);
  hipFree(w->hrowf);
  hipFree(w->hsum);
  hipFree(w->y);
  delete w;
}

size_t prefill_placed_bytes(const moe_config& cfg, int n_tok) { return placement(cfg, n_tok).total; }

void prefill_place(PrefillWorkspace* w, const moe_config& c, int T, uint8_t* base, int32_t** route_idx,
                   float** route_w, float** route_gamma) {
  const Placement p = placement(c, T);
  w->logits = reinterpret_cast<float*>(base + p.off[0]);
  w->xscale = reinterpret_cast<float*>(base + p.off[1]);
  w->xp = reinterpret_cast<uint16_t*>(base + p.off[2]);
  w->cnt = reinterpret_cast<int32_t*>(base + p.off[3]);
  w->chunk_off = reinterpret_cast<int32_t*>(base + p.off[4]);
  w->perm = reinterpret_cast<int32_t*>(base + p.off[5]);
  w->wperm = reinterpret_cast<float*>(base + p.off[6]);
  w->tiles = reinterpret_cast<int32_t*>(base + p.off[7]);
  w->h16 = reinterpret_cast<uint16_t*>(base + p.off[8]);
  w->hscale = reinterpret_cast<float*>(base + p.off[9]);
  w->hrowf = reinterpret_cast<float*>(base + p.off[10]);
  w->hsum = reinterpret_cast<float*>(base + p.off[11]);
  w->y = reinterpret_cast<float*>(base + p.off[12]);
  *route_idx = reinterpret_cast<int32_t*>(base + p.off[13]);
  *route_w = reinterpret_cast<float*>(base + p.off[14]);
  *route_gamma = reinterpret_cast<float*>(base + p.off[15]);
  w->T = T;
  w->E = c.n_experts;
  w->k = c.top_k;
  w->H = c.hidden;
  w->I = c.inter;
  w->max_tiles = max_tiles_for(c, T);
}

moe_status prefill_reserve(void** wsp, const moe_config& c, int T) {
  Workspace* w = ws_of(*wsp);
  if (!w) {
    w = new Workspace();
    *wsp = w;
  }
  const int E = c.n_experts, k = c.top_k, H = c.hidden, I = c.inter;
  if (w->T >= T && w->E == E && w->k == k && w->H == H && w->I == I) return MOE_OK;
  if (hipDeviceSynchronize() != hipSuccess) return MOE_EHIP;
  const size_t P = (size_t)T * k, rows = P + T;
  const int nchunk = (int)((P + CHUNK - 1) / CHUNK);
  const int max_tiles = max_tiles_for(c, T);
  w->T = 0;  // invalid until every buffer is in place
  const bool ok = grow(w->logits, (size_t)T * (E + 1)) && grow(w->xscale, (size_t)T) && grow(w->xp, (size_t)T * H) &&
                  grow(w->cnt, (size_t)nchunk * E) && grow(w->chunk_off, (size_t)nchunk * E) &&
                  grow(w->perm, P) && grow(w->wperm, P) &&
                  grow(w->tiles, (size_t)4 + 4 * max_tiles) &&
                  grow(w->h16, rows * I) && grow(w->hscale, (size_t)max_tiles * (I / 64)) &&
                  grow(w->hrowf, rows * (I / 64)) && grow(w->hsum, rows * (I / 64)) &&
                  grow(w->y, rows * H);
  if (!ok) return MOE_ENOMEM;
  w->T = T;
  w->E = E;
  w->k = k;
  w->H = H;
  w->I = I;
  w->max_tiles = max_tiles;
  return MOE_OK;
}

hipError_t prefill_xprep(void* ws, const PrefillArgs& pa, hipStream_t s) {
  Workspace* w = ws_of(ws);
  const int T = pa.n_tok, H = pa.cfg.hidden;
  const dim3 grid((T + 3) / 4), block(256);
  switch (H <= 512 ? 1 : H / 512) {
    case 1: launch(xprep_kernel<1>, grid, block, 0, s, pa.x, T, H, w->xscale, w->xp); break;
    case 2: launch(xprep_kernel<2>, grid, block, 0, s, pa.x, T, H, w->xscale, w->xp); break;
    case 4: launch(xprep_kernel<4>, grid, block, 0, s, pa.x, T, H, w->xscale, w->xp); break;
    case 8: launch(xprep_kernel<8>, grid, block, 0, s, pa.x, T, H, w->xscale, w->xp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t prefill_router(void* ws, const PrefillArgs& pa, hipStream_t s) {
  Workspace* w = ws_of(ws);
  const int T = pa.n_tok, H = pa.cfg.hidden, E = pa.cfg.n_experts;
  if (T <= kRouterRowsMaxT) {
    const dim3 grid((E + 1 + 3) / 4), block(512);
#define ROWS_LAUNCH(NIT, U) \
  launch(router_rows_kernel<NIT, U>, grid, block, 0, s, pa.wr_rows, pa.bias, pa.x, T, H, E, w->logits)
    switch ((H / 4 + 63) / 64) {  // float4 loads per lane
      case 1: ROWS_LAUNCH(1, 4); break;
      case 2: ROWS_LAUNCH(2, 4); break;
      case 4: ROWS_LAUNCH(4, 4); break;
      case 8: ROWS_LAUNCH(8, 4); break;
      case 16: ROWS_LAUNCH(16, 2); break;
      default: return hipErrorInvalidValue;
    }
#undef ROWS_LAUNCH
    return hipGetLastError();
  }
  launch(router_gemm_kernel, dim3((T + 127) / 128, (E + 1 + 63) / 64), dim3(512), 0, s, pa.x, pa.wr_split, pa.bias, T,
         H, E, w->logits);
  return hipGetLastError();
}

hipError_t prefill_route(void* ws, const PrefillArgs& pa, hipStream_t s) {
  Workspace* w = ws_of(ws);
  return launch_route(pa.geo, w->logits, pa.cfg.n_experts + 1, pa.n_tok, pa.route_idx, pa.route_w, pa.route_gamma,
                      nullptr, s);
}

hipError_t prefill_count(void* ws, const PrefillArgs& pa, hipStream_t s) {
  Workspace* w = ws_of(ws);
  const int E = pa.cfg.n_experts, P = pa.n_tok * pa.cfg.top_k;
  launch(bucket_count_kernel, dim3(n_chunks(pa)), dim3(CHUNK), (uint32_t)(E * sizeof(int32_t)), s, pa.route_idx, P, E,
         w->cnt);
  return hipGetLastError();
}

hipError_t prefill_scan(void* ws, const PrefillArgs& pa, hipStream_t s) {
  Workspace* w = ws_of(ws);
  launch(bucket_scan_kernel, dim3(1), dim3(1024), 0, s, w->cnt, n_chunks(pa), pa.cfg.n_experts, pa.n_tok,
         w->chunk_off, w->tiles, w->max_tiles);
  return hipGetLastError();
}

hipError_t prefill_scatter(void* ws, const PrefillArgs& pa, hipStream_t s) {
  Workspace* w = ws_of(ws);
  const int E = pa.cfg.n_experts, P = pa.n_tok * pa.cfg.top_k;
  launch(bucket_scatter_kernel, dim3(n_chunks(pa)), dim3(CHUNK), (uint32_t)((CHUNK / 64) * E * sizeof(int32_t)), s,
         pa.route_idx, pa.route_w, P, E, w->chunk_off, w->perm, w->wperm);
  return hipGetLastError();
}

hipError_t prefill_gateup(void* ws, const PrefillArgs& pa, hipStream_t s) {
  Workspace* w = ws_of(ws);
  const size_t lds = gateup_lds_bytes();
  // dynamic LDS above 64 KB has to be allowed per kernel (LDS is 160 KB per CU)
  static size_t attr_bytes = 0;
  if (attr_bytes < lds) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_gateup_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_bytes = lds;
  }
  if (pa.scalar) {
    const int nt = (pa.cfg.inter + GU_BN - 1) / GU_BN;
    launch(gemm_gateup_plain_kernel, dim3((unsigned)(w->max_tiles * nt)), dim3(64), 0, s, gemm_args(w, pa));
    return hipGetLastError();
  }
  const int nblk = xcd_grid(w->max_tiles, (pa.n_tok + BM - 1) / BM, (pa.cfg.inter + GU_BN - 1) / GU_BN);
  launch(gemm_gateup_kernel, dim3((unsigned)nblk), dim3(256), (uint32_t)lds, s, gemm_args(w, pa));
  return hipGetLastError();
}

hipError_t prefill_down(void* ws, const PrefillArgs& pa, hipStream_t s) {
  Workspace* w = ws_of(ws);
  const size_t lds = down_lds_bytes(pa.cfg.inter / 64);
  static size_t attr_bytes = 0;
  if (attr_bytes < lds) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_down_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_bytes = lds;
  }
  if (pa.scalar) {
    launch(gemm_down_plain_kernel, dim3((unsigned)(w->max_tiles * (pa.cfg.hidden / DN_BN))), dim3(64), 0, s,
           gemm_args(w, pa));
    return hipGetLastError();
  }
  const int nblk = xcd_grid(w->max_tiles, (pa.n_tok + BM - 1) / BM, pa.cfg.hidden / DN_BN);
  launch(gemm_down_kernel, dim3((unsigned)nblk), dim3(256), (uint32_t)lds, s, gemm_args(w, pa));
  return hipGetLastError();
}

hipError_t prefill_combine(void* ws, const PrefillArgs& pa, hipStream_t s) {
  Workspace* w = ws_of(ws);
  const size_t n4 = (size_t)pa.n_tok * pa.cfg.hidden / 4;
  launch(combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, w->y, pa.n_tok,
                     pa.cfg.top_k, pa.cfg.hidden, pa.out);
  return hipGetLastError();
}

}  // namespace moe
