// Plainly written ("scalar") variants of the decode expert kernel and of the
// batched path's grouped GEMMs, bit-identical to the fast kernels on the same
// inputs.
//
// Pages: the runtime keeps a fast and a scalar variant of its GPU kernels and
// its fixtures require the two to produce identical output (paotong.dev
// commentary, paragraph on the test fixtures). Here the scalar variants are a
// debugging reference on the GPU itself: no LDS staging, no DMA rings, no
// register pipelining, no cross-lane tricks; one thread per output value
// (decode) or one wave per MFMA output tile read straight from global memory
// (grouped GEMMs). They repeat the fast kernels' arithmetic operation for
// operation: the same per-chunk and per-group expressions (decode_math.h),
// the same association of every sum (a cross-lane reduction of the fast
// kernel becomes the same pairwise tree over an array here), the same MFMA
// instructions fed the same operands in the same K order. Selection results
// (top-k) are exact comparisons, so any correct algorithm gives the same
// picks; the weights repeat the fast routine's arithmetic.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_math.h"
#include "kernels.h"
#include "launch.h"
#include "scalar.h"

namespace moe {
namespace {

constexpr int kSlice = 32;  // I rows per partial row of the fused decode path

// Sum of v[0..n) (n a power of two <= 64) associated as the DPP reduction over
// n lanes: adjacent pairs, then adjacent pairs of pairs, and so on.
__device__ float tree_sum(float* v, int n) {
  for (int w = 1; w < n; w *= 2)
    for (int i = 0; i < n; i += 2 * w) v[i] = v[i] + v[i + w];
  return v[0];
}

// Order key of a logit (unsigned order = logit order; NaN ranks with -inf,
// -0 with +0) and its inverse, as in the fast routine.
__device__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) u = 0xFF800000u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ float key_value(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

// ------------------------------------------------------------ decode route ---
// One thread: the k largest (key, -e) in selection order by k passes over all
// E logits, then the renormalised weights exp(l - l_max) / sum, the sum
// associated as the fast routine's 64-lane reduction (lane q holds pick q,
// lanes >= k hold 0; norm_topk = 0: lane l holds the sum of exp(l_e - l_max)
// over e = l, l + 64, ... in that order).
__global__ void route_scalar_kernel(const float* __restrict__ logits, int E, int k, int norm_topk, int32_t* idx,
                                    float* w, float* gamma) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  uint32_t pk[16];
  int pe[16];
  uint64_t prev = ~0ull;
  for (int q = 0; q < k; ++q) {
    uint64_t best = 0;
    for (int e = 0; e < E; ++e) {
      const uint64_t p = ((uint64_t)order_key(logits[e]) << 32) | (uint32_t)~(uint32_t)e;
      if (p < prev && p > best) best = p;
    }
    prev = best;
    pk[q] = (uint32_t)(best >> 32);
    pe[q] = (int)~(uint32_t)best;
  }
  const float lmax = key_value(pk[0]);
  float lanes[64];
  float z[16];
  for (int l = 0; l < 64; ++l) lanes[l] = 0.f;
  for (int q = 0; q < k; ++q) z[q] = expf(key_value(pk[q]) - lmax);
  if (norm_topk) {
    for (int q = 0; q < k; ++q) lanes[q] = z[q];
  } else {
    for (int l = 0; l < 64; ++l) {
      float part = 0.f;
      for (int e = l; e < E; e += 64) part += expf(logits[e] - lmax);
      lanes[l] = part;
    }
  }
  const float s = tree_sum(lanes, 64);
  for (int q = 0; q < k; ++q) {
    idx[q] = pe[q];
    w[q] = z[q] / s;
  }
  gamma[0] = 1.0f / (1.0f + expf(-logits[E]));
}

// ----------------------------------------------------------- decode gate/up ---
// Thread (slot j, row i): h[j][i] = swiglu(gate_i . x, up_i . x), each dot the
// sum over LPR lane partials (lane c takes chunks c, c + LPR, ...: the chunk
// term s * sum(q x) + c * sum(x) of chunk_term, on the same activation pairs)
// associated as the fast kernel's reduction.
template <int BITS>
__global__ void gateup_scalar_kernel(Geometry g, const uint8_t* __restrict__ experts, uint64_t stride,
                                     int64_t gid_base, const uint8_t* __restrict__ shared_rec,
                                     const uint16_t* __restrict__ x, const int32_t* __restrict__ idx, float* h) {
  constexpr int EPC = 128 / BITS;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (g.k + 1) * g.I) return;
  const int j = t / g.I, i = t % g.I;
  const uint8_t* rec = j == g.k ? shared_rec : experts + (uint64_t)(gid_base + idx[j]) * stride;
  const int chunks = g.H * BITS / 128;
  const int lpr = chunks < 64 ? chunks : 64;
  const int groups = g.H / 64;
  const size_t row_bytes = (size_t)g.H * BITS / 8;
  float pg[64], pu[64];
  for (int c = 0; c < lpr; ++c) {
    float ag = 0.f, au = 0.f;
    for (int ch = c; ch < chunks; ch += lpr) {
      uint32_t xr[EPC / 2];
      for (int q = 0; q < EPC / 2; ++q) xr[q] = (uint32_t)x[ch * EPC + 2 * q] | ((uint32_t)x[ch * EPC + 2 * q + 1] << 16);
      const XChunk<BITS> xc = x_chunk<BITS>(xr);
      const uint4 cg = *reinterpret_cast<const uint4*>(rec + g.gate_codes + (size_t)i * row_bytes + 16 * ch);
      const uint4 cu = *reinterpret_cast<const uint4*>(rec + g.up_codes + (size_t)i * row_bytes + 16 * ch);
      const int grp = ch * EPC / 64;
      const uint32_t sg = *reinterpret_cast<const uint32_t*>(rec + g.gate_sc + ((size_t)i * groups + grp) * 4);
      const uint32_t su = *reinterpret_cast<const uint32_t*>(rec + g.up_sc + ((size_t)i * groups + grp) * 4);
      ag += chunk_term<BITS>(cg, sg, xc);
      au += chunk_term<BITS>(cu, su, xc);
    }
    pg[c] = ag;
    pu[c] = au;
  }
  h[(size_t)j * g.I + i] = swiglu(tree_sum(pg, lpr), tree_sum(pu, lpr));
}

// ------------------------------------------------------------- decode down ---
// Thread (slot j, 32-row slice sl, output n): the partial row the fast kernel's
// block (j, sl) writes at n: w_j * (s * sum_c chunk_dot(tile c of row n, h) +
// c * sum(h)) over the slice.
template <int BITS>
__global__ void down_scalar_kernel(Geometry g, const uint8_t* __restrict__ experts, uint64_t stride,
                                   int64_t gid_base, const uint8_t* __restrict__ shared_rec,
                                   const int32_t* __restrict__ idx, const float* __restrict__ w,
                                   const float* __restrict__ gamma, const float* __restrict__ h, float* partial) {
  constexpr int EPC = 128 / BITS;
  constexpr int DCH = kSlice / EPC;
  const int nsl = g.I / kSlice;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)(g.k + 1) * nsl * g.H) return;
  const int n = (int)(t % g.H);
  const int sl = (int)((t / g.H) % nsl);
  const int j = (int)(t / ((int64_t)g.H * nsl));
  const uint8_t* rec = j == g.k ? shared_rec : experts + (uint64_t)(gid_base + idx[j]) * stride;
  float hv[kSlice];
  for (int q = 0; q < kSlice; ++q) hv[q] = h[(size_t)j * g.I + sl * kSlice + q];
  float hs = 0.f;
  for (int q = 0; q < kSlice; ++q) hs += hv[q];
  float d = 0.f;
  for (int c = 0; c < DCH; ++c) {
    const uint4 cd = *reinterpret_cast<const uint4*>(rec + g.down_codes + ((size_t)(sl * DCH + c) * g.H + n) * 16);
    d += chunk_dot<BITS>(cd, hv + c * EPC);
  }
  const uint32_t sd = *reinterpret_cast<const uint32_t*>(rec + g.down_sc + ((size_t)(sl * kSlice / 64) * g.H + n) * 4);
  const float wj = j == g.k ? gamma[0] : w[j];
  partial[((size_t)j * nsl + sl) * g.H + n] = wj * group_term(sd, d, hs);
}

}  // namespace

hipError_t launch_expert_scalar(const Geometry& g, const uint8_t* experts, uint64_t stride, int64_t gid_base,
                                const uint8_t* shared_rec, const StepBuffers& b, float* h, hipStream_t s) {
  launch(route_scalar_kernel, dim3(1), dim3(64), 0, s, (const float*)b.logits, g.E, g.k, g.norm_topk, b.route_idx,
         b.route_w, b.route_gamma);
  const int n_gu = (g.k + 1) * g.I;
  const int64_t n_dn = (int64_t)(g.k + 1) * (g.I / kSlice) * g.H;
  const dim3 gu_grid((n_gu + 255) / 256), dn_grid((unsigned)((n_dn + 255) / 256)), blk(256);
  if (g.bits == 4) {
    launch(gateup_scalar_kernel<4>, gu_grid, blk, 0, s, g, experts, stride, gid_base, shared_rec, b.x,
           (const int32_t*)b.route_idx, h);
    launch(down_scalar_kernel<4>, dn_grid, blk, 0, s, g, experts, stride, gid_base, shared_rec,
           (const int32_t*)b.route_idx, (const float*)b.route_w, (const float*)b.route_gamma, (const float*)h,
           b.partial);
  } else {
    launch(gateup_scalar_kernel<8>, gu_grid, blk, 0, s, g, experts, stride, gid_base, shared_rec, b.x,
           (const int32_t*)b.route_idx, h);
    launch(down_scalar_kernel<8>, dn_grid, blk, 0, s, g, experts, stride, gid_base, shared_rec,
           (const int32_t*)b.route_idx, (const float*)b.route_w, (const float*)b.route_gamma, (const float*)h,
           b.partial);
  }
  return hipGetLastError();
}

}  // namespace moe
