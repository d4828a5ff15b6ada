// Single-wave exact top-k of router logits with renormalised softmax weights.
//
// Selection order: logit descending, expert index ascending on ties; NaN ranks
// with -inf and -0 with +0 (one total order over all values). Pages: each layer
// routes a token to the top 10 of 512 experts (80B) or 8 of 256 (35B)
// (cheshm.ai news article, paragraph on how it works); the weights of the
// chosen experts are renormalised (norm_topk_prob, alphalab.site field test,
// section on the 35B correctness fix).
//
// Method. Each logit maps to a 32-bit key whose unsigned order is the logit
// order. k rounds of: per-lane max of its keys, wave max with DPP (one v_max
// per step), the lowest expert index holding that key by a DPP wave min over
// per-lane candidates, and the owning lane clears it. The picks come out in selection order; everything is
// wave-local (registers, DPP, ballots), with no LDS round trips on the path.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dpp.h"

namespace moe {

constexpr int kTopkMax = 16;
constexpr int kRouteLds = 2 * kTopkMax;   // uint32 of LDS per routing wave
constexpr int kRouteOrdered = 0;          // pick q at lds[kRouteOrdered + 2q + 1]

// Straight-line arithmetic (no data-dependent branches): NaN -> -inf, -0 -> +0,
// then flip all bits of negatives and the sign bit of non-negatives.
__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t u = __float_as_uint(v);
  u = ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0xFF800000u : u;  // NaN ranks with -inf
  u = (u == 0x80000000u) ? 0u : u;                           // -0 ranks with +0
  const uint32_t flip = (uint32_t)((int32_t)u >> 31) | 0x80000000u;
  return u ^ flip;
}

__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// One wave routes one token. logits: E values (global memory). lds: kRouteLds
// uint32 of this wave's LDS; on return lds[kRouteOrdered + 2q + 1] holds pick q
// (selection order) and lds[kRouteOrdered + 2q] the bits of its weight, for
// q < k. When out_idx is non-NULL, lane q < k also writes out_idx[q] and
// out_w[q] (and host_idx[q] when that is non-NULL too).
template <int NPL>
__device__ __forceinline__ void wave_route(const float* __restrict__ logits, int E, int k, int norm_topk, uint32_t* lds,
                                           int32_t* out_idx, float* out_w, int32_t* host_idx) {
  const int lane = threadIdx.x & 63;
  float lv[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) lv[i] = logits[min(lane + 64 * i, E - 1)];
  uint32_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) key[i] = logit_key(lv[i]) & ((lane + 64 * i < E) ? 0xFFFFFFFFu : 0u);

  uint32_t pick_k = 0u, pick_e = 0u;  // lane q keeps pick q
#pragma unroll
  for (int j = 0; j < kTopkMax; ++j) {
    if (j < k) {
      uint32_t lm = key[0];
#pragma unroll
      for (int i = 1; i < NPL; ++i) lm = key[i] > lm ? key[i] : lm;
      const uint32_t wm = dpp::wave_max_u32(lm);
      // lowest expert index holding wm: per-lane candidate, then a wave min
      uint32_t li = 0xFFFFFFFFu;
#pragma unroll
      for (int i = NPL - 1; i >= 0; --i) li = (key[i] == wm) ? (uint32_t)(lane + 64 * i) : li;
      const int e = (int)dpp::wave_min_u32(li);
#pragma unroll
      for (int i = 0; i < NPL; ++i) key[i] = (lane + 64 * i == e) ? 0u : key[i];
      pick_k = (lane == j) ? wm : pick_k;
      pick_e = (lane == j) ? (uint32_t)e : pick_e;
    }
  }
  // weights: exp(l - l_max) over the picks (norm_topk) or over all E logits
  const float l = key_logit(pick_k);
  const float lmax = key_logit(__builtin_amdgcn_readfirstlane(pick_k));
  const float z = (lane < k) ? expf(l - lmax) : 0.f;
  float s;
  if (norm_topk) {
    s = dpp::wave_sum(z);
  } else {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i < E) part += expf(lv[i] - lmax);
    s = dpp::wave_sum(part);
  }
  if (lane < k) {
    const float wq = z / s;
    lds[kRouteOrdered + 2 * lane] = __float_as_uint(wq);
    lds[kRouteOrdered + 2 * lane + 1] = pick_e;
    if (out_idx) {
      out_idx[lane] = (int32_t)pick_e;
      out_w[lane] = wq;
      if (host_idx) host_idx[lane] = (int32_t)pick_e;
    }
  }
}

inline int topk_npl(int E) {
  const int n = (E + 63) / 64;
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

}  // namespace moe
