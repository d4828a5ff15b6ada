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
// order; packing the key above the complemented expert index gives one
// unsigned 64-bit value per expert whose order is the selection order, so
// every comparison below is a single unsigned compare with no ties.
//   1. Each lane holds NPL experts (e = lane + 64 i) and takes their maximum.
//   2. The lane maxima are written to LDS and each lane counts how many beat
//      its own (reads of one address by all lanes are LDS broadcasts). The
//      k-th best lane maximum T is a lower bound of the whole top-k: the k
//      lane maxima at or above T are k distinct experts.
//   3. When exactly k experts reach T (the top-k sit in k different lanes)
//      they are the k best lane maxima, already ranked by step 2; when k + 1
//      do, the one that is not a lane maximum is placed among them with two
//      ballots. Otherwise the experts at or above T are compacted into LDS
//      with ballots (at most k * NPL of them, usually little more than k),
//      each is ranked against the others the same way, and rank r < k is
//      pick r.
//   4. When more than kRouteCand experts reach T (many of the best logits in
//      a few lanes; only possible when k * NPL > kRouteCand), k rounds of
//      wave max / lowest-index selection with DPP take over.
// The picks come out in selection order; the whole routine is one wave.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dpp.h"

namespace moe {

constexpr int kTopkMax = 16;
constexpr int kRouteCand = 128;           // candidates ranked by the threshold pass
constexpr int kRouteOut = 2 * kTopkMax;   // uint32: (weight bits, pick) per selection slot
// uint32 of LDS per routing wave: the output, then u64 scratch for the 64 lane
// maxima, the candidates and the ranked picks, then 64 rank counters
constexpr int kRouteLds = kRouteOut + 2 * (64 + kRouteCand + kTopkMax) + 64;
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

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// LDS written by this wave becomes readable by all its lanes (LDS operations
// of one wave complete in order; the fence keeps the compiler from moving
// accesses across this point).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Per-lane state of one routing wave: the logits and packed values of the
// lane's NPL experts and their maximum.
template <int NPL>
struct RouteLane {
  float lv[NPL];
  uint64_t p[NPL];
  uint64_t pm;
};

// The lane's NPL logits (loads only).
template <int NPL>
__device__ __forceinline__ void route_issue(const float* __restrict__ logits, int E, RouteLane<NPL>& r) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NPL; ++i) r.lv[i] = logits[min(lane + 64 * i, E - 1)];
}

// Packed values and the lane maximum of logits loaded by route_issue.
template <int NPL>
__device__ __forceinline__ void route_keys(int E, RouteLane<NPL>& r) {
  const int lane = threadIdx.x & 63;
  // packed (key, ~e): padding (e >= E) gets key 0, below every real logit
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const uint32_t e = (uint32_t)(lane + 64 * i);
    const uint32_t key = logit_key(r.lv[i]) & (e < (uint32_t)E ? 0xFFFFFFFFu : 0u);
    r.p[i] = ((uint64_t)key << 32) | (uint32_t)~e;
  }
  r.pm = r.p[0];
#pragma unroll
  for (int i = 1; i < NPL; ++i) r.pm = r.p[i] > r.pm ? r.p[i] : r.pm;
}

template <int NPL>
__device__ __forceinline__ void route_load(const float* __restrict__ logits, int E, RouteLane<NPL>& r) {
  route_issue<NPL>(logits, E, r);
  route_keys<NPL>(E, r);
}

__device__ __forceinline__ uint64_t* route_lane_best(uint32_t* lds) { return reinterpret_cast<uint64_t*>(lds + kRouteOut); }
__device__ __forceinline__ uint32_t* route_rank_count(uint32_t* lds) {
  return lds + kRouteOut + 2 * (64 + kRouteCand + kTopkMax);
}

// Number of the values v[0..n) greater than c. v is read 16 values at a
// time, the eight 16-byte LDS reads of a batch issued together so that a
// batch costs one LDS round trip (a read-then-wait loop pays one per pair);
// v must hold round_up(n, 16) readable values, those at or past n are not
// counted.
__device__ __forceinline__ int count_greater(const uint64_t* v, int n, uint64_t c) {
  int q = 0;
  for (int j0 = 0; j0 < n; j0 += 16) {
    ulonglong2 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = *reinterpret_cast<const ulonglong2*>(v + j0 + 2 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      q += (j0 + 2 * u < n && w[u].x > c) ? 1 : 0;
      q += (j0 + 2 * u + 1 < n && w[u].y > c) ? 1 : 0;
    }
  }
  return q;
}

// Steps 3-4, given the threshold T and the lane's rank among the 64 lane
// maxima (one wave): lane q < k ends with pick q (its key and its expert) and
// writes the expert to lds[kRouteOrdered + 2q + 1].
template <int NPL>
__device__ __forceinline__ void route_select(const RouteLane<NPL>& r, uint64_t T, int rank, int k, uint32_t* lds,
                                             uint32_t& pick_k, uint32_t& pick_e) {
  const int lane = threadIdx.x & 63;
  uint64_t* cand = route_lane_best(lds) + 64;
  uint64_t* ranked = cand + kRouteCand;
  uint64_t m[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) m[i] = __ballot(r.p[i] >= T);
  int n_cand = 0;  // uniform
#pragma unroll
  for (int i = 0; i < NPL; ++i) n_cand += __popcll(m[i]);

  pick_k = 0u;  // lane q keeps pick q
  pick_e = 0u;
  if (n_cand == k) {
    // the only experts at or above T are the k lane maxima of rank < k (the
    // top-k sit in k different lanes, about half the tokens at 10 of 512):
    // their ranks among the lane maxima are the selection order
    if (rank < k) ranked[rank] = r.pm;
    wave_lds_sync();
    const uint64_t pq = ranked[min(lane, k - 1)];
    if (lane < k) {
      pick_k = (uint32_t)(pq >> 32);
      pick_e = ~(uint32_t)pq;
    }
  } else if (n_cand == k + 1) {
    // one expert x at or above T is not a lane maximum (one lane holds two of
    // the best k + 1). A lane maximum of rank r < k has r + [x above it]
    // candidates above it; x has the lane maxima above it (those of rank >= k
    // are below T).
    uint64_t xv = 0ull;  // candidate values are never 0: the low word is ~e
#pragma unroll
    for (int i = 0; i < NPL; ++i) xv = (r.p[i] >= T && r.p[i] != r.pm) ? r.p[i] : xv;
    const uint64_t x = readlane_u64(xv, __builtin_ctzll(__ballot(xv != 0ull)));
    const int fx = __popcll(__ballot(rank < k && r.pm > x));
    const int f = rank + (x > r.pm ? 1 : 0);
    if (rank < k && f < k) ranked[f] = r.pm;
    if (lane == 0 && fx < k) ranked[fx] = x;
    wave_lds_sync();
    const uint64_t pq = ranked[min(lane, k - 1)];
    if (lane < k) {
      pick_k = (uint32_t)(pq >> 32);
      pick_e = ~(uint32_t)pq;
    }
  } else if (n_cand <= kRouteCand) {
    // 3. compaction of the experts at or above T (prefix offsets from the
    //    ballots), then each ranked against the others
#pragma unroll
    for (int i = 0, base = 0; i < NPL; ++i) {
      const int pos = base + (int)lanes_below(m[i]);
      if ((m[i] >> lane) & 1ull) cand[pos] = r.p[i];
      base += __popcll(m[i]);
    }
    wave_lds_sync();
    const uint64_t c0 = lane < n_cand ? cand[lane] : 0ull;
    const uint64_t c1 = lane + 64 < n_cand ? cand[lane + 64] : 0ull;
    const int q0 = count_greater(cand, n_cand, c0);
    const int q1 = n_cand > 64 ? count_greater(cand, n_cand, c1) : k;
    if (lane < n_cand && q0 < k) ranked[q0] = c0;
    if (lane + 64 < n_cand && q1 < k) ranked[q1] = c1;
    wave_lds_sync();
    const uint64_t pq = ranked[min(lane, k - 1)];
    if (lane < k) {
      pick_k = (uint32_t)(pq >> 32);
      pick_e = ~(uint32_t)pq;
    }
  } else {
    // 4. k rounds of wave max, lowest index holding it, owner clears it
    uint32_t key[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) key[i] = (uint32_t)(r.p[i] >> 32);
#pragma unroll
    for (int j = 0; j < kTopkMax; ++j) {
      if (j < k) {
        uint32_t lm = key[0];
#pragma unroll
        for (int i = 1; i < NPL; ++i) lm = key[i] > lm ? key[i] : lm;
        const uint32_t wm = dpp::wave_max_u32(lm);
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
  }
  if (lane < k) lds[kRouteOrdered + 2 * lane + 1] = pick_e;
}

// The weights of the picks (one wave, the one that ran route_select, with
// its lane state and picks): exp(l - l_max) over the picks, normalised by
// their sum (norm_topk) or by the sum over all E logits. Lane q < k writes
// the bits of weight q to lds[kRouteOrdered + 2q] and, when out_idx is
// non-NULL, out_idx[q] and out_w[q] (and host_idx[q] when that is non-NULL).
template <int NPL>
__device__ __forceinline__ void route_weights(const RouteLane<NPL>& r, uint32_t pick_k, uint32_t pick_e, int E, int k,
                                              int norm_topk, uint32_t* lds, int32_t* out_idx, float* out_w,
                                              int32_t* host_idx) {
  const int lane = threadIdx.x & 63;
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
      if (lane + 64 * i < E) part += expf(r.lv[i] - lmax);
    s = dpp::wave_sum(part);
  }
  if (lane < k) {
    const float wq = z / s;
    lds[kRouteOrdered + 2 * lane] = __float_as_uint(wq);
    if (out_idx) {
      out_idx[lane] = (int32_t)pick_e;
      out_w[lane] = wq;
      if (host_idx) host_idx[lane] = (int32_t)pick_e;
    }
  }
}

// Steps 3-4 and the weights, given the threshold T and the lane's rank
// among the lane maxima (one wave).
template <int NPL>
__device__ __forceinline__ void route_finish(const RouteLane<NPL>& r, uint64_t T, int rank, int E, int k,
                                             int norm_topk, uint32_t* lds, int32_t* out_idx, float* out_w,
                                             int32_t* host_idx) {
  uint32_t pick_k, pick_e;
  route_select<NPL>(r, T, rank, k, lds, pick_k, pick_e);
  route_weights<NPL>(r, pick_k, pick_e, E, k, norm_topk, lds, out_idx, out_w, host_idx);
}

// T: the lane maximum of rank k - 1 (one lane has it: the 64 values are distinct).
__device__ __forceinline__ uint64_t route_threshold(uint64_t pm, int rank, int k) {
  const uint64_t tmask = __ballot(rank == k - 1);
  return readlane_u64(pm, __builtin_ctzll(tmask));
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
  RouteLane<NPL> r;
  route_load<NPL>(logits, E, r);
  uint64_t* lane_best = route_lane_best(lds);
  lane_best[lane] = r.pm;
  wave_lds_sync();
  const int rank = count_greater(lane_best, 64, r.pm);
  route_finish<NPL>(r, route_threshold(r.pm, rank, k), rank, E, k, norm_topk, lds, out_idx, out_w, host_idx);
}

// The selection by a whole block of NW waves (every thread calls it; it
// synchronises the block): wave 0, whose logits the caller has loaded with
// route_issue, does steps 1, 3 and 4; the ranks of the 64 lane maxima are
// counted by all NW waves, each against 64 / NW of them, and summed with LDS
// atomics. On return the picks are in lds as for wave_route, visible to the
// whole block, and wave 0 holds its lane state r and, in lane q, pick q
// (pick_k, pick_e): the caller runs route_weights in wave 0 when it suits it,
// and the weights become visible to the block at its next barrier.
template <int NPL, int NW>
__device__ __forceinline__ void block_route_select(int E, int k, uint32_t* lds, RouteLane<NPL>& r, uint32_t& pick_k,
                                                   uint32_t& pick_e) {
  static_assert(64 % NW == 0, "the lane maxima are split evenly over the waves");
  constexpr int PER = 64 / NW;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  uint64_t* lane_best = route_lane_best(lds);
  uint32_t* rank_count = route_rank_count(lds);
  if (wv == 0) {
    route_keys<NPL>(E, r);
    lane_best[lane] = r.pm;
    rank_count[lane] = 0u;
  }
  __syncthreads();
  {
    const uint64_t mine = lane_best[lane];
    int c = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) c += lane_best[wv * PER + j] > mine ? 1 : 0;
    if (c) atomicAdd(&rank_count[lane], (uint32_t)c);
  }
  __syncthreads();
  if (wv == 0) {
    const int rank = (int)rank_count[lane];
    route_select<NPL>(r, route_threshold(r.pm, rank, k), rank, k, lds, pick_k, pick_e);
  }
  __syncthreads();
}

inline int topk_npl(int E) {
  const int n = (E + 63) / 64;
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

}  // namespace moe
