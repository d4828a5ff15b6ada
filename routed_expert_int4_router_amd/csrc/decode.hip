// Batch-1 decode kernels of the routed MoE step for gfx950 (wave64).
//
// One token-layer runs as three dependent launches:
//   router   : E+1 fp64-accumulated dot products (router logits + shared gate)
//   gateup   : per wave, top-k of the logits (wave shuffles), then the int4/int8
//              group-dequant GEMV of gate and up rows and SwiGLU -> h (fp32)
//   down     : down-projection GEMV of the k+1 experts on h, weighted combine
//              with the renormalised router weights and the sigmoid shared gate,
//              optional residual update of a layer stack.
// Pages: top-k routing per layer (10 of 512 / 8 of 256), resident router and
// shared experts, fixed-stride expert blobs, MLX-style int4/int8 group
// quantisation (cheshm.ai news article, paragraphs on how it works and on the
// code base; paotong.dev commentary, paragraphs on the principle and the fetch
// path); renormalised top-k weights (alphalab.site field test, section on the
// 35B correctness fix). The decode loop being dispatch-bound (paotong.dev,
// paragraph on the bounded pool) is why the token-layer is only three launches.
//
// Weight reads are 16-byte (dwordx4) loads of packed codes; each lane owns a
// contiguous 16-byte chunk of a code row, consecutive lanes own consecutive
// chunks, so a wave-wide load covers contiguous row bytes. The group scale and
// bias are applied once per chunk: dot = s * sum(q * x) + c * sum(x). For the
// int4 gate/up rows the chunk's products run on the dot-product unit, two codes
// (as the exact bf16 values 128 + q) against two bf16 activations per
// instruction (x_chunk / chunk_term); the down rows multiply fp32 h, so there
// and for int8 the codes become floats exactly (v_cvt_f32_ubyte*) and meet
// their operands in fp32 FMAs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_math.h"
#include "dpp.h"
#include "kernels.h"
#include "launch.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kWave = 64;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The activations of a chunk from the 16-byte words they were loaded as.
template <int BITS>
__device__ __forceinline__ XChunk<BITS> x_chunk_of(const uint4 (&raw)[128 / BITS / 8]) {
  uint32_t xr[128 / BITS / 2];
#pragma unroll
  for (int q = 0; q < 128 / BITS / 8; ++q) {
    xr[4 * q] = raw[q].x;
    xr[4 * q + 1] = raw[q].y;
    xr[4 * q + 2] = raw[q].z;
    xr[4 * q + 3] = raw[q].w;
  }
  return x_chunk<BITS>(xr);
}

template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  return dpp::group_sum<LPR>(v);
}

// ------------------------------------------------------------------ router ---
// One wave per output row; lanes stride over the hidden dimension in float4 /
// 4 x bf16 steps. Products of a bf16 and an fp32 are exact in fp64, so the
// fp64 sum rounded once to fp32 is the exactly rounded logit except in
// vanishingly rare near-ties.
template <int NIT>
__global__ void __launch_bounds__(256) router_kernel(Geometry g, const float* __restrict__ wr,
                                                     const float* __restrict__ bias, StepBuffers b) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row > g.E) return;
  const float4* w4 = reinterpret_cast<const float4*>(wr + (size_t)row * g.H);
  const uint2* x4 = reinterpret_cast<const uint2*>(b.x);
  const int n4 = g.H / 4;
  float4 w[NIT];
  uint2 xv[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int i = min(lane + kWave * it, n4 - 1);  // clamped: every load issues unconditionally
    w[it] = w4[i];
    xv[it] = x4[i];
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    if (lane + kWave * it >= n4) {
      w[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      xv[it] = make_uint2(0u, 0u);
    }
  }
  double acc = 0.0;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    acc += (double)bf16f(xv[it].x & 0xFFFFu) * (double)w[it].x;
    acc += (double)bf16f(xv[it].x >> 16) * (double)w[it].y;
    acc += (double)bf16f(xv[it].y & 0xFFFFu) * (double)w[it].z;
    acc += (double)bf16f(xv[it].y >> 16) * (double)w[it].w;
  }
  acc = dpp::wave_sum(acc);
  if (lane == 0) {
    if (row < g.E && bias) acc += (double)bias[row];
    b.logits[row] = (float)acc;
  }
}

// ---------------------------------------------------------------- routing ---
// One wave per token: top-k + weights + shared gate (route_* at token offsets).
// Used where the route must exist before the expert kernels are launched: the
// pool (the host reads the picks through host_route) and batched prefill.
template <int NPL>
__global__ void __launch_bounds__(64) route_kernel(Geometry g, const float* __restrict__ logits, int ld_logits,
                                                   int32_t* route_idx, float* route_w, float* route_gamma,
                                                   int32_t* host_route) {
  __shared__ __align__(16) uint32_t lds[kRouteLds];
  const int t = blockIdx.x;
  const float* lg = logits + (size_t)t * ld_logits;
  wave_route<NPL>(lg, g.E, g.k, g.norm_topk, lds, route_idx + (size_t)t * g.k, route_w + (size_t)t * g.k,
                  host_route ? host_route + (size_t)t * g.k : nullptr);
  if (threadIdx.x == 0) route_gamma[t] = 1.0f / (1.0f + expf(-lg[g.E]));
}

// Record of selection slot j: table[j] (pool slots) or gid_base + e (resident).
// The table is read with static indices only (kernel-argument scalar loads);
// a dynamic index would turn it into a dependent vector load.
__device__ __forceinline__ const uint8_t* expert_record(const ExpertSource& src, int j, int e) {
  int64_t r = src.gid_base + e;
  if (src.use_table) {
#pragma unroll
    for (int q = 0; q < kMaxTopK; ++q)
      if (q == j) r = src.table[q];
  }
  return src.base + (uint64_t)r * src.stride;
}

// ------------------------------------------------------------------ gateup ---
// Wave task: RPW * RW consecutive rows i of one expert slot j (slot k = shared).
// Lane (r, c): r = lane / LPR selects the row inside a group of RPW rows,
// c = lane % LPR the first 16-byte chunk; it owns chunks c + LPR * it.
template <int BITS, int LPR, int IT, int RW, int NPL>
__global__ void __launch_bounds__(256) gateup_kernel(Geometry g, ExpertSource src, const uint8_t* __restrict__ shared_rec,
                                                     StepBuffers b, int waves_per_expert, int total_waves) {
  constexpr int EPC = 128 / BITS;  // elements per 16-byte chunk
  constexpr int RPW = kWave / LPR;
  __shared__ __align__(16) uint32_t lds_route[kRouteLds];
  const int wave_raw = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const bool idle = wave_raw >= total_waves;  // padding waves: join the barrier, then leave
  const int wave = min(wave_raw, total_waves - 1);
  const int lane = threadIdx.x & 63;
  const int j = __builtin_amdgcn_readfirstlane(wave / waves_per_expert);
  const int row0 = (wave % waves_per_expert) * (RPW * RW);
  const int rsub = lane / LPR, c0 = lane % LPR;

  // Activations first: they do not depend on the routing, and loads issued
  // before the weight loads can be waited on without waiting for the weights.
  uint4 xraw[IT][EPC / 8];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const uint4* xp = reinterpret_cast<const uint4*>(b.x + (size_t)(c0 + LPR * it) * EPC);
#pragma unroll
    for (int q = 0; q < EPC / 8; ++q) xraw[it][q] = xp[q];
  }

  // Resident routing: wave 0 of the block computes the token's top-k and the
  // block shares the picks through LDS (block 0 also publishes the route for
  // the down kernel). Slots only grow with the wave index and slot k (the
  // shared expert) is last, so "the block's first slot is routed" is uniform
  // over the block and every wave reaches the barrier.
  const int j_first = (blockIdx.x * 4) / waves_per_expert;
  if (!src.use_table && j_first < g.k) {
    if (threadIdx.x < 64) {
      const bool pub = blockIdx.x == 0;
      wave_route<NPL>(b.logits, g.E, g.k, g.norm_topk, lds_route, pub ? b.route_idx : nullptr,
                      pub ? b.route_w : nullptr, nullptr);
      if (pub && threadIdx.x == 0) b.route_gamma[0] = 1.0f / (1.0f + expf(-b.logits[g.E]));
    }
    __syncthreads();
  }
  if (idle) return;
  const uint8_t* rec;
  if (j == g.k) {
    rec = shared_rec;
  } else if (src.use_table) {
    rec = expert_record(src, j, 0);
  } else {
    rec = expert_record(src, j, __builtin_amdgcn_readfirstlane((int)lds_route[kRouteOrdered + 2 * j + 1]));
  }

  const size_t row_bytes = (size_t)g.H * BITS / 8;
  const int groups = g.H / 64;
  uint4 cg[RW][IT], cu[RW][IT];
  uint32_t sg[RW][IT], su[RW][IT];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    const int i = row0 + rsub + RPW * rr;
    const uint8_t* grow = rec + g.gate_codes + (size_t)i * row_bytes;
    const uint8_t* urow = rec + g.up_codes + (size_t)i * row_bytes;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int ch = c0 + LPR * it;
      cg[rr][it] = ld_stream(grow + 16 * ch);
      cu[rr][it] = ld_stream(urow + 16 * ch);
      const int grp = ch * EPC / 64;
      sg[rr][it] = *reinterpret_cast<const uint32_t*>(rec + g.gate_sc + ((size_t)i * groups + grp) * 4);
      su[rr][it] = *reinterpret_cast<const uint32_t*>(rec + g.up_sc + ((size_t)i * groups + grp) * 4);
    }
  }
  XChunk<BITS> xc[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) xc[it] = x_chunk_of<BITS>(xraw[it]);
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    float ag = 0.f, au = 0.f;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      ag += chunk_term<BITS>(cg[rr][it], sg[rr][it], xc[it]);
      au += chunk_term<BITS>(cu[rr][it], su[rr][it], xc[it]);
    }
    ag = group_sum<LPR>(ag);
    au = group_sum<LPR>(au);
    if (c0 == LPR - 1) {
      const int i = row0 + rsub + RPW * rr;
      b.h[(size_t)j * g.I + i] = swiglu(ag, au);
    }
  }
}

// -------------------------------------------------------------------- down ---
// Block: RPW * R output rows, 4 waves; wave w handles expert slots j = w, w+4, ...
// (slot k = shared expert, weight gamma). Lane (r, c) owns chunks c + LPR * it of
// rows r + RPW * rr. Each wave stages the h of its own slots in LDS.
template <int BITS, int LPR, int IT, int R>
__global__ void __launch_bounds__(256) down_kernel(Geometry g, ExpertSource src, const uint8_t* __restrict__ shared_rec,
                                                   StepBuffers b, ResidualArgs res) {
  constexpr int EPC = 128 / BITS;
  constexpr int RPW = kWave / LPR;
  constexpr int RB = RPW * R;
  constexpr int I = LPR * IT * EPC;                 // down rows hold I codes: LPR * IT chunks
  constexpr int HU = I / 4 >= kWave ? I / 4 / kWave : 1;  // 1 KiB wave loads per slot's h
  constexpr int RS = I >= 256 ? I : 256;            // LDS floats per slot (a wave load fills 1 KiB)
  constexpr int MS = (kMaxTopK + 1 + 3) / 4;        // slots per wave at most (k <= 16)
  extern __shared__ __align__(16) float smem[];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rsub = lane / LPR, c0 = lane % LPR;
  const int hrow0 = blockIdx.x * RB;
  const int nslots = g.k + 1;
  const int msw = (nslots + 3) / 4;                 // slots per wave in use
  float* sh_h = smem + (size_t)wv * msw * RS;       // this wave's slots: [msw][RS]
  float* sh_part = smem + (size_t)4 * msw * RS;     // [4][RB]

  // 1. the step's route (lane q < k holds slot q), one vector load per array
  const int qk = min(lane, g.k - 1);
  const int r_idx = src.use_table ? 0 : b.route_idx[qk];
  const float r_w = b.route_w[qk];
  const float r_gamma = b.route_gamma[0];
  // 2. h of this wave's slots straight into LDS (global_load_lds: no registers,
  //    in flight together with the weight loads below)
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    if (m < msw) {
      const int j = min(wv + 4 * m, nslots - 1);
#pragma unroll
      for (int u = 0; u < HU; ++u) {
        const float* gsrc = b.h + (size_t)j * I + 4 * min(lane + kWave * u, I / 4 - 1);
        __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)(sh_h + (size_t)m * RS + 256 * u),
                                         16, 0, 0);
      }
    }
  }
  // 3. expert ids of this wave's slots, all read out before the first weight
  //    load (the empty asm pins each id in an SGPR here, so the wait for the
  //    route happens once instead of before every slot's loads)
  int e_of[MS];
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const int j = min(wv + 4 * m, g.k - 1);
    e_of[m] = __builtin_amdgcn_readlane(r_idx, j);
    asm volatile("" ::"s"(e_of[m]));
  }
  const uint8_t* recs[MS];
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const int j = wv + 4 * m;
    recs[m] = (j >= g.k) ? shared_rec : expert_record(src, j, e_of[m]);
  }
  uint4 cd[MS][R][IT];
  uint32_t sd[MS][R][IT];
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const int j = wv + 4 * m;
    if (j < nslots) {
      const uint8_t* rec = recs[m];
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const int hr = hrow0 + rsub + RPW * rr;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int ch = c0 + LPR * it;  // tile ch of row hr: [I*bits/128][H][16 B]; (s, c) [I/64][H]
          cd[m][rr][it] = ld_stream(rec + g.down_codes + ((size_t)ch * g.H + hr) * 16);
          sd[m][rr][it] = *reinterpret_cast<const uint32_t*>(rec + g.down_sc + ((size_t)(ch * EPC / 64) * g.H + hr) * 4);
        }
      }
    }
  }
  // 4. the LDS copies land through the vector-memory counter: wait for all loads
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __builtin_amdgcn_wave_barrier();

  float acc[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) acc[rr] = 0.f;
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const int j = wv + 4 * m;
    if (j < nslots) {
      const float wj = (j == g.k) ? r_gamma : __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(r_w), min(j, g.k - 1)));
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int ch = c0 + LPR * it;
        float hv[EPC];
        const float4* hp = reinterpret_cast<const float4*>(sh_h + (size_t)m * RS + ch * EPC);
#pragma unroll
        for (int q = 0; q < EPC / 4; ++q) {
          const float4 v = hp[q];
          hv[4 * q] = v.x;
          hv[4 * q + 1] = v.y;
          hv[4 * q + 2] = v.z;
          hv[4 * q + 3] = v.w;
        }
        float hs = 0.f;
#pragma unroll
        for (int q = 0; q < EPC; ++q) hs += hv[q];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          const float d = chunk_dot<BITS>(cd[m][rr][it], hv);
          const float c = group_term(sd[m][rr][it], d, hs);
          acc[rr] = fmaf(wj, c, acc[rr]);
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const float v = group_sum<LPR>(acc[rr]);
    if (c0 == LPR - 1) sh_part[wv * RB + rsub + RPW * rr] = v;
  }
  __syncthreads();
  if (threadIdx.x < RB) {
    const int hr = hrow0 + threadIdx.x;
    const float o = ((sh_part[threadIdx.x] + sh_part[RB + threadIdx.x]) + sh_part[2 * RB + threadIdx.x]) +
                    sh_part[3 * RB + threadIdx.x];
    if (res.r_in || res.x_res) {
      const float r = (res.r_in ? res.r_in[hr] : bf16f(res.x_res[hr])) + o;
      res.out[hr] = r;
      if (res.x_next) res.x_next[hr] = to_bf16_rne(r);
    } else {
      res.out[hr] = o;
    }
  }
}

// ------------------------------------------------------------------ expert ---
// Fused expert step. Block (slot j, slice sl): I rows [sl * SL, sl * SL + SL)
// of expert slot j (slot k = the shared expert), 16 waves (enough waves per
// SIMD to overlap one wave's dequantisation arithmetic with another's
// loads). The block
//   1. routes the token (top-k of the logits by the whole block, picks in
//      LDS; wave 0 computes their weights once the block's weight loads are
//      in flight; a pool step reads the route and the record table instead),
//   2. issues the gate/up code rows of its SL rows and the down codes of the
//      slice (16 bytes of every down row) together, so the weight latency is
//      paid once,
//   3. computes h = silu(gate . x) * (up . x) for its rows into LDS,
//   4. writes w_j * (down[:, slice] . h[slice]) for all H outputs as one
//      partial row (w_k = gamma for the shared expert).
// The reduce kernel sums the (k + 1) * (I / SL) partial rows in a fixed
// order, so results do not depend on scheduling. SL = 32: the down slice of a
// row is DCH = SL * BITS / 128 16-byte tiles (1 int4, 2 int8) inside one
// quantisation group.
constexpr int kExpertWaves = 16;
constexpr int kSlice = 32;

template <int BITS, int LPR, int IT, int NPL, int DQ>
__global__ void __launch_bounds__(64 * kExpertWaves) expert_kernel(Geometry g, ExpertSource src,
                                                                  const uint8_t* __restrict__ shared_rec,
                                                                  StepBuffers b) {
  constexpr int EPC = 128 / BITS;  // codes per 16-byte chunk
  constexpr int SL = kSlice;       // I rows per block
  constexpr int DCH = SL / EPC;    // 16-byte down tiles per row slice
  constexpr int NT = 64 * kExpertWaves;
  constexpr int RPWV = SL / kExpertWaves;  // gate/up rows per wave
  constexpr int RPW = kWave / LPR; // rows per wave pass
  constexpr int RW = (RPWV + RPW - 1) / RPW;
  __shared__ __align__(16) uint32_t lds_route[kRouteLds];
  __shared__ __align__(16) float sh_h[SL];
  const int nsl = g.I / SL;
  const int jb = (int)blockIdx.x / nsl;
  const int j = __builtin_amdgcn_readfirstlane(src.n_sel ? src.sel[jb] : jb);
  const int sl = __builtin_amdgcn_readfirstlane((int)blockIdx.x % nsl);
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int rsub = lane / LPR, c0 = lane % LPR;

  // the logits (wave 0 of a routed block) and the activations first: neither
  // depends on the routing
  const bool routed = j < g.k && !src.use_table;  // block-uniform
  RouteLane<NPL> rl;
  if (routed && wv == 0) route_issue<NPL>(b.logits, g.E, rl);
  uint4 xraw[IT][EPC / 8];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const uint4* xp = reinterpret_cast<const uint4*>(b.x + (size_t)(c0 + LPR * it) * EPC);
#pragma unroll
    for (int q = 0; q < EPC / 8; ++q) xraw[it][q] = xp[q];
  }
  // 1. route: the picks now, their weights once the weight loads are issued
  uint32_t pick_k = 0u, pick_e = 0u;
  if (routed) block_route_select<NPL, kExpertWaves>(g.E, g.k, lds_route, rl, pick_k, pick_e);
  const uint8_t* rec;
  if (j == g.k) {
    rec = shared_rec;
  } else if (src.use_table) {
    rec = expert_record(src, j, 0);
  } else {
    rec = expert_record(src, j, __builtin_amdgcn_readfirstlane((int)lds_route[kRouteOrdered + 2 * j + 1]));
  }

  // 2. all weight loads of the block
  const size_t row_bytes = (size_t)g.H * BITS / 8;
  const int groups = g.H / 64;
  uint4 cg[RW][IT], cu[RW][IT];
  uint32_t sg[RW][IT], su[RW][IT];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    const int i = sl * SL + wv * RPWV + min(rsub + RPW * rr, RPWV - 1);  // idle lanes re-read a valid row
    const uint8_t* grow = rec + g.gate_codes + (size_t)i * row_bytes;
    const uint8_t* urow = rec + g.up_codes + (size_t)i * row_bytes;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int ch = c0 + LPR * it;
      cg[rr][it] = ld_stream(grow + 16 * ch);
      cu[rr][it] = ld_stream(urow + 16 * ch);
      const int grp = ch * EPC / 64;
      sg[rr][it] = *reinterpret_cast<const uint32_t*>(rec + g.gate_sc + ((size_t)i * groups + grp) * 4);
      su[rr][it] = *reinterpret_cast<const uint32_t*>(rec + g.up_sc + ((size_t)i * groups + grp) * 4);
    }
  }
  // down tiles sl * DCH .. of every row: contiguous in the record (tiles
  // [I * BITS / 128][H][16 B], (s, c) group-major [I/64][H])
  const uint8_t* dtile = rec + g.down_codes + (size_t)sl * DCH * g.H * 16;
  const uint32_t* dsc = reinterpret_cast<const uint32_t*>(rec + g.down_sc) + (size_t)(sl * SL / 64) * g.H;
  uint4 cd[DQ][DCH];
  uint32_t sd[DQ];
#pragma unroll
  for (int q = 0; q < DQ; ++q) {
    const int n = min((int)threadIdx.x + NT * q, g.H - 1);
#pragma unroll
    for (int c = 0; c < DCH; ++c) cd[q][c] = ld_stream(dtile + ((size_t)c * g.H + n) * 16);
    sd[q] = dsc[n];
  }
  // the slot's weight (and the published shared gate) only after every weight
  // load is in flight; nothing is scheduled across this point. In a routed
  // block wave 0 computes the picks' weights now; they reach the other waves
  // through the barrier that ends the gate/up phase.
  __builtin_amdgcn_sched_barrier(0);
  float wjv = 0.f;
  if (j == g.k)
    wjv = src.use_table ? b.route_gamma[0] : 1.0f / (1.0f + expf(-b.logits[g.E]));
  else if (src.use_table)
    wjv = b.route_w[j];
  if (routed && wv == 0) {
    const bool pub = blockIdx.x == 0;
    route_weights<NPL>(rl, pick_k, pick_e, g.E, g.k, g.norm_topk, lds_route, pub ? b.route_idx : nullptr,
                       pub ? b.route_w : nullptr, nullptr);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && !src.use_table) b.route_gamma[0] = 1.0f / (1.0f + expf(-b.logits[g.E]));

  // 3. gate/up dots, SwiGLU -> h of the slice in LDS
  XChunk<BITS> xc[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) xc[it] = x_chunk_of<BITS>(xraw[it]);
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    float ag = 0.f, au = 0.f;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      ag += chunk_term<BITS>(cg[rr][it], sg[rr][it], xc[it]);
      au += chunk_term<BITS>(cu[rr][it], su[rr][it], xc[it]);
    }
    ag = group_sum<LPR>(ag);
    au = group_sum<LPR>(au);
    const int r = rsub + RPW * rr;
    if (c0 == LPR - 1 && r < RPWV) sh_h[wv * RPWV + r] = swiglu(ag, au);
  }
  __syncthreads();
  const float wj = routed ? __uint_as_float(lds_route[kRouteOrdered + 2 * j]) : wjv;

  // 4. partial down projection of the slice for every output row
  float hv[SL];
#pragma unroll
  for (int q = 0; q < SL / 4; ++q) {
    const float4 v = reinterpret_cast<const float4*>(sh_h)[q];
    hv[4 * q] = v.x;
    hv[4 * q + 1] = v.y;
    hv[4 * q + 2] = v.z;
    hv[4 * q + 3] = v.w;
  }
  float hs = 0.f;
#pragma unroll
  for (int q = 0; q < SL; ++q) hs += hv[q];
  float* part = b.partial + ((size_t)j * nsl + sl) * g.H;
#pragma unroll
  for (int q = 0; q < DQ; ++q) {
    const int n = (int)threadIdx.x + NT * q;
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < DCH; ++c) d += chunk_dot<BITS>(cd[q][c], hv + c * EPC);
    const float v = group_term(sd[q], d, hs);
    if (n < g.H) part[n] = wj * v;
  }
}

// ------------------------------------------------------------------ reduce ---
// out[n] = sum of the nparts partial rows at column n, in a fixed order, plus
// the residual update of a layer stack. Block: 64 columns, 16 waves; wave w
// owns rows p = w, w + 16, ...; it loads up to 16 of them at once (one round
// of memory latency for up to 256 rows) and adds them in row order; the 16
// wave sums are then added in wave order.
constexpr int kReduceWaves = 16;
constexpr int kReduceBatch = 16;
__global__ void __launch_bounds__(64 * kReduceWaves) reduce_kernel(int H, int nparts, const float* __restrict__ partial,
                                                                   ResidualArgs res) {
  __shared__ float sh[kReduceWaves][64];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * 64 + lane;
  const float* p = partial + n;
  constexpr int S = kReduceWaves;
  float acc = 0.f;
  for (int q0 = wv; q0 < nparts; q0 += S * kReduceBatch) {
    float v[kReduceBatch];
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) {
      const int q = min(q0 + S * u, nparts - 1);  // clamped: every load issues unconditionally
      v[u] = p[(size_t)q * H];
    }
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u)
      if (q0 + S * u < nparts) acc += v[u];
  }
  sh[wv][lane] = acc;
  __syncthreads();
  if (wv == 0) {
    float o = sh[0][lane];
#pragma unroll
    for (int w = 1; w < S; ++w) o += sh[w][lane];
    if (res.r_in || res.x_res) {
      const float r = (res.r_in ? res.r_in[n] : bf16f(res.x_res[n])) + o;
      res.out[n] = r;
      if (res.x_next) res.x_next[n] = to_bf16_rne(r);
    } else {
      res.out[n] = o;
    }
  }
}

// ------------------------------------------------------------- dispatchers ---

int lpr_for(int chunks) { return chunks < 64 ? chunks : 64; }

template <int BITS, int LPR, int IT, int NPL>
hipError_t gateup_rwn(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                      hipStream_t s) {
  constexpr int RPW = kWave / LPR;
  int rw = g.I / RPW;
  rw = rw >= 4 ? 4 : (rw >= 2 ? 2 : 1);
  const int wpe = g.I / (RPW * rw);
  const int total = (g.k + 1) * wpe;
  const dim3 grid((total + 3) / 4), block(256);
  if (rw == 4) launch((gateup_kernel<BITS, LPR, IT, 4, NPL>), grid, block, 0, s, g, src, shared_rec, b, wpe, total);
  else if (rw == 2) launch((gateup_kernel<BITS, LPR, IT, 2, NPL>), grid, block, 0, s, g, src, shared_rec, b, wpe, total);
  else launch((gateup_kernel<BITS, LPR, IT, 1, NPL>), grid, block, 0, s, g, src, shared_rec, b, wpe, total);
  return hipGetLastError();
}

template <int BITS, int LPR, int IT>
hipError_t gateup_rw(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                     hipStream_t s) {
  switch (topk_npl(g.E)) {
    case 1: return gateup_rwn<BITS, LPR, IT, 1>(g, src, shared_rec, b, s);
    case 2: return gateup_rwn<BITS, LPR, IT, 2>(g, src, shared_rec, b, s);
    case 4: return gateup_rwn<BITS, LPR, IT, 4>(g, src, shared_rec, b, s);
    case 8: return gateup_rwn<BITS, LPR, IT, 8>(g, src, shared_rec, b, s);
    case 16: return gateup_rwn<BITS, LPR, IT, 16>(g, src, shared_rec, b, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS>
hipError_t gateup_bits(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                       hipStream_t s) {
  const int chunks = g.H * BITS / 128;
  const int lpr = lpr_for(chunks), it = chunks / lpr;
  if (it == 1) {
    switch (lpr) {
      case 2: return gateup_rw<BITS, 2, 1>(g, src, shared_rec, b, s);
      case 4: return gateup_rw<BITS, 4, 1>(g, src, shared_rec, b, s);
      case 8: return gateup_rw<BITS, 8, 1>(g, src, shared_rec, b, s);
      case 16: return gateup_rw<BITS, 16, 1>(g, src, shared_rec, b, s);
      case 32: return gateup_rw<BITS, 32, 1>(g, src, shared_rec, b, s);
      case 64: return gateup_rw<BITS, 64, 1>(g, src, shared_rec, b, s);
    }
  } else if (it == 2) {
    return gateup_rw<BITS, 64, 2>(g, src, shared_rec, b, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS, int LPR, int IT>
hipError_t down_r(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                  const ResidualArgs& r, hipStream_t s) {
  constexpr int RPW = kWave / LPR;
  int R = g.H / (RPW * 256);
  R = R >= 4 ? 4 : (R >= 2 ? 2 : 1);
  while (R > 1 && g.H % (RPW * R)) R >>= 1;
  const int RB = RPW * R;
  if (g.H % RB) return hipErrorInvalidValue;
  const size_t rs = g.I >= 256 ? g.I : 256;
  const size_t lds = ((size_t)4 * ((g.k + 1 + 3) / 4) * rs + 4 * RB) * sizeof(float);
  const dim3 grid(g.H / RB), block(256);
  if (R == 4) launch((down_kernel<BITS, LPR, IT, 4>), grid, block, lds, s, g, src, shared_rec, b, r);
  else if (R == 2) launch((down_kernel<BITS, LPR, IT, 2>), grid, block, lds, s, g, src, shared_rec, b, r);
  else launch((down_kernel<BITS, LPR, IT, 1>), grid, block, lds, s, g, src, shared_rec, b, r);
  return hipGetLastError();
}

template <int BITS>
hipError_t down_bits(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                     const ResidualArgs& r, hipStream_t s) {
  const int chunks = g.I * BITS / 128;
  const int lpr = lpr_for(chunks), it = chunks / lpr;
  if (it == 1) {
    switch (lpr) {
      case 2: return down_r<BITS, 2, 1>(g, src, shared_rec, b, r, s);
      case 4: return down_r<BITS, 4, 1>(g, src, shared_rec, b, r, s);
      case 8: return down_r<BITS, 8, 1>(g, src, shared_rec, b, r, s);
      case 16: return down_r<BITS, 16, 1>(g, src, shared_rec, b, r, s);
      case 32: return down_r<BITS, 32, 1>(g, src, shared_rec, b, r, s);
      case 64: return down_r<BITS, 64, 1>(g, src, shared_rec, b, r, s);
    }
  } else if (it == 2) {
    return down_r<BITS, 64, 2>(g, src, shared_rec, b, r, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS, int LPR, int IT, int NPL>
hipError_t expert_dq(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                     hipStream_t s) {
  const dim3 grid((src.n_sel ? src.n_sel : g.k + 1) * (g.I / kSlice)), block(64 * kExpertWaves);
  switch (g.H <= 64 * kExpertWaves ? 1 : g.H / (64 * kExpertWaves)) {
    case 1: launch((expert_kernel<BITS, LPR, IT, NPL, 1>), grid, block, 0, s, g, src, shared_rec, b); break;
    case 2: launch((expert_kernel<BITS, LPR, IT, NPL, 2>), grid, block, 0, s, g, src, shared_rec, b); break;
    case 4: launch((expert_kernel<BITS, LPR, IT, NPL, 4>), grid, block, 0, s, g, src, shared_rec, b); break;
    case 8: launch((expert_kernel<BITS, LPR, IT, NPL, 8>), grid, block, 0, s, g, src, shared_rec, b); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS, int LPR, int IT>
hipError_t expert_npl(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                      hipStream_t s) {
  switch (topk_npl(g.E)) {
    case 1: return expert_dq<BITS, LPR, IT, 1>(g, src, shared_rec, b, s);
    case 2: return expert_dq<BITS, LPR, IT, 2>(g, src, shared_rec, b, s);
    case 4: return expert_dq<BITS, LPR, IT, 4>(g, src, shared_rec, b, s);
    case 8: return expert_dq<BITS, LPR, IT, 8>(g, src, shared_rec, b, s);
    case 16: return expert_dq<BITS, LPR, IT, 16>(g, src, shared_rec, b, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS>
hipError_t expert_bits(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                       hipStream_t s) {
  const int chunks = g.H * BITS / 128;
  const int lpr = lpr_for(chunks), it = chunks / lpr;
  if (it == 1) {
    switch (lpr) {
      case 2: return expert_npl<BITS, 2, 1>(g, src, shared_rec, b, s);
      case 4: return expert_npl<BITS, 4, 1>(g, src, shared_rec, b, s);
      case 8: return expert_npl<BITS, 8, 1>(g, src, shared_rec, b, s);
      case 16: return expert_npl<BITS, 16, 1>(g, src, shared_rec, b, s);
      case 32: return expert_npl<BITS, 32, 1>(g, src, shared_rec, b, s);
      case 64: return expert_npl<BITS, 64, 1>(g, src, shared_rec, b, s);
    }
  } else if (it == 2 && BITS == 8) {
    return expert_npl<BITS, 64, 2>(g, src, shared_rec, b, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_shape_supported(const Geometry& g) {
  if (g.bits != 4 && g.bits != 8) return false;
  const int cg = g.H * g.bits / 128, cd = g.I * g.bits / 128;
  if (cg < 2 || cg > 128 || cd < 2 || cd > 128) return false;
  if (g.k < 1 || g.k > kMaxTopK || g.E > 1024 || g.E < g.k) return false;
  if ((size_t)(g.k + 1) * g.I > 15360) return false;  // h staged in <= 60 KiB of LDS
  return true;
}

hipError_t launch_router(const Geometry& g, const float* wr_rows, const float* bias, const StepBuffers& b,
                         hipStream_t s) {
  const dim3 grid((g.E + 1 + 3) / 4), block(256);
  const int nit = (g.H / 4 + kWave - 1) / kWave;  // float4 loads per lane
  switch (nit) {
    case 1: launch(router_kernel<1>, grid, block, 0, s, g, wr_rows, bias, b); break;
    case 2: launch(router_kernel<2>, grid, block, 0, s, g, wr_rows, bias, b); break;
    case 4: launch(router_kernel<4>, grid, block, 0, s, g, wr_rows, bias, b); break;
    case 8: launch(router_kernel<8>, grid, block, 0, s, g, wr_rows, bias, b); break;
    case 16: launch(router_kernel<16>, grid, block, 0, s, g, wr_rows, bias, b); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_route(const Geometry& g, const float* logits, int ld_logits, int n_tok, int32_t* route_idx,
                        float* route_w, float* route_gamma, int32_t* host_route, hipStream_t s) {
  const dim3 grid(n_tok), block(64);
  switch (topk_npl(g.E)) {
    case 1: launch(route_kernel<1>, grid, block, 0, s, g, logits, ld_logits, route_idx, route_w, route_gamma, host_route); break;
    case 2: launch(route_kernel<2>, grid, block, 0, s, g, logits, ld_logits, route_idx, route_w, route_gamma, host_route); break;
    case 4: launch(route_kernel<4>, grid, block, 0, s, g, logits, ld_logits, route_idx, route_w, route_gamma, host_route); break;
    case 8: launch(route_kernel<8>, grid, block, 0, s, g, logits, ld_logits, route_idx, route_w, route_gamma, host_route); break;
    case 16: launch(route_kernel<16>, grid, block, 0, s, g, logits, ld_logits, route_idx, route_w, route_gamma, host_route); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool fused_expert_supported(const Geometry& g) {
  // H <= 2048: the down rows of a larger H do not fit in registers; those
  // shapes keep the two-kernel path
  return g.H <= 2048 && g.I % kSlice == 0;
}

hipError_t launch_expert(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                         hipStream_t s) {
  return g.bits == 4 ? expert_bits<4>(g, src, shared_rec, b, s) : expert_bits<8>(g, src, shared_rec, b, s);
}

hipError_t launch_reduce(const Geometry& g, const StepBuffers& b, const ResidualArgs& r, hipStream_t s) {
  const int nparts = (g.k + 1) * (g.I / kSlice);
  launch(reduce_kernel, dim3(g.H / 64), dim3(64 * kReduceWaves), 0, s, g.H, nparts, (const float*)b.partial, r);
  return hipGetLastError();
}

hipError_t launch_gateup(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec,
                         const StepBuffers& b, hipStream_t s) {
  return g.bits == 4 ? gateup_bits<4>(g, src, shared_rec, b, s) : gateup_bits<8>(g, src, shared_rec, b, s);
}

hipError_t launch_down(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                       const ResidualArgs& r, hipStream_t s) {
  return g.bits == 4 ? down_bits<4>(g, src, shared_rec, b, r, s) : down_bits<8>(g, src, shared_rec, b, r, s);
}

}  // namespace moe
