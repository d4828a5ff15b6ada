// Gated grouped-query attention decode step with an fp16 KV cache, for gfx950:
// the full-attention layers beside the routed MoE (12 of the 80B model's 48).
//
// Pages: those layers are the only ones with a growing K/V cache, budgeted at
// 24 KiB per token in fp16 (alphalab.site field test, section explaining MoE
// expert streaming); the model pairs linear attention with gated attention
// (cheshm.ai article, paragraph on the code base). The pages print no
// formula; the step is the decode form of the Qwen3-Next gated attention
// layer: per-head RMS norms of q and k, rotary embedding of the first `rot`
// dims (pairs (i, i + rot/2), angle p * 1e7^(-2i/rot), computed in fp64), the
// new K/V row stored in fp16, softmax attention of each query head over its KV
// group's cached rows, and the sigmoid output gate.
//
// Split-K decoding, bound by reading the cache (2 * d * 2 bytes per cached
// position and KV group). Kernel 1: one wave per (KV group, 32 positions)
// loads its K rows and V columns straight into MFMA operand registers, 16
// bytes per load, and contracts them with the group's G query heads on
// v_mfma_f32_16x16x32_f16: scores S[j][h] = K[j] . q_h, then
// O[d][h] = sum_j V[j][d] P[h][j]. The G heads sharing one KV group make this
// a real contraction (8 heads per group at the 80B shape): the vector ALU
// would need 8 fp32 FMAs per cached byte. fp16 operands: the cache is fp16;
// q and the softmax weights P are carried as fp16 hi + lo pairs (two MFMAs
// each), so scores and weighted sums keep close to fp32 accuracy. Each wave
// writes softmax partials (max, sum of exp, weighted sum of V); kernel 2 merges
// the partials per query head and applies the output gate.
//
// Cache layout: K [n_kv][max_pos][d] (a position's row contiguous, as the
// score contracts over d), V transposed [n_kv][d][pitch] (a dim's positions
// contiguous, as the weighted sum contracts over positions), pitch = max_pos
// rounded up to 32. The wave whose 32 positions hold the new one computes that
// row itself (norm, rotation, fp16), writes it to the cache and patches it into
// its own registers.
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

constexpr int kSpan = 32;  // positions per wave of kernel 1
constexpr int kCombineDims = 64;
constexpr int kCombineGroups = 4;

__device__ __forceinline__ float bfv(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

struct AttnLayer {
  const float* wq;  // [d]
  const float* wk;  // [d]
  uint16_t* kc;     // [n_kv][max_pos][d] fp16
  uint16_t* vt;     // [n_kv][d][pitch] fp16
};

struct AttnIo {
  const uint16_t* q;     // [n_q][d] bf16
  const uint16_t* gate;  // [n_q][d]
  const uint16_t* k;     // [n_kv][d]
  const uint16_t* v;     // [n_kv][d]
  float* out;            // [n_q][d]
};

struct AttnWork {
  float* ml;      // [n_kv][max_split][G][2]: max, sum of exp
  float* o;       // [n_kv][max_split][G][d]
  int max_split;
};

// RMS norm with weight, then rotation by position of the first `rot` dims, of
// the rows x[R][D] held one value per (row, lane + 64c); writes the results
// (times `scale`) to out[R][D] in LDS. cs/sn: cos, sin of this lane's angles.
template <int D>
__device__ __forceinline__ void norm_rope_rows(const float* x, int R, const float* w, int rot, const float* cs,
                                               const float* sn, float scale, float* tmp, float* out) {
  constexpr int C = D / 64;
  const int lane = threadIdx.x;
  for (int r = 0; r < R; ++r) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) ss = fmaf(x[r * C + c], x[r * C + c], ss);
    ss = dpp::wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + 1e-6f);
#pragma unroll
    for (int c = 0; c < C; ++c) tmp[r * D + lane + 64 * c] = x[r * C + c] * inv * w[c];
  }
  __syncthreads();
  const int half = rot / 2;
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int d = lane + 64 * c;
      const float xn = tmp[r * D + d];
      float y = xn;
      if (d < half) y = xn * cs[c] - tmp[r * D + d + half] * sn[c];
      else if (d < rot) y = xn * cs[c] + tmp[r * D + d - half] * sn[c];
      out[r * D + d] = y * scale;
    }
  }
  __syncthreads();
}

// One wave: KV group g = blockIdx.x % n_kv, positions [j0, j0 + 32) with
// j0 = 32 * (blockIdx.x / n_kv), all of them <= pos except in the last span.
//
// MFMA 16x16x32 operand map (lane = r + 16 * gq, r < 16, gq < 4): A supplies
// row r, B column r, each 8 consecutive k-values of the lane's group gq; C
// gives lane rows 4 * gq + i (i < 4) of column r. Which k-values a group's 8
// slots stand for is free as long as A and B agree, so:
// - scores, C = S[j][h]: row r of tile t is position j0 + 8 * (r / 4) + 4 * t
//   + r % 4, so that C lane (r, gq) holds head r at positions j0 + 8 * gq +
//   e (e = 4 t + i < 8); k-slots of step s are dims 32 s + 8 gq + [0, 8);
// - weighted sums, C = O[d][h], tile n covers dims 16 n + [0, 16); k-slots are
//   positions j0 + 8 gq + [0, 8): A is 16 contiguous bytes of the transposed
//   V row of dim 16 n + r, B the lane's own 8 weights of head r.
template <int D, int G>
__global__ void __launch_bounds__(64) attn_split_kernel(AttnLayer L, AttnIo io, AttnWork W, int n_kv, int max_pos,
                                                        int pitch, int rot, int pos) {
  static_assert(D % 64 == 0 && D <= 256 && G <= 16, "shape");
  constexpr int NS = D / 32;  // score k-steps
  constexpr int NT = D / 16;  // weighted-sum tiles
  constexpr int C = D / 64;   // values per lane of a D-row
  constexpr int QP = D + 8;   // fp16 pitch of the q rows in LDS
  __shared__ float s_tmp[G * D];
  __shared__ float s_qf[G * D];
  __shared__ __align__(16) _Float16 s_qh[G * QP];
  __shared__ __align__(16) _Float16 s_ql[G * QP];
  __shared__ __align__(16) uint16_t s_new[2 * D];  // the new position's K row, V row (fp16)

  const int lane = threadIdx.x, r = lane & 15, gq = lane >> 4;
  const int g = blockIdx.x % n_kv, split = blockIdx.x / n_kv;
  const int j0 = split * kSpan;
  const bool last = pos < j0 + kSpan;

  // 1. loads: the small inputs first (their wait then leaves the cache loads
  //    in flight), then the span's K rows and V columns
  float qx[G * C], wq[C], wk[C], kx[C], vx[C];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < C; ++c) qx[h * C + c] = bfv(io.q[(size_t)(g * G + h) * D + lane + 64 * c]);
#pragma unroll
  for (int c = 0; c < C; ++c) {
    wq[c] = L.wq[lane + 64 * c];
    wk[c] = last ? L.wk[lane + 64 * c] : 0.f;
    kx[c] = last ? bfv(io.k[(size_t)g * D + lane + 64 * c]) : 0.f;
    vx[c] = last ? bfv(io.v[(size_t)g * D + lane + 64 * c]) : 0.f;
  }
  uint4 ka[2][NS], va[NT];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int p = min(j0 + 8 * (r >> 2) + 4 * t + (r & 3), pos);
    const uint16_t* row = L.kc + ((size_t)g * max_pos + p) * D + 8 * gq;
#pragma unroll
    for (int s = 0; s < NS; ++s) ka[t][s] = *reinterpret_cast<const uint4*>(row + 32 * s);
  }
#pragma unroll
  for (int n = 0; n < NT; ++n)
    va[n] = *reinterpret_cast<const uint4*>(L.vt + ((size_t)g * D + 16 * n + r) * pitch + j0 + 8 * gq);

  // 2. rotation angles of this lane's dims (fp64), the G query rows normed,
  //    rotated and scaled by 1 / sqrt(D), split into fp16 hi + lo
  float cs[C], sn[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int d = lane + 64 * c, i = d < rot / 2 ? d : d - rot / 2;
    cs[c] = 1.f;
    sn[c] = 0.f;
    if (d < rot) {
      double sd, cd;
      sincos((double)pos * pow(1.0e7, -2.0 * i / rot), &sd, &cd);
      cs[c] = (float)cd;
      sn[c] = (float)sd;
    }
  }
  norm_rope_rows<D>(qx, G, wq, rot, cs, sn, 1.0f / sqrtf((float)D), s_tmp, s_qf);
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int d = lane + 64 * c;
      const float y = s_qf[h * D + d];
      const _Float16 hi = (_Float16)y;
      s_qh[h * QP + d] = hi;
      s_ql[h * QP + d] = (_Float16)(y - (float)hi);
    }
  // 3. the new position's row (last span only): fp16 K = rotated, normed k;
  //    fp16 V = v; both to the cache and to LDS
  if (last) {
    norm_rope_rows<D>(kx, 1, wk, rot, cs, sn, 1.0f, s_tmp, s_qf);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int d = lane + 64 * c;
      const uint16_t kh = f2h(s_qf[d]), vh = f2h(vx[c]);
      L.kc[((size_t)g * max_pos + pos) * D + d] = kh;
      L.vt[((size_t)g * D + d) * pitch + pos] = vh;
      s_new[d] = kh;
      s_new[D + d] = vh;
    }
  }
  __syncthreads();
  if (last) {
    // K rows: the lane whose row is the new position takes it from LDS
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (j0 + 8 * (r >> 2) + 4 * t + (r & 3) == pos)
#pragma unroll
        for (int s = 0; s < NS; ++s) ka[t][s] = *reinterpret_cast<const uint4*>(s_new + 32 * s + 8 * gq);
    // V columns: the new position from LDS, later positions zero
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      uint16_t e8[8];
      __builtin_memcpy(e8, &va[n], 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int p = j0 + 8 * gq + e;
        e8[e] = p == pos ? s_new[D + 16 * n + r] : (p > pos ? (uint16_t)0 : e8[e]);
      }
      __builtin_memcpy(&va[n], e8, 16);
    }
  }

  // 4. scores S[j][h] = K[j] . q_h (q as hi + lo)
  f32x4 sc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    f16x8 bh = {}, bl = {};
    if (r < G) {
      bh = *reinterpret_cast<const f16x8*>(s_qh + r * QP + 32 * s + 8 * gq);
      bl = *reinterpret_cast<const f16x8*>(s_ql + r * QP + 32 * s + 8 * gq);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f16x8 a = __builtin_bit_cast(f16x8, ka[t][s]);
      sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh, sc[t], 0, 0, 0);
      sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl, sc[t], 0, 0, 0);
    }
  }

  // 5. softmax partials of head r over the span: lane (r, gq) holds positions
  //    j0 + 8 gq + e, e = 4 t + i; positions past pos are masked
  float sv[8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * t + i;
      sv[e] = j0 + 8 * gq + e <= pos ? sc[t][i] : -INFINITY;
    }
  float m = sv[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) m = fmaxf(m, sv[e]);
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));  // finite: position j0 is always live
  f16x8 ph, pl;
  float l = 0.f;
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

  // 6. weighted sums O[d][h] = sum_j V[j][d] P[h][j]
  const size_t part = ((size_t)g * W.max_split + split) * G;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const f16x8 a = __builtin_bit_cast(f16x8, va[n]);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    o = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ph, o, 0, 0, 0);
    o = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pl, o, 0, 0, 0);
    if (r < G) *reinterpret_cast<f32x4*>(W.o + (part + r) * D + 16 * n + 4 * gq) = o;
  }
  if (r < G && gq == 0) {
    W.ml[(part + r) * 2] = m;
    W.ml[(part + r) * 2 + 1] = l;
  }
}

// Block (query head hq, 64 dims), 256 threads = 4 groups of spans x 64 dims:
// each thread folds its spans' partials with a running max, the four groups
// merge through LDS, then out = o / l * sigmoid(gate).
template <int D, int G>
__global__ void __launch_bounds__(kCombineDims * kCombineGroups) attn_combine_kernel(AttnIo io, AttnWork W,
                                                                                     int n_split) {
  __shared__ float s_m[kCombineGroups][kCombineDims], s_l[kCombineGroups][kCombineDims],
      s_o[kCombineGroups][kCombineDims];
  const int hq = blockIdx.x / (D / kCombineDims), d0 = (blockIdx.x % (D / kCombineDims)) * kCombineDims;
  const int g = hq / G, h = hq % G;
  const int dl = threadIdx.x % kCombineDims, grp = threadIdx.x / kCombineDims, d = d0 + dl;
  float M = -INFINITY, l = 0.f, o = 0.f;
  for (int s = grp; s < n_split; s += kCombineGroups) {
    const size_t part = ((size_t)g * W.max_split + s) * G + h;
    const float ms = W.ml[part * 2], ls = W.ml[part * 2 + 1], os = W.o[part * D + d];
    const float Mn = fmaxf(M, ms);
    const float a = expf(M - Mn), b = expf(ms - Mn);
    l = fmaf(l, a, ls * b);
    o = fmaf(o, a, os * b);
    M = Mn;
  }
  s_m[grp][dl] = M;
  s_l[grp][dl] = l;
  s_o[grp][dl] = o;
  __syncthreads();
  if (grp != 0) return;
  float Mt = s_m[0][dl];
#pragma unroll
  for (int q = 1; q < kCombineGroups; ++q) Mt = fmaxf(Mt, s_m[q][dl]);
  float lt = 0.f, ot = 0.f;
#pragma unroll
  for (int q = 0; q < kCombineGroups; ++q) {
    const float f = s_m[q][dl] == -INFINITY ? 0.f : expf(s_m[q][dl] - Mt);
    lt = fmaf(s_l[q][dl], f, lt);
    ot = fmaf(s_o[q][dl], f, ot);
  }
  const float gt = bfv(io.gate[(size_t)hq * D + d]);
  io.out[(size_t)hq * D + d] = ot / lt / (1.0f + expf(-gt));
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
  int pitch = 0;           // positions per transposed V row
  float* norms = nullptr;  // [L][2][d]: q norm weight, k norm weight
  uint16_t* kc = nullptr;  // [L][n_kv][max_pos][d]
  uint16_t* vt = nullptr;  // [L][n_kv][d][pitch]
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

template <int D, int G>
hipError_t launch_dg(moe_attn* a, const AttnLayer& L, const AttnIo& io, int pos, hipStream_t s) {
  const int n_kv = a->cfg.n_kv_heads, n_split = pos / kSpan + 1;
  record(a, a->prof_split);
  launch(attn_split_kernel<D, G>, dim3(n_kv * n_split), dim3(64), 0, s, L, io, a->work, n_kv, a->cfg.max_pos,
         a->pitch, a->cfg.rot_dim, pos);
  record(a, a->prof_combine);
  launch(attn_combine_kernel<D, G>, dim3(a->cfg.n_q_heads * (D / kCombineDims)), dim3(kCombineDims * kCombineGroups),
         0, s, io, a->work, n_split);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(moe_attn* a, const AttnLayer& L, const AttnIo& io, int pos, hipStream_t s) {
  switch (a->cfg.n_q_heads / a->cfg.n_kv_heads) {
    case 1: return launch_dg<D, 1>(a, L, io, pos, s);
    case 2: return launch_dg<D, 2>(a, L, io, pos, s);
    case 4: return launch_dg<D, 4>(a, L, io, pos, s);
    case 8: return launch_dg<D, 8>(a, L, io, pos, s);
    default: return launch_dg<D, 16>(a, L, io, pos, s);
  }
}

AttnLayer layer_args(moe_attn* a, int layer) {
  const size_t D = a->cfg.head_dim, KV = a->cfg.n_kv_heads;
  const float* w = a->norms + (size_t)layer * 2 * D;
  return AttnLayer{w, w + D, a->kc + (size_t)layer * KV * a->cfg.max_pos * D, a->vt + (size_t)layer * KV * D * a->pitch};
}

hipError_t launch_attn(moe_attn* a, int layer, const AttnIo& io, int pos, hipStream_t s) {
  const AttnLayer L = layer_args(a, layer);
  switch (a->cfg.head_dim) {
    case 64: return launch_d<64>(a, L, io, pos, s);
    case 128: return launch_d<128>(a, L, io, pos, s);
    default: return launch_d<256>(a, L, io, pos, s);
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
  a->pitch = (cfg->max_pos + kSpan - 1) / kSpan * kSpan;
  const size_t L = cfg->n_layers, D = cfg->head_dim, KV = cfg->n_kv_heads, P = cfg->max_pos;
  const size_t G = (size_t)(cfg->n_q_heads / cfg->n_kv_heads);
  a->work.max_split = a->pitch / kSpan;
  a->set.assign(L, 0);
  const size_t kbytes = L * KV * P * D * 2, vbytes = L * KV * D * a->pitch * 2;
  bool ok = hipMalloc(&a->norms, L * 2 * D * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&a->kc, kbytes) == hipSuccess;
  ok = ok && hipMalloc(&a->vt, vbytes) == hipSuccess;
  ok = ok && hipMalloc(&a->work.ml, KV * a->work.max_split * G * 2 * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&a->work.o, KV * a->work.max_split * G * D * sizeof(float)) == hipSuccess;
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
  const size_t D = a->cfg.head_dim, KV = a->cfg.n_kv_heads, P = a->cfg.max_pos, pitch = a->pitch;
  const AttnLayer L = layer_args(a, layer);
  // V goes in transposed: one strided 2D copy per group
  for (size_t g = 0; g < KV; ++g) {
    const uint16_t* kg = k + g * n * D;
    const uint16_t* vg = v + g * n * D;
    std::vector<uint16_t> vtg(D * (size_t)n);
    for (int p = 0; p < n; ++p)
      for (size_t d = 0; d < D; ++d) vtg[d * n + p] = vg[(size_t)p * D + d];
    if (hipMemcpy(L.kc + (g * P + first_pos) * D, kg, (size_t)n * D * 2, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy2D(L.vt + g * D * pitch + first_pos, pitch * 2, vtg.data(), (size_t)n * 2, (size_t)n * 2, D,
                    hipMemcpyHostToDevice) != hipSuccess)
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
  const size_t D = a->cfg.head_dim, KV = a->cfg.n_kv_heads, P = a->cfg.max_pos, pitch = a->pitch;
  const AttnLayer L = layer_args(a, layer);
  for (size_t g = 0; g < KV; ++g) {
    if (k && hipMemcpy(k + g * n * D, L.kc + (g * P + first_pos) * D, (size_t)n * D * 2, hipMemcpyDeviceToHost) !=
                 hipSuccess)
      return fail(MOE_EHIP, "moe_attn_read_cache: copy");
    if (v) {
      std::vector<uint16_t> vtg(D * (size_t)n);
      if (hipMemcpy2D(vtg.data(), (size_t)n * 2, L.vt + g * D * pitch + first_pos, pitch * 2, (size_t)n * 2, D,
                      hipMemcpyDeviceToHost) != hipSuccess)
        return fail(MOE_EHIP, "moe_attn_read_cache: copy");
      for (int p = 0; p < n; ++p)
        for (size_t d = 0; d < D; ++d) v[g * n * D + (size_t)p * D + d] = vtg[d * n + p];
    }
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
  auto enqueue = [&](hipStream_t qs) -> moe_status {
    for (int t = 0; t < n_tok; ++t)
      for (int l = first_layer; l < first_layer + n_layers; ++l) {
        const size_t r = (size_t)t * n_layers + (l - first_layer);
        const AttnIo io{q + r * QD, gate + r * QD, k + r * KD, v + r * KD, out + r * QD};
        const hipError_t e = launch_attn(a, l, io, pos0 + t, qs);
        if (e != hipSuccess) return fail(MOE_EHIP, std::string("moe_attn_decode: launch: ") + hipGetErrorString(e));
      }
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
  hipFree(a->kc);
  hipFree(a->vt);
  hipFree(a->work.ml);
  hipFree(a->work.o);
  delete a;
}

}  // extern "C"
