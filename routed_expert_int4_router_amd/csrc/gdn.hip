// Gated DeltaNet decode step for gfx950: the linear-attention layers that sit
// beside the routed MoE in 36 of the 80B model's 48 layers.
//
// Pages: those layers keep a fixed-size recurrent state, about 72 MiB over the
// 36 layers, instead of a growing KV cache (alphalab.site field test, section
// explaining MoE expert streaming); the model is a hybrid of linear attention
// (Gated DeltaNet) and gated attention with a sparse MoE (cheshm.ai article,
// paragraph on the code base). The pages print no formula; the step follows
// the published gated delta rule (Yang, Kautz and Hatamizadeh, 2024) in the
// decode form of the Qwen3-Next linear-attention layer, per value head h:
//   conv     a 4-tap causal depthwise convolution + SiLU over the q, k, v
//            channels (the last three inputs of every channel kept as state)
//   norms    q and k L2-normalised per head (epsilon 1e-6), q / sqrt(d_k)
//   gates    alpha = exp(-exp(A_log) * softplus(a + dt_bias)), beta = sigmoid(b)
//   state    S <- alpha S; u = beta (v - S^T k); S <- S + k u^T; o = S^T q
//   output   o / sqrt(mean(o^2) + 1e-6) * w_norm * silu(z)
//
// A step is two kernels. The state kernel spreads each head's fp32 state
// [d_v][d_k] (64 KiB at the 80B shape) over NC blocks of R rows (8 blocks of
// 16 rows: 256 blocks for 32 heads, one per CU); each block holds its rows in
// registers between one read and one write, so the state crosses HBM exactly
// once each way: HBM-bound, 4 MiB per layer and token at the 80B shape. TPV =
// d_k / 16 threads share a state row v; thread i of a row owns k = 4 i + 4 TPV
// j (j < 4), so every float4 load of a wave covers whole 128-byte runs; the
// sums over k are DPP reductions within the row's TPV lanes. Every block
// recomputes its key head's q and k (a few hundred channels), cheaper than an
// exchange between blocks. The gated RMS norm needs all d_v outputs of a
// head, which lie in 8 blocks, so each step's kernel also applies the norm of
// the step before it (its outputs are complete by then: a few hundred bytes
// per block, read while the state loads are in flight); a call's last step
// is normed by a small kernel of its own (one block per head). Folding the
// norm into one block per head instead (32 blocks of 1024 threads, 64 KiB of
// state each) was slower: 32 CUs move the state at a fraction of 256's rate.
#include <hip/hip_runtime.h>

#include <algorithm>
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

__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

// One output of the gated RMS norm of a head whose d_v outputs before the
// norm have sum of squares ss; the same expression wherever a step is normed
// (the next step's kernel or the call's last norm kernel), so outputs do not
// depend on how a sequence is split into calls.
template <int DV>
__device__ __forceinline__ float gated_norm(float o, float ss, float w, float z) {
  const float inv = 1.0f / sqrtf(ss / (float)DV + 1e-6f);
  return o * inv * w * silu_f(z);
}

struct GdnLayer {
  const float* conv_w;   // [C][4]
  const float* a_log;    // [Hv]
  const float* dt_bias;  // [Hv]
  const float* norm_w;   // [dv]
  float* state;          // [Hv][dv][dk]
  const float* win_in;   // [C][3] conv inputs t-3, t-2, t-1
  float* win_out;        // [C][3] conv inputs t-2, t-1, t
};

struct GdnIo {
  const uint16_t* qkv;   // [C] bf16
  const uint16_t* z;     // [Hv * dv]
  const uint16_t* a;     // [Hv]
  const uint16_t* b;     // [Hv]
  float* out;            // [Hv * dv]
};

// The previous step's gated norm, applied by the next step's kernel: its
// outputs before the norm, its z, its layer's norm weight and its output.
// With valid = 0 the pointers are any readable ones and nothing is written.
struct GdnPrevNorm {
  const float* o;        // [Hv][dv]
  const uint16_t* z;     // [Hv * dv]
  const float* norm_w;   // [dv]
  float* out;            // [Hv * dv]
  int valid;
};

// Threads per block and state rows per block of the state kernel.
template <int DK, int DV>
struct GdnTile {
  static constexpr int TPV = DK / 16;                       // threads per state row
  static constexpr int NT = DV * TPV < 128 ? DV * TPV : 128;
  static constexpr int R = NT / TPV;                        // rows per block
  static constexpr int NC = DV / R;                         // blocks per head
};

// Block (head h, row chunk) of the state kernel: the conv, norms and gates
// of head h (every block of the head recomputes them, a few hundred
// channels), then rows [R c, R c + R) of the head's state: decay, S^T k,
// delta-rule write, S^T q. Writes o before the norm to o_pre; with
// prev.valid, also writes rows [R c, R c + R) of head h of the previous
// step's normed output.
template <int DK, int DV>
__global__ void __launch_bounds__(DV * (DK / 16) < 128 ? DV * (DK / 16) : 128) gdn_state_kernel(GdnLayer L, GdnIo io, float* o_pre, GdnPrevNorm prev,
                                                                         int n_k, int n_v) {
  using Tl = GdnTile<DK, DV>;
  constexpr int TPV = Tl::TPV, NT = Tl::NT, R = Tl::R, NC = Tl::NC;
  static_assert(TPV >= 1 && TPV <= 16 && (TPV & (TPV - 1)) == 0, "state rows are reduced within a DPP row");
  static_assert(NT % 64 == 0, "whole waves");
  __shared__ float s_q[DK], s_k[DK], s_v[R];
  __shared__ float s_red[3][NT / 64];
  const int h = blockIdx.x / NC, chunk = blockIdx.x % NC;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int kh = h / (n_v / n_k);
  const int v = chunk * R + t / TPV, i = t % TPV;
  const int nq = n_k * DK;

  // 1. the block's state rows first: the longest wait of the step
  float* srow = L.state + ((size_t)h * DV + v) * DK;
  float4 s[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s[j] = *reinterpret_cast<const float4*>(srow + 4 * i + 4 * TPV * j);

  // gate inputs of the head, also before any wait
  const float a_in = bf(io.a[h]), b_in = bf(io.b[h]), dt = L.dt_bias[h], alog = L.a_log[h];
  // the previous step's outputs of head h before its norm (thread t < DV: row
  // t; NT >= DV), and z and the norm weight of this block's rows (t < R)
  const float po_all = prev.o[(size_t)h * DV + min(t, DV - 1)];   // unconditional load, then select
  const float po = t < DV ? po_all : 0.f;
  const int pv = chunk * R + min(t, R - 1);
  const float pz = bf(prev.z[(size_t)h * DV + pv]), pw = prev.norm_w[pv];
  const float po_row = prev.o[(size_t)h * DV + pv];

  // 2. convolution + SiLU: q and k of the key head, v of the block's rows. The
  //    history moves on in the other buffer, each channel's by one block only
  //    (q/k: the key head's first value head, chunk 0).
  //    Every load of every channel is issued before any arithmetic or store,
  //    so the block waits for memory once.
  constexpr int CH = 2 * DK + R, IT = (CH + NT - 1) / NT;
  const bool owns_qk = (h % (n_v / n_k)) == 0 && chunk == 0;
  int chn[IT];
  float xin[IT], w0[IT][4], w1[IT][3];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = min(t + NT * it, CH - 1);  // clamped: every load issues unconditionally
    chn[it] = c < DK ? kh * DK + c
                     : (c < 2 * DK ? nq + kh * DK + (c - DK) : 2 * nq + h * DV + chunk * R + (c - 2 * DK));
    xin[it] = bf(io.qkv[chn[it]]);
    const float4 w = *reinterpret_cast<const float4*>(L.conv_w + (size_t)chn[it] * 4);
    w0[it][0] = w.x;
    w0[it][1] = w.y;
    w0[it][2] = w.z;
    w0[it][3] = w.w;
    const float* wi = L.win_in + (size_t)chn[it] * 3;
    w1[it][0] = wi[0];
    w1[it][1] = wi[1];
    w1[it][2] = wi[2];
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = t + NT * it;
    if (c >= CH) continue;
    const float x = xin[it];
    const float y = silu_f(((w0[it][0] * w1[it][0] + w0[it][1] * w1[it][1]) + w0[it][2] * w1[it][2]) + w0[it][3] * x);
    if (c < DK) s_q[c] = y;
    else if (c < 2 * DK) s_k[c - DK] = y;
    else s_v[c - 2 * DK] = y;
    if (c >= 2 * DK || owns_qk) {
      float* wo = L.win_out + (size_t)chn[it] * 3;
      wo[0] = w1[it][1];
      wo[1] = w1[it][2];
      wo[2] = x;
    }
  }
  __syncthreads();
  // 3. L2 norms of q and k, and the previous step's sum of o^2 (wave sums,
  //    then the waves in order)
  {
    float sq = 0.f, sk = 0.f;
    for (int c = t; c < DK; c += NT) {
      sq += s_q[c] * s_q[c];
      sk += s_k[c] * s_k[c];
    }
    sq = dpp::wave_sum(sq);
    sk = dpp::wave_sum(sk);
    const float so = dpp::wave_sum(po * po);
    if (lane == 0) {
      s_red[0][wv] = sq;
      s_red[1][wv] = sk;
      s_red[2][wv] = so;
    }
  }
  __syncthreads();
  float nq2 = 0.f, nk2 = 0.f, no2 = 0.f;
  for (int w = 0; w < NT / 64; ++w) {
    nq2 += s_red[0][w];
    nk2 += s_red[1][w];
    no2 += s_red[2][w];
  }
  if (prev.valid && t < R) prev.out[(size_t)h * DV + pv] = gated_norm<DV>(po_row, no2, pw, pz);
  const float qs = 1.0f / (sqrtf(nq2 + 1e-6f) * sqrtf((float)DK));
  const float ks = 1.0f / sqrtf(nk2 + 1e-6f);
  // 4. gates of the head
  const float ga = a_in + dt;
  const float sp = ga > 20.f ? ga : log1pf(expf(ga));
  const float alpha = expf(-expf(alog) * sp);
  const float beta = 1.0f / (1.0f + expf(-b_in));
  // 5. decay, S^T k, delta-rule write, S^T q
  float sv[16], kk[16], qq[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kk[4 * j + e] = s_k[4 * i + 4 * TPV * j + e] * ks;
      qq[4 * j + e] = s_q[4 * i + 4 * TPV * j + e] * qs;
    }
    sv[4 * j] = s[j].x * alpha;
    sv[4 * j + 1] = s[j].y * alpha;
    sv[4 * j + 2] = s[j].z * alpha;
    sv[4 * j + 3] = s[j].w * alpha;
  }
  float kv = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) kv = fmaf(sv[e], kk[e], kv);
  kv = dpp::group_sum<TPV>(kv);
  const float u = beta * (s_v[v - chunk * R] - kv);
  float o = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    sv[e] = fmaf(kk[e], u, sv[e]);
    o = fmaf(sv[e], qq[e], o);
  }
  o = dpp::group_sum<TPV>(o);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<float4*>(srow + 4 * i + 4 * TPV * j) = make_float4(sv[4 * j], sv[4 * j + 1], sv[4 * j + 2],
                                                                         sv[4 * j + 3]);
  if (i == 0) o_pre[(size_t)h * DV + v] = o;
}

// One block per head: out = o / sqrt(mean(o^2) + 1e-6) * w_norm * silu(z).
// Whole waves: a block of d_v < 64 rows still runs 64 threads, the extra
// ones adding zeros.
template <int DV>
__global__ void __launch_bounds__(DV < 64 ? 64 : DV) gdn_norm_kernel(const float* __restrict__ o_pre,
                                                                     const float* __restrict__ norm_w,
                                                                     const uint16_t* __restrict__ z, float* out) {
  constexpr int NW = (DV + 63) / 64;
  __shared__ float s_red[NW];
  const int h = blockIdx.x, v = threadIdx.x, lane = v & 63;
  const bool live = v < DV;
  const float o = live ? o_pre[(size_t)h * DV + v] : 0.f;
  float o2 = dpp::wave_sum(o * o);
  if (lane == 0) s_red[v >> 6] = o2;
  __syncthreads();
  float ss = 0.f;
  for (int q = 0; q < NW; ++q) ss += s_red[q];
  if (live) out[(size_t)h * DV + v] = gated_norm<DV>(o, ss, norm_w[v], bf(z[(size_t)h * DV + v]));
}

struct GdnGraph {
  int layer0, n_layers, n_tok, parity;
  const void* qkv;
  const void* z;
  const void* a;
  const void* b;
  void* out;
  hipGraphExec_t exec;
  hipEvent_t done;
  uint64_t stamp;
};

}  // namespace
}  // namespace moe

using namespace moe;

struct moe_gdn {
  uint64_t magic = 0x4d4f4547444e2121ull;
  moe_gdn_config cfg{};
  int device = 0;
  size_t C = 0;
  float* params = nullptr;   // per layer: conv_w [C][4], a_log [Hv], dt_bias [Hv], norm_w [dv]
  size_t params_per_layer = 0;
  float* state = nullptr;    // [L][Hv][dv][dk]
  float* window = nullptr;   // [L][2][C][3]
  float* o_pre = nullptr;    // [2][Hv][dv]: steps' outputs before the norm (even, odd steps of a call)
  std::vector<int64_t> pos;  // tokens each layer has taken
  std::vector<uint8_t> set;
  std::vector<GdnGraph> graphs;
  hipStream_t cap_stream = nullptr;
  uint64_t clock = 0;
  bool prof = false;                                // time every launch (graphs bypassed)
  std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_events;
};

namespace {

std::mutex g_gdn_mu;
std::set<const moe_gdn*> g_gdn_live;

moe_status gdn_check(const moe_gdn* g, const char* fn) {
  if (!g) return fail(MOE_EINVAL, std::string(fn) + ": handle is NULL");
  std::lock_guard<std::mutex> l(g_gdn_mu);
  if (!g_gdn_live.count(g)) return fail(MOE_ESTATE, std::string(fn) + ": not a live DeltaNet handle");
  return MOE_OK;
}

std::string gdn_config_error(const moe_gdn_config* c) {
  if (!c) return "config is NULL";
  if (c->n_layers < 1 || c->n_layers > 4096) return "n_layers must be in [1, 4096]";
  if (c->n_k_heads < 1 || c->n_v_heads < c->n_k_heads || c->n_v_heads % c->n_k_heads)
    return "n_v_heads must be a positive multiple of n_k_heads";
  if (c->n_v_heads > 4096) return "n_v_heads must be <= 4096";
  const bool ok = (c->d_k == 128 && c->d_v == 128) || (c->d_k == 64 && c->d_v == 64) ||
                  (c->d_k == 32 && c->d_v == 32);
  if (!ok) return "(d_k, d_v) must be (32, 32), (64, 64) or (128, 128)";
  return "";
}

GdnLayer layer_args(moe_gdn* g, int l, int parity) {
  const size_t C = g->C, Hv = g->cfg.n_v_heads, dv = g->cfg.d_v, dk = g->cfg.d_k;
  const float* p = g->params + (size_t)l * g->params_per_layer;
  GdnLayer L;
  L.conv_w = p;
  L.a_log = p + C * 4;
  L.dt_bias = L.a_log + Hv;
  L.norm_w = L.dt_bias + Hv;
  L.state = g->state + (size_t)l * Hv * dv * dk;
  L.win_in = g->window + ((size_t)l * 2 + parity) * C * 3;
  L.win_out = g->window + ((size_t)l * 2 + (parity ^ 1)) * C * 3;
  return L;
}

template <int D>
hipError_t launch_step_d(moe_gdn* g, const GdnLayer& L, const GdnIo& io, float* o_pre, const GdnPrevNorm& prev,
                         hipStream_t s) {
  using Tl = GdnTile<D, D>;
  const int Hv = g->cfg.n_v_heads, Hk = g->cfg.n_k_heads;
  if (g->prof) {
    // the state kernel's launch fills the pair with its own begin/end timestamps
    LaunchEvents ev{};
    if (hipEventCreate(&ev.start) != hipSuccess || hipEventCreate(&ev.stop) != hipSuccess) return hipErrorOutOfMemory;
    launch_events() = ev;
    g->prof_events.emplace_back(ev.start, ev.stop);
  }
  launch(gdn_state_kernel<D, D>, dim3(Hv * Tl::NC), dim3(Tl::NT), 0, s, L, io, o_pre, prev, Hk, Hv);
  return hipGetLastError();
}

template <int D>
hipError_t launch_norm_d(moe_gdn* g, const GdnPrevNorm& last, hipStream_t s) {
  launch(gdn_norm_kernel<D>, dim3(g->cfg.n_v_heads), dim3(D < 64 ? 64 : D), 0, s, last.o, last.norm_w, last.z,
         last.out);
  return hipGetLastError();
}

hipError_t launch_norm(moe_gdn* g, const GdnPrevNorm& last, hipStream_t s) {
  switch (g->cfg.d_k) {
    case 128: return launch_norm_d<128>(g, last, s);
    case 64: return launch_norm_d<64>(g, last, s);
    default: return launch_norm_d<32>(g, last, s);
  }
}

hipError_t launch_step(moe_gdn* g, const GdnLayer& L, const GdnIo& io, float* o_pre, const GdnPrevNorm& prev,
                       hipStream_t s) {
  switch (g->cfg.d_k) {
    case 128: return launch_step_d<128>(g, L, io, o_pre, prev, s);
    case 64: return launch_step_d<64>(g, L, io, o_pre, prev, s);
    default: return launch_step_d<32>(g, L, io, o_pre, prev, s);
  }
}

}  // namespace

extern "C" {

moe_status moe_gdn_create(const moe_gdn_config* cfg, moe_gdn** out) {
  clear_error();
  if (!out) return fail(MOE_EINVAL, "moe_gdn_create: out is NULL");
  *out = nullptr;
  const std::string why = gdn_config_error(cfg);
  if (!why.empty()) return fail(MOE_EINVAL, "moe_gdn_create: " + why);
  moe_gdn* g = new moe_gdn();
  g->cfg = *cfg;
  hipGetDevice(&g->device);
  const size_t L = cfg->n_layers, Hv = cfg->n_v_heads, Hk = cfg->n_k_heads, dk = cfg->d_k, dv = cfg->d_v;
  g->C = 2 * Hk * dk + Hv * dv;
  g->params_per_layer = (g->C * 4 + 2 * Hv + dv + 3) / 4 * 4;  // each layer's conv_w 16-byte aligned
  g->pos.assign(L, 0);
  g->set.assign(L, 0);
  bool ok = hipMalloc(&g->params, L * g->params_per_layer * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&g->state, L * Hv * dv * dk * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&g->window, L * 2 * g->C * 3 * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&g->o_pre, 2 * Hv * dv * sizeof(float)) == hipSuccess;
  ok = ok && hipMemset(g->params, 0, L * g->params_per_layer * sizeof(float)) == hipSuccess;
  ok = ok && hipMemset(g->state, 0, L * Hv * dv * dk * sizeof(float)) == hipSuccess;
  ok = ok && hipMemset(g->window, 0, L * 2 * g->C * 3 * sizeof(float)) == hipSuccess;
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  {
    std::lock_guard<std::mutex> l(g_gdn_mu);
    g_gdn_live.insert(g);
  }
  if (!ok) {
    moe_gdn_destroy(g);
    return fail(MOE_ENOMEM, "moe_gdn_create: allocation failed");
  }
  *out = g;
  return MOE_OK;
}

moe_status moe_gdn_set_layer(moe_gdn* g, int32_t layer, const float* conv_w, const float* a_log, const float* dt_bias,
                             const float* norm_w) {
  clear_error();
  moe_status st = gdn_check(g, "moe_gdn_set_layer");
  if (st) return st;
  if (layer < 0 || layer >= g->cfg.n_layers) return fail(MOE_EINVAL, "moe_gdn_set_layer: layer out of range");
  if (!conv_w || !a_log || !dt_bias || !norm_w) return fail(MOE_EINVAL, "moe_gdn_set_layer: NULL pointer");
  const size_t C = g->C, Hv = g->cfg.n_v_heads, dv = g->cfg.d_v;
  std::vector<float> p(g->params_per_layer);
  std::memcpy(p.data(), conv_w, C * 4 * sizeof(float));
  std::memcpy(p.data() + C * 4, a_log, Hv * sizeof(float));
  std::memcpy(p.data() + C * 4 + Hv, dt_bias, Hv * sizeof(float));
  std::memcpy(p.data() + C * 4 + 2 * Hv, norm_w, dv * sizeof(float));
  const hipError_t e = hipMemcpy(g->params + (size_t)layer * g->params_per_layer, p.data(), p.size() * sizeof(float),
                                 hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(MOE_EHIP, std::string("moe_gdn_set_layer: ") + hipGetErrorString(e));
  g->set[(size_t)layer] = 1;
  return MOE_OK;
}

moe_status moe_gdn_reset(moe_gdn* g) {
  clear_error();
  moe_status st = gdn_check(g, "moe_gdn_reset");
  if (st) return st;
  const size_t L = g->cfg.n_layers, Hv = g->cfg.n_v_heads, dk = g->cfg.d_k, dv = g->cfg.d_v;
  bool ok = hipDeviceSynchronize() == hipSuccess;
  ok = ok && hipMemset(g->state, 0, L * Hv * dv * dk * sizeof(float)) == hipSuccess;
  ok = ok && hipMemset(g->window, 0, L * 2 * g->C * 3 * sizeof(float)) == hipSuccess;
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  if (!ok) return fail(MOE_EHIP, "moe_gdn_reset: clearing the state failed");
  std::fill(g->pos.begin(), g->pos.end(), 0);
  return MOE_OK;
}

moe_status moe_gdn_decode(moe_gdn* g, int32_t first_layer, int32_t n_layers, const uint16_t* qkv, const uint16_t* z,
                          const uint16_t* a, const uint16_t* b, int32_t n_tok, float* out, void* stream) {
  clear_error();
  moe_status st = gdn_check(g, "moe_gdn_decode");
  if (st) return st;
  if (first_layer < 0 || n_layers < 1 || first_layer + n_layers > g->cfg.n_layers)
    return fail(MOE_EINVAL, "moe_gdn_decode: layer range outside [0, n_layers)");
  if (n_tok < 0 || n_tok > 65536) return fail(MOE_EINVAL, "moe_gdn_decode: n_tok must be in [0, 65536]");
  if (n_tok == 0) return MOE_OK;
  if (!qkv || !z || !a || !b || !out) return fail(MOE_EINVAL, "moe_gdn_decode: NULL pointer");
  for (int l = first_layer; l < first_layer + n_layers; ++l)
    if (!g->set[(size_t)l]) return fail(MOE_ESTATE, "moe_gdn_decode: moe_gdn_set_layer was not called for a layer");
  const size_t C = g->C, Z = (size_t)g->cfg.n_v_heads * g->cfg.d_v, Hv = g->cfg.n_v_heads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // every layer's window parity moves on by n_tok; a captured sequence is
  // valid for the parity it started from
  const int parity = (int)(g->pos[(size_t)first_layer] & 1);
  for (int l = first_layer; l < first_layer + n_layers; ++l)
    if ((int)(g->pos[(size_t)l] & 1) != parity)
      return fail(MOE_ESTATE, "moe_gdn_decode: the layers of one call must have taken the same number of tokens");
  // step k (token-major) writes its outputs before the norm to o_pre half
  // k % 2 and norms step k - 1's; the call's last step is normed on its own
  auto enqueue = [&](hipStream_t q) -> moe_status {
    GdnPrevNorm prev{g->o_pre, z, nullptr, out, 0};
    for (int t = 0; t < n_tok; ++t) {
      for (int l = first_layer; l < first_layer + n_layers; ++l) {
        const size_t r = (size_t)t * n_layers + (l - first_layer);
        GdnIo io{qkv + r * C, z + r * Z, a + r * Hv, b + r * Hv, out + r * Z};
        const GdnLayer L = layer_args(g, l, (parity + t) & 1);
        float* o_cur = g->o_pre + (r & 1) * Hv * g->cfg.d_v;
        if (!prev.norm_w) prev.norm_w = L.norm_w;   // first step: any readable weight
        const hipError_t e = launch_step(g, L, io, o_cur, prev, q);
        if (e != hipSuccess) return fail(MOE_EHIP, std::string("moe_gdn_decode: launch: ") + hipGetErrorString(e));
        prev = GdnPrevNorm{o_cur, io.z, L.norm_w, io.out, 1};
      }
    }
    const hipError_t e = launch_norm(g, prev, q);
    if (e != hipSuccess) return fail(MOE_EHIP, std::string("moe_gdn_decode: launch: ") + hipGetErrorString(e));
    return MOE_OK;
  };
  if ((int64_t)n_tok * n_layers < 16 || g->prof) {
    st = enqueue(s);
    if (st) return st;
  } else {
    GdnGraph* hit = nullptr;
    for (auto& e : g->graphs)
      if (e.layer0 == first_layer && e.n_layers == n_layers && e.n_tok == n_tok && e.parity == parity &&
          e.qkv == qkv && e.z == z && e.a == a && e.b == b && e.out == out)
        hit = &e;
    if (!hit) {
      if (!g->cap_stream && hipStreamCreateWithFlags(&g->cap_stream, hipStreamNonBlocking) != hipSuccess)
        return fail(MOE_EHIP, "moe_gdn_decode: capture stream");
      if (hipStreamBeginCapture(g->cap_stream, hipStreamCaptureModeThreadLocal) != hipSuccess)
        return fail(MOE_EHIP, "moe_gdn_decode: capture begin");
      st = enqueue(g->cap_stream);
      hipGraph_t graph = nullptr;
      const hipError_t e = hipStreamEndCapture(g->cap_stream, &graph);
      if (st) {
        if (graph) hipGraphDestroy(graph);
        return st;
      }
      if (e != hipSuccess) return fail(MOE_EHIP, "moe_gdn_decode: capture end");
      GdnGraph ent{first_layer, n_layers, n_tok, parity, qkv, z, a, b, out, nullptr, nullptr, 0};
      const hipError_t ei = hipGraphInstantiate(&ent.exec, graph, nullptr, nullptr, 0);
      hipGraphDestroy(graph);
      if (ei != hipSuccess) return fail(MOE_EHIP, "moe_gdn_decode: graph instantiate");
      if (hipEventCreateWithFlags(&ent.done, hipEventDisableTiming) != hipSuccess) {
        hipGraphExecDestroy(ent.exec);
        return fail(MOE_EHIP, "moe_gdn_decode: graph event");
      }
      if (g->graphs.size() >= 8) {
        auto lru = std::min_element(g->graphs.begin(), g->graphs.end(),
                                    [](const GdnGraph& x, const GdnGraph& y) { return x.stamp < y.stamp; });
        hipEventSynchronize(lru->done);  // its last launch may still run
        hipGraphExecDestroy(lru->exec);
        hipEventDestroy(lru->done);
        g->graphs.erase(lru);
      }
      g->graphs.push_back(ent);
      hit = &g->graphs.back();
    }
    hit->stamp = ++g->clock;
    if (hipGraphLaunch(hit->exec, s) != hipSuccess) return fail(MOE_EHIP, "moe_gdn_decode: graph launch");
    if (hipEventRecord(hit->done, s) != hipSuccess) return fail(MOE_EHIP, "moe_gdn_decode: graph event record");
  }
  for (int l = first_layer; l < first_layer + n_layers; ++l) g->pos[(size_t)l] += n_tok;
  return MOE_OK;
}

moe_status moe_gdn_profile(moe_gdn* g, int32_t enable, double* total_ms, uint64_t* launches) {
  clear_error();
  moe_status st = gdn_check(g, "moe_gdn_profile");
  if (st) return st;
  if (enable != 0 && enable != 1) return fail(MOE_EINVAL, "moe_gdn_profile: enable must be 0 or 1");
  double ms = 0.0;
  uint64_t n = 0;
  for (auto& pr : g->prof_events) {
    float t = 0.f;
    if (hipEventSynchronize(pr.second) == hipSuccess && hipEventElapsedTime(&t, pr.first, pr.second) == hipSuccess) {
      ms += t;
      ++n;
    }
    hipEventDestroy(pr.first);
    hipEventDestroy(pr.second);
  }
  g->prof_events.clear();
  if (total_ms) *total_ms = ms;
  if (launches) *launches = n;
  g->prof = enable != 0;
  return MOE_OK;
}

moe_status moe_gdn_read_state(moe_gdn* g, int32_t layer, float* state, float* window) {
  clear_error();
  moe_status st = gdn_check(g, "moe_gdn_read_state");
  if (st) return st;
  if (layer < 0 || layer >= g->cfg.n_layers) return fail(MOE_EINVAL, "moe_gdn_read_state: layer out of range");
  if (hipDeviceSynchronize() != hipSuccess) return fail(MOE_EHIP, "moe_gdn_read_state: sync");
  const size_t C = g->C, Hv = g->cfg.n_v_heads, dk = g->cfg.d_k, dv = g->cfg.d_v;
  const GdnLayer L = layer_args(g, layer, (int)(g->pos[(size_t)layer] & 1));
  if (state && hipMemcpy(state, L.state, Hv * dv * dk * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(MOE_EHIP, "moe_gdn_read_state: copy");
  if (window && hipMemcpy(window, L.win_in, C * 3 * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(MOE_EHIP, "moe_gdn_read_state: copy");
  return MOE_OK;
}

void moe_gdn_destroy(moe_gdn* g) {
  {
    std::lock_guard<std::mutex> l(g_gdn_mu);
    if (!g || !g_gdn_live.count(g)) return;
    g_gdn_live.erase(g);
  }
  hipDeviceSynchronize();
  for (auto& pr : g->prof_events) {
    hipEventDestroy(pr.first);
    hipEventDestroy(pr.second);
  }
  for (auto& e : g->graphs) {
    hipGraphExecDestroy(e.exec);
    hipEventDestroy(e.done);
  }
  if (g->cap_stream) hipStreamDestroy(g->cap_stream);
  hipFree(g->params);
  hipFree(g->state);
  hipFree(g->window);
  hipFree(g->o_pre);
  delete g;
}

}  // extern "C"
