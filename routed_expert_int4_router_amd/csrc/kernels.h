// Launchers of the HIP kernels (defined in decode.hip and prefill.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

constexpr int kMaxTopK = 16;

// Where the k routed experts of one step are read from.
struct ExpertSource {
  const uint8_t* base;   // routed records: resident blob, or the pool's slot arena
  uint64_t stride;       // bytes between records
  int64_t gid_base;      // resident: record index = gid_base + expert id
  int32_t use_table;     // 1: record index of selection j is table[j] (pool slots)
  int32_t n_sel;         // 0: the fused expert kernel runs every slot j = 0..k (k = shared);
                         // else only slots sel[0..n_sel) (a pool step's hits, then its misses)
  int64_t table[kMaxTopK];
  int32_t sel[kMaxTopK + 1];
};

struct Geometry {
  int32_t H, I, E, k, bits, norm_topk;
  // byte offsets inside a record
  uint64_t gate_codes, up_codes, down_codes, gate_sc, up_sc, down_sc;
};

struct StepBuffers {
  const uint16_t* x;      // bf16 [H] activations of this step
  float* logits;          // [E+1]; entry E is the shared-gate logit
  int32_t* route_idx;     // [k] selection of this step
  float* route_w;         // [k]
  float* route_gamma;     // [1] sigmoid(x . g_s)
  float* h;               // two-kernel path: [(k+1)][I] SwiGLU activations, slot k = shared expert
  float* partial;         // fused path: [(k+1) * I * bits / 128][H] weighted partial down rows
};

struct ResidualArgs {
  float* out;             // plain layer: out[H]; stack: r_out[H]
  const float* r_in;      // stack, layer > 0: r_l [H]; NULL otherwise
  const uint16_t* x_res;  // stack, layer 0: r_0 = x0 (bf16 [H]); NULL otherwise
  uint16_t* x_next;       // stack: bf16(r_{l+1}) [H], or NULL
};

// logits[e] = fp32( sum_h x[h] * wr[e][h] + bias[e] ) for e < E, accumulated in
// fp64; logits[E] = the shared-gate logit (wr row E, no bias).
hipError_t launch_router(const Geometry& g, const float* wr_rows, const float* bias, const StepBuffers& b,
                         hipStream_t s);

// Top-k routing of n_tok tokens, one wave each: logits row t at
// logits + t * ld_logits (E + 1 entries, the last being the shared-gate logit);
// writes route_idx/route_w [t][k] in selection order, route_gamma[t] =
// sigmoid(shared-gate logit), and, when host_route is non-NULL (pinned,
// device-visible), the picks there too.
hipError_t launch_route(const Geometry& g, const float* logits, int ld_logits, int n_tok, int32_t* route_idx,
                        float* route_w, float* route_gamma, int32_t* host_route, hipStream_t s);

// Gate/up GEMV + SwiGLU for the k routed experts and the shared expert -> h.
// Resident source: each block routes the token from the logits itself (block 0
// also writes route_idx/w/gamma for the down kernel). Table source (pool): the
// records are the table's slots and the route must already be written.
hipError_t launch_gateup(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec,
                         const StepBuffers& b, hipStream_t s);

// Down GEMV of the k + 1 experts, weighted combine, optional residual update.
hipError_t launch_down(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                       const ResidualArgs& r, hipStream_t s);

bool decode_shape_supported(const Geometry& g);

// Fused decode path: expert (route + gate/up + SwiGLU + partial down rows of
// one I slice per block) then reduce (fixed-order sum of the partial rows,
// residual update). Used for every shape fused_expert_supported accepts; the
// others run launch_gateup + launch_down.
bool fused_expert_supported(const Geometry& g);
hipError_t launch_expert(const Geometry& g, const ExpertSource& src, const uint8_t* shared_rec, const StepBuffers& b,
                         hipStream_t s);
hipError_t launch_reduce(const Geometry& g, const StepBuffers& b, const ResidualArgs& r, hipStream_t s);

}  // namespace moe
