// Batched (prefill) path of the routed MoE step: router GEMM, top-k, bucketing
// of (token, slot) pairs by expert, MFMA grouped GEMMs, combine.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"
#include "moe.h"

namespace moe {

struct PrefillArgs {
  moe_config cfg;
  Geometry geo;
  const uint8_t* experts;   // device, routed records of this layer (E records at stride)
  uint64_t stride;
  const uint8_t* shared;    // device, shared-expert record of this layer
  const float* wr_rows;     // device fp32 [E+1][H]: the router rows (row E = shared gate)
  const uint16_t* wr_split; // device bf16 [3][E+1][H]: the router rows as hi + mid + lo (exact)
  const float* bias;        // device [E]
  const uint16_t* x;        // device bf16 [n_tok][H]
  int32_t n_tok;
  float* out;               // device fp32 [n_tok][H]
  int32_t* route_idx;       // device [n_tok][k]
  float* route_w;           // device [n_tok][k]
  float* route_gamma;       // device [n_tok]
  int32_t scalar;           // 1: the plainly written grouped GEMMs (bit-identical, slow)
};

// Device arrays of the batched path for batches of up to T tokens.
struct PrefillWorkspace {
  int T = 0, E = 0, k = 0, H = 0, I = 0;
  float* logits = nullptr;      // [T][E+1]
  float* xscale = nullptr;      // [T] power-of-two scale of each token
  uint16_t* xp = nullptr;       // [T][H] fp16 bits of x / xscale, k-permuted
  int32_t* cnt = nullptr;       // [nchunk][E]
  int32_t* chunk_off = nullptr; // [nchunk][E]
  int32_t* perm = nullptr;      // [T*k] sorted position -> pair id
  float* wperm = nullptr;       // [T*k] sorted position -> router weight of the pair
  int32_t* tiles = nullptr;     // [4 + 4 max_tiles]: count (3 unused), then per tile (expert, row0, base, rows)
  uint16_t* h16 = nullptr;      // [T*k + T][I] fp16 bits, h / range scale
  float* hscale = nullptr;      // [max_tiles][I/64] power-of-two scale of each (tile, group), sign = mixed
  float* hrowf = nullptr;       // [T*k + T][I/64] power-of-two factor of each row relative to its tile-group
  float* hsum = nullptr;        // [T*k + T][I/64]
  float* y = nullptr;           // [T*k + T][H]
  int max_tiles = 0;
};

bool prefill_supported(const moe_config& cfg);

// Bytes of a workspace for batches of up to n_tok tokens laid out in one
// block of device memory, route arrays ([n_tok][k] idx and w, [n_tok] gamma)
// included; prefill_place points w and the route arrays into such a block.
// Nothing needs clearing: every kernel writes what a later one reads.
size_t prefill_placed_bytes(const moe_config& cfg, int n_tok);
void prefill_place(PrefillWorkspace* w, const moe_config& cfg, int n_tok, uint8_t* base, int32_t** route_idx,
                   float** route_w, float** route_gamma);

// Workspace for batches of up to n_tok tokens (grown on demand; synchronises
// the device when it has to reallocate).
moe_status prefill_reserve(void** workspace, const moe_config& cfg, int n_tok);
void prefill_free(void* workspace);

// The stages, one kernel each, in this order on one stream.
hipError_t prefill_xprep(void* workspace, const PrefillArgs& a, hipStream_t s);    // per-token scale, fp16 copy of x
hipError_t prefill_router(void* workspace, const PrefillArgs& a, hipStream_t s);   // logits [T][E+1] (MFMA)
hipError_t prefill_route(void* workspace, const PrefillArgs& a, hipStream_t s);    // top-k, weights, shared gate
hipError_t prefill_count(void* workspace, const PrefillArgs& a, hipStream_t s);    // pairs per (chunk, expert)
hipError_t prefill_scan(void* workspace, const PrefillArgs& a, hipStream_t s);     // offsets and the tile list
hipError_t prefill_scatter(void* workspace, const PrefillArgs& a, hipStream_t s);  // stable placement of pairs
hipError_t prefill_gateup(void* workspace, const PrefillArgs& a, hipStream_t s);   // grouped gate/up GEMM + SwiGLU
hipError_t prefill_down(void* workspace, const PrefillArgs& a, hipStream_t s);     // grouped down GEMM x weight
hipError_t prefill_combine(void* workspace, const PrefillArgs& a, hipStream_t s);  // per-token sum

}  // namespace moe
