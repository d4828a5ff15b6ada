// Cross-lane reductions for wave64 on gfx950 built from DPP row operations
// (no LDS round trip), and the wave-wide argmax used by the top-k.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {
namespace dpp {

// DPP control words (GFX9 encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm(1,0,3,2)
constexpr int kQuadXor2 = 0x4E;       // quad_perm(2,3,0,1)
constexpr int kRowMirror = 0x140;     // lane i <- 15 - i within a row of 16
constexpr int kRowHalfMirror = 0x141; // lane i <- 7 - i within each half row
constexpr int kRowBcast15 = 0x142;    // lane 15 of row r -> row r + 1
constexpr int kRowBcast31 = 0x143;    // lane 31 -> rows 2 and 3

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t mov(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float add_f32(float v) {
  return v + __uint_as_float(mov<CTRL, ROW_MASK>(0u, __float_as_uint(v)));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double add_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = mov<CTRL, ROW_MASK>(0u, (uint32_t)u);
  const uint32_t hi = mov<CTRL, ROW_MASK>(0u, (uint32_t)(u >> 32));
  return v + __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over each aligned group of LPR lanes (LPR a power of two <= 64). The
// total is valid in the group's last lane (in every lane when LPR <= 16).
// The association order is fixed, so results are run-to-run identical.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPR >= 2) v = add_f32<kQuadXor1, 0xF>(v);
  if constexpr (LPR >= 4) v = add_f32<kQuadXor2, 0xF>(v);
  if constexpr (LPR >= 8) v = add_f32<kRowHalfMirror, 0xF>(v);
  if constexpr (LPR >= 16) v = add_f32<kRowMirror, 0xF>(v);
  if constexpr (LPR >= 32) v = add_f32<kRowBcast15, 0xA>(v);
  if constexpr (LPR >= 64) v = add_f32<kRowBcast31, 0xC>(v);
  return v;
}

// Inclusive prefix sum over the 64 lanes (lane 0 first), Hillis-Steele within
// rows of 16 then the row carries.
__device__ __forceinline__ uint32_t wave_prefix_u32(uint32_t v) {
  v += mov<0x111, 0xF>(0u, v);  // row_shr:1
  v += mov<0x112, 0xF>(0u, v);  // row_shr:2
  v += mov<0x114, 0xF>(0u, v);  // row_shr:4
  v += mov<0x118, 0xF>(0u, v);  // row_shr:8
  v += mov<kRowBcast15, 0xA>(0u, v);
  v += mov<kRowBcast31, 0xC>(0u, v);
  return v;
}

// Wave-wide max of u32 values, returned uniform. Each step is a DPP-moved
// operand into v_max (masked-out rows and lanes read 0, the identity of max).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t max_step(uint32_t v) {
  const uint32_t o = mov<CTRL, ROW_MASK>(0u, v);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max_step<kQuadXor1, 0xF>(v);
  v = max_step<kQuadXor2, 0xF>(v);
  v = max_step<kRowHalfMirror, 0xF>(v);
  v = max_step<kRowMirror, 0xF>(v);
  v = max_step<kRowBcast15, 0xA>(v);
  v = max_step<kRowBcast31, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

// Wave-wide min of u32 values, returned uniform (masked rows read 0xFFFFFFFF).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t min_step(uint32_t v) {
  const uint32_t o = mov<CTRL, ROW_MASK>(0xFFFFFFFFu, v);
  return o < v ? o : v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min_step<kQuadXor1, 0xF>(v);
  v = min_step<kQuadXor2, 0xF>(v);
  v = min_step<kRowHalfMirror, 0xF>(v);
  v = min_step<kRowMirror, 0xF>(v);
  v = min_step<kRowBcast15, 0xA>(v);
  v = min_step<kRowBcast31, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

// Whole-wave sums broadcast to every lane (via lane 63).
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<64>(v);
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

__device__ __forceinline__ double wave_sum(double v) {
  v = add_f64<kQuadXor1, 0xF>(v);
  v = add_f64<kQuadXor2, 0xF>(v);
  v = add_f64<kRowHalfMirror, 0xF>(v);
  v = add_f64<kRowMirror, 0xF>(v);
  v = add_f64<kRowBcast15, 0xA>(v);
  v = add_f64<kRowBcast31, 0xC>(v);
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), 63);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Lexicographic max of (key, tag) pairs; masked-out rows compare with themselves.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void kv_max(uint32_t& key, uint32_t& tag) {
  const uint32_t ok = mov<CTRL, ROW_MASK>(key, key);
  const uint32_t ot = mov<CTRL, ROW_MASK>(tag, tag);
  const bool take = (ok > key) || (ok == key && ot > tag);
  key = take ? ok : key;
  tag = take ? ot : tag;
}

// Wave-wide lexicographic max of (key, tag), returned uniform (SGPR values).
__device__ __forceinline__ void wave_kv_max(uint32_t& key, uint32_t& tag) {
  kv_max<kQuadXor1, 0xF>(key, tag);
  kv_max<kQuadXor2, 0xF>(key, tag);
  kv_max<kRowHalfMirror, 0xF>(key, tag);
  kv_max<kRowMirror, 0xF>(key, tag);
  kv_max<kRowBcast15, 0xA>(key, tag);
  kv_max<kRowBcast31, 0xC>(key, tag);
  key = __builtin_amdgcn_readlane(key, 63);
  tag = __builtin_amdgcn_readlane(tag, 63);
}

}  // namespace dpp
}  // namespace moe
