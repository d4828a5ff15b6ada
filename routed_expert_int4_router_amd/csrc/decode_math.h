// Arithmetic of the decode kernels that the plainly written (scalar)
// variants repeat operation for operation, so both produce the same bits:
// format conversions, the 16-byte chunk dot product on integer codes, the
// group scale and bias applied to a chunk, and SwiGLU.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

__device__ __forceinline__ float bf16f(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xFFu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }

// sum over the chunk of code * x; x holds EPC = 128 / BITS consecutive elements.
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4 c, const float* x) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float a0 = 0.f, a1 = 0.f;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t lo = w[t] & 0x0F0F0F0Fu, hi = (w[t] >> 4) & 0x0F0F0F0Fu;
      const float* xx = x + 8 * t;
      a0 = fmaf(ub0(lo), xx[0], a0);
      a1 = fmaf(ub0(hi), xx[1], a1);
      a0 = fmaf(ub1(lo), xx[2], a0);
      a1 = fmaf(ub1(hi), xx[3], a1);
      a0 = fmaf(ub2(lo), xx[4], a0);
      a1 = fmaf(ub2(hi), xx[5], a1);
      a0 = fmaf(ub3(lo), xx[6], a0);
      a1 = fmaf(ub3(hi), xx[7], a1);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float* xx = x + 4 * t;
      a0 = fmaf(ub0(w[t]), xx[0], a0);
      a1 = fmaf(ub1(w[t]), xx[1], a1);
      a0 = fmaf(ub2(w[t]), xx[2], a0);
      a1 = fmaf(ub3(w[t]), xx[3], a1);
    }
  }
  return a0 + a1;
}

// s * d + c * xs for one chunk: (s, c) the fp16 pair of its quantisation group
// (s in the low half), d = sum(q * x) over the chunk, xs = sum(x).
__device__ __forceinline__ float group_term(uint32_t sc, float d, float xs) {
  return fmaf(f16f(sc & 0xFFFFu), d, f16f(sc >> 16) * xs);
}

// silu(g) * u with silu(g) = g / (1 + e^-g).
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace moe
