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

// ------------------------------------------------ gate/up chunk against x ---
// The activations of one 16-byte code chunk, prepared once for every row that
// multiplies them, and the chunk's term s * sum(q x) + c * sum(x).
//
// int4 runs on the dot-product unit: v_dot2 takes two bf16 pairs and adds
// their two products to an fp32 accumulator. A nibble q becomes the bf16 value
// 128 + q (bit pattern 0x4300 | q, exact), so a masked shift of an 8-code word
// gives two codes at once: nibbles j and j + 4 land in the two halves. The
// activations are re-paired the same way, (x_j, x_{j+4}) within each word, and
// their sum comes from the same unit against (1, 1). The chunk's dot is then
// d' = sum((128 + q) x) = d + 128 sum(x), and the term s * d + c * sum(x) is
// s * d' + (c - 128 s) * sum(x). Every product of a code and a bf16 value is
// exact; the offset costs the fp32 sums about five bits, far below the fp16
// rounding of s and c themselves.
// int8 keeps the float path: codes up to 255 have no such one-operation bf16
// form.
template <int BITS>
struct XChunk;
template <>
struct XChunk<4> {
  uint32_t p[16];  // p[4t + j] = bf16 pair (x_{8t+j}, x_{8t+j+4}), j < 4
  float s;         // sum of the 32 activations
};
template <>
struct XChunk<8> {
  float v[16];
  float s;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// xr: the chunk's activations as stored (bf16, two per word, element order).
template <int BITS>
__device__ __forceinline__ XChunk<BITS> x_chunk(const uint32_t (&xr)[128 / BITS / 2]) {
  XChunk<BITS> r;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t a = xr[4 * t + u], b = xr[4 * t + u + 2];
        r.p[4 * t + 2 * u] = (a & 0xFFFFu) | (b << 16);
        r.p[4 * t + 2 * u + 1] = (a >> 16) | (b & 0xFFFF0000u);
      }
    }
    constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1, 1)
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int m = 0; m < 16; m += 2) {
      s0 = dot2bf(r.p[m], kOnes, s0);
      s1 = dot2bf(r.p[m + 1], kOnes, s1);
    }
    r.s = s0 + s1;
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      r.v[2 * m] = bf16f(xr[m] & 0xFFFFu);
      r.v[2 * m + 1] = bf16f(xr[m] >> 16);
    }
    float sx = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) sx += r.v[q];
    r.s = sx;
  }
  return r;
}

// The 32 int4 codes of a chunk as bf16 pairs (128 + q_{8t+j}, 128 + q_{8t+j+4})
// at q[4t + j], the pairing of XChunk<4>.
__device__ __forceinline__ void code_pairs4(const uint4 c, uint32_t (&q)[16]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) q[4 * t + j] = ((w[t] >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
  }
}

// s * sum((128 + q) x) + (c - 128 s) * sum(x) = s * sum(q x) + c * sum(x) of a
// chunk from its code pairs and activation pairs (even pairs into one
// accumulator, odd into another, each in order).
__device__ __forceinline__ float pairs_term(const uint32_t (&q)[16], uint32_t sc, const uint32_t (&xp)[16],
                                            float xs) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int m = 0; m < 16; m += 2) {
    a0 = dot2bf(q[m], xp[m], a0);
    a1 = dot2bf(q[m + 1], xp[m + 1], a1);
  }
  const float s = f16f(sc & 0xFFFFu);
  return fmaf(s, a0 + a1, fmaf(-128.0f, s, f16f(sc >> 16)) * xs);
}

// s * sum(q x) + c * sum(x) of one chunk; sc = the fp16 (s, c) pair of its
// quantisation group (s in the low half).
template <int BITS>
__device__ __forceinline__ float chunk_term(const uint4 c, uint32_t sc, const XChunk<BITS>& x) {
  if constexpr (BITS == 4) {
    uint32_t q[16];
    code_pairs4(c, q);
    return pairs_term(q, sc, x.p, x.s);
  } else {
    return group_term(sc, chunk_dot<8>(c, x.v), x.s);
  }
}

// silu(g) * u with silu(g) = g / (1 + e^-g).
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace moe
