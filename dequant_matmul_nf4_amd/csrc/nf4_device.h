// Device helpers shared by the NF4 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "nf4_internal.h"

namespace nf4i {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round-to-nearest-even float32 -> bfloat16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// fl32(q / 127) for an int8 q: from y = fl32(1/127), q0 = fl32(q y) and the
// exact residual r = q - q0 * 127, fl32(q0 + r y) is the correctly rounded
// quotient (Markstein's theorem; also checked for all 256 values of q).
__device__ __forceinline__ float div127(int q) {
  const float f = static_cast<float>(q);
  const float y = 1.0f / 127.0f;
  const float q0 = f * y;
  const float r = fmaf(-q0, 127.0f, f);
  return fmaf(r, y, q0);
}

// The float8 reading's ratio table (make_e4m3_ratio in nf4_internal.h).
static __device__ const E4m3Ratio kE4m3Ratio = make_e4m3_ratio();

// The first factor of a_hat: q / 127 for an int8 code, e4m3(q) / 448 for a
// float8 code (q's low byte).
__device__ __forceinline__ float code_ratio(int q, int f8) { return f8 ? kE4m3Ratio.v[q & 0xFF] : div127(q); }

// The scale of block b: either the stored fp32 absmax, or the double-quantized
// form a_hat = fl32(fl32(fl32(q / 127) * s2) + mean), three separate roundings
// (q / 127 replaced by e4m3(q) / 448 for float8 codes).
__device__ __forceinline__ float block_scale(const Scales& sc, int64_t b, float mean) {
  if (sc.absmax) return sc.absmax[b];
  const float t = code_ratio(sc.q[b], sc.f8);
  const float u = t * sc.absmax2[b >> 8];
  return u + mean;
}

// Hides a value from the optimizer so that byte-field extracts of a masked
// word stay single v_bfe_u32 instructions instead of being re-derived from
// the unmasked word with shift-and-mask pairs.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int kWidth>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = 1; off < kWidth; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Batched launches: the item (weight or scale array) a workgroup belongs to,
// the last j < count with first[j] <= blk (first[] holds each item's first
// workgroup, ascending).
template <int N>
__device__ __forceinline__ int batch_item_of(const int (&first)[N + 1], int count, int blk) {
  int j = 0;
#pragma unroll
  for (int k = 1; k < N; ++k) j = (k < count && first[k] <= blk) ? k : j;
  return j;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace nf4i
