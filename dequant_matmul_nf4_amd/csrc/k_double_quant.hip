// Double quantization of the block scales (bitsandbytes tool page, "Double
// quantization", with the int8 scheme of its "A worked example": scale by 127,
// round half away from zero).  The scales are first centred on their mean.
//
// The mean must not depend on summation order, so the scales are summed
// exactly: each float32 is an integer m * 2^p times 2^-149 (m < 2^24,
// 0 <= p <= 253), added into 32-bit digits of a wide fixed-point integer held
// in 64-bit accumulators (no carries until the end).  The last block to finish
// propagates the carries, rounds the integer once to float64, divides by the
// count in float64 and rounds to float32.
//
// Kernels: k_dq_clear (fill kernel for the workspace), k_dq_sum (exact sum and
// mean), k_dq_quant (one wave per group of 256 scales).
#include "nf4_device.h"

namespace nf4i {
namespace {

__global__ void k_dq_clear(unsigned long long* ws) {
  if (threadIdx.x < 16) ws[threadIdx.x] = 0ull;
}

__device__ __forceinline__ void scale_to_digits(float a, int* d, uint32_t* lo, uint32_t* hi) {
  const uint32_t u = __float_as_uint(a) & 0x7FFFFFFFu;
  const uint32_t e = u >> 23;
  const uint32_t mant = e ? ((u & 0x7FFFFFu) | 0x800000u) : (u & 0x7FFFFFu);
  const uint32_t p = e ? e - 1 : 0;  // value = mant * 2^p * 2^-149
  const unsigned long long v = static_cast<unsigned long long>(mant) << (p & 31);
  *d = static_cast<int>(p >> 5);
  *lo = static_cast<uint32_t>(v);
  *hi = static_cast<uint32_t>(v >> 32);
}

// Rounds the non-negative integer sum_k digit[k] 2^(32k) to the nearest
// float64 (ties to even) and scales it by 2^-149.
__device__ double digits_to_double(const uint32_t* dig, int ndig) {
  int top = -1;
  for (int k = ndig - 1; k >= 0 && top < 0; --k)
    if (dig[k]) top = 32 * k + (31 - __clz(dig[k]));
  if (top < 0) return 0.0;
  auto bit = [&](int i) -> uint32_t { return (i < 0) ? 0u : (dig[i >> 5] >> (i & 31)) & 1u; };
  unsigned long long mant = 0;
  const int low = top - 52;  // lowest kept bit (may be negative: then exact)
  for (int i = top; i >= low && i >= 0; --i) mant = (mant << 1) | bit(i);
  int scale = 0;
  if (low > 0) {
    const uint32_t round = bit(low - 1);
    uint32_t sticky = 0;
    for (int i = low - 2; i >= 0 && !sticky; --i) sticky |= bit(i);
    if (round && (sticky || (mant & 1ull))) ++mant;
    scale = low;
  }
  return ldexp(static_cast<double>(mant), scale - 149);
}

__global__ __launch_bounds__(256) void k_dq_sum(const float* __restrict__ absmax, int64_t nb,
                                                unsigned long long* __restrict__ ws,
                                                float* __restrict__ mean_out) {
  __shared__ unsigned long long acc[kDqDigits];
  __shared__ int is_last;
  if (threadIdx.x < kDqDigits) acc[threadIdx.x] = 0ull;
  __syncthreads();
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nb; i += stride) {
    int d;
    uint32_t lo, hi;
    scale_to_digits(absmax[i], &d, &lo, &hi);
    if (lo) atomicAdd(&acc[d], static_cast<unsigned long long>(lo));
    if (hi) atomicAdd(&acc[d + 1], static_cast<unsigned long long>(hi));
  }
  __syncthreads();
  if (threadIdx.x < kDqDigits && acc[threadIdx.x]) atomicAdd(&ws[threadIdx.x], acc[threadIdx.x]);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long prev = atomicAdd(&ws[kDqDoneSlot], 1ull);
    is_last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (!is_last || threadIdx.x != 0) return;
  __threadfence();
  uint32_t dig[kDqDigits];
  unsigned long long carry = 0;
  for (int k = 0; k < kDqDigits; ++k) {
    const unsigned long long t =
        __hip_atomic_load(&ws[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + carry;
    dig[k] = static_cast<uint32_t>(t);
    carry = t >> 32;
  }
  const double total = digits_to_double(dig, kDqDigits);
  *mean_out = static_cast<float>(total / static_cast<double>(nb));
}

__global__ __launch_bounds__(256) void k_dq_quant(const float* __restrict__ absmax, int64_t nb,
                                                  const float* __restrict__ mean_p,
                                                  int8_t* __restrict__ q, float* __restrict__ absmax2) {
  const int lane = threadIdx.x & 63;
  const int64_t ngroups = (nb + 255) >> 8;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const float mu = *mean_p;
  for (int64_t g = wave; g < ngroups; g += nwaves) {
    const int64_t i0 = g * 256 + lane * 4;
    float c[4];
    if (i0 + 4 <= nb) {
      const float4 a = *reinterpret_cast<const float4*>(absmax + i0);
      c[0] = a.x - mu; c[1] = a.y - mu; c[2] = a.z - mu; c[3] = a.w - mu;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = (i0 + j < nb) ? absmax[i0 + j] - mu : 0.0f;
    }
    float s = fmaxf(fmaxf(fabsf(c[0]), fabsf(c[1])), fmaxf(fabsf(c[2]), fabsf(c[3])));
    s = group_max<64>(s);
    uint32_t word = 0;
    if (s > 0.0f) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float t = (c[j] / s) * 127.0f;
        const float at = fabsf(t);
        const float fl = floorf(at);
        float r = fl + ((at - fl) >= 0.5f ? 1.0f : 0.0f);  // half away from zero
        r = fminf(r, 127.0f);
        const int qi = (t < 0.0f) ? -static_cast<int>(r) : static_cast<int>(r);
        word |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * j);
      }
    }
    if (i0 + 4 <= nb) {
      *reinterpret_cast<uint32_t*>(q + i0) = word;
    } else {
      for (int j = 0; j < 4; ++j)
        if (i0 + j < nb) q[i0 + j] = static_cast<int8_t>(word >> (8 * j));
    }
    if (lane == 0) absmax2[g] = s;
  }
}

}  // namespace

hipError_t launch_double_quant(const float* absmax, int64_t nb, int8_t* q, float* absmax2,
                               float* mean, unsigned long long* ws, hipStream_t s) {
  hipLaunchKernelGGL(k_dq_clear, dim3(1), dim3(64), 0, s, ws);
  int64_t want = (nb + 255) / 256;
  int grid = static_cast<int>(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(k_dq_sum, dim3(grid), dim3(256), 0, s, absmax, nb, ws, mean);
  const int64_t groups = (nb + 255) >> 8;
  want = (groups + 3) / 4;  // 4 waves per workgroup
  grid = static_cast<int>(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(k_dq_quant, dim3(grid), dim3(256), 0, s, absmax, nb, mean, q, absmax2);
  return hipGetLastError();
}

}  // namespace nf4i
