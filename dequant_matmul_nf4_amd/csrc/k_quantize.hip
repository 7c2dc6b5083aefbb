// Blockwise NF4 quantization (bitsandbytes tool page, "How it works",
// Steps 1-4): per block of 64 values, the largest |x| is the scale; each value
// is divided by it (IEEE float32 division) and replaced by the index of the
// nearest NF4 level; two indices are packed per byte, the first in the high
// nibble.
//
// Layout: each lane owns 8 consecutive values (one 16-byte bf16 load or two
// 16-byte fp32 loads) and writes one 32-bit word of packed codes; 8 adjacent
// lanes form one 64-block and reduce its absmax with lane shuffles.
#include "nf4_device.h"

namespace nf4i {
namespace {

template <bool kBf16>
__device__ __forceinline__ void load8(const void* xv, int64_t e0, int64_t n, float v[8]) {
  if (e0 + 8 <= n) {
    if constexpr (kBf16) {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + e0);
      const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(q[i] << 16);
        v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(xv) + e0);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (e0 + i < n) {
        if constexpr (kBf16) v[i] = bf16_to_f32(static_cast<const uint16_t*>(xv)[e0 + i]);
        else v[i] = static_cast<const float*>(xv)[e0 + i];
      } else {
        v[i] = 0.0f;  // padding: does not change the absmax, never stored
      }
    }
  }
}

__device__ __forceinline__ uint32_t nearest_code(float v, const Codebook& cb) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) c += (v >= cb.thresh[i]) ? 1u : 0u;
  return c;
}

template <bool kBf16>
__global__ __launch_bounds__(256) void k_quantize(const void* __restrict__ x, int64_t n,
                                                  uint8_t* __restrict__ packed,
                                                  float* __restrict__ absmax, Codebook cb) {
  const int64_t nblocks = (n + 63) >> 6;
  const int64_t noct = nblocks * 8;  // whole blocks, so 8-lane groups stay together
  const int64_t nbytes = (n + 1) >> 1;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; o < noct; o += stride) {
    float v[8];
    load8<kBf16>(x, o * 8, n, v);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = group_max<8>(m);
    uint32_t word = 0x77777777u;  // all codes 7 when the block is all zero
    if (m > 0.0f) {
      word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t c = nearest_code(v[i] / m, cb);
        // element 2j -> high nibble of byte j, element 2j+1 -> low nibble
        word |= c << (8 * (i >> 1) + ((i & 1) ? 0 : 4));
      }
    }
    const int64_t byte0 = o * 4;
    if (byte0 + 4 <= nbytes) {
      *reinterpret_cast<uint32_t*>(packed + byte0) = word;
    } else {
      for (int j = 0; j < 4; ++j)
        if (byte0 + j < nbytes) packed[byte0 + j] = static_cast<uint8_t>(word >> (8 * j));
    }
    if ((threadIdx.x & 7) == 0) absmax[o >> 3] = m;
  }
}

}  // namespace

hipError_t launch_quantize(const void* x, int x_bf16, int64_t n, uint8_t* packed, float* absmax,
                           hipStream_t s) {
  const int64_t noct = ((n + 63) >> 6) * 8;
  const int64_t want = (noct + 255) / 256;
  const int grid = static_cast<int>(want < 16384 ? want : 16384);
  const Codebook& cb = codebook();
  if (x_bf16)
    hipLaunchKernelGGL(k_quantize<true>, dim3(grid), dim3(256), 0, s, x, n, packed, absmax, cb);
  else
    hipLaunchKernelGGL(k_quantize<false>, dim3(grid), dim3(256), 0, s, x, n, packed, absmax, cb);
  return hipGetLastError();
}

}  // namespace nf4i
