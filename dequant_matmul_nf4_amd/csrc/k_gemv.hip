// Fused dequantize-and-multiply for decode, y[m][r] = sum_k x[m][k] * w[r][k]
// (bitsandbytes tool page, "How it works", Step 5: a block is expanded with
// its scale and code book and multiplied; the expanded copy never leaves the
// registers).
//
// Layout: a workgroup of 4 waves owns 16 consecutive rows, 4 per wave.  Lane l
// of a wave walks the row in 16-byte chunks l, l+64, ... (32 codes, half of a
// 64-block).  Within a chunk the level values are summed against x in float32
// and the block scale is applied once per chunk; the per-lane partial sums are
// reduced across the wave with shuffles at the end.
#include "nf4_device.h"

namespace nf4i {
namespace {

constexpr int kRowsPerWave = 4;
constexpr int kRowsPerGroup = 4 * kRowsPerWave;

__device__ __forceinline__ void load_x32(const uint16_t* __restrict__ xrow, int64_t k0, float xv[32]) {
  const uint4* p = reinterpret_cast<const uint4*>(xrow + k0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = p[i];
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[8 * i + 2 * j] = __uint_as_float(q[j] << 16);
      xv[8 * i + 2 * j + 1] = __uint_as_float(q[j] & 0xFFFF0000u);
    }
  }
}

// Sum over the 32 codes of a 16-byte chunk of level[code] * x.
__device__ __forceinline__ float chunk_dot(const uint4 w, const float xv[32], const float* lv) {
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t byte = (q[i] >> (8 * b)) & 0xFFu;
      s = fmaf(lv[byte >> 4], xv[8 * i + 2 * b], s);
      s = fmaf(lv[byte & 0xFu], xv[8 * i + 2 * b + 1], s);
    }
  }
  return s;
}

template <int kMG, bool kBf16Out>
__global__ __launch_bounds__(256) void k_gemv(const uint8_t* __restrict__ packed, int64_t rows,
                                              int64_t cols, Scales sc, const uint16_t* __restrict__ x,
                                              int m_total, void* __restrict__ y, Codebook cb) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = cb.level[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowsPerGroup + wave * kRowsPerWave;
  const float mean = sc.absmax ? 0.0f : *sc.mean;
  const int64_t nchunk = cols / 32;
  const int64_t row_bytes = cols / 2;
  const int64_t row_blocks = cols / 64;

  for (int m0 = 0; m0 < m_total; m0 += kMG) {
    float acc[kRowsPerWave][kMG];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
      for (int j = 0; j < kMG; ++j) acc[r][j] = 0.0f;

    for (int64_t c = lane; c < nchunk; c += 64) {
      uint4 w[kRowsPerWave];
      float a[kRowsPerWave];
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        const int64_t row = r0 + r;
        if (row < rows) {
          w[r] = *reinterpret_cast<const uint4*>(packed + row * row_bytes + c * 16);
          a[r] = block_scale(sc, row * row_blocks + (c >> 1), mean);
        } else {
          w[r] = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
          a[r] = 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < kMG; ++j) {
        if (m0 + j >= m_total) break;
        float xv[32];
        load_x32(x + static_cast<int64_t>(m0 + j) * cols, c * 32, xv);
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) acc[r][j] = fmaf(chunk_dot(w[r], xv, lv), a[r], acc[r][j]);
      }
    }

#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
#pragma unroll
      for (int j = 0; j < kMG; ++j) {
        const float s = wave_sum(acc[r][j]);
        const int64_t row = r0 + r;
        if (lane == 0 && row < rows && m0 + j < m_total) {
          const int64_t idx = static_cast<int64_t>(m0 + j) * rows + row;
          if constexpr (kBf16Out) static_cast<uint16_t*>(y)[idx] = static_cast<uint16_t>(f32_to_bf16(s));
          else static_cast<float*>(y)[idx] = s;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemv(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x,
                       int64_t m, void* y, int y_bf16, hipStream_t s) {
  const int64_t groups = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(groups));
  const Codebook& cb = codebook();
  const int mm = static_cast<int>(m);
  if (m == 1) {
    if (y_bf16) hipLaunchKernelGGL((k_gemv<1, true>), grid, dim3(256), 0, s, packed, rows, cols, sc, x, mm, y, cb);
    else hipLaunchKernelGGL((k_gemv<1, false>), grid, dim3(256), 0, s, packed, rows, cols, sc, x, mm, y, cb);
  } else {
    if (y_bf16) hipLaunchKernelGGL((k_gemv<4, true>), grid, dim3(256), 0, s, packed, rows, cols, sc, x, mm, y, cb);
    else hipLaunchKernelGGL((k_gemv<4, false>), grid, dim3(256), 0, s, packed, rows, cols, sc, x, mm, y, cb);
  }
  return hipGetLastError();
}

}  // namespace nf4i
