// Dequantize-into-LDS bf16 matrix-core GEMM with an optional fused LoRA term:
//   y = x . deq(W)^T + s . (x . A^T) . B^T
// (bitsandbytes tool page, "How it works", Step 5: matrix hardware works best
// on 16-bit numbers, so each block is expanded to 16-bit and multiplied; the
// tutorial page, "QLoRA: Fine-Tuning a 4-bit Model": low-rank adapters on the
// frozen 4-bit base, their output multiplied by a scale factor.)
//
// Tiling: a workgroup of 4 waves computes a 128 x 128 tile of y.  Each K step
// covers one 64-column block of W, so each W row of the tile has exactly one
// scale per step.  The x tile (bf16) is copied to LDS; the W tile is read as
// packed nibbles, expanded to bf16 (round-to-nearest-even of fl32(level * a))
// and written to LDS; each wave then runs 2 x 4 x 4 v_mfma_f32_16x16x32_bf16
// on its 64 x 64 sub-tile.  LoRA: T = x . A^T is formed in float32 first by
// k_lora_xa; the epilogue adds s * T[m] . B[n] before the bf16 store.
#include "nf4_device.h"

namespace nf4i {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsStride = kBK + 8;  // bf16 elements per LDS row (padding against bank conflicts)

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  union { uint4 u; bf16x8 b; } c;
  c.u = v;
  return c.b;
}

__global__ __launch_bounds__(256) void k_gemm(const uint8_t* __restrict__ packed, int64_t rows,
                                              int64_t cols, Scales sc, const uint16_t* __restrict__ x,
                                              int64_t m_total, uint16_t* __restrict__ y,
                                              const float* __restrict__ t_lora,
                                              const uint16_t* __restrict__ lora_b, int r,
                                              float lora_scale, Codebook cb) {
  __shared__ uint16_t xs[kBM * kLdsStride];
  __shared__ uint16_t ws[kBN * kLdsStride];
  __shared__ float lv[16];
  const int tid = threadIdx.x;
  if (tid < 16) lv[tid] = cb.level[tid];
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (rows + kBN - 1) / kBN;
  const int64_t m0 = (static_cast<int64_t>(blockIdx.x) / tiles_n) * kBM;
  const int64_t n0 = (static_cast<int64_t>(blockIdx.x) % tiles_n) * kBN;
  const float mean = sc.absmax ? 0.0f : *sc.mean;
  const int64_t row_blocks = cols / 64;

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  __syncthreads();
  for (int64_t k0 = 0; k0 < cols; k0 += kBK) {
    // x tile: 128 rows x 64 bf16 = 1024 x 16 bytes, 4 per thread
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + 256 * it;
      const int row = idx >> 3, c8 = idx & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + row < m_total) v = *reinterpret_cast<const uint4*>(x + (m0 + row) * cols + k0 + c8 * 8);
      *reinterpret_cast<uint4*>(&xs[row * kLdsStride + c8 * 8]) = v;
    }
    // W tile: 128 rows x 32 bytes; thread -> (row, half block of 32 codes)
    {
      const int row = tid >> 1, half = tid & 1;
      uint4 out[4] = {};
      if (n0 + row < rows) {
        const uint4 w = *reinterpret_cast<const uint4*>(packed + ((n0 + row) * cols + k0) / 2 + half * 16);
        const float a = block_scale(sc, (n0 + row) * row_blocks + k0 / 64, mean);
        const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t o[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (q[i] >> (8 * b)) & 0xFFu;
            o[b] = pack_bf16x2(lv[byte >> 4] * a, lv[byte & 0xFu] * a);
          }
          out[i] = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(&ws[row * kLdsStride + half * 32 + i * 8]) = out[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 af[4], bfr[4];
      const int kl = kk + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&xs[(wm * 64 + i * 16 + (lane & 15)) * kLdsStride + kl]));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const uint4*>(&ws[(wn * 64 + j * 16 + (lane & 15)) * kLdsStride + kl]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // epilogue: lane holds D[4*(lane/16) + q][lane % 16] of each 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + q;
        if (row < m_total && col < rows) {
          float v = acc[i][j][q];
          if (r > 0) {
            float l = 0.0f;
            for (int t = 0; t < r; ++t)
              l = fmaf(t_lora[row * r + t], bf16_to_f32(lora_b[col * r + t]), l);
            v = fmaf(lora_scale, l, v);
          }
          y[row * rows + col] = static_cast<uint16_t>(f32_to_bf16(v));
        }
      }
    }
  }
}

// T[m][t] = sum_k x[m][k] * A[t][k] in float32: one wave per (m, t).
__global__ __launch_bounds__(256) void k_lora_xa(const uint16_t* __restrict__ x, const uint16_t* __restrict__ a,
                                                 int64_t m_total, int64_t cols, int r, float* __restrict__ t_out) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (wave >= m_total * r) return;
  const int64_t m = wave / r;
  const int t = static_cast<int>(wave % r);
  const uint16_t* xr = x + m * cols;
  const uint16_t* ar = a + static_cast<int64_t>(t) * cols;
  float s = 0.0f;
  for (int64_t k = lane * 8; k < cols; k += 64 * 8) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xr + k);
    const uint4 av = *reinterpret_cast<const uint4*>(ar + k);
    const uint32_t xq[4] = {xv.x, xv.y, xv.z, xv.w};
    const uint32_t aq[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = fmaf(__uint_as_float(xq[i] << 16), __uint_as_float(aq[i] << 16), s);
      s = fmaf(__uint_as_float(xq[i] & 0xFFFF0000u), __uint_as_float(aq[i] & 0xFFFF0000u), s);
    }
  }
  s = wave_sum(s);
  if (lane == 0) t_out[m * r + t] = s;
}

}  // namespace

hipError_t launch_gemm(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x,
                       int64_t m, uint16_t* y, const uint16_t* lora_a, const uint16_t* lora_b, int r,
                       float lora_scale, float* t_ws, hipStream_t s) {
  if (r > 0) {
    const int64_t waves = m * r;
    const int64_t blocks = (waves + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_lora_xa, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, x, lora_a, m, cols, r, t_ws);
  }
  const int64_t tiles = ((rows + kBN - 1) / kBN) * ((m + kBM - 1) / kBM);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const Codebook& cb = codebook();
  hipLaunchKernelGGL(k_gemm, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, s, packed,
                     rows, cols, sc, x, m, y, t_ws, lora_b, r, lora_scale, cb);
  return hipGetLastError();
}

}  // namespace nf4i
