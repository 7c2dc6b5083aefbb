// The thin factor of a LoRA term: T = s . x . A^T for x [m][len] bf16 and the
// r rows of A [r][len] bf16 (tutorial page "bitsandbytes quantization
// tutorial: 4-bit and 8-bit models", section "QLoRA: Fine-Tuning a 4-bit
// Model": the adapter output is multiplied by a scale factor).  The forward
// GEMM uses it with (x, A), the input gradient with (dY, B^T), the adapter
// gradients in both orientations.
//
// It is a tall-skinny product (r <= 64), so it runs on the matrix cores with
// both operands loaded straight into v_mfma_f32_16x16x32_bf16 fragments: a
// lane's 8 consecutive reduction indices are 16 contiguous bytes of a row of
// x and of a row of A.  A workgroup owns 16 rows of x; its 8 waves take
// interleaved 32-wide reduction steps (8 per iteration, loads first) and
// their partial sums are added in LDS.  The number of 16-wide rank tiles is
// a template parameter, so a rank-16 adapter holds only the registers it
// uses.  Products of bf16 values are exact in float32; sums are float32.
//
// Outputs: the bf16 pair form u[i][.] = (hi | lo | 0) used by the fused GEMMs
// (hi = bf16(sT) at column j, lo = bf16(sT - hi) at column r_pad + j, zero
// elsewhere in the row of kl values), or float32 rows of r_pad values (zero
// for j >= r).
#include "nf4_device.h"

namespace nf4i {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kPW = 8;   // waves per workgroup
constexpr int kPU = 8;   // reduction steps per wave per iteration
constexpr int kPJ = 4;   // at most 4 tiles of 16 rank entries (r <= 64)

template <bool kF32, int kNJ>
__global__ __launch_bounds__(kPW * kWave) void k_lora_prep(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ la, int64_t m, int64_t len,
                                                           int r, int r_pad, int kl, float scale, void* __restrict__ out) {
  __shared__ floatx4_t red[kPW][kNJ][kWave];  // 8 KB per rank tile
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, kq = lane >> 4;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t row = i0 + li < m ? i0 + li : m - 1;  // rows past the end: never stored
  const uint16_t* xr = x + row * len + 8 * kq;
  const uint16_t* ar[kNJ];
  bool jlive[kNJ];
#pragma unroll
  for (int jt = 0; jt < kNJ; ++jt) {
    const int j = 16 * jt + li;
    jlive[jt] = j < r;
    ar[jt] = la + static_cast<int64_t>(jlive[jt] ? j : 0) * len + 8 * kq;
  }
  floatx4_t acc[kNJ];
#pragma unroll
  for (int jt = 0; jt < kNJ; ++jt) acc[jt] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t steps = (len + 31) / 32;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  for (int64_t s0 = wave; s0 < steps; s0 += kPW * kPU) {
    uint4 xv[kPU], av[kPU][kNJ];
#pragma unroll
    for (int u = 0; u < kPU; ++u) {
      const int64_t k = 32 * (s0 + kPW * u);  // this lane reads k + 8 kq .. + 7; len % 8 == 0
      const bool in = k + 8 * kq < len;
      xv[u] = in ? *reinterpret_cast<const uint4*>(xr + k) : zero;
#pragma unroll
      for (int jt = 0; jt < kNJ; ++jt)
        av[u][jt] = (in && jlive[jt]) ? *reinterpret_cast<const uint4*>(ar[jt] + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < kPU; ++u)
#pragma unroll
      for (int jt = 0; jt < kNJ; ++jt)
        acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv[u]),
                                                           __builtin_bit_cast(bf16x8_t, av[u][jt]), acc[jt], 0, 0, 0);
  }
#pragma unroll
  for (int jt = 0; jt < kNJ; ++jt) red[wave][jt][lane] = acc[jt];
  __syncthreads();
  if (wave != 0) return;
  // lane holds T[i0 + 4 kq + e][16 jt + li] for e = 0..3
#pragma unroll
  for (int jt = 0; jt < kNJ; ++jt) {
    floatx4_t t = red[0][jt][lane];
#pragma unroll
    for (int w = 1; w < kPW; ++w) t += red[w][jt][lane];
    const int j = 16 * jt + li;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + 4 * kq + e;
      if (i >= m) continue;
      const float v = j < r ? t[e] * scale : 0.0f;
      if constexpr (kF32) {
        static_cast<float*>(out)[i * r_pad + j] = v;
      } else {
        uint16_t* urow = static_cast<uint16_t*>(out) + i * kl;
        const __bf16 hi = static_cast<__bf16>(v);
        const __bf16 lo = static_cast<__bf16>(v - static_cast<float>(hi));
        urow[j] = __builtin_bit_cast(uint16_t, hi);
        urow[r_pad + j] = __builtin_bit_cast(uint16_t, lo);
      }
    }
  }
  if constexpr (!kF32) {
    // the padding columns [2 r_pad, kl) of the workgroup's rows
    for (int c = 2 * r_pad + li; c < kl; c += 16)
      for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + 4 * kq + e;
        if (i < m) static_cast<uint16_t*>(out)[i * kl + c] = 0;
      }
  }
}

template <bool kF32>
hipError_t launch_prep(const uint16_t* x, const uint16_t* a, int64_t m, int64_t len, int r, float scale, void* out,
                       hipStream_t s) {
  const int64_t groups = (m + 15) / 16;
  if (groups > 0x7FFFFFFF || r < 1 || r > 16 * kPJ) return hipErrorInvalidValue;
  const int r_pad = (r + 15) / 16 * 16;
  const int kl = static_cast<int>(gemm_lora_cols(r));
  const dim3 grid(static_cast<unsigned>(groups)), block(kPW * kWave);
  switch (r_pad / 16) {
    case 1: hipLaunchKernelGGL((k_lora_prep<kF32, 1>), grid, block, 0, s, x, a, m, len, r, r_pad, kl, scale, out); break;
    case 2: hipLaunchKernelGGL((k_lora_prep<kF32, 2>), grid, block, 0, s, x, a, m, len, r, r_pad, kl, scale, out); break;
    case 3: hipLaunchKernelGGL((k_lora_prep<kF32, 3>), grid, block, 0, s, x, a, m, len, r, r_pad, kl, scale, out); break;
    default: hipLaunchKernelGGL((k_lora_prep<kF32, 4>), grid, block, 0, s, x, a, m, len, r, r_pad, kl, scale, out);
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_lora_u(const uint16_t* x, const uint16_t* a, int64_t m, int64_t len, int r, float scale,
                         uint16_t* u, hipStream_t s) {
  return launch_prep<false>(x, a, m, len, r, scale, u, s);
}

hipError_t launch_lora_t32(const uint16_t* x, const uint16_t* a, int64_t m, int64_t len, int r, float scale,
                           float* t, hipStream_t s) {
  return launch_prep<true>(x, a, m, len, r, scale, t, s);
}

}  // namespace nf4i
