// LoRA merge (tutorial page "bitsandbytes quantization tutorial: 4-bit and
// 8-bit models", section "Merging LoRA Adapters After Fine-Tuning": after
// training the adapters are folded into one dense 16-bit copy of the base,
// which needs the base dequantized first; tool page "bitsandbytes", section
// "Practical guidance and best practices": merging adds a rounding step):
//
//   out[n][k] = round( deq[n][k] + s * sum_j B[n][j] * A[j][k] )
//
// deq[n][k] = fl32(level[code] * a_hat), the value nf4_dequantize writes.  The
// rank-r sum is formed in float64 with j ascending (each bf16 x bf16 product
// is exact in float64, so a fused multiply-add rounds exactly as a multiply
// followed by an add), then t = fl64(s * sum) and v = fl64(deq + t), and v is
// rounded once to nearest even into bf16 or fp16: first to float32 rounding
// to odd (keep the truncated value and set its last bit when inexact), then
// to the 16-bit format by the hardware's nearest-even conversion; float32's
// 24 significant bits are at least two more than either target's, which makes
// the two steps one correct rounding (Boldo and Melquiond, "Emulation of FMA
// and correctly rounded sums: proved algorithms using rounding to odd").
//
// Layout: a workgroup of 256 threads covers kRows consecutive rows (grid x)
// and 2048 columns (grid y); each thread owns 8 consecutive columns of those
// rows (16 bytes of output per row).  For each j the thread loads
// A[j][8 columns] once (one j ahead of its use) and updates its kRows x 8
// float64 sums; the workgroup's kRows rows of B sit in LDS and are read as
// broadcasts.  The work is float64 arithmetic (r multiply-adds per output
// value) next to 0.52 bytes read and 2 bytes written per value.
#include "scale_forms.h"

namespace nf4i {
namespace {

constexpr int kRows = 4;        // rows per workgroup
constexpr int kMergeThreads = 256;
constexpr int kColsPerWg = 8 * kMergeThreads;

// Round-to-odd float64 -> float32: the truncated value with the last bit set
// when the conversion is inexact (same result as round-toward-zero with a
// sticky bit).
__device__ __forceinline__ float to_f32_round_odd(double v) {
  const float f = static_cast<float>(v);  // nearest even
  const double back = static_cast<double>(f);
  uint32_t u = __float_as_uint(f);
  if (back != v) {
    if (fabs(back) > fabs(v)) u -= 1u;  // rounded away from zero: one ulp back toward it
    u |= 1u;
  }
  return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t to_16(double v, bool f16) {
  const float f = to_f32_round_odd(v);
  if (f16) return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // nearest even, subnormals kept
  return f32_to_bf16(f);                                                   // nearest even
}

template <bool kF16Out, bool kDQ, bool kF8>
__global__ __launch_bounds__(kMergeThreads) void k_lora_merge(const uint8_t* __restrict__ packed, int64_t rows,
                                                              int64_t cols, Scales sc,
                                                              const uint16_t* __restrict__ la,
                                                              const uint16_t* __restrict__ lb, int r, float scale,
                                                              uint16_t* __restrict__ out, Codebook cb) {
  __shared__ float lv[16];
  __shared__ uint16_t bsh[kRows * 64];  // B[n0 + i][j] at i * 64 + j
  const int64_t k0 = static_cast<int64_t>(blockIdx.y) * kColsPerWg + 8 * static_cast<int64_t>(threadIdx.x);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int nr = static_cast<int>(rows - n0 < kRows ? rows - n0 : kRows);
  if (threadIdx.x < 16) lv[threadIdx.x] = cb.level[threadIdx.x];
  for (int t = threadIdx.x; t < kRows * r; t += kMergeThreads) {
    const int i = t / r, j = t - (t / r) * r;
    const int64_t n = n0 + (i < nr ? i : nr - 1);  // rows past the end repeat the last (never stored)
    bsh[i * 64 + j] = lb[n * r + j];
  }
  __syncthreads();
  if (k0 >= cols) return;  // cols % 8 == 0: a thread's 8 columns are all in range or all out

  double acc[kRows][8];
#pragma unroll
  for (int i = 0; i < kRows; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.0;
  // A[j][8 columns] is loaded one j ahead of its use (clamped at the end)
  const uint16_t* ap = la + k0;
  uint4 a_next = *reinterpret_cast<const uint4*>(ap);
  for (int j = 0; j < r; ++j) {
    const uint4 a4 = a_next;
    a_next = *reinterpret_cast<const uint4*>(ap + static_cast<int64_t>(j + 1 < r ? j + 1 : j) * cols);
    const uint32_t aw[4] = {a4.x, a4.y, a4.z, a4.w};
    double a[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      a[2 * c] = static_cast<double>(__uint_as_float(aw[c] << 16));
      a[2 * c + 1] = static_cast<double>(__uint_as_float(aw[c] & 0xFFFF0000u));
    }
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const double b = static_cast<double>(__uint_as_float(static_cast<uint32_t>(bsh[i * 64 + j]) << 16));
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[i][c] = fma(b, a[c], acc[i][c]);
    }
  }

  const float mean = kDQ ? *sc.mean : 0.0f;
  const double s = static_cast<double>(scale);
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    if (i >= nr) break;
    const int64_t e0 = (n0 + i) * cols + k0;  // first of the 8 elements; e0 % 8 == 0
    const uint32_t word = *reinterpret_cast<const uint32_t*>(packed + e0 / 2);
    const float ah = block_scale_t<kDQ, kF8>(sc, e0 >> 6, mean);
    uint32_t h[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t code = (word >> (8 * (c >> 1) + ((c & 1) ? 0 : 4))) & 0xFu;
      const float deq = lv[code] * ah;        // fl32(level * a_hat)
      const double t = s * acc[i][c];         // fl64(s * sum)
      const double v = static_cast<double>(deq) + t;
      h[c] = to_16(v, kF16Out);
    }
    const uint4 o = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    *reinterpret_cast<uint4*>(out + e0) = o;
  }
}

}  // namespace

hipError_t launch_lora_merge(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* lora_a,
                             const uint16_t* lora_b, int r, float scale, uint16_t* out, int out_f16,
                             hipStream_t s) {
  const int64_t gx = (rows + kRows - 1) / kRows;             // row groups
  const int64_t gy = (cols + kColsPerWg - 1) / kColsPerWg;   // column chunks
  if (gx > (int64_t(1) << 24) || gy > 65535) return hipErrorInvalidValue;  // work-items fit 32 bits
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
  const Codebook& cb = codebook(sc.fp4);
#define NF4_MERGE(H, D, F) \
  hipLaunchKernelGGL((k_lora_merge<H, D, F>), grid, dim3(kMergeThreads), 0, s, packed, rows, cols, sc, lora_a, lora_b, \
                     r, scale, out, cb)
  if (out_f16) {
    if (sc.absmax) NF4_MERGE(true, false, false); else if (sc.f8) NF4_MERGE(true, true, true); else NF4_MERGE(true, true, false);
  } else {
    if (sc.absmax) NF4_MERGE(false, false, false); else if (sc.f8) NF4_MERGE(false, true, true); else NF4_MERGE(false, true, false);
  }
#undef NF4_MERGE
  return hipGetLastError();
}

}  // namespace nf4i
