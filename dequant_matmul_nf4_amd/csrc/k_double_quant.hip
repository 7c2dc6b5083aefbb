// Double quantization of the block scales (bitsandbytes tool page, "Double
// quantization", with the int8 scheme of its "A worked example": scale by 127,
// round half away from zero).  The scales are first centred on their mean.
// The float8 variant (tutorial page "bitsandbytes quantization tutorial:
// 4-bit and 8-bit models", section "How NF4 Works": float32 to float8) scales
// by 448 instead and stores the nearest E4M3 code.
//
// The mean must not depend on summation order, so the scales are summed
// exactly: each float32 is an integer m * 2^p times 2^-149 (m < 2^24,
// 0 <= p <= 253), added into 32-bit digits of a wide fixed-point integer held
// in 64-bit accumulators (no carries until the end).  Each summing workgroup
// writes its digit sums to its own workspace row (no atomics: device-wide
// atomics on one address serialize in memory).  Every workgroup of the
// quantizing kernel then adds the rows itself, propagates the carries, rounds
// the integer once to float64, divides by the count in float64 and rounds to
// float32 -- the same value in every workgroup, so no third launch is needed.
//
// Kernels: k_dq_partial (digit sums per workgroup), k_dq_quant (the mean,
// then one wave per group of 256 scales).
#include "nf4_device.h"

namespace nf4i {
namespace {

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

// Rounds the non-negative integer I = sum_k dig[k] 2^(32k) (12 digits, all
// indexing static so everything stays in registers) to the nearest float64,
// ties to even, and returns I * 2^-149.  The top three digits give a 96-bit
// window holding the 53 result bits plus the round bit; everything below
// only feeds the sticky bit.
__device__ double digits_to_double(const uint32_t (&dig)[kDqDigits]) {
  int top = -1;
#pragma unroll
  for (int k = 0; k < kDqDigits; ++k)
    if (dig[k]) top = k;
  if (top < 0) return 0.0;
  uint32_t d2 = 0, d1 = 0, d0 = 0, below = 0;
#pragma unroll
  for (int k = 0; k < kDqDigits; ++k) {
    d2 = (k == top) ? dig[k] : d2;
    d1 = (k == top - 1) ? dig[k] : d1;
    d0 = (k == top - 2) ? dig[k] : d0;
    below |= (k < top - 2) ? dig[k] : 0u;
  }
  // window N = (H:L) with H = d2:d1, L = d0:0, so I = N * 2^(32 (top - 2) - 32)
  const unsigned long long H = (static_cast<unsigned long long>(d2) << 32) | d1;
  const unsigned long long L = static_cast<unsigned long long>(d0) << 32;
  const int lz = __clzll(H);  // 0..31 because d2 != 0
  const unsigned long long nh = lz ? (H << lz) | (L >> (64 - lz)) : H;
  const unsigned long long nl = L << lz;
  unsigned long long mant = nh >> 11;  // top 53 bits of the 128-bit window
  const unsigned long long round = (nh >> 10) & 1ull;
  const bool sticky = (nh & 0x3FFull) || nl || below;
  if (round && (sticky || (mant & 1ull))) ++mant;
  const int exp2 = 75 + 32 * (top - 2) - 32 - lz - 149;
  return ldexp(static_cast<double>(mant), exp2);
}

// Adds the 256 threads' digit vectors held in vec and returns the total of
// digit t in threads t < 12: first thread t < 192 adds digit t % 12 of rows
// 16 c .. 16 c + 15 (c = t / 12), then 12 threads add the 16 chunk sums.
// Each step issues all of its LDS reads before adding, so the sum costs two
// LDS round trips rather than one per row.  Contains two barriers.
constexpr int kSumChunks = 16;  // rows per chunk and number of chunks (16 x 16 = 256)

__device__ __forceinline__ unsigned long long block_digit_sum(unsigned long long (*vec)[kDqDigits + 1],
                                                              unsigned long long (*tot)[kDqDigits]) {
  const int t = threadIdx.x;
  if (t < kSumChunks * kDqDigits) {
    const int k = t % kDqDigits, c = t / kDqDigits;
    unsigned long long v[kSumChunks];
#pragma unroll
    for (int i = 0; i < kSumChunks; ++i) v[i] = vec[kSumChunks * c + i][k];
    unsigned long long sum = 0ull;
#pragma unroll
    for (int i = 0; i < kSumChunks; ++i) sum += v[i];
    tot[c][k] = sum;
  }
  __syncthreads();
  unsigned long long sum = 0ull;
  if (t < kDqDigits) {
    unsigned long long v[kSumChunks];
#pragma unroll
    for (int c = 0; c < kSumChunks; ++c) v[c] = tot[c][t];
#pragma unroll
    for (int c = 0; c < kSumChunks; ++c) sum += v[c];
  }
  __syncthreads();
  return sum;
}

// Digit sums of the workgroup's scales: each thread adds kPerThread scales
// (all loads issued first) into registers, then the 256 threads' digit
// vectors are added through LDS into the workgroup's row.
//
// A contribution lands in digits d and d + 1.  The scales of one weight
// mostly share one or two exponent ranges, so each thread also keeps a
// window of three digits starting at the digit d of its first nonzero scale
// and adds a contribution there when d is the window's first or second digit
// (three selects); any other contribution takes the selects over all 12
// digits.  The window is added into the 12 digits at the end, so the sum is
// the same integer either way.  The window pays off from about 8 scales per
// thread (measured: 8192^2 weights 15.4 -> 14.6 us; at 4 per thread the
// final fold costs more than it saves), so the launcher picks it by size.
constexpr int kPerThread = 4;

template <bool kWindow>
__global__ __launch_bounds__(256) void k_dq_partial(const float* __restrict__ absmax, int64_t nb,
                                                    unsigned long long* __restrict__ ws) {
  __shared__ unsigned long long vec[256][kDqDigits + 1];  // +1: spreads the banks
  __shared__ unsigned long long tot[kSumChunks][kDqDigits];
  const int t = threadIdx.x;
  unsigned long long acc[kDqDigits];
#pragma unroll
  for (int k = 0; k < kDqDigits; ++k) acc[k] = 0ull;
  int base = -1;  // the window's first digit (placed by the first nonzero scale)
  unsigned long long w0 = 0ull, w1 = 0ull, w2 = 0ull;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + t; i0 < nb; i0 += kPerThread * stride) {
    float v[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int64_t i = i0 + u * stride;
      v[u] = (i < nb) ? absmax[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      int d;
      uint32_t lo, hi;
      scale_to_digits(v[u], &d, &lo, &hi);
      if (kWindow && base < 0 && (lo | hi) != 0u) base = d;
      const int rel = d - base;  // a zero scale adds nothing wherever it goes
      if (kWindow && (rel == 0 || rel == 1)) {
        w0 += rel == 0 ? lo : 0u;
        w1 += rel == 0 ? hi : lo;
        w2 += rel == 0 ? 0u : hi;
      } else {
        // selects keep the indexing static
#pragma unroll
        for (int k = 0; k < kDqDigits; ++k)
          acc[k] += static_cast<unsigned long long>((k == d ? lo : 0u)) + static_cast<unsigned long long>((k == d + 1 ? hi : 0u));
      }
    }
  }
  if constexpr (kWindow) {
#pragma unroll
    for (int k = 0; k < kDqDigits; ++k)
      acc[k] += (k == base ? w0 : 0ull) + (k == base + 1 ? w1 : 0ull) + (k == base + 2 ? w2 : 0ull);
  }
#pragma unroll
  for (int k = 0; k < kDqDigits; ++k) vec[t][k] = acc[k];
  __syncthreads();
  const unsigned long long sum = block_digit_sum(vec, tot);
  if (t < kDqDigits) ws[blockIdx.x * kDqDigits + t] = sum;
}

// The mean from the partial rows (at most 256), in a workgroup of 256
// threads: thread t loads row t, the rows are added per digit, and thread 0
// propagates the carries, rounds and divides.  Returns the mean in every
// thread.
__device__ float dq_mean(const unsigned long long* __restrict__ ws, int nparts, int64_t nb) {
  __shared__ unsigned long long vec[256][kDqDigits + 1];
  __shared__ unsigned long long tot[kSumChunks][kDqDigits];
  __shared__ unsigned long long dsum[kDqDigits];
  __shared__ float mean_s;
  const int t = threadIdx.x;
  {
    unsigned long long row[kDqDigits];
    if (t < nparts) {
      const ulonglong2* p = reinterpret_cast<const ulonglong2*>(ws + t * kDqDigits);
#pragma unroll
      for (int k = 0; k < kDqDigits / 2; ++k) {
        const ulonglong2 v = p[k];
        row[2 * k] = v.x;
        row[2 * k + 1] = v.y;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kDqDigits; ++k) row[k] = 0ull;
    }
#pragma unroll
    for (int k = 0; k < kDqDigits; ++k) vec[t][k] = row[k];
  }
  __syncthreads();
  const unsigned long long s = block_digit_sum(vec, tot);
  if (t < kDqDigits) dsum[t] = s;
  __syncthreads();
  if (t == 0) {
    uint32_t dig[kDqDigits];
    unsigned long long carry = 0;
#pragma unroll
    for (int k = 0; k < kDqDigits; ++k) {
      const unsigned long long v = dsum[k] + carry;
      dig[k] = static_cast<uint32_t>(v);
      carry = v >> 32;
    }
    const double total = digits_to_double(dig);
    mean_s = static_cast<float>(total / static_cast<double>(nb));
  }
  __syncthreads();
  return mean_s;
}

// E4M3 code of t, |t| <= 448, nearest with ties to the even mantissa (the
// float8 reading): subnormals (|t| < 2^-6) are multiples of 2^-9, rounded by
// rintf on t * 2^9 (exact scaling); normal values round the float32
// significand to 3 bits at bit 20 (a carry moves into the exponent).  448 is
// the largest finite E4M3 value, so the NaN pattern is never produced.
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
  const uint32_t sign = (__float_as_uint(t) >> 24) & 0x80u;
  const float a = fabsf(t);
  if (a < 0x1p-6f) return sign | static_cast<uint32_t>(rintf(a * 512.0f));  // 0..8; 8 is 2^-6 = code 0x08
  const uint32_t b = __float_as_uint(a);
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  return sign | ((((r >> 23) - 127u + 7u) << 3) | ((r >> 20) & 7u));
}

template <bool kF8>
__global__ __launch_bounds__(256) void k_dq_quant(const float* __restrict__ absmax, int64_t nb,
                                                  const unsigned long long* __restrict__ ws, int nparts,
                                                  float* __restrict__ mean_out, int8_t* __restrict__ q,
                                                  float* __restrict__ absmax2) {
  const int lane = threadIdx.x & 63;
  const int64_t ngroups = (nb + 255) >> 8;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  // the scales of the wave's first group are loaded before the mean is known
  auto load4 = [&](int64_t g, float (&a)[4]) {
    const int64_t i0 = g * 256 + lane * 4;
    if (i0 + 4 <= nb) {
      const float4 v = *reinterpret_cast<const float4*>(absmax + i0);
      a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = (i0 + j < nb) ? absmax[i0 + j] : 0.0f;
    }
  };
  float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (wave < ngroups) load4(wave, a);
  const float mu = dq_mean(ws, nparts, nb);
  if (blockIdx.x == 0 && threadIdx.x == 0) *mean_out = mu;
  for (int64_t g = wave; g < ngroups; g += nwaves) {
    if (g != wave) load4(g, a);
    const int64_t i0 = g * 256 + lane * 4;
    float c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = (i0 + j < nb) ? a[j] - mu : 0.0f;
    float s = fmaxf(fmaxf(fabsf(c[0]), fabsf(c[1])), fmaxf(fabsf(c[2]), fabsf(c[3])));
    s = group_max<64>(s);
    uint32_t word = 0;
    if (s > 0.0f) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (kF8) {
          const float t = (c[j] / s) * 448.0f;  // two roundings, as the int8 step
          word |= e4m3_rne(t) << (8 * j);
        } else {
          const float t = (c[j] / s) * 127.0f;
          const float at = fabsf(t);
          const float fl = floorf(at);
          float r = fl + ((at - fl) >= 0.5f ? 1.0f : 0.0f);  // half away from zero
          r = fminf(r, 127.0f);
          const int qi = (t < 0.0f) ? -static_cast<int>(r) : static_cast<int>(r);
          word |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * j);
        }
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
                               float* mean, unsigned long long* ws, int f8, hipStream_t s) {
  int64_t want = (nb + 256 * kPerThread - 1) / (256 * kPerThread);
  int grid = static_cast<int>(want < kDqMaxGroups ? want : kDqMaxGroups);
  if (nb >= static_cast<int64_t>(grid) * 256 * 8)
    hipLaunchKernelGGL(k_dq_partial<true>, dim3(grid), dim3(256), 0, s, absmax, nb, ws);
  else
    hipLaunchKernelGGL(k_dq_partial<false>, dim3(grid), dim3(256), 0, s, absmax, nb, ws);
  const int64_t groups = (nb + 255) >> 8;
  want = (groups + 3) / 4;  // 4 waves per workgroup
  const int qgrid = static_cast<int>(want < 1024 ? want : 1024);
  if (f8) hipLaunchKernelGGL(k_dq_quant<true>, dim3(qgrid), dim3(256), 0, s, absmax, nb, ws, grid, mean, q, absmax2);
  else hipLaunchKernelGGL(k_dq_quant<false>, dim3(qgrid), dim3(256), 0, s, absmax, nb, ws, grid, mean, q, absmax2);
  return hipGetLastError();
}

}  // namespace nf4i
