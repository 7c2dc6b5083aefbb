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
// then one wave per group of 256 scales).  For several scale arrays at once,
// k_dq_partial_batch, k_dq_mean_batch (one workgroup per array: its mean,
// written to the array's mean output) and k_dq_quant_batch (reads that mean)
// do the same in three launches: each workgroup belongs to one array, found
// from per-array workgroup offsets; each array has its own partial rows.
#include <mutex>

#include "nf4_device.h"

namespace nf4i {
namespace {

// Partial digit rows of the allocation-free entry point: one call's worth
// (kDqMaxGroups rows of kDqDigits u64, 24 KiB) per device, alive until the
// process ends.  Host code never passes this name to a kernel; it passes the
// address dq_scratch() obtained for the current device.
static __device__ __align__(256) unsigned long long scratch[kDqMaxGroups * kDqDigits];
static_assert(sizeof(scratch) >= kDqWorkspaceBytes, "scratch holds the partial rows of any call");

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

// Both kernels run in workgroups of kThreads = 256 (small scale arrays: more
// workgroups, so more of the chip pulls the few bytes) or 1024 threads (large
// ones: fewer partial rows, so less for every quantizing workgroup to re-read).

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Adds the workgroup's digit vectors (acc in every thread) and returns the
// total of digit t in threads t < 12.
//  - 256 threads: the vectors go to LDS; thread t < 192 adds digit t % 12 of
//    rows 16 c .. 16 c + 15 (c = t / 12), then 12 threads add the 16 chunk
//    sums; each step issues all of its LDS reads before adding.
//  - 1024 threads (too many rows for LDS): each wave adds its 64 lanes with
//    cross-lane 64-bit adds, skipping a digit that is zero in all of its
//    lanes (the scales of one weight touch two or three digits), and the 16
//    wave sums of each digit are added through LDS.
// Contains two barriers (256 threads) or one (1024).
constexpr int kSumChunks = 16;  // rows per chunk and number of chunks (16 x 16 = 256)

template <int kThreads>
__device__ __forceinline__ unsigned long long block_digit_sum(const unsigned long long (&acc)[kDqDigits]) {
  static_assert(kThreads == 256 || kThreads == 1024, "two workgroup sizes");
  const int t = threadIdx.x;
  unsigned long long sum = 0ull;
  if constexpr (kThreads == 256) {
    __shared__ unsigned long long vec[256][kDqDigits + 1];  // +1: spreads the banks
    __shared__ unsigned long long tot[kSumChunks][kDqDigits];
#pragma unroll
    for (int k = 0; k < kDqDigits; ++k) vec[t][k] = acc[k];
    __syncthreads();
    if (t < kSumChunks * kDqDigits) {
      const int k = t % kDqDigits, c = t / kDqDigits;
      unsigned long long v[kSumChunks];
#pragma unroll
      for (int i = 0; i < kSumChunks; ++i) v[i] = vec[kSumChunks * c + i][k];
      unsigned long long cs = 0ull;
#pragma unroll
      for (int i = 0; i < kSumChunks; ++i) cs += v[i];
      tot[c][k] = cs;
    }
    __syncthreads();
    if (t < kDqDigits) {
      unsigned long long v[kSumChunks];
#pragma unroll
      for (int c = 0; c < kSumChunks; ++c) v[c] = tot[c][t];
#pragma unroll
      for (int c = 0; c < kSumChunks; ++c) sum += v[c];
    }
  } else {
    constexpr int kWaves = kThreads / kWave;
    __shared__ unsigned long long wsum[kWaves][kDqDigits];
    const int lane = t & (kWave - 1), wave = t / kWave;
#pragma unroll
    for (int k = 0; k < kDqDigits; ++k) {
      unsigned long long v = acc[k];
      if (__any(v != 0ull)) v = wave_sum_u64(v);
      if (lane == 0) wsum[wave][k] = v;
    }
    __syncthreads();
    if (t < kDqDigits) {
      unsigned long long v[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v[w] = wsum[w][t];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += v[w];
    }
  }
  return sum;
}

// Digit sums of the workgroup's scales: each thread adds its scales, read as
// 16-byte vectors with kVec of them requested before any is used, into
// registers; the workgroup's digit vectors are then added into its row.
//
// A contribution lands in digits d and d + 1.  The scales of one weight
// mostly share one or two exponent ranges, so each thread also keeps a
// window of three digits starting at the digit d of its first nonzero scale
// and adds a contribution there when d is the window's first or second digit
// (three selects); any other contribution takes the selects over all 12
// digits.  The window is added into the 12 digits at the end, so the sum is
// the same integer either way.  The window pays off from about 8 scales per
// thread, so the launcher picks it by size.  kVec: 2 vectors in flight for
// small arrays, 4 for large ones (16 scales per thread: one round trip).
// Workgroup `blk` of `grid` summing workgroups over absmax[0, nb); its row
// goes to ws[blk].
// One thread's digit sums: 12 digits, plus (kWindow) the three-digit window.
template <bool kWindow>
struct DigitAcc {
  unsigned long long acc[kDqDigits];
  int base = -1;  // the window's first digit (placed by the first nonzero scale)
  unsigned long long w0 = 0ull, w1 = 0ull, w2 = 0ull;

  __device__ __forceinline__ DigitAcc() {
#pragma unroll
    for (int k = 0; k < kDqDigits; ++k) acc[k] = 0ull;
  }
  __device__ __forceinline__ void add(float a) {
    int d;
    uint32_t lo, hi;
    scale_to_digits(a, &d, &lo, &hi);
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
  // The window added into the 12 digits: the same integer either way.
  __device__ __forceinline__ void fold() {
    if constexpr (kWindow) {
#pragma unroll
      for (int k = 0; k < kDqDigits; ++k)
        acc[k] += (k == base ? w0 : 0ull) + (k == base + 1 ? w1 : 0ull) + (k == base + 2 ? w2 : 0ull);
    }
  }
};

template <int kThreads, bool kWindow, int kVec>
__device__ __forceinline__ void dq_partial_body(const float* __restrict__ absmax, int64_t nb,
                                                unsigned long long* __restrict__ ws, int blk, int grid) {
  const int t = threadIdx.x;
  DigitAcc<kWindow> da;
  auto add = [&](float a) { da.add(a); };
  const int64_t n4 = nb >> 2;  // whole 16-byte vectors; absmax is 16-byte aligned
  const float4* a4 = reinterpret_cast<const float4*>(absmax);
  const int64_t stride = static_cast<int64_t>(grid) * kThreads;
  for (int64_t i0 = static_cast<int64_t>(blk) * kThreads + t; i0 < n4; i0 += kVec * stride) {
    float4 v[kVec];
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const int64_t i = i0 + u * stride;
      v[u] = (i < n4) ? a4[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      add(v[u].x);
      add(v[u].y);
      add(v[u].z);
      add(v[u].w);
    }
  }
  // the last nb % 4 scales, in the first workgroup
  if (blk == 0 && t < static_cast<int>(nb & 3)) add(absmax[(n4 << 2) + t]);
  da.fold();
  const unsigned long long sum = block_digit_sum<kThreads>(da.acc);
  if (t < kDqDigits) ws[static_cast<int64_t>(blk) * kDqDigits + t] = sum;
}

template <int kThreads, bool kWindow, int kVec>
__global__ __launch_bounds__(kThreads) void k_dq_partial(const float* __restrict__ absmax, int64_t nb,
                                                         unsigned long long* __restrict__ ws) {
  dq_partial_body<kThreads, kWindow, kVec>(absmax, nb, ws, blockIdx.x, gridDim.x);
}

// The mean from the partial rows (at most 256, one per thread of the
// workgroup at most): thread t < nparts loads row t, the rows are added per digit, and thread 0 propagates the carries,
// rounds and divides.  Returns the mean in every thread.
template <int kThreads>
__device__ float dq_mean(const unsigned long long* __restrict__ ws, int nparts, int64_t nb) {
  __shared__ unsigned long long dsum[kDqDigits];
  __shared__ float mean_s;
  const int t = threadIdx.x;
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
  const unsigned long long s = block_digit_sum<kThreads>(row);
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

// One wave per group of 256 scales; a wave's first kQuantPre groups are
// requested before the mean is known, so their loads overlap the mean.
constexpr int kQuantPre = 4;

// Workgroup `blk` of `grid` quantizing workgroups of one scale array: the
// mean from the nparts partial rows at ws (written to mean_out by workgroup
// 0), or, with kMeanGiven, read from mean_out, where an earlier launch put it.
template <int kThreads, bool kF8, bool kMeanGiven = false>
__device__ __forceinline__ void dq_quant_body(const float* __restrict__ absmax, int64_t nb,
                                              const unsigned long long* __restrict__ ws, int nparts,
                                              float* __restrict__ mean_out, int8_t* __restrict__ q,
                                              float* __restrict__ absmax2, int blk, int grid) {
  constexpr int kWaves = kThreads / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t ngroups = (nb + 255) >> 8;
  const int64_t wave = static_cast<int64_t>(blk) * kWaves + threadIdx.x / kWave;
  const int64_t nwaves = static_cast<int64_t>(grid) * kWaves;
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
  auto quant_group = [&](int64_t g, const float (&a)[4], float mu) {
    const int64_t i0 = g * 256 + lane * 4;
    const bool full = (g + 1) * 256 <= nb;  // the same for the whole wave
    float c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = (full || i0 + j < nb) ? a[j] - mu : 0.0f;
    float s = fmaxf(fmaxf(fabsf(c[0]), fabsf(c[1])), fmaxf(fabsf(c[2]), fabsf(c[3])));
    s = group_max<64>(s);
    uint32_t word = 0;
    if (s > 0.0f) {
      // fl32(c / s) from one reciprocal per group: y = fl32(1 / s), q0 =
      // fl32(c y), r = fma(-q0, s, c) (exact) and fma(r, y, q0) is the
      // correctly rounded quotient (Markstein's theorem) while no
      // intermediate underflows: for 2^-80 <= s < 2^126 that holds for
      // |c / s| >= 2^-20, and below that the quotient only decides codes
      // that are 0 either way (|t| < 127 * 2^-20 or 448 * 2^-20, far under
      // half of the smallest nonzero code).  Other s: IEEE division per value.
      const bool fast = s >= 0x1p-80f && s < 0x1p126f;  // the same for the whole wave
      const float y = 1.0f / s;
      auto quotient = [&](float cj) {
        if (!fast) return cj / s;
        const float q0 = cj * y;
        const float r = fmaf(-q0, s, cj);
        return fmaf(r, y, q0);
      };
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (kF8) {
          const float t = quotient(c[j]) * 448.0f;  // two roundings, as the int8 step
          word |= e4m3_rne(t) << (8 * j);
        } else {
          const float t = quotient(c[j]) * 127.0f;
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
  };
  float a[kQuantPre][4];
#pragma unroll
  for (int p = 0; p < kQuantPre; ++p) {
    const int64_t g = wave + p * nwaves;
    if (g < ngroups) load4(g, a[p]);
  }
  float mu;
  if constexpr (kMeanGiven) {
    mu = *mean_out;
  } else {
    mu = dq_mean<kThreads>(ws, nparts, nb);
    if (blk == 0 && threadIdx.x == 0) *mean_out = mu;
  }
#pragma unroll
  for (int p = 0; p < kQuantPre; ++p) {
    const int64_t g = wave + p * nwaves;
    if (g < ngroups) quant_group(g, a[p], mu);
  }
  for (int64_t g = wave + kQuantPre * nwaves; g < ngroups; g += nwaves) {
    float b[4];
    load4(g, b);
    quant_group(g, b, mu);
  }
}

template <int kThreads, bool kF8>
__global__ __launch_bounds__(kThreads) void k_dq_quant(const float* __restrict__ absmax, int64_t nb,
                                                         const unsigned long long* __restrict__ ws, int nparts,
                                                         float* __restrict__ mean_out, int8_t* __restrict__ q,
                                                         float* __restrict__ absmax2) {
  dq_quant_body<kThreads, kF8>(absmax, nb, ws, nparts, mean_out, q, absmax2, blockIdx.x, gridDim.x);
}

// Several scale arrays in one pair of launches.  part0[j] and quant0[j] are
// the first summing and quantizing workgroups of array j (part0[count] and
// quant0[count] the totals); array j's partial rows are ws rows
// part0[j] .. part0[j + 1] - 1.
struct DqBatch {
  int count;
  const float* absmax[kDqMaxJobs];
  int64_t nb[kDqMaxJobs];
  int8_t* q[kDqMaxJobs];
  float* absmax2[kDqMaxJobs];
  float* mean[kDqMaxJobs];
  int window[kDqMaxJobs];  // the summing kernel's digit window pays off (about 8 or more scales per thread)
  int part0[kDqMaxJobs + 1];
  int quant0[kDqMaxJobs + 1];
};

constexpr int kDqBatchThreads = 1024;
constexpr int kDqBatchVec = 4;
constexpr int kDqBatchPerThread = 64;   // scales per summing thread (four vectors in flight at a time)

__global__ __launch_bounds__(kDqBatchThreads) void k_dq_partial_batch(DqBatch b, unsigned long long* __restrict__ ws) {
  const int blk = blockIdx.x;
  const int j = batch_item_of<kDqMaxJobs>(b.part0, b.count, blk);
  const int local = blk - b.part0[j], grid = b.part0[j + 1] - b.part0[j];
  unsigned long long* rows = ws + static_cast<int64_t>(b.part0[j]) * kDqDigits;
  if (b.window[j]) dq_partial_body<kDqBatchThreads, true, kDqBatchVec>(b.absmax[j], b.nb[j], rows, local, grid);
  else dq_partial_body<kDqBatchThreads, false, kDqBatchVec>(b.absmax[j], b.nb[j], rows, local, grid);
}

// One workgroup per array: the mean from its partial rows (at most
// kDqMaxGroups, one per thread).
__global__ __launch_bounds__(kDqMaxGroups) void k_dq_mean_batch(DqBatch b, const unsigned long long* __restrict__ ws) {
  const int j = blockIdx.x;
  const unsigned long long* rows = ws + static_cast<int64_t>(b.part0[j]) * kDqDigits;
  const float mu = dq_mean<kDqMaxGroups>(rows, b.part0[j + 1] - b.part0[j], b.nb[j]);
  if (threadIdx.x == 0) *b.mean[j] = mu;
}

// Sized so that every wave has at most kQuantPre groups, all requested at once.
template <bool kF8>
__global__ __launch_bounds__(kDqBatchThreads) void k_dq_quant_batch(DqBatch b) {
  const int blk = blockIdx.x;
  const int j = batch_item_of<kDqMaxJobs>(b.quant0, b.count, blk);
  const int local = blk - b.quant0[j], grid = b.quant0[j + 1] - b.quant0[j];
  dq_quant_body<kDqBatchThreads, kF8, true>(b.absmax[j], b.nb[j], nullptr, 0, b.mean[j], b.q[j], b.absmax2[j], local,
                                            grid);
}

}  // namespace

hipError_t dq_scratch(unsigned long long** out) {
  // device address of `scratch`, looked up once per device with that device
  // current (each device holds its own copy of the array)
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = static_cast<unsigned long long*>(addr[dev]);
  return hipSuccess;
}

namespace {

template <int kThreads, int kVec>
void launch_dq(const float* absmax, int64_t nb, int8_t* q, float* absmax2, float* mean, unsigned long long* ws,
               int f8, int per_thread, int max_qgrid, hipStream_t s) {
  constexpr int kWaves = kThreads / kWave;
  // at least per_thread scales per summing thread, at most kDqMaxGroups partial rows
  int64_t want = (nb + kThreads * per_thread - 1) / (kThreads * per_thread);
  const int grid = static_cast<int>(want < kDqMaxGroups ? want : kDqMaxGroups);
  if (nb >= static_cast<int64_t>(grid) * kThreads * 8)
    hipLaunchKernelGGL((k_dq_partial<kThreads, true, kVec>), dim3(grid), dim3(kThreads), 0, s, absmax, nb, ws);
  else
    hipLaunchKernelGGL((k_dq_partial<kThreads, false, kVec>), dim3(grid), dim3(kThreads), 0, s, absmax, nb, ws);
  // one group per wave, up to max_qgrid workgroups (each re-reads the partial rows)
  const int64_t groups = (nb + 255) >> 8;
  want = (groups + kWaves - 1) / kWaves;
  const int qgrid = static_cast<int>(want < max_qgrid ? want : max_qgrid);
  if (f8)
    hipLaunchKernelGGL((k_dq_quant<kThreads, true>), dim3(qgrid), dim3(kThreads), 0, s, absmax, nb, ws, grid, mean, q,
                       absmax2);
  else
    hipLaunchKernelGGL((k_dq_quant<kThreads, false>), dim3(qgrid), dim3(kThreads), 0, s, absmax, nb, ws, grid, mean, q,
                       absmax2);
}

}  // namespace

hipError_t launch_double_quant(const float* absmax, int64_t nb, int8_t* q, float* absmax2,
                               float* mean, unsigned long long* ws, int f8, hipStream_t s) {
  if (nb >= (int64_t{1} << 21))
    launch_dq<1024, 4>(absmax, nb, q, absmax2, mean, ws, f8, 16, 256, s);
  else
    launch_dq<256, 2>(absmax, nb, q, absmax2, mean, ws, f8, 4, 1024, s);
  return hipGetLastError();
}

hipError_t launch_double_quant_batch(const DqJob* jobs, int count, unsigned long long* ws, int f8, hipStream_t s) {
  if (count < 1 || count > kDqMaxJobs) return hipErrorInvalidValue;
  DqBatch b{};
  b.count = count;
  int parts = 0, quants = 0;
  for (int j = 0; j < count; ++j) {
    const int64_t nb = jobs[j].nblocks;
    b.absmax[j] = jobs[j].absmax;
    b.nb[j] = nb;
    b.q[j] = jobs[j].q;
    b.absmax2[j] = jobs[j].absmax2;
    b.mean[j] = jobs[j].mean;
    // summing workgroups: about kDqBatchPerThread scales per thread, at most kDqMaxGroups rows
    const int64_t pw = (nb + int64_t{kDqBatchThreads} * kDqBatchPerThread - 1) /
                       (int64_t{kDqBatchThreads} * kDqBatchPerThread);
    const int g = static_cast<int>(pw < kDqMaxGroups ? pw : kDqMaxGroups);
    b.window[j] = nb >= static_cast<int64_t>(g) * kDqBatchThreads * 8 ? 1 : 0;
    // quantizing workgroups: at most kQuantPre groups of 256 scales per wave
    const int64_t groups = (nb + 255) >> 8;
    const int64_t per_wg = int64_t{kDqBatchThreads / kWave} * kQuantPre;
    const int qg = static_cast<int>((groups + per_wg - 1) / per_wg);  // nb < 2^31: at most 2^13
    b.part0[j] = parts;
    b.quant0[j] = quants;
    parts += g;
    quants += qg;
  }
  for (int j = count; j <= kDqMaxJobs; ++j) {
    b.part0[j] = parts;
    b.quant0[j] = quants;
  }
  hipLaunchKernelGGL(k_dq_partial_batch, dim3(parts), dim3(kDqBatchThreads), 0, s, b, ws);
  hipLaunchKernelGGL(k_dq_mean_batch, dim3(count), dim3(kDqMaxGroups), 0, s, b, ws);
  if (f8) hipLaunchKernelGGL(k_dq_quant_batch<true>, dim3(quants), dim3(kDqBatchThreads), 0, s, b);
  else hipLaunchKernelGGL(k_dq_quant_batch<false>, dim3(quants), dim3(kDqBatchThreads), 0, s, b);
  return hipGetLastError();
}

}  // namespace nf4i
