// Blockwise NF4 quantization (bitsandbytes tool page, "How it works",
// Steps 1-4): per block of 64 values, the largest |x| is the scale; each value
// is divided by it and replaced by the index of the nearest NF4 level; two
// indices are packed per byte, the first in the high nibble.  The FP4 code book
// (the tool page's "What it is" and "Glossary"; read as E2M1 / 6) takes the
// same steps; its ascending level index is stored as the E2M1 pattern.
//
// Layout: each lane owns 16 consecutive values (two 16-byte bf16 loads or
// four 16-byte fp32 loads) and writes 8 bytes of packed codes; 4 adjacent
// lanes form one 64-block and reduce its absmax with DPP quad permutes.
//
// Division: the normalized value must be the IEEE float32 quotient
// fl32(x / a).  With y = fl32(1 / a) correctly rounded (one IEEE division per
// lane and block), q0 = fl32(x * y), r = fma(-q0, a, x) and q = fma(r, y, q0)
// give exactly fl32(x / a) (Markstein's theorem: y within half an ulp of 1/a,
// q0 within one ulp of x/a, r exact) whenever no intermediate underflows.
// That holds for 2^-98 <= a < 2^126 and |x / a| >= 2^-5; below 2^-5 every
// value maps to the zero level whatever its last bits.  Blocks whose absmax
// lies outside that range take the IEEE division per value.
//
// Nearest level: a 2048-entry bucket table in LDS indexed by the top 11 bits
// of the normalized value (sign, exponent, two significand bits); each bucket
// holds at most one decision threshold, so code = base + (q >= thr).
#include "nf4_device.h"

namespace nf4i {
namespace {

constexpr int kPerLane = 16;

__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));  // lane ^ 1
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));  // lane ^ 2
  return v;
}

template <bool kBf16>
__device__ __forceinline__ void load16(const void* xv, int64_t e0, int64_t, float v[kPerLane]) {
  {
    if constexpr (kBf16) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + e0);
      const uint4 a = p[0], b = p[1];
      const uint32_t q[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[2 * i] = __uint_as_float(q[i] << 16);
        v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(xv) + e0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 t = p[i];
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
      }
    }
  }
}

__device__ __forceinline__ uint32_t code_of(float q, const uint2* lut) {
  const uint2 e = lut[__float_as_uint(q) >> 21];
  return e.y + ((q >= __uint_as_float(e.x)) ? 1u : 0u);
}

// Quantizes one 16-value segment held by a lane (its quad holds the block)
// and stores its 8 packed bytes and, from the quad's first lane, the absmax.
template <bool kFp4>
__device__ __forceinline__ void quantize_segment(const float v[kPerLane], int64_t sg, uint8_t* __restrict__ packed,
                                                 float* __restrict__ absmax, const uint2* lut, int64_t nbytes,
                                                 bool full) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) a = fmaxf(a, fabsf(v[i]));
  a = quad_max(a);
  constexpr uint32_t kZero = kFp4 ? 0u : 0x77777777u;  // the zero level's code in every nibble
  uint32_t w0 = kZero, w1 = kZero;  // all-zero block
  if (a > 0.0f) {
    uint32_t c[kPerLane];
    if (a >= 0x1p-98f && a < 0x1p126f) {
      const float y = 1.0f / a;
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) {
        const float q0 = v[i] * y;
        const float r = fmaf(-q0, a, v[i]);
        c[i] = code_of(fmaf(r, y, q0), lut);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) c[i] = code_of(v[i] / a, lut);
    }
    if constexpr (kFp4) {
      // ascending index -> E2M1 pattern
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) c[i] = c[i] >= 7u ? c[i] - 7u : 15u - c[i];
    }
    w0 = 0;
    w1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // element 2j -> high nibble of byte j, element 2j+1 -> low nibble
      const int sh = 8 * (i >> 1) + ((i & 1) ? 0 : 4);
      w0 |= c[i] << sh;
      w1 |= c[i + 8] << sh;
    }
  }
  const int64_t byte0 = sg * (kPerLane / 2);
  if (full) {
    *reinterpret_cast<uint2*>(packed + byte0) = make_uint2(w0, w1);
  } else {
    for (int j = 0; j < 8; ++j)
      if (byte0 + j < nbytes) packed[byte0 + j] = static_cast<uint8_t>((j < 4 ? w0 : w1) >> (8 * (j & 3)));
  }
  if ((threadIdx.x & 3) == 0) absmax[sg >> 2] = a;
}

// The bucket table in LDS (ends with a barrier).
__device__ __forceinline__ void fill_lut(uint2* lut, const QuantLut& tab) {
  for (int i = threadIdx.x; i < kLutBuckets; i += blockDim.x) lut[i] = make_uint2(0x7F800000u, 7u);
  __syncthreads();
  if (threadIdx.x < kLutSpecial)
    lut[lut_special_index(threadIdx.x)] = make_uint2(__float_as_uint(tab.thr[threadIdx.x]), tab.base[threadIdx.x]);
  __syncthreads();
}

// Workgroup `blk` of `grid` over one tensor.  Main loop over the blocks that
// hold 64 values: each lane takes two segments per iteration and issues both
// loads before using either; there is no branch around any load.  A partial
// last block is done afterwards by the first quad of workgroup 0 with
// guarded loads and stores.
template <bool kBf16, bool kFp4>
__device__ __forceinline__ void quantize_body(const void* __restrict__ x, int64_t n, uint8_t* __restrict__ packed,
                                              float* __restrict__ absmax, const uint2* lut, int blk, int grid) {
  const int64_t nfull = n >> 6;
  const int64_t nseg = nfull * 4;
  const int64_t nbytes = (n + 1) >> 1;
  const int64_t stride = static_cast<int64_t>(grid) * blockDim.x;
  for (int64_t sg0 = static_cast<int64_t>(blk) * blockDim.x + threadIdx.x; sg0 < nseg; sg0 += 2 * stride) {
    const int64_t sg1 = sg0 + stride;
    const int64_t sg1c = sg1 < nseg ? sg1 : sg0;  // clamped: the load is always issued
    float v0[kPerLane], v1[kPerLane];
    load16<kBf16>(x, sg0 * kPerLane, n, v0);
    load16<kBf16>(x, sg1c * kPerLane, n, v1);
    quantize_segment<kFp4>(v0, sg0, packed, absmax, lut, nbytes, true);
    if (sg1 < nseg) quantize_segment<kFp4>(v1, sg1, packed, absmax, lut, nbytes, true);
  }
  if ((n & 63) && blk == 0 && threadIdx.x < 4) {
    const int64_t sg = nseg + threadIdx.x;
    float v[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int64_t e = sg * kPerLane + i;
      if constexpr (kBf16) v[i] = e < n ? bf16_to_f32(static_cast<const uint16_t*>(x)[e]) : 0.0f;
      else v[i] = e < n ? static_cast<const float*>(x)[e] : 0.0f;
    }
    quantize_segment<kFp4>(v, sg, packed, absmax, lut, nbytes, false);
  }
}

template <bool kBf16, bool kFp4>
__global__ __launch_bounds__(256) void k_quantize(const void* __restrict__ x, int64_t n,
                                                  uint8_t* __restrict__ packed,
                                                  float* __restrict__ absmax, QuantLut tab) {
  __shared__ uint2 lut[kLutBuckets];
  fill_lut(lut, tab);
  quantize_body<kBf16, kFp4>(x, n, packed, absmax, lut, blockIdx.x, gridDim.x);
}

// Several tensors in one launch: wg0[j] is the first workgroup of tensor j
// (wg0[count] the total).
struct QuantBatch {
  int count;
  const void* x[kQuantMaxJobs];
  int64_t n[kQuantMaxJobs];
  uint8_t* packed[kQuantMaxJobs];
  float* absmax[kQuantMaxJobs];
  int wg0[kQuantMaxJobs + 1];
};

template <bool kBf16, bool kFp4>
__global__ __launch_bounds__(256) void k_quantize_batch(QuantBatch b, QuantLut tab) {
  __shared__ uint2 lut[kLutBuckets];
  fill_lut(lut, tab);
  const int blk = blockIdx.x;
  const int j = batch_item_of<kQuantMaxJobs>(b.wg0, b.count, blk);
  quantize_body<kBf16, kFp4>(b.x[j], b.n[j], b.packed[j], b.absmax[j], lut, blk - b.wg0[j], b.wg0[j + 1] - b.wg0[j]);
}

}  // namespace

namespace {
// two segments per lane and one pass per lane: a loop would make the next
// loads wait for the previous stores (their registers are reused)
int64_t quantize_grid(int64_t n) {
  const int64_t nseg = (n >> 6) * 4;
  const int64_t want = (nseg + 511) / 512;
  return want < 1 ? 1 : want;
}
}  // namespace

hipError_t launch_quantize(const void* x, int x_bf16, int64_t n, uint8_t* packed, float* absmax,
                           const QuantLut& tab, int fp4, hipStream_t s) {
  const int64_t want = quantize_grid(n);
  if (want > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int grid = static_cast<int>(want);
  if (fp4) {
    if (x_bf16) hipLaunchKernelGGL((k_quantize<true, true>), dim3(grid), dim3(256), 0, s, x, n, packed, absmax, tab);
    else hipLaunchKernelGGL((k_quantize<false, true>), dim3(grid), dim3(256), 0, s, x, n, packed, absmax, tab);
  } else {
    if (x_bf16) hipLaunchKernelGGL((k_quantize<true, false>), dim3(grid), dim3(256), 0, s, x, n, packed, absmax, tab);
    else hipLaunchKernelGGL((k_quantize<false, false>), dim3(grid), dim3(256), 0, s, x, n, packed, absmax, tab);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_batch(const QuantJob* jobs, int count, int x_bf16, const QuantLut& tab, int fp4,
                                 hipStream_t s) {
  if (count < 1 || count > kQuantMaxJobs) return hipErrorInvalidValue;
  QuantBatch b{};
  b.count = count;
  int64_t total = 0;
  for (int j = 0; j < count; ++j) {
    b.x[j] = jobs[j].x;
    b.n[j] = jobs[j].n;
    b.packed[j] = jobs[j].packed;
    b.absmax[j] = jobs[j].absmax;
    b.wg0[j] = static_cast<int>(total);
    total += quantize_grid(jobs[j].n);
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  }
  for (int j = count; j <= kQuantMaxJobs; ++j) b.wg0[j] = static_cast<int>(total);
  const dim3 grid(static_cast<unsigned>(total));
  if (fp4) {
    if (x_bf16) hipLaunchKernelGGL((k_quantize_batch<true, true>), grid, dim3(256), 0, s, b, tab);
    else hipLaunchKernelGGL((k_quantize_batch<false, true>), grid, dim3(256), 0, s, b, tab);
  } else {
    if (x_bf16) hipLaunchKernelGGL((k_quantize_batch<true, false>), grid, dim3(256), 0, s, b, tab);
    else hipLaunchKernelGGL((k_quantize_batch<false, false>), grid, dim3(256), 0, s, b, tab);
  }
  return hipGetLastError();
}

}  // namespace nf4i
