// Dequantization (bitsandbytes tool page, "How it works", Step 5): each code
// is replaced by level[code] times its block's scale, w = fl32(level * a_hat),
// written as float32 or rounded once (nearest even) to bf16.
//
// Layout: each lane expands one 32-bit word of packed codes (8 values) and
// writes 16 bytes (bf16) or 32 bytes (fp32); the code book sits in LDS.
#include "scale_forms.h"

namespace nf4i {
namespace {

template <bool kBf16Out, bool kDQ, bool kF8>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ packed, int64_t n,
                                                    Scales sc, void* __restrict__ out, Codebook cb) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = cb.level[threadIdx.x];
  __syncthreads();
  const float mean = kDQ ? *sc.mean : 0.0f;
  const int64_t noct = (n + 7) >> 3;
  const int64_t nbytes = (n + 1) >> 1;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; o < noct; o += stride) {
    const int64_t byte0 = o * 4;
    uint32_t word;
    if (byte0 + 4 <= nbytes) {
      word = *reinterpret_cast<const uint32_t*>(packed + byte0);
    } else {
      word = 0x77777777u;
      for (int j = 0; j < 4; ++j)
        if (byte0 + j < nbytes)
          word = (word & ~(0xFFu << (8 * j))) | (static_cast<uint32_t>(packed[byte0 + j]) << (8 * j));
    }
    const float a = block_scale_t<kDQ, kF8>(sc, (o * 8) >> 6, mean);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (word >> (8 * (i >> 1) + ((i & 1) ? 0 : 4))) & 0xFu;
      v[i] = lv[c] * a;
    }
    const int64_t e0 = o * 8;
    if constexpr (kBf16Out) {
      uint16_t* dst = static_cast<uint16_t*>(out) + e0;
      if (e0 + 8 <= n) {
        uint4 w4;
        w4.x = pack_bf16x2(v[0], v[1]);
        w4.y = pack_bf16x2(v[2], v[3]);
        w4.z = pack_bf16x2(v[4], v[5]);
        w4.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(dst) = w4;
      } else {
        for (int i = 0; i < 8; ++i)
          if (e0 + i < n) dst[i] = static_cast<uint16_t>(f32_to_bf16(v[i]));
      }
    } else {
      float* dst = static_cast<float*>(out) + e0;
      if (e0 + 8 <= n) {
        reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
      } else {
        for (int i = 0; i < 8; ++i)
          if (e0 + i < n) dst[i] = v[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* packed, int64_t n, Scales sc, void* out, int out_bf16,
                             hipStream_t s) {
  const int64_t noct = (n + 7) >> 3;
  const int64_t want = (noct + 255) / 256;
  const int grid = static_cast<int>(want < 16384 ? want : 16384);
  const Codebook& cb = codebook(sc.fp4);
  const dim3 gd(static_cast<unsigned>(grid)), bd(256);
#define NF4_DEQ(B, D, F) hipLaunchKernelGGL((k_dequantize<B, D, F>), gd, bd, 0, s, packed, n, sc, out, cb)
  if (out_bf16) {
    if (sc.absmax) NF4_DEQ(true, false, false); else if (sc.f8) NF4_DEQ(true, true, true); else NF4_DEQ(true, true, false);
  } else {
    if (sc.absmax) NF4_DEQ(false, false, false); else if (sc.f8) NF4_DEQ(false, true, true); else NF4_DEQ(false, true, false);
  }
#undef NF4_DEQ
  return hipGetLastError();
}

}  // namespace nf4i
