// Device pieces of the streaming decode GEMV shared by the single-weight
// kernel (k_gemv.hip) and the kernel that takes several weights in one launch
// (k_gemv_batch.hip): the fp16 level-pair table, the per-row loads, the
// per-row dot product and the power-of-two scaling of x to fp16.
#pragma once

#include "nf4_device.h"

namespace nf4i {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// Sum over the wave; the total is exact in lane 63 only.
__device__ __forceinline__ float wave_sum_to_last(float v) {
  v = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true)) + v;   // quad [1,0,3,2]
  v = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true)) + v;   // quad [2,3,0,1]
  v = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, true)) + v;  // row_ror:4
  v = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true)) + v;  // row_ror:8
  // rows 1 and 3 add the total of the row below, then rows 2 and 3 that of rows 0-1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

// 256 fp16 level pairs (element 2j = high nibble in the low half), one copy
// per lane slot: entry e occupies 64 consecutive words.  Each thread builds the
// pair of entry threadIdx % 256 in registers and writes its share of the 64
// copies with 16-byte stores, starting at a chunk rotated by the entry so that
// 16 consecutive lanes cover every bank.  Ends with a barrier.
template <int kThreads>
__device__ __forceinline__ void fill_half_table(uint32_t* tab, const Codebook& cb) {
  static_assert(kThreads % 256 == 0 && kThreads <= 1024, "whole entries per pass");
  constexpr int kParts = kThreads / 256;
  const int e = threadIdx.x & 255;
  const int p = threadIdx.x >> 8;
  float l0 = cb.level[0], l1 = cb.level[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    l0 = ((e >> 4) == i) ? cb.level[i] : l0;
    l1 = ((e & 15) == i) ? cb.level[i] : l1;
  }
  const half2_t h = {static_cast<_Float16>(l0), static_cast<_Float16>(l1)};  // round to nearest even
  const uint32_t v = __builtin_bit_cast(uint32_t, h);
  const uint4 v4 = {v, v, v, v};
#pragma unroll
  for (int j = 0; j < 16 / kParts; ++j) {
    const int c = (j * kParts + p + e) & 15;
    *reinterpret_cast<uint4*>(tab + e * 64 + 4 * c) = v4;
  }
  __syncthreads();
}

struct RowItem {
  uint4 w[2];    // piece j: 16 bytes of codes at segment offset 1024 j + 16 lane
  float am[2];   // absmax of each piece's block (plain scales)
  int q[2];      // second-level scale codes (double quant)
  float s2[2];   // second-level scales
};

// The lane's fixed offsets within any row: piece j's code bytes
// (blk[j] * 32 + 16 * half) and its block (blk[j]).
struct LaneOffs {
  uint32_t code[2];
  uint32_t blk[2];
};

// Loads of one row.  The row's first block row_blk0 = row * nblk is
// wave-uniform, so each address is a uniform base plus the lane's 32-bit
// offset (no 64-bit arithmetic per lane); the scale group of piece j is
// (row_blk0 % 256 + blk[j]) / 256 groups past that of the row's first block.
template <bool kDQ>
__device__ __forceinline__ void row_load(RowItem& it, const uint8_t* packed, int64_t row_blk0, const LaneOffs& lo,
                                         Scales sc) {
  const uint8_t* crow = packed + row_blk0 * 32;
  const uint32_t g0 = static_cast<uint32_t>(row_blk0 & 255);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    it.w[j] = *reinterpret_cast<const uint4*>(crow + lo.code[j]);
    if constexpr (kDQ) {
      it.q[j] = (sc.q + row_blk0)[lo.blk[j]];
      it.s2[j] = (sc.absmax2 + (row_blk0 >> 8))[(g0 + lo.blk[j]) >> 8];
    } else {
      it.am[j] = (sc.absmax + row_blk0)[lo.blk[j]];
    }
  }
}

// First factor of a_hat: q / 127 for int8 codes, the E4M3 ratio table (copied
// to LDS) for float8 codes.
template <bool kF8>
__device__ __forceinline__ float row_ratio(int q, const float* rtab) {
  if constexpr (kF8) return rtab[q & 0xFF];
  else return div127(q);
}

// Products of one row item with MC rows of x (the lookups are shared):
// out[c] = sum_j on[j] ? a_hat_j * xinv[c][j] * sum_k level[code_k] * xh[c][j][k] : 0.
template <int MC, bool kDQ, bool kF8>
__device__ __forceinline__ void row_dot(const RowItem& it, const uint32_t (&xh)[MC][2][16], const char* tab,
                                        uint32_t slot, float mean, const float* rtab, const float (&xinv)[MC][2],
                                        const bool (&on)[2], float (&out)[MC]) {
#pragma unroll
  for (int c = 0; c < MC; ++c) out[c] = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t q[4] = {it.w[j].x, it.w[j].y, it.w[j].z, it.w[j].w};
    uint32_t e[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t addr = __builtin_amdgcn_perm(q[u >> 2], slot, 0x0C0C0000u | ((4u + (u & 3)) << 8));
      e[u] = *reinterpret_cast<const uint32_t*>(tab + addr);
    }
    float a;
    if constexpr (kDQ) a = (row_ratio<kF8>(it.q[j], rtab) * it.s2[j]) + mean;  // a_hat
    else a = it.am[j];
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int u = 0; u < 16; u += 2) {
        s0 = dot2h(e[u], xh[c][j][u], s0);
        s1 = dot2h(e[u + 1], xh[c][j][u + 1], s1);
      }
      const float v = (s0 + s1) * (a * xinv[c][j]);
      out[c] += on[j] ? v : 0.0f;
    }
  }
}

// 32 values of x (16 bf16 pairs) to fp16 pairs scaled by 2^k, k chosen so
// that the largest |x| lies in [2^14, 2^15); xinv = 2^-k.
__device__ __forceinline__ void x_piece_to_half(const uint4 (&xv)[4], uint32_t (&xh)[16], float& xinv) {
  uint32_t xw[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) { xw[4 * i] = xv[i].x; xw[4 * i + 1] = xv[i].y; xw[4 * i + 2] = xv[i].z; xw[4 * i + 3] = xv[i].w; }
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = max(mx, max(xw[i] & 0x7FFF0000u, (xw[i] << 16) & 0x7FFF0000u));
  int k = 14 - (static_cast<int>(mx >> 23) - 127);
  k = k < -126 ? -126 : (k > 126 ? 126 : k);
  const float sc2 = __uint_as_float(static_cast<uint32_t>(127 + k) << 23);
  xinv = __uint_as_float(static_cast<uint32_t>(127 - k) << 23);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float lo = __uint_as_float(xw[i] << 16) * sc2;         // exact: a power of two
    const float hi = __uint_as_float(xw[i] & 0xFFFF0000u) * sc2;
    xh[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
}

}  // namespace
}  // namespace nf4i
