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

// A workgroup barrier for LDS data only: this wave's LDS accesses complete,
// then s_barrier.  __syncthreads() also waits for every global load in flight
// (its workgroup-scope fence), which would drain the rows a kernel requested
// before building its tables.  The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 256 fp16 level pairs (element 2j = high nibble in the low half), one copy
// per lane slot: entry e occupies 64 consecutive words.  Each thread builds the
// pair of entry threadIdx % 256 in registers and writes its share of the 64
// copies with 16-byte stores, starting at a chunk rotated by the entry so that
// 16 consecutive lanes cover every bank.  Ends with a barrier: __syncthreads,
// or with kLdsBarrier the LDS-only barrier above, which leaves the caller's
// global loads in flight.
template <int kThreads, bool kLdsBarrier = false>
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
  if constexpr (kLdsBarrier) lds_barrier();
  else __syncthreads();
}

struct RowItem {
  uint4 w[2];    // piece j: 16 bytes of codes at segment offset 1024 j + 16 lane
  float am;      // absmax of the block this lane scales (plain scales)
  int q;         // its second-level scale code (double quant)
  float s2;      // its second-level scale
};

// The lane's fixed offsets within any row: piece j's code bytes
// (blk[j] * 32 + 16 * half) and the block whose scale the lane applies.
// Lanes 2k and 2k + 1 hold the two halves of the same two blocks (k and
// 32 + k of the segment): after their partial sums are added pairwise, lane
// 2k scales block k and lane 2k + 1 block 32 + k, so each lane loads and
// applies one block scale per row.
struct LaneOffs {
  uint32_t code[2];
  uint32_t sblk;
};

// The lane's offsets for a segment of seg_blocks blocks starting at block
// seg0 of the row, seg_end of them present: piece j covers half (lane & 1)
// of block 32 j + lane / 2 (clamped to the last present block, flagged off).
__device__ __forceinline__ void make_lane_offs(int seg0, int seg_end, int lane, LaneOffs& lo, bool (&on)[2],
                                               int (&blk)[2]) {
  const int half = lane & 1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int bj = 32 * j + (lane >> 1);
    on[j] = bj < seg_end;
    blk[j] = seg0 + (on[j] ? bj : seg_end - 1);
    lo.code[j] = static_cast<uint32_t>(blk[j]) * 32u + 16u * static_cast<uint32_t>(half);
  }
  const uint32_t b0 = opaque(static_cast<uint32_t>(blk[0])), b1 = opaque(static_cast<uint32_t>(blk[1]));
  lo.sblk = half ? b1 : b0;  // a select, not an index: blk stays in registers
}

// 16 bytes of weight codes, which a decode GEMV reads exactly once: a
// non-temporal load, so that the stream does not push out of the caches
// what every wave re-reads (x, the scale tables).  Measured on the 70B-shaped
// layer in one launch: 93.5 -> 88.5 us.
__device__ __forceinline__ uint4 load_codes16(const uint8_t* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Loads of one row.  The row's first block row_blk0 = row * nblk is
// wave-uniform, so each address is a uniform base plus the lane's 32-bit
// offset (no 64-bit arithmetic per lane); the scale group of the lane's block
// is (row_blk0 % 256 + sblk) / 256 groups past that of the row's first block.
template <bool kDQ>
__device__ __forceinline__ void row_load(RowItem& it, const uint8_t* packed, int64_t row_blk0, const LaneOffs& lo,
                                         Scales sc) {
  const uint8_t* crow = packed + row_blk0 * 32;
  const uint32_t g0 = static_cast<uint32_t>(row_blk0 & 255);
#pragma unroll
  for (int j = 0; j < 2; ++j) it.w[j] = load_codes16(crow + lo.code[j]);
  if constexpr (kDQ) {
    it.q = (sc.q + row_blk0)[lo.sblk];
    it.s2 = (sc.absmax2 + (row_blk0 >> 8))[(g0 + lo.sblk) >> 8];
  } else {
    it.am = (sc.absmax + row_blk0)[lo.sblk];
  }
}

// The first factor of a_hat for every second-level code, in LDS: q / 127
// for int8 codes (div127, the correctly rounded quotient), the E4M3 ratio
// table for float8 codes.  Indexed by the code's low byte.
template <bool kF8>
__device__ __forceinline__ void fill_ratio_table(float* rtab, int nthreads) {
  for (int i = threadIdx.x; i < 256; i += nthreads)
    rtab[i] = kF8 ? kE4m3Ratio.v[i] : div127(static_cast<int>(static_cast<int8_t>(i)));
}

__device__ __forceinline__ float pair_sum(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true)) + v;  // lane ^ 1
}

// The per-lane factors row_dot applies: the x scale of the block the lane
// scales (piece lane & 1), zero when that block lies past the segment's end
// (its loads were clamped).  Selected once with the values held in registers
// (opaque), so the choice stays a select and the small arrays are never
// indexed by a lane-dependent value.
template <int MC>
__device__ __forceinline__ void lane_x_scales(const float (&xinv)[MC][2], const bool (&on)[2], float (&xsel)[MC]) {
  const bool odd = (threadIdx.x & 1) != 0;
  const bool live = odd ? on[1] : on[0];
#pragma unroll
  for (int c = 0; c < MC; ++c) {
    const float x0 = __uint_as_float(opaque(__float_as_uint(xinv[c][0])));
    const float x1 = __uint_as_float(opaque(__float_as_uint(xinv[c][1])));
    xsel[c] = live ? (odd ? x1 : x0) : 0.0f;
  }
}

// Products of one row item with MC rows of x (the lookups are shared).  Per
// piece the lane forms sum_k level[code_k] * xh[c][j][k]; the pair of lanes
// holding the two halves of a block adds its sums, and each lane scales the
// block it owns (piece lane & 1):
//   out[c] = pairsum_(lane & 1) * (a_hat * xsel[c]).
template <int MC, bool kDQ>
__device__ __forceinline__ void row_dot(const RowItem& it, const uint32_t (&xh)[MC][2][16], const char* tab,
                                        uint32_t slot, float mean, const float* rtab, const float (&xsel)[MC],
                                        float (&out)[MC]) {
  float sa[MC], sb[MC];  // pair sums of piece 0 and piece 1
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t q[4] = {it.w[j].x, it.w[j].y, it.w[j].z, it.w[j].w};
    uint32_t e[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t addr = __builtin_amdgcn_perm(q[u >> 2], slot, 0x0C0C0000u | ((4u + (u & 3)) << 8));
      e[u] = *reinterpret_cast<const uint32_t*>(tab + addr);
    }
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int u = 0; u < 16; u += 2) {
        s0 = dot2h(e[u], xh[c][j][u], s0);
        s1 = dot2h(e[u + 1], xh[c][j][u + 1], s1);
      }
      if (j == 0) sa[c] = pair_sum(s0 + s1);
      else sb[c] = pair_sum(s0 + s1);
    }
  }
  const bool odd = (threadIdx.x & 1) != 0;
  float a;
  if constexpr (kDQ) a = (rtab[it.q & 0xFF] * it.s2) + mean;  // a_hat
  else a = it.am;
#pragma unroll
  for (int c = 0; c < MC; ++c) out[c] = (odd ? sb[c] : sa[c]) * (a * xsel[c]);
}

// 32 values of x (16 bf16 pairs, half of a 64-value block; the other half is
// held by the neighbouring lane, lane ^ 1) to fp16 pairs scaled by 2^k, k
// chosen so that the largest |x| of the whole block lies in [2^14, 2^15);
// xinv = 2^-k, the same in both lanes.  Must be called by all lanes of the
// wave together.
__device__ __forceinline__ void x_half_block_to_half(const uint4 (&xv)[4], uint32_t (&xh)[16], float& xinv) {
  uint32_t xw[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) { xw[4 * i] = xv[i].x; xw[4 * i + 1] = xv[i].y; xw[4 * i + 2] = xv[i].z; xw[4 * i + 3] = xv[i].w; }
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = max(mx, max(xw[i] & 0x7FFF0000u, (xw[i] << 16) & 0x7FFF0000u));
  mx = max(mx, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(mx), 0xB1, 0xF, 0xF, true)));
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

// The same conversion for a whole 64-value block held by one thread (the
// batched kernel's stage): identical scale and fp16 values.
__device__ __forceinline__ void x_block_to_half(const uint4 (&xv)[8], uint32_t (&xh)[32], float& xinv) {
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) mx = max(mx, max(w[t] & 0x7FFF0000u, (w[t] << 16) & 0x7FFF0000u));
  }
  int k = 14 - (static_cast<int>(mx >> 23) - 127);
  k = k < -126 ? -126 : (k > 126 ? 126 : k);
  const float sc2 = __uint_as_float(static_cast<uint32_t>(127 + k) << 23);
  xinv = __uint_as_float(static_cast<uint32_t>(127 - k) << 23);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float lo = __uint_as_float(w[t] << 16) * sc2;
      const float hi = __uint_as_float(w[t] & 0xFFFF0000u) * sc2;
      xh[4 * i + t] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
  }
}

}  // namespace
}  // namespace nf4i
