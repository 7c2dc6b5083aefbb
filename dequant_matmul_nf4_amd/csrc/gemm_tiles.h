// Pieces shared by the two dequantize-and-multiply GEMMs (the forward
// y = x . deq(W)^T and the input gradient dX = dY . deq(W)): the activation
// tile staged in LDS by direct global-to-LDS loads, its MFMA fragments, the
// 8 x 2 tile of v_mfma_f32_32x32x16_bf16 a wave accumulates, and the bf16
// epilogue.  In both kernels a workgroup of 4 waves computes a (32 MI) x 256
// output tile; wave w owns output columns [64 w, 64 w + 64) for all 32 MI
// rows (MI x 2 tiles of 32 x 32), and one reduction step covers 64 indices.
#pragma once

#include "nf4_device.h"

namespace nf4i {
namespace gt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in registers

constexpr int kTileN = 256;      // output columns of a workgroup
constexpr int kStep = 64;        // reduction indices per step
constexpr int kThreads = 256;    // 4 waves
constexpr int kActRowBytes = kStep * 2;  // 128: swizzled activation rows
// A stage holds ROWS rows of 128 bytes.
template <int ROWS>
constexpr int act_stage_bytes() { return ROWS * kActRowBytes; }

__device__ __forceinline__ bf16x8 lds_frag(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const bf16x2 p = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // round to nearest even
  return __builtin_bit_cast(uint32_t, p);
}

// Activation tile of one step (ROWS rows of 64 bf16) by direct global-to-LDS
// loads, P 16-byte pieces per thread: wave w's instruction i (i < P) fills
// tile rows 8 (P w + i) .. + 7 (1 KB); its lane l takes row 8 (P w + i) + l / 8,
// LDS slot l % 8, i.e. the row's 16-byte piece (l % 8) ^ ((row / 2) % 8), so
// that the fragment reads of 16 consecutive rows hit distinct banks.  Rows
// past the end re-read the last valid one (they only feed outputs that are
// never stored).
template <int P>
struct ActPtrs {
  const uint8_t* base;  // the tile's first row (bytes), the same for the whole workgroup
  uint32_t off[P];      // byte offset of the lane's piece for instruction i from base
};

// Global piece index (0..7: reduction indices 8 p .. 8 p + 7 of the step)
// that the lane's instruction i reads.
__device__ __forceinline__ int act_piece(int i, int lane) { return (lane & 7) ^ (((8 * i + (lane >> 3)) >> 1) & 7); }

// act: bf16 [m][ld]; the tile's rows start at m0.  Offsets are 32-bit:
// 256 * ld * 2 < 2^32 (ld < 2^23).
template <int P, int ROWS>
__device__ __forceinline__ ActPtrs<P> make_act_ptrs(const uint16_t* act, int64_t ld, int64_t m, int64_t m0, int wave,
                                                    int lane) {
  ActPtrs<P> p;
  p.base = reinterpret_cast<const uint8_t*>(act + m0 * ld);
  const int last = static_cast<int>(m - 1 - m0 < ROWS - 1 ? m - 1 - m0 : ROWS - 1);  // last tile row that exists
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int tr = 8 * (P * wave + i) + (lane >> 3);  // tile row
    const int rc = tr < last ? tr : last;
    p.off[i] = static_cast<uint32_t>(rc) * static_cast<uint32_t>(ld * 2) + (static_cast<uint32_t>(act_piece(i, lane)) << 4);
  }
  return p;
}

// One direct global-to-LDS load of 16 bytes per lane (kept out of templates:
// the host pass of a template that uses this builtin loses kernel stubs).
__device__ __forceinline__ void dma16(const uint8_t* g, char* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

template <int P>
__device__ __forceinline__ void dma_act(const ActPtrs<P>& p, int64_t ks, char* stage, int wave) {
  const uint8_t* b = p.base + ks * (kStep * 2);
#pragma unroll
  for (int i = 0; i < P; ++i) dma16(b + p.off[i], stage + (P * wave + i) * 1024);
}

// The same loads through a buffer descriptor (buffer_load_dwordx4 ... lds)
// whose base is the step's first byte; each lane adds its offset.  The
// input-gradient kernel measured faster with this form, the forward GEMM
// with the global form above.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

template <int P>
__device__ __forceinline__ void dma_act_buf(const ActPtrs<P>& p, int64_t ks, char* stage, int wave) {
  // word 3 of a raw buffer descriptor on gfx9; no range limit
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.base + ks * (kStep * 2)), static_cast<short>(0), -1, 0x00020000);
#pragma unroll
  for (int i = 0; i < P; ++i) dma16_buf(r, p.off[i], stage + (P * wave + i) * 1024);
}

// Waits for this wave's direct-to-LDS loads (and all other vector memory
// loads); a barrier after it then covers every wave's.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Activation fragments of 16-wide step s: rows 32 i + lane % 32 of the
// swizzled tile, logical piece 4 h + s (h = lane / 32) at slot
// (4 h + s) ^ sw, where sw = ((lane % 32) / 2) % 8 is the same for every i.
// So lane half h holds reduction indices 32 h + 8 s .. + 7 at step s; the
// other operand's fragments must use the same order.
template <int MI>
__device__ __forceinline__ void read_act(const char* xa, int s, uint32_t sw, uint32_t h4, bf16x8 (&f)[MI]) {
  const char* p = xa + (((h4 + s) ^ sw) << 4);
#pragma unroll
  for (int i = 0; i < MI; ++i) f[i] = lds_frag(p + i * 32 * kActRowBytes);
}

// The MFMAs compute transposed output tiles (the weight fragment as the A
// operand, the activation fragment as B), so that each lane ends up holding
// 4 consecutive output columns of one output row.
template <int MI>
__device__ __forceinline__ void mfma16(const bf16x8 (&af)[MI], const bf16x8 (&bf)[2], floatx16 (&acc)[MI][2]) {
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[0], af[i], acc[i][0], 0, 0, 0);
    acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[1], af[i], acc[i][1], 0, 0, 0);
  }
}

template <int MI>
__device__ __forceinline__ void zero_acc(floatx16 (&acc)[MI][2]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
}

// Epilogue into out bf16 [m][ncols]: of each 32 x 32 tile the lane holds
// element e at output column (e % 4) + 4 (lane / 32) + 8 (e / 4) and output
// row lane % 32: four consecutive columns per group of four e, written as one
// 8-byte store when the row holds them all and is 8-byte aligned.
template <int MI>
__device__ __forceinline__ void store_acc(const floatx16 (&acc)[MI][2], uint16_t* out, int64_t m, int64_t ncols,
                                          int64_t m0, int64_t c0, int wave, int lane) {
  const bool vec = (ncols & 3) == 0;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int64_t row = m0 + i * 32 + (lane & 31);
    if (row >= m) continue;
    uint16_t* orow = out + row * ncols;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t col = c0 + wave * 64 + j * 32 + 4 * (lane >> 5) + 8 * g;
        const uint32_t p0 = bf16_pair(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
        const uint32_t p1 = bf16_pair(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        if (vec && col + 3 < ncols) {
          *reinterpret_cast<uint2*>(orow + col) = make_uint2(p0, p1);
        } else {
          const uint16_t v[4] = {static_cast<uint16_t>(p0), static_cast<uint16_t>(p0 >> 16),
                                 static_cast<uint16_t>(p1), static_cast<uint16_t>(p1 >> 16)};
          for (int u = 0; u < 4; ++u)
            if (col + u < ncols) orow[col + u] = v[u];
        }
      }
    }
  }
}

}  // namespace gt
}  // namespace nf4i
