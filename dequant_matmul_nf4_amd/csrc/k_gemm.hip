// Dequantize-into-LDS bf16 matrix-core GEMM with an optional fused LoRA term:
//   y = x . deq(W)^T + s . (x . A^T) . B^T
// (bitsandbytes tool page, "How it works", Step 5: matrix hardware works best
// on 16-bit numbers, so each block is expanded to 16-bit and multiplied; the
// tutorial page, "QLoRA: Fine-Tuning a 4-bit Model": low-rank adapters on the
// frozen 4-bit base, their output multiplied by a scale factor.)
//
// Tiling: a workgroup of 4 waves computes a 256 x 256 tile of y; wave (wm, wn)
// owns the 128 x 128 quarter and runs 4 x 4 v_mfma_f32_32x32x16_bf16 per
// 16-wide k step (256 fp32 accumulators per lane).  A K step covers 64
// columns, i.e. exactly one NF4 block of every weight row, so thread t
// expands row t of the W tile: 64 codes -> level (16-entry LDS table) times
// the block scale, rounded to bf16 (the same value nf4_dequantize writes) ->
// LDS.  The x tile is copied to LDS as is.  LDS holds two stages (x and W,
// 256 rows of 64 bf16 each, rows padded to 144 bytes so the 16-byte fragment
// reads of 16 consecutive rows hit distinct banks); the global loads of step
// k+1 are issued before the MFMAs of step k and written to the other stage
// after them.
//
// LoRA: the low-rank term is folded in as extra K columns,
//   [x | s T_hi | s T_lo] . [deq(W) | B | B]^T  with T = x . A^T,
// where s T is split into two bf16 parts (hi = bf16(sT), lo = bf16(sT - hi))
// by k_lora_prep, so the adapter product keeps about 16 significant bits.
// Those columns (2 r rounded up to a multiple of 64) run as one or two more
// K steps with bf16 operands read directly.
#include "nf4_device.h"

namespace nf4i {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in registers

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kRowBytes = 144;                  // 64 bf16 + 16 bytes of padding
constexpr int kTileBytes = 256 * kRowBytes;     // one operand tile in LDS
constexpr int kStageBytes = 2 * kTileBytes;     // x tile + W tile
constexpr int kLdsBytes = 2 * kStageBytes + 64; // two stages + the level table

__device__ __forceinline__ bf16x8 lds_frag(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const bf16x2 p = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // round to nearest even
  return __builtin_bit_cast(uint32_t, p);
}

struct GemmArgs {
  const uint8_t* packed;
  int64_t rows, cols;    // W [rows][cols]; y has `rows` columns
  Scales sc;
  const uint16_t* x;     // [m][cols]
  int64_t m;
  uint16_t* y;           // [m][rows]
  const uint16_t* u;     // LoRA columns of x: [m][kl] (s T hi | s T lo | 0), or null
  const uint16_t* lb;    // LoRA B [rows][r]
  int r, r_pad, kl;      // rank, rank rounded up to 16, extra K (multiple of 64)
  Codebook cb;
};

// Global loads of one K step into registers: 8 x 16 bytes of the x tile (rows
// t/8 + 32 i, 16-byte piece t%8) and the 32 bytes of codes of W row t.
// Rows past the end of x or W are clamped to the last one: they only feed
// outputs that are never written.
struct StepRegs {
  u32x4 xv[8];
  u32x4 wv[2];
  float am;      // absmax (plain scales)
  int q;         // int8 scale code (double quant)
  float s2;
};

struct StepPtrs {
  const uint8_t* x0;      // x piece 0 of step 0 (bytes)
  int64_t x_stride32;     // bytes between pieces i and i+1 (32 rows)
  int i_max;              // last piece whose row exists; later pieces re-read it
  const uint8_t* w0;      // codes of W row t, step 0
  int64_t blk0;           // block index of W row t, step 0
};

template <bool kDQ>
__device__ __forceinline__ void load_step(StepRegs& st, const StepPtrs& p, const GemmArgs& a, int64_t ks) {
  const uint8_t* xp = p.x0 + ks * (kBK * 2);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ii = i < p.i_max ? i : p.i_max;
    st.xv[i] = *reinterpret_cast<const u32x4*>(xp + ii * p.x_stride32);
  }
  const u32x4* wp = reinterpret_cast<const u32x4*>(p.w0 + ks * (kBK / 2));
  st.wv[0] = wp[0];
  st.wv[1] = wp[1];
  const int64_t blk = p.blk0 + ks;
  if constexpr (kDQ) {
    st.q = a.sc.q[blk];
    st.s2 = a.sc.absmax2[blk >> 8];
  } else {
    st.am = a.sc.absmax[blk];
  }
}

// Writes a step's operands to an LDS stage, expanding the thread's W row.
template <bool kDQ>
__device__ __forceinline__ void store_step(const StepRegs& st, char* stage, const float* lv, float mean) {
  const int t = threadIdx.x;
  char* xs = stage;
  char* wrow = stage + kTileBytes + t * kRowBytes;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4*>(xs + ((t >> 3) + 32 * i) * kRowBytes + (t & 7) * 16) = st.xv[i];
  float sa;
  if constexpr (kDQ) sa = (div127(st.q) * st.s2) + mean;  // a_hat, three roundings
  else sa = st.am;
  const uint32_t q[8] = {st.wv[0][0], st.wv[0][1], st.wv[0][2], st.wv[0][3],
                         st.wv[1][0], st.wv[1][1], st.wv[1][2], st.wv[1][3]};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // byte b of word j holds elements 8j + 2b (high nibble) and 8j + 2b + 1
    const uint32_t hi4 = opaque((q[j] >> 2) & 0x3C3C3C3Cu);
    const uint32_t lo4 = opaque((q[j] << 2) & 0x3C3C3C3Cu);
    uint32_t o[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float e0 = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lv) + __builtin_amdgcn_ubfe(hi4, 8 * b, 8));
      const float e1 = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lv) + __builtin_amdgcn_ubfe(lo4, 8 * b, 8));
      o[b] = bf16_pair(e0 * sa, e1 * sa);
    }
    const u32x4 ov = {o[0], o[1], o[2], o[3]};
    *reinterpret_cast<u32x4*>(wrow + 16 * j) = ov;
  }
}

// One LoRA step (64 extra K columns): x columns from u, W columns [B | B]
// (zero past the rank), loaded and stored directly.
__device__ __forceinline__ void lora_step_to_lds(char* stage, const GemmArgs& a, int64_t m0, int64_t n0, int64_t k0) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = m0 + (t >> 3) + 32 * i;
    const int64_t rc = row < a.m ? row : a.m - 1;
    const u32x4 v = *reinterpret_cast<const u32x4*>(a.u + rc * a.kl + k0 + (t & 7) * 8);
    *reinterpret_cast<u32x4*>(stage + ((t >> 3) + 32 * i) * kRowBytes + (t & 7) * 16) = v;
  }
  const int64_t n = n0 + t;
  const int64_t nc = n < a.rows ? n : a.rows - 1;
  const uint16_t* bp = a.lb + nc * a.r;
  char* wrow = stage + kTileBytes + t * kRowBytes;
  for (int c = 0; c < kBK; ++c) {
    const int64_t col = k0 + c;
    const int64_t j = col < a.r_pad ? col : col - a.r_pad;
    const bool live = col < 2 * a.r_pad && j < a.r;
    reinterpret_cast<uint16_t*>(wrow)[c] = live ? bp[j] : static_cast<uint16_t>(0);
  }
}

__device__ __forceinline__ void mfma_stage(const char* stage, floatx16 (&acc)[4][4], int wm, int wn, int lane) {
  const char* xs = stage;
  const char* ws = stage + kTileBytes;
  const int frag_row = lane & 31;
  const int frag_k = 8 * (lane >> 5);  // bf16 offset of the lane's 8 k values
#pragma unroll
  for (int kk = 0; kk < kBK; kk += 16) {
    bf16x8 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = lds_frag(xs + (wm * 128 + i * 32 + frag_row) * kRowBytes + (kk + frag_k) * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bfr[j] = lds_frag(ws + (wn * 128 + j * 32 + frag_row) * kRowBytes + (kk + frag_k) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
}

template <bool kDQ>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  extern __shared__ __align__(16) char smem[];
  float* lv = reinterpret_cast<float*>(smem + 2 * kStageBytes);
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if (t < 16) lv[t] = a.cb.level[t];

  // tile order: consecutive workgroups of one XCD (dispatch is round-robin
  // over the 8 XCDs) take neighbouring tiles along N, so they share x rows
  const int64_t tiles_n = (a.rows + kBN - 1) / kBN;
  const int64_t tiles = tiles_n * ((a.m + kBM - 1) / kBM);
  int64_t tid = blockIdx.x;
  if (tiles % 8 == 0) tid = (tid % 8) * (tiles / 8) + tid / 8;
  const int64_t m0 = (tid / tiles_n) * kBM;
  const int64_t n0 = (tid % tiles_n) * kBN;

  const float mean = kDQ ? *a.sc.mean : 0.0f;
  const int64_t nk = a.cols / kBK;

  StepPtrs ptr;
  {
    const int64_t xr = m0 + (t >> 3);
    const int64_t xrc = xr < a.m ? xr : a.m - 1;
    ptr.x0 = reinterpret_cast<const uint8_t*>(a.x + xrc * a.cols + (t & 7) * 8);
    ptr.x_stride32 = 32 * a.cols * 2;
    // ragged M: pieces whose row is past the end re-read the last valid one
    // (they only feed outputs that are never stored)
    const int64_t last = xr < a.m ? (a.m - 1 - xr) / 32 : 0;
    ptr.i_max = static_cast<int>(last < 7 ? last : 7);
    const int64_t n = n0 + t;
    const int64_t nc = n < a.rows ? n : a.rows - 1;
    ptr.w0 = a.packed + nc * (a.cols / 2);
    ptr.blk0 = nc * (a.cols / 64);
  }

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  StepRegs st;
  load_step<kDQ>(st, ptr, a, 0);
  __syncthreads();  // level table
  store_step<kDQ>(st, smem, lv, mean);
  __syncthreads();
  for (int64_t ks = 0; ks < nk; ++ks) {
    // the next step's loads are always issued (clamped on the last step) so
    // that no branch separates them from the MFMAs
    const int64_t kn = ks + 1 < nk ? ks + 1 : ks;
    load_step<kDQ>(st, ptr, a, kn);
    mfma_stage(smem + (ks & 1) * kStageBytes, acc, wm, wn, lane);
    store_step<kDQ>(st, smem + ((ks + 1) & 1) * kStageBytes, lv, mean);
    __syncthreads();
  }
  for (int64_t k0 = 0; k0 < a.kl; k0 += kBK) {
    lora_step_to_lds(smem, a, m0, n0, k0);
    __syncthreads();
    mfma_stage(smem, acc, wm, wn, lane);
    __syncthreads();
  }

  // epilogue: lane holds D[(e % 4) + 4 (lane / 32) + 8 (e / 4)][lane % 32] of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 128 + i * 32 + (e & 3) + 4 * (lane >> 5) + 8 * (e >> 2);
        if (row < a.m && col < a.rows)
          a.y[row * a.rows + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[i][j][e]));
      }
    }
  }
}

// u[m][.] = (hi(sT) | lo(sT) | 0) with T = x . A^T in float32, one
// workgroup per row of x: the row's extra columns are zeroed, then each wave
// computes rank entries j (lanes split K, shuffle reduction) and writes
// hi = bf16(s T) at column j and lo = bf16(s T - hi) at column r_pad + j.
__global__ __launch_bounds__(256) void k_lora_prep(const uint16_t* __restrict__ x, const uint16_t* __restrict__ la,
                                                   int64_t cols, int r, int r_pad, int kl, float scale,
                                                   uint16_t* __restrict__ u) {
  const int64_t m = blockIdx.x;
  uint16_t* urow = u + m * kl;
  if (threadIdx.x < kl) urow[threadIdx.x] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* xr = x + m * cols;
  for (int j = wave; j < r; j += 4) {
    const uint16_t* ar = la + static_cast<int64_t>(j) * cols;
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
    s = wave_sum(s) * scale;
    if (lane == 0) {
      const __bf16 hi = static_cast<__bf16>(s);
      const __bf16 lo = static_cast<__bf16>(s - static_cast<float>(hi));
      urow[j] = __builtin_bit_cast(uint16_t, hi);
      urow[r_pad + j] = __builtin_bit_cast(uint16_t, lo);
    }
  }
}

}  // namespace

size_t gemm_lora_cols(int r) {
  if (r <= 0) return 0;
  const int r_pad = (r + 15) / 16 * 16;
  return static_cast<size_t>((2 * r_pad + kBK - 1) / kBK * kBK);
}

hipError_t launch_gemm(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x,
                       int64_t m, uint16_t* y, const uint16_t* lora_a, const uint16_t* lora_b, int r,
                       float lora_scale, uint16_t* u_ws, hipStream_t s) {
  // the two stages take 144 KiB of the 160 KiB LDS; the attribute is per
  // function and idempotent, so setting it on every call is safe across threads
  for (const void* f : {reinterpret_cast<const void*>(k_gemm<true>), reinterpret_cast<const void*>(k_gemm<false>)}) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
  }
  GemmArgs a{};
  a.packed = packed; a.rows = rows; a.cols = cols; a.sc = sc; a.x = x; a.m = m; a.y = y;
  a.cb = codebook();
  if (r > 0) {
    a.r = r;
    a.r_pad = (r + 15) / 16 * 16;
    a.kl = static_cast<int>(gemm_lora_cols(r));
    a.u = u_ws;
    a.lb = lora_b;
    if (m > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_lora_prep, dim3(static_cast<unsigned>(m)), dim3(256), 0, s, x, lora_a, cols, r, a.r_pad,
                       a.kl, lora_scale, u_ws);
  }
  const int64_t tiles = ((rows + kBN - 1) / kBN) * ((m + kBM - 1) / kBM);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (sc.absmax) hipLaunchKernelGGL(k_gemm<false>, dim3(static_cast<unsigned>(tiles)), dim3(256), kLdsBytes, s, a);
  else hipLaunchKernelGGL(k_gemm<true>, dim3(static_cast<unsigned>(tiles)), dim3(256), kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace nf4i
