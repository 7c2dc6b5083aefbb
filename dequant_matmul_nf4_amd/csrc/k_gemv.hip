// Fused dequantize-and-multiply for decode, y[m][r] = sum_k x[m][k] * w[r][k]
// (bitsandbytes tool page, "How it works", Step 5: a block is expanded with
// its scale and code book and multiplied; the expanded copy never leaves the
// registers).
//
// Layout: a workgroup of 4 waves owns 16 consecutive rows, 4 per wave.  Lane l
// of a wave walks the row in 16-byte chunks l, l+64, ... (32 codes, half of a
// 64-block).  Within a chunk the level values are summed against x in float32
// and the block scale is applied once per chunk; the per-lane partial sums are
// reduced across the wave with shuffles at the end.
#include "nf4_device.h"

namespace nf4i {
namespace {

constexpr int kRowsPerWave = 4;
constexpr int kRowsPerGroup = 4 * kRowsPerWave;

__device__ __forceinline__ void load_x32(const uint16_t* __restrict__ xrow, int64_t k0, float xv[32]) {
  const uint4* p = reinterpret_cast<const uint4*>(xrow + k0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = p[i];
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[8 * i + 2 * j] = __uint_as_float(q[j] << 16);
      xv[8 * i + 2 * j + 1] = __uint_as_float(q[j] & 0xFFFF0000u);
    }
  }
}

// Sum over the 32 codes of a 16-byte chunk of level[code] * x.
__device__ __forceinline__ float chunk_dot(const uint4 w, const float xv[32], const float* lv) {
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t byte = (q[i] >> (8 * b)) & 0xFFu;
      s = fmaf(lv[byte >> 4], xv[8 * i + 2 * b], s);
      s = fmaf(lv[byte & 0xFu], xv[8 * i + 2 * b + 1], s);
    }
  }
  return s;
}

template <int kMG, bool kBf16Out>
__global__ __launch_bounds__(256) void k_gemv(const uint8_t* __restrict__ packed, int64_t rows,
                                              int64_t cols, Scales sc, const uint16_t* __restrict__ x,
                                              int m_total, void* __restrict__ y, Codebook cb) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = cb.level[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowsPerGroup + wave * kRowsPerWave;
  const float mean = sc.absmax ? 0.0f : *sc.mean;
  const int64_t nchunk = cols / 32;
  const int64_t row_bytes = cols / 2;
  const int64_t row_blocks = cols / 64;

  for (int m0 = 0; m0 < m_total; m0 += kMG) {
    float acc[kRowsPerWave][kMG];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
      for (int j = 0; j < kMG; ++j) acc[r][j] = 0.0f;

    for (int64_t c = lane; c < nchunk; c += 64) {
      uint4 w[kRowsPerWave];
      float a[kRowsPerWave];
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        const int64_t row = r0 + r;
        if (row < rows) {
          w[r] = *reinterpret_cast<const uint4*>(packed + row * row_bytes + c * 16);
          a[r] = block_scale(sc, row * row_blocks + (c >> 1), mean);
        } else {
          w[r] = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
          a[r] = 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < kMG; ++j) {
        if (m0 + j >= m_total) break;
        float xv[32];
        load_x32(x + static_cast<int64_t>(m0 + j) * cols, c * 32, xv);
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) acc[r][j] = fmaf(chunk_dot(w[r], xv, lv), a[r], acc[r][j]);
      }
    }

#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
#pragma unroll
      for (int j = 0; j < kMG; ++j) {
        const float s = wave_sum(acc[r][j]);
        const int64_t row = r0 + r;
        if (lane == 0 && row < rows && m0 + j < m_total) {
          const int64_t idx = static_cast<int64_t>(m0 + j) * rows + row;
          if constexpr (kBf16Out) static_cast<uint16_t*>(y)[idx] = static_cast<uint16_t>(f32_to_bf16(s));
          else static_cast<float*>(y)[idx] = s;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- m == 1
//
// Decode GEMV.  Each level is split into two bf16 parts, hi = bf16(level) and
// lo = bf16(level - hi) (together within 2^-17 of the float32 level), and a
// byte of packed codes (two elements) indexes a table of (hi pair, lo pair)
// words.  x stays in its bf16 pairs, so a pair of weights costs one
// v_perm_b32 (table address), one 8-byte LDS read and two v_dot2c_f32_bf16.
// The table is replicated 32 times with lane slot c at bytes [8c, 8c + 8) of
// every 256-byte row, so the 16 lanes served together always hit distinct
// banks: address = (byte << 8) | (8 * (lane % 32)), a single byte permute.
//
// Work: a wave owns R consecutive rows (a row group) and walks their 64-blocks
// in segments of 64 (lane l takes block l of a segment); row groups are dealt
// round-robin to the persistent waves, and each wave prefetches the next
// (row group, segment) item into a second register set while it computes the
// current one.

constexpr int kTabSlots = 32;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int R>
struct GemvItem {
  uint4 w[R][2];   // 32 bytes of packed codes per row
  float am[R];     // absmax (plain scales)
  int q[R];        // int8 scale code (double quant), kept as loaded
  float s2[R];     // second-level scale (double quant)
  uint32_t x[32];  // bf16 pairs of x for the lane's block (several segments only)
};

__device__ __forceinline__ void load_x_block(uint32_t xr[32], const uint16_t* __restrict__ x, int64_t bc) {
  const uint4* xp = reinterpret_cast<const uint4*>(x + bc * 64);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 t = xp[i];
    xr[4 * i] = t.x; xr[4 * i + 1] = t.y; xr[4 * i + 2] = t.z; xr[4 * i + 3] = t.w;
  }
}

// Builds the replicated table in two phases so that every LDS write of a wave
// goes to consecutive addresses (a direct write of entry e to all its slots
// would put the lanes of a wave 256 bytes apart, all in one bank): the 256
// distinct entries first, then the copies.  Ends with a barrier.
__device__ __forceinline__ void fill_pair_table(uint2* tab, uint2* base, const Codebook& cb) {
  if (threadIdx.x < 256) {
    // entry for byte e: element 2j takes level[e >> 4], element 2j + 1 level[e & 15]
    // (levels picked with static indices so they stay in scalar registers)
    const int e = threadIdx.x;
    float l0 = cb.level[0], l1 = cb.level[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      l0 = ((e >> 4) == i) ? cb.level[i] : l0;
      l1 = ((e & 15) == i) ? cb.level[i] : l1;
    }
    const uint32_t h0 = f32_to_bf16(l0), h1 = f32_to_bf16(l1);
    const uint32_t r0 = f32_to_bf16(l0 - bf16_to_f32(h0)), r1 = f32_to_bf16(l1 - bf16_to_f32(h1));
    base[e] = make_uint2(h0 | (h1 << 16), r0 | (r1 << 16));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 256 * kTabSlots; i += blockDim.x) tab[i] = base[i / kTabSlots];
  __syncthreads();
}

// Issues the loads of one (row group, segment) item.  Indices are clamped so
// that no branch separates the loads (a branch would make the compiler wait
// for them at the merge point); the raw scale inputs are kept and turned into
// the block scale only when the item is consumed.
template <int R, bool kDQ, bool kLoadX>
__device__ __forceinline__ void gemv_load(GemvItem<R>& it, const uint8_t* __restrict__ packed, int64_t rows,
                                          int64_t nblk, int64_t row0, int64_t b, Scales sc,
                                          const uint16_t* __restrict__ x) {
  const int64_t bc = b < nblk ? b : nblk - 1;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = (row0 + r < rows) ? row0 + r : rows - 1;
    const uint4* p = reinterpret_cast<const uint4*>(packed + row * (nblk * 32) + bc * 32);
    it.w[r][0] = p[0];
    it.w[r][1] = p[1];
    const int64_t blk = row * nblk + bc;
    if constexpr (kDQ) {
      it.q[r] = sc.q[blk];
      it.s2[r] = sc.absmax2[blk >> 8];
    } else {
      it.am[r] = sc.absmax[blk];
    }
  }
  if constexpr (kLoadX) load_x_block(it.x, x, bc);
}

template <int R, bool kDQ>
__device__ __forceinline__ void gemv_compute(const GemvItem<R>& it, const uint32_t* __restrict__ xr, bool active,
                                             const char* tab, uint32_t slot, float mean, float acc[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t q[8] = {it.w[r][0].x, it.w[r][0].y, it.w[r][0].z, it.w[r][0].w,
                           it.w[r][1].x, it.w[r][1].y, it.w[r][1].z, it.w[r][1].w};
    float sh = 0.0f, sl = 0.0f;
    // 8 lookups in flight before their products are taken
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      uint2 e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t addr = __builtin_amdgcn_perm(q[j + (u >> 2)], slot, 0x0C0C0000u | ((4u + (u & 3)) << 8));
        e[u] = *reinterpret_cast<const uint2*>(tab + addr);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sh = dot2(e[u].x, xr[4 * j + u], sh);
        sl = dot2(e[u].y, xr[4 * j + u], sl);
      }
    }
    float a;
    if constexpr (kDQ) a = (div127(it.q[r]) * it.s2[r]) + mean;  // a_hat
    else a = it.am[r];
    acc[r] = fmaf(sh + sl, active ? a : 0.0f, acc[r]);
  }
}

// Work split: wave w owns the contiguous rows [w per, (w+1) per) (at most 64;
// the grid grows beyond one workgroup per CU otherwise) and takes them in
// batches of R rows.  For each batch it walks the row segments (64 blocks,
// lane l on block l); each (batch, segment) step issues the R x 32-byte code
// loads and the 128-byte x load of every lane at once, then consumes them.
// Sixteen waves per CU keep enough of these steps in flight to cover the
// memory latency.  The first step's loads go out before the table is built.
// Finished rows are parked in a register (lane k holds row k) and stored
// once at the end.
template <int R, bool kDQ, bool kBf16Out>
__global__ __launch_bounds__(1024) void k_gemv_m1(const uint8_t* __restrict__ packed, int64_t rows,
                                                  int64_t cols, Scales sc, const uint16_t* __restrict__ x,
                                                  void* __restrict__ y, Codebook cb) {
  __shared__ uint2 tab[256 * kTabSlots];
  __shared__ uint2 tab_base[256];
  const char* smem = reinterpret_cast<const char*>(tab);
  const int lane = threadIdx.x & 63;
  const uint32_t slot = static_cast<uint32_t>(lane & 31) << 3;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
  const int64_t per = (rows + nwaves - 1) / nwaves;
  const int64_t r_begin = wave * per;
  const int64_t r_end = (r_begin + per < rows) ? r_begin + per : rows;
  const int64_t nblk = cols / 64;
  const int64_t nseg = (nblk + 63) / 64;

  GemvItem<R> it;
  // first step's loads, then the table
  gemv_load<R, kDQ, true>(it, packed, rows, nblk, r_begin < rows ? r_begin : rows - 1, lane, sc, x);
  fill_pair_table(tab, tab_base, cb);
  if (r_begin >= r_end) return;
  const float mean = kDQ ? *sc.mean : 0.0f;

  float res = 0.0f;  // lane k <-> row r_begin + k
  int nres = 0;
  for (int64_t rb = r_begin; rb < r_end; rb += R) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    for (int64_t sg = 0; sg < nseg; ++sg) {
      if (rb != r_begin || sg != 0) gemv_load<R, kDQ, true>(it, packed, rows, nblk, rb, sg * 64 + lane, sc, x);
      gemv_compute<R, kDQ>(it, it.x, sg * 64 + lane < nblk, smem, slot, mean, acc);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float s = wave_sum(acc[r]);
      res = (lane == nres + r) ? s : res;
    }
    nres += R;
  }
  const int64_t row = r_begin + lane;
  if (lane < nres && row < r_end) {
    if constexpr (kBf16Out) static_cast<uint16_t*>(y)[row] = static_cast<uint16_t>(f32_to_bf16(res));
    else static_cast<float*>(y)[row] = res;
  }
}

// Variant with x staged in LDS (cols <= kXLdsMaxCols): the workgroup copies
// x once into LDS, block c's 64 values at byte c * 144 (16 bytes of padding
// per block keep the lanes' 16-byte reads in distinct banks), next to the
// pair table.  The global loads of a step are then only the R rows' codes and
// scales, and each wave prefetches the next step into a second register set
// while it computes the current one.
constexpr int64_t kXLdsMaxCols = 32768;
constexpr int kXStride = 144;

__device__ __forceinline__ void lds_x_block(uint32_t xr[32], const char* xs, int64_t b) {
  const char* p = xs + b * kXStride;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 t = *reinterpret_cast<const uint4*>(p + 16 * i);
    xr[4 * i] = t.x; xr[4 * i + 1] = t.y; xr[4 * i + 2] = t.z; xr[4 * i + 3] = t.w;
  }
}

template <int R, bool kDQ, bool kBf16Out>
__global__ __launch_bounds__(1024) void k_gemv_m1_xl(const uint8_t* __restrict__ packed, int64_t rows,
                                                     int64_t cols, Scales sc, const uint16_t* __restrict__ x,
                                                     void* __restrict__ y, Codebook cb) {
  __shared__ uint2 tab[256 * kTabSlots];
  __shared__ uint2 tab_base[256];
  __shared__ __align__(16) char xs[(kXLdsMaxCols / 64) * kXStride + 16];  // + a dummy slot
  const char* smem = reinterpret_cast<const char*>(tab);
  const int lane = threadIdx.x & 63;
  const uint32_t slot = static_cast<uint32_t>(lane & 31) << 3;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
  const int64_t per = (rows + nwaves - 1) / nwaves;
  const int64_t r_begin = wave * per;
  const int64_t r_end = (r_begin + per < rows) ? r_begin + per : rows;
  const int64_t nblk = cols / 64;
  const int64_t nseg = (nblk + 63) / 64;
  const int64_t nbatch = r_end > r_begin ? (r_end - r_begin + R - 1) / R : 0;
  const int64_t n_items = nbatch * nseg;
  const int64_t last = n_items > 0 ? n_items - 1 : 0;
  auto row0_of = [&](int64_t t) { const int64_t r0 = r_begin + (t / nseg) * R; return r0 < rows ? r0 : rows - 1; };
  auto blk_of = [&](int64_t t) { return (t % nseg) * 64 + lane; };

  GemvItem<R> A, B;
  // Prologue: x loads (at most 4 pieces of 16 bytes per thread with 1024
  // threads) and the first step's loads are issued, then x and the pair
  // table go to LDS.
  constexpr int kXPieces = static_cast<int>(kXLdsMaxCols / 8 / 1024);
  const int64_t npieces = nblk * 8;
  uint4 xv[kXPieces];
#pragma unroll
  for (int u = 0; u < kXPieces; ++u) {
    const int64_t p = threadIdx.x + static_cast<int64_t>(u) * blockDim.x;
    xv[u] = reinterpret_cast<const uint4*>(x)[p < npieces ? p : npieces - 1];
  }
  gemv_load<R, kDQ, false>(A, packed, rows, nblk, row0_of(0), blk_of(0), sc, x);
#pragma unroll
  for (int u = 0; u < kXPieces; ++u) {
    // unconditional store (pieces past the end go to the dummy slot)
    const int64_t p = threadIdx.x + static_cast<int64_t>(u) * blockDim.x;
    const int64_t off = p < npieces ? (p >> 3) * kXStride + (p & 7) * 16 : (kXLdsMaxCols / 64) * kXStride;
    *reinterpret_cast<uint4*>(xs + off) = xv[u];
  }
  fill_pair_table(tab, tab_base, cb);  // ends with a barrier
  if (n_items == 0) return;
  const float mean = kDQ ? *sc.mean : 0.0f;

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  float res = 0.0f;  // lane k <-> row r_begin + k
  int nres = 0;
  uint32_t xr[32];
  auto step = [&](const GemvItem<R>& it, int64_t t) {
    const int64_t b = blk_of(t);
    const bool active = b < nblk;
    lds_x_block(xr, xs, active ? b : 0);
    gemv_compute<R, kDQ>(it, xr, active, smem, slot, mean, acc);
    if ((t % nseg) == nseg - 1) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float sum = wave_sum(acc[r]);
        res = (lane == nres + r) ? sum : res;
        acc[r] = 0.0f;
      }
      nres += R;
    }
  };
  for (int64_t t = 0; t < n_items; t += 2) {
    const int64_t t1 = (t + 1 < last) ? t + 1 : last;
    gemv_load<R, kDQ, false>(B, packed, rows, nblk, row0_of(t1), blk_of(t1), sc, x);
    step(A, t);
    if (t + 1 >= n_items) break;
    const int64_t t2 = (t + 2 < last) ? t + 2 : last;
    gemv_load<R, kDQ, false>(A, packed, rows, nblk, row0_of(t2), blk_of(t2), sc, x);
    step(B, t + 1);
  }
  const int64_t row = r_begin + lane;
  if (lane < nres && row < r_end) {
    if constexpr (kBf16Out) static_cast<uint16_t*>(y)[row] = static_cast<uint16_t>(f32_to_bf16(res));
    else static_cast<float*>(y)[row] = res;
  }
}

template <int R, bool kDQ>
void launch_m1_xl(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x, void* y,
                  int y_bf16, hipStream_t s) {
  const int64_t cus = device_cus();
  const int64_t wpg = 16;  // 1024 threads: the x copy assumes it
  const int64_t need = (rows + wpg * 64 - 1) / (wpg * 64);
  const int64_t want = (rows + wpg * R - 1) / (wpg * R);
  int64_t g = want < cus ? want : cus;
  if (g < need) g = need;
  if (g < 1) g = 1;
  if (g > 0x7FFFFFFF) return;
  const Codebook& cb = codebook();
  const dim3 gd(static_cast<unsigned>(g)), b(static_cast<unsigned>(64 * wpg));
  if (y_bf16) hipLaunchKernelGGL((k_gemv_m1_xl<R, kDQ, true>), gd, b, 0, s, packed, rows, cols, sc, x, y, cb);
  else hipLaunchKernelGGL((k_gemv_m1_xl<R, kDQ, false>), gd, b, 0, s, packed, rows, cols, sc, x, y, cb);
}

template <int R, bool kDQ>
void launch_m1(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x, void* y,
               int y_bf16, int waves_per_group, hipStream_t s) {
  // one workgroup per CU (one 64 KiB table per CU); a wave takes at most 64
  // rows, so very tall matrices get more workgroups
  const int64_t cus = device_cus();
  const int64_t wpg = waves_per_group;
  const int64_t need = (rows + wpg * 64 - 1) / (wpg * 64);
  const int64_t want = (rows + wpg * R - 1) / (wpg * R);
  int64_t g = want < cus ? want : cus;
  if (g < need) g = need;
  if (g < 1) g = 1;
  if (g > 0x7FFFFFFF) return;
  const Codebook& cb = codebook();
  const dim3 gd(static_cast<unsigned>(g)), b(static_cast<unsigned>(64 * wpg));
  if (y_bf16) hipLaunchKernelGGL((k_gemv_m1<R, kDQ, true>), gd, b, 0, s, packed, rows, cols, sc, x, y, cb);
  else hipLaunchKernelGGL((k_gemv_m1<R, kDQ, false>), gd, b, 0, s, packed, rows, cols, sc, x, y, cb);
}

}  // namespace

hipError_t launch_gemv(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x,
                       int64_t m, void* y, int y_bf16, hipStream_t s) {
  const int64_t groups = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(groups));
  const Codebook& cb = codebook();
  const int mm = static_cast<int>(m);
  if (m == 1) {
    // rows per batch and waves per workgroup from the shape, so that every CU
    // gets work: up to 16 waves per CU, then 2 and 4 rows per batch
    const int64_t cus = device_cus();
    const int64_t per_cu = (rows + cus - 1) / cus;
    if (cols <= kXLdsMaxCols && per_cu > 16) {
      if (per_cu <= 32) {
        if (sc.absmax) launch_m1_xl<1, false>(packed, rows, cols, sc, x, y, y_bf16, s);
        else launch_m1_xl<1, true>(packed, rows, cols, sc, x, y, y_bf16, s);
      } else {
        if (sc.absmax) launch_m1_xl<2, false>(packed, rows, cols, sc, x, y, y_bf16, s);
        else launch_m1_xl<2, true>(packed, rows, cols, sc, x, y, y_bf16, s);
      }
    } else if (per_cu <= 16) {
      const int wpg = static_cast<int>(((per_cu + 3) / 4) * 4);  // multiple of 4 waves (256 threads)
      if (sc.absmax) launch_m1<1, false>(packed, rows, cols, sc, x, y, y_bf16, wpg, s);
      else launch_m1<1, true>(packed, rows, cols, sc, x, y, y_bf16, wpg, s);
    } else if (per_cu <= 32) {
      if (sc.absmax) launch_m1<2, false>(packed, rows, cols, sc, x, y, y_bf16, 16, s);
      else launch_m1<2, true>(packed, rows, cols, sc, x, y, y_bf16, 16, s);
    } else {
      if (sc.absmax) launch_m1<4, false>(packed, rows, cols, sc, x, y, y_bf16, 16, s);
      else launch_m1<4, true>(packed, rows, cols, sc, x, y, y_bf16, 16, s);
    }
  } else {
    if (y_bf16) hipLaunchKernelGGL((k_gemv<4, true>), grid, dim3(256), 0, s, packed, rows, cols, sc, x, mm, y, cb);
    else hipLaunchKernelGGL((k_gemv<4, false>), grid, dim3(256), 0, s, packed, rows, cols, sc, x, mm, y, cb);
  }
  return hipGetLastError();
}

}  // namespace nf4i
