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
#include "gemv_rows.h"

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
                                             const char* tab, uint32_t slot, float mean, int f8, float acc[R]) {
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
    if constexpr (kDQ) a = (code_ratio(it.q[r], f8) * it.s2[r]) + mean;  // a_hat
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
      gemv_compute<R, kDQ>(it, it.x, sg * 64 + lane < nblk, smem, slot, mean, sc.f8, acc);
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

// ---------------------------------------------------------------- rows
//
// Decode GEMV with the load schedule of a streaming copy.  A workgroup owns a
// contiguous range of rows; its waves split the columns into segments of up
// to 64 blocks (2 KiB of codes per row) and the rows into equal parts, so each
// wave walks a run of rows over one fixed column segment:
//  - a row's segment is read with two fully coalesced 1 KiB loads: lane l
//    takes the 16 bytes at offsets 16 l and 1024 + 16 l, i.e. half l & 1 of
//    blocks l / 2 and 32 + l / 2 (two pieces of 32 codes, each with its own
//    block scale);
//  - the lane's 2 x 32 values of x stay in registers for the whole run, as
//    fp16 pairs, each piece scaled by a power of two chosen from its largest
//    magnitude (so the scaling is exact and nothing overflows; it is undone on
//    the piece's partial sum);
//  - a byte of packed codes (two elements) indexes a 256-entry table of fp16
//    level pairs in LDS, one copy per lane (address = byte * 256 + lane * 4,
//    a single byte permute, every lane in its own bank), and one
//    v_dot2c_f32_f16 takes both products; fp16 keeps 11 significant bits of
//    each level;
//  - a ring of U + 1 register slots keeps U rows of loads in flight: each step
//    first requests the row U places ahead into the slot the previous step
//    used, then works on its own row (indices clamped so that no branch
//    separates the loads from their use); the first U rows are requested
//    before the table is built.  One row ahead measured fastest: deeper rings
//    were slower on every shape tried;
//  - each row's per-lane partial sum is reduced across the wave with DPP
//    (total in lane 63) and parked in LDS per (row, segment); at the end the
//    segments of each row are added in a fixed order, so the result does not
//    depend on timing.

constexpr int kRowsMaxWg = 512;   // rows per workgroup (LDS for the partial sums)
constexpr int kSegMax = 16;       // column segments per workgroup (cols <= 65536)

struct RowsPlan {
  int grid;          // number of workgroups
  int nseg;          // column segments
  int seg_blocks;    // blocks per segment (<= 64)
  int wpr;           // waves per segment (row parts)
};

// MC rows of x per launch (x and y point at the first of them; the x rows
// are cols apart, the y rows `rows` apart).
template <int U, int kWaves, int MC, bool kDQ, bool kF8, bool kBf16Out>
__global__ __launch_bounds__(kWaves * 64) void k_gemv_rows(const uint8_t* packed, int64_t rows,
                                                           int64_t cols, Scales sc, const uint16_t* x,
                                                           void* __restrict__ y, Codebook cb, RowsPlan pl) {
  constexpr int kRowsWg = kRowsMaxWg / MC;
  __shared__ uint32_t tab[256 * 64];
  __shared__ float part[kRowsWg * kSegMax * MC];
  __shared__ float rtab[kDQ ? 256 : 1];
  const char* smem = reinterpret_cast<const char*>(tab);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t slot = static_cast<uint32_t>(lane) << 2;
  const int64_t nblk = cols / 64;
  // Row parts are interleaved over the whole grid: part p takes rows p,
  // p + NP, p + 2 NP, ... so that at any time the grid reads one contiguous
  // window of rows, as a streaming copy does.
  const int64_t np = static_cast<int64_t>(gridDim.x) * pl.wpr;
  const int64_t kmax = (rows + np - 1) / np;  // rows per part, at most
  const int seg = wave % pl.nseg;
  const int prt = wave / pl.nseg;
  const int64_t gp = static_cast<int64_t>(blockIdx.x) * pl.wpr + prt;
  const int64_t n = (prt < pl.wpr && gp < rows) ? (rows - gp + np - 1) / np : 0;
  // piece j of the lane: half `half` of block 32 j + lane / 2 of the segment
  const int half = lane & 1;
  const int seg_end = static_cast<int>(nblk - seg * pl.seg_blocks < pl.seg_blocks ? nblk - seg * pl.seg_blocks
                                                                                   : pl.seg_blocks);
  bool on[2];
  int blk[2];
  LaneOffs lo;
  make_lane_offs(seg * pl.seg_blocks, seg_end, lane, lo, on, blk);
  const int64_t row0 = gp < rows ? gp : rows - 1;
  const int64_t last = n > 0 ? row0 + (n - 1) * np : row0;  // loads are clamped to it

  // x of the lane's pieces (MC rows), the first U rows, then the tables.  x
  // goes first: its conversion, which the compiler may place before the
  // tables' barrier, then waits for x alone, and the barrier waits for LDS
  // only, so the rows stay in flight while the tables are built.
  constexpr int S = U + 1;  // ring slots: U rows in flight plus the one in use
  uint4 xv[MC][2][4];
#pragma unroll
  for (int c = 0; c < MC; ++c)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4* xp = reinterpret_cast<const uint4*>(x + c * cols + static_cast<int64_t>(blk[j]) * 64 + 32 * half);
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[c][j][i] = xp[i];
    }
  RowItem it[S];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = row0 + u * np;
    row_load<kDQ>(it[u], packed, (r < last ? r : last) * nblk, lo, sc);
  }
  if constexpr (kDQ) fill_ratio_table<kF8>(rtab, kWaves * 64);
  fill_half_table<kWaves * 64, true>(tab, cb);  // ends with the LDS-only barrier

  uint32_t xh[MC][2][16];
  float xinv[MC][2];
#pragma unroll
  for (int c = 0; c < MC; ++c)
#pragma unroll
    for (int j = 0; j < 2; ++j) x_half_block_to_half(xv[c][j], xh[c][j], xinv[c][j]);
  float xsel[MC];
  lane_x_scales<MC>(xinv, on, xsel);
  const float mean = kDQ ? *sc.mean : 0.0f;

  // step i: request row i + U into the slot freed by step i - 1, then use
  // row i; the loop is unrolled by the ring size so that every slot keeps its
  // registers (no copies, each wait covers only the row about to be used)
  for (int64_t i0 = 0; i0 < n; i0 += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int64_t i = i0 + u;
      const int64_t r = row0 + (i + U) * np;
      row_load<kDQ>(it[(u + U) % S], packed, (r < last ? r : last) * nblk, lo, sc);
      __builtin_amdgcn_sched_barrier(0);
      if (i < n) {  // wave-uniform
        float v[MC];
        row_dot<MC, kDQ>(it[u], xh, smem, slot, mean, rtab, xsel, v);
#pragma unroll
        for (int c = 0; c < MC; ++c) {
          const float t = wave_sum_to_last(v[c]);
          if (lane == 63) part[((prt * kmax + i) * kSegMax + seg) * MC + c] = t;
        }
      }
    }
  }
  __syncthreads();
  for (int64_t t = threadIdx.x; t < pl.wpr * kmax * MC; t += blockDim.x) {
    const int64_t rt = t / MC;
    const int c = static_cast<int>(t % MC);
    const int64_t row = static_cast<int64_t>(blockIdx.x) * pl.wpr + rt / kmax + (rt % kmax) * np;
    if (row >= rows) continue;
    float s = part[(rt * kSegMax) * MC + c];
    for (int k = 1; k < pl.nseg; ++k) s += part[(rt * kSegMax + k) * MC + c];
    if constexpr (kBf16Out) static_cast<uint16_t*>(y)[c * rows + row] = static_cast<uint16_t>(f32_to_bf16(s));
    else static_cast<float*>(y)[c * rows + row] = s;
  }
}

// Plan for k_gemv_rows: rows split evenly over at least one workgroup per CU
// (at most rows_wg rows each), columns into the fewest segments of at most 64
// blocks, balanced, and the waves spread over the segments.
RowsPlan rows_plan(int64_t rows, int64_t cols, int waves, int rows_wg) {
  const int64_t cus = device_cus();
  const int64_t nblk = cols / 64;
  RowsPlan pl{};
  pl.nseg = static_cast<int>((nblk + 63) / 64);
  pl.seg_blocks = static_cast<int>((nblk + pl.nseg - 1) / pl.nseg);
  pl.wpr = waves / pl.nseg;
  // grid: one workgroup per CU, more if a workgroup would own more than
  // rows_wg rows (wpr parts of ceil(rows / (grid * wpr)) rows each)
  int64_t g = cus;
  while (pl.wpr > 0 && pl.wpr * ((rows + g * pl.wpr - 1) / (g * pl.wpr)) > rows_wg) ++g;
  pl.grid = static_cast<int>(g);
  return pl;
}

template <int U, int kWaves, int MC, bool kDQ, bool kF8>
hipError_t launch_rows(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x, void* y,
                       int y_bf16, hipStream_t s) {
  const RowsPlan pl = rows_plan(rows, cols, kWaves, kRowsMaxWg / MC);
  if (pl.nseg > kSegMax || pl.wpr < 1 || (cols / 64) * 32 >= (int64_t{1} << 32)) return hipErrorInvalidValue;
  const int64_t g = pl.grid;
  const Codebook& cb = codebook(sc.fp4);
  const dim3 gd(static_cast<unsigned>(g)), bd(64 * kWaves);
  if (y_bf16)
    hipLaunchKernelGGL((k_gemv_rows<U, kWaves, MC, kDQ, kF8, true>), gd, bd, 0, s, packed, rows, cols, sc, x, y, cb, pl);
  else
    hipLaunchKernelGGL((k_gemv_rows<U, kWaves, MC, kDQ, kF8, false>), gd, bd, 0, s, packed, rows, cols, sc, x, y, cb, pl);
  return hipGetLastError();
}

// The scale form of a launch: plain absmax, int8 or float8 second level.
template <int U, int kWaves, int MC>
hipError_t launch_rows_sc(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x, void* y,
                          int y_bf16, hipStream_t s) {
  if (sc.absmax) return launch_rows<U, kWaves, MC, false, false>(packed, rows, cols, sc, x, y, y_bf16, s);
  if (sc.f8) return launch_rows<U, kWaves, MC, true, true>(packed, rows, cols, sc, x, y, y_bf16, s);
  return launch_rows<U, kWaves, MC, true, false>(packed, rows, cols, sc, x, y, y_bf16, s);
}

// ---------------------------------------------------------------- m = 2..16
//
// Skinny products on the matrix cores: v_mfma_f32_16x16x32_bf16 with x (its
// m <= 16 rows; rows past m repeat row m - 1 and are never stored) as the A
// operand and 16 weight rows as the B operand, D[x row][weight row].
//  - B is the dequantized weight rounded once to bf16, bf16(fl32(level * a))
//    with a the block's scale, as the GEMM expands it: a byte of codes
//    indexes a table of fp32 level pairs (one permute, one LDS read), both
//    levels are multiplied by a and the pair is rounded to one operand word.
//    With the scale inside the operand an MFMA may span two blocks, so a lane
//    loads 16 contiguous code bytes and a wave instruction reads 64 bytes of
//    each of its 16 rows.
//  - k order of a 4-block segment: lane group g = lane / 16 takes, for
//    h = 0, 1, codes 32 (g % 2) .. + 31 of block 2 h + g / 2 (code bytes
//    16 (g % 2) .. + 15), 8 per MFMA, and x the same columns, so that x
//    needs no conversion.
//  - Weight rows go in groups of 16, interleaved over the grid (group p of a
//    workgroup is p-th of its share); waves walk the workgroup's groups for
//    each of their segments and park each (group, segment) partial tile in
//    LDS; the segments are added in a fixed order at the end.  Where those
//    tiles do not fit (wide rows: more than 64 per workgroup), each wave adds
//    its segments, in order, into one tile per (group, wave) instead, and the
//    16 waves' tiles are added in a fixed order at the end.
// First factor of a_hat: q / 127 for int8 codes, the E4M3 ratio table (copied
// to LDS) for float8 codes.
template <bool kF8>
__device__ __forceinline__ float row_ratio(int q, const float* rtab) {
  if constexpr (kF8) return rtab[q & 0xFF];
  else return div127(q);
}

constexpr int kPartTiles = 64;   // 16 x 16 float partial tiles per workgroup (64 KiB)
constexpr int kMfmaSeg = 4;      // blocks per column segment (x kept in registers)
constexpr int kMfmaWaves = 16;
constexpr int kMfmaMaxGroups = kPartTiles / kMfmaWaves;  // row groups per workgroup with (group, wave) tiles

typedef float floatx4 __attribute__((ext_vector_type(4)));

struct MfmaPlan {
  int grid;          // workgroups
  int nseg;          // column segments
  int seg_blocks;    // blocks per segment (<= kMfmaSeg)
  int kmax;          // row groups per workgroup, at most
  int accum;         // tiles per (group, wave), summed over the wave's segments (else per (group, segment))
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t sk_bf16_pair(float lo, float hi) {
  const bf16x2_t p = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, p);
}

// The loads of one (row group, segment): for weight row ln = lane % 16 the
// 16 code bytes 16 (g % 2) .. + 15 of blocks 2 h + g / 2 (h = 0, 1) of the
// segment and those blocks' scale inputs, kept as loaded until they are used.
// kQ4: the segment is 4 blocks starting at a multiple of 4 in the flattened
// block order, so the 4 int8 codes (or 4 absmax) are one aligned load and the
// group scales are the two that can occur.
template <bool kDQ>
struct SegItem {
  uint4 c[2];
  uint32_t q4;    // kQ4, double quant: the segment's 4 int8 codes
  float4 a4;      // kQ4, plain scales: the segment's 4 absmax
  int q[2];       // otherwise, per h: int8 code and group scale, or absmax
  float am[2];
  float s2lo, s2hi;
  int cross;      // blocks j >= cross of the segment use s2hi
};

template <bool kDQ, bool kQ4>
__device__ __forceinline__ void seg_load(SegItem<kDQ>& it, const uint8_t* __restrict__ packed, int64_t nblk,
                                         int64_t row, int64_t b0, int nb, int g, Scales sc, int64_t ngroups2) {
  const int64_t rb = row * nblk + b0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int pj = 2 * h + (g >> 1);
    const int64_t b = rb + (pj < nb ? pj : nb - 1);
    it.c[h] = *reinterpret_cast<const uint4*>(packed + b * 32 + 16 * (g & 1));
  }
  if constexpr (kQ4) {
    if constexpr (kDQ) {
      it.q4 = *reinterpret_cast<const uint32_t*>(sc.q + rb);
      const int64_t g0 = rb >> 8;
      it.s2lo = sc.absmax2[g0];
      it.s2hi = sc.absmax2[g0 + 1 < ngroups2 ? g0 + 1 : g0];
      it.cross = 256 - static_cast<int>(rb & 255);
    } else {
      it.a4 = *reinterpret_cast<const float4*>(sc.absmax + rb);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int pj = 2 * h + (g >> 1);
      const int64_t b = rb + (pj < nb ? pj : nb - 1);
      if constexpr (kDQ) {
        it.q[h] = sc.q[b];
        it.am[h] = sc.absmax2[b >> 8];
      } else {
        it.am[h] = sc.absmax[b];
      }
    }
  }
}

template <int kWaves, bool kDQ, bool kF8, bool kQ4, bool kBf16Out, bool kAccum>
__global__ __launch_bounds__(kWaves * 64) void k_gemv_mfma(const uint8_t* __restrict__ packed, int64_t rows,
                                                           int64_t cols, Scales sc, const uint16_t* __restrict__ x,
                                                           int m, void* __restrict__ y, Codebook cb, MfmaPlan pl) {
  __shared__ __align__(16) float2 tab[256 * 32];
  __shared__ float part[kPartTiles * 256];
  __shared__ float rtab[kF8 ? 256 : 1];
  const char* smem = reinterpret_cast<const char*>(tab);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int ln = lane & 15;
  const uint32_t slot = static_cast<uint32_t>(lane & 31) << 3;
  const int64_t nblk = cols / 64;
  const int64_t ngroups = (rows + 15) / 16;
  const int64_t G = gridDim.x;
  const int64_t kmine = (static_cast<int64_t>(blockIdx.x) < ngroups) ? (ngroups - blockIdx.x + G - 1) / G : 0;
  const int64_t ngroups2 = (rows * nblk + 255) / 256;
  const float mean = kDQ ? *sc.mean : 0.0f;
  if constexpr (kF8)
    for (int i = threadIdx.x; i < 256; i += kWaves * 64) rtab[i] = kE4m3Ratio.v[i];
  {
    // the 256 fp32 level pairs (element 2j = high nibble first), 32 copies:
    // entry e of copy c at byte 256 e + 8 c, a lane reads copy lane % 32
    const int e = threadIdx.x & 255;
    const int pp = threadIdx.x >> 8;
    constexpr int kParts = kWaves * 64 / 256;
    float l0 = cb.level[0], l1 = cb.level[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      l0 = ((e >> 4) == i) ? cb.level[i] : l0;
      l1 = ((e & 15) == i) ? cb.level[i] : l1;
    }
    const float2 v = make_float2(l0, l1);
#pragma unroll
    for (int j = 0; j < 32 / kParts; ++j) tab[e * 32 + ((j * kParts + pp + e) & 31)] = v;
  }
  // (group, wave) tiles start at zero: a wave adds each of its segments
  if constexpr (kAccum)
    for (int i = threadIdx.x; i < kPartTiles * 64; i += kWaves * 64)
      reinterpret_cast<float4*>(part)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  __syncthreads();

  for (int seg = wave; seg < pl.nseg; seg += kWaves) {
    const int64_t b0 = static_cast<int64_t>(seg) * pl.seg_blocks;
    const int nb = static_cast<int>(nblk - b0 < pl.seg_blocks ? nblk - b0 : pl.seg_blocks);
    // x of the segment as the A operand: lane (row ln, group g) holds, for
    // h = 0, 1, columns 32 (g % 2) .. + 31 of block 2 h + g / 2
    uint4 xv[2][4];
    {
      // rows past m repeat row m - 1: a row of A only reaches the same row of D,
      // and those rows are never stored
      const uint16_t* xr = x + static_cast<int64_t>(ln < m ? ln : m - 1) * cols;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int pj = 2 * h + (g >> 1);
        const int64_t blk = b0 + (pj < nb ? pj : nb - 1);
        const uint4* p = reinterpret_cast<const uint4*>(xr + blk * 64 + 32 * (g & 1));
#pragma unroll
        for (int u = 0; u < 4; ++u) xv[h][u] = p[u];
      }
    }
    // groups in order, the loads of group gi + 1 issued before group gi is
    // multiplied (clamped to the last group, whose loads are then repeated)
    auto load_group = [&](SegItem<kDQ>& it, int64_t gi) {
      const int64_t gl = gi < kmine ? gi : (kmine > 0 ? kmine - 1 : 0);
      const int64_t grp = blockIdx.x + gl * G;
      const int64_t rowc = grp * 16 + ln < rows ? grp * 16 + ln : rows - 1;
      seg_load<kDQ, kQ4>(it, packed, nblk, rowc, b0, nb, g, sc, ngroups2);
    };
    // per h: the lane's block scale, its 16 lookups, then 4 MFMAs whose B
    // words are the level pairs times the scale, each rounded once to bf16
    auto mult_group = [&](const SegItem<kDQ>& it, int64_t gi) {
      floatx4 acc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int pj = 2 * h + (g >> 1);
        float a;
        if constexpr (kDQ) {
          int q;
          float s2;
          if constexpr (kQ4) {
            q = static_cast<int>(static_cast<int8_t>(it.q4 >> (8 * pj)));
            s2 = pj >= it.cross ? it.s2hi : it.s2lo;
          } else {
            q = it.q[h];
            s2 = it.am[h];
          }
          a = (row_ratio<kF8>(q, rtab) * s2) + mean;
        } else if constexpr (kQ4) {
          a = pj == 0 ? it.a4.x : pj == 1 ? it.a4.y : pj == 2 ? it.a4.z : it.a4.w;
        } else {
          a = it.am[h];
        }
        a = pj < nb ? a : 0.0f;  // clamped loads past the segment's end
        float2 l[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const uint32_t word = u == 0 ? it.c[h].x : u == 1 ? it.c[h].y : u == 2 ? it.c[h].z : it.c[h].w;
            const uint32_t addr = __builtin_amdgcn_perm(word, slot, 0x0C0C0000u | ((4u + bb) << 8));
            l[u][bb] = *reinterpret_cast<const float2*>(smem + addr);
          }
        acc[h] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 bw = make_uint4(sk_bf16_pair(l[u][0].x * a, l[u][0].y * a), sk_bf16_pair(l[u][1].x * a, l[u][1].y * a),
                                      sk_bf16_pair(l[u][2].x * a, l[u][2].y * a), sk_bf16_pair(l[u][3].x * a, l[u][3].y * a));
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv[h][u]),
                                                           __builtin_bit_cast(bf16x8_t, bw), acc[h], 0, 0, 0);
        }
      }
      if constexpr (kAccum) {
        // tile of (group gi, wave): element (x row 4 g + i, weight row ln) at
        // ln * 16 + 4 g + i, so that a lane's four values are one 16-byte word
        float4* pt = reinterpret_cast<float4*>(part + (gi * kWaves + wave) * 256 + ln * 16 + 4 * g);
        float4 t = *pt;
        t.x += acc[0][0] + acc[1][0];
        t.y += acc[0][1] + acc[1][1];
        t.z += acc[0][2] + acc[1][2];
        t.w += acc[0][3] + acc[1][3];
        *pt = t;
      } else {
        // tile of (group gi, segment): element (x row 4 g + i, weight row ln)
        float* pt = part + (gi * pl.nseg + seg) * 256;
#pragma unroll
        for (int i = 0; i < 4; ++i) pt[(4 * g + i) * 16 + ln] = acc[0][i] + acc[1][i];
      }
    };
    SegItem<kDQ> ia, ib;
    load_group(ia, 0);
    for (int64_t gi = 0; gi < kmine; gi += 2) {
      load_group(ib, gi + 1);
      mult_group(ia, gi);
      if (gi + 1 >= kmine) break;
      load_group(ia, gi + 2);
      mult_group(ib, gi + 1);
    }
  }
  __syncthreads();
  if constexpr (kAccum) {
    // each thread adds one 16-byte word (x rows 4 q .. 4 q + 3 of weight
    // row wn) over the 16 waves' tiles in order: consecutive threads read
    // consecutive words
    const float4* part4 = reinterpret_cast<const float4*>(part);
    for (int64_t t = threadIdx.x; t < kmine * 64; t += blockDim.x) {
      const int64_t gi = t >> 6;
      const int wn = static_cast<int>((t >> 2) & 15);
      const int q = static_cast<int>(t & 3);
      const int64_t row = (blockIdx.x + gi * G) * 16 + wn;
      if (4 * q >= m || row >= rows) continue;
      float4 sum = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      const float4* src = part4 + gi * kWaves * 64 + wn * 4 + q;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float4 v = src[w * 64];
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
      }
      const float r[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int xm = 4 * q + i;
        if (xm >= m) continue;
        if constexpr (kBf16Out) static_cast<uint16_t*>(y)[xm * rows + row] = static_cast<uint16_t>(f32_to_bf16(r[i]));
        else static_cast<float*>(y)[xm * rows + row] = r[i];
      }
    }
  } else {
    for (int64_t t = threadIdx.x; t < kmine * 256; t += blockDim.x) {
      const int64_t gi = t >> 8;
      const int xm = static_cast<int>((t >> 4) & 15);
      const int wn = static_cast<int>(t & 15);
      const int64_t row = (blockIdx.x + gi * G) * 16 + wn;
      if (xm >= m || row >= rows) continue;
      float sum = 0.0f;
      for (int sg = 0; sg < pl.nseg; ++sg) sum += part[(gi * pl.nseg + sg) * 256 + xm * 16 + wn];
      if constexpr (kBf16Out) static_cast<uint16_t*>(y)[xm * rows + row] = static_cast<uint16_t>(f32_to_bf16(sum));
      else static_cast<float*>(y)[xm * rows + row] = sum;
    }
  }
}

// Plan: segments of at most kMfmaSeg blocks (balanced); grid of one
// workgroup per CU (fewer for few groups).  If a workgroup's (group, segment)
// tiles do not fit, the kernel keeps (group, wave) tiles instead and the grid
// grows until a workgroup has at most kMfmaMaxGroups groups.
MfmaPlan mfma_plan(int64_t rows, int64_t cols) {
  const int64_t cus = device_cus();
  const int64_t nblk = cols / 64;
  MfmaPlan pl{};
  pl.nseg = static_cast<int>((nblk + kMfmaSeg - 1) / kMfmaSeg);
  pl.seg_blocks = static_cast<int>((nblk + pl.nseg - 1) / pl.nseg);
  const int64_t ngroups = (rows + 15) / 16;
  int64_t g = cus < ngroups ? cus : ngroups;
  pl.accum = ((ngroups + g - 1) / g) * pl.nseg > kPartTiles ? 1 : 0;
  if (pl.accum)
    while ((ngroups + g - 1) / g > kMfmaMaxGroups) ++g;
  pl.grid = static_cast<int>(g);
  pl.kmax = static_cast<int>((ngroups + g - 1) / g);
  return pl;
}

// One launch of the skinny kernel with the plan's tiles (kAccum: one per
// (group, wave)) and the scale arrays' load form (kQ4).
template <bool kDQ, bool kAccum>
void launch_mfma_tiles(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x, int mi,
                       void* y, int y_bf16, const Codebook& cb, const MfmaPlan& pl, bool q4, dim3 gd, dim3 bd,
                       hipStream_t s) {
#define NF4_MFMA(Q4, BF) \
  do { \
    if (sc.f8) hipLaunchKernelGGL((k_gemv_mfma<kMfmaWaves, kDQ, kDQ, Q4, BF, kAccum>), gd, bd, 0, s, packed, rows, cols, \
                                  sc, x, mi, y, cb, pl); \
    else hipLaunchKernelGGL((k_gemv_mfma<kMfmaWaves, kDQ, false, Q4, BF, kAccum>), gd, bd, 0, s, packed, rows, cols, sc, \
                            x, mi, y, cb, pl); \
  } while (0)
  if (q4) {
    if (y_bf16) NF4_MFMA(true, true); else NF4_MFMA(true, false);
  } else {
    if (y_bf16) NF4_MFMA(false, true); else NF4_MFMA(false, false);
  }
#undef NF4_MFMA
}

template <bool kDQ>
hipError_t launch_mfma(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x, int64_t m,
                       void* y, int y_bf16, hipStream_t s) {
  const MfmaPlan pl = mfma_plan(rows, cols);
  if (pl.accum ? pl.kmax > kMfmaMaxGroups : pl.kmax * pl.nseg > kPartTiles) return hipErrorInvalidValue;
  const Codebook& cb = codebook(sc.fp4);
  const dim3 gd(static_cast<unsigned>(pl.grid)), bd(64 * kMfmaWaves);
  const int mi = static_cast<int>(m);
  // whole 4-block segments at multiples of 4 blocks in every row, and scale
  // arrays aligned for one 4-byte (int8 codes) or 16-byte (absmax) load
  const uintptr_t sa = kDQ ? reinterpret_cast<uintptr_t>(sc.q) : reinterpret_cast<uintptr_t>(sc.absmax);
  const bool q4 = pl.seg_blocks == kMfmaSeg && (cols / 64) % kMfmaSeg == 0 && (sa & (kDQ ? 3u : 15u)) == 0;
  if (pl.accum) launch_mfma_tiles<kDQ, true>(packed, rows, cols, sc, x, mi, y, y_bf16, cb, pl, q4, gd, bd, s);
  else launch_mfma_tiles<kDQ, false>(packed, rows, cols, sc, x, mi, y, y_bf16, cb, pl, q4, gd, bd, s);
  return hipGetLastError();
}

// Skinny products (m > 1): passes of up to 4 rows of x over W, 8 waves.
hipError_t launch_rows_multi(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x,
                             int64_t m, void* y, int y_bf16, hipStream_t s) {
  const size_t ysz = y_bf16 ? 2 : 4;
  for (int64_t c0 = 0; c0 < m; c0 += 4) {
    const int64_t mc = m - c0 < 4 ? m - c0 : 4;
    const uint16_t* xc = x + c0 * cols;
    void* yc = static_cast<char*>(y) + c0 * rows * ysz;
    hipError_t e;
    if (mc == 4) e = launch_rows_sc<1, 8, 4>(packed, rows, cols, sc, xc, yc, y_bf16, s);
    else if (mc == 3) e = launch_rows_sc<1, 8, 3>(packed, rows, cols, sc, xc, yc, y_bf16, s);
    else if (mc == 2) e = launch_rows_sc<1, 8, 2>(packed, rows, cols, sc, xc, yc, y_bf16, s);
    else e = launch_rows_sc<1, 8, 1>(packed, rows, cols, sc, xc, yc, y_bf16, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
  const Codebook& cb = codebook(sc.fp4);
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
  const Codebook& cb = codebook(sc.fp4);
  const int mm = static_cast<int>(m);
  if (m == 1) {
    const int64_t nseg = (cols / 64 + 63) / 64;
    if (nseg == 1) {
      // one column segment: 8 waves
      return launch_rows_sc<1, 8, 1>(packed, rows, cols, sc, x, y, y_bf16, s);
    }
    if (nseg <= kSegMax) {
      // 16 waves, or 8 where 16 would leave row parts without rows
      if (nseg <= 8 && rows < device_cus() * (16 / nseg))
        return launch_rows_sc<1, 8, 1>(packed, rows, cols, sc, x, y, y_bf16, s);
      return launch_rows_sc<1, 16, 1>(packed, rows, cols, sc, x, y, y_bf16, s);
    }
    // wider than 16 segments (cols > 65536): one row group per wave
    const int64_t cus = device_cus();
    const int64_t per_cu = (rows + cus - 1) / cus;
    if (per_cu <= 16) {
      const int wpg = static_cast<int>(((per_cu + 3) / 4) * 4);  // multiple of 4 waves (256 threads)
      if (sc.absmax) launch_m1<1, false>(packed, rows, cols, sc, x, y, y_bf16, wpg, s);
      else launch_m1<1, true>(packed, rows, cols, sc, x, y, y_bf16, wpg, s);
    } else {
      if (sc.absmax) launch_m1<2, false>(packed, rows, cols, sc, x, y, y_bf16, 16, s);
      else launch_m1<2, true>(packed, rows, cols, sc, x, y, y_bf16, 16, s);
    }
  } else {
    // m = 2 (and m <= 4 on matrices of at least 2^27 weights): the streaming
    // kernel with the x rows sharing each lookup, which measured faster there
    // than the matrix cores (e.g. 28672x8192: 31 against 59 us at m = 2, 46
    // against 63 us at m = 4; 14336x4096 at m = 4: 17.8 against 15.0 us).
    // Rows wider than 32768 columns there take the per-row-group kernel.
    // Every other skinny product runs on the matrix cores.
    const bool rows_first = m <= 2 || (m <= 4 && rows * cols >= (int64_t{1} << 27));
    if (rows_first) {
      if ((cols / 64 + 63) / 64 <= 8) return launch_rows_multi(packed, rows, cols, sc, x, m, y, y_bf16, s);
      if (y_bf16) hipLaunchKernelGGL((k_gemv<4, true>), grid, dim3(256), 0, s, packed, rows, cols, sc, x, mm, y, cb);
      else hipLaunchKernelGGL((k_gemv<4, false>), grid, dim3(256), 0, s, packed, rows, cols, sc, x, mm, y, cb);
      return hipGetLastError();
    }
    return sc.absmax ? launch_mfma<false>(packed, rows, cols, sc, x, m, y, y_bf16, s)
                     : launch_mfma<true>(packed, rows, cols, sc, x, m, y, y_bf16, s);
  }
  return hipGetLastError();
}

}  // namespace nf4i
