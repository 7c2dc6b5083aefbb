// Dequantize-and-multiply bf16 matrix-core GEMM with an optional fused LoRA
// term:
//   y = x . deq(W)^T + s . (x . A^T) . B^T
// (bitsandbytes tool page, "How it works", Step 5: matrix hardware works best
// on 16-bit numbers, so each block is expanded to 16-bit and multiplied; the
// tutorial page, "QLoRA: Fine-Tuning a 4-bit Model": low-rank adapters on the
// frozen 4-bit base, their output multiplied by a scale factor.)
//
// Tiling: a workgroup of 4 waves computes a (32 MI) x 256 tile of y.  Wave w
// owns the 64 output columns [64 w, 64 w + 64) for all 32 MI rows: MI x 2
// tiles of v_mfma_f32_32x32x16_bf16 per 16-wide k step (MI = 8: 256 fp32
// accumulators per lane).  A K step covers 64 columns, exactly one NF4 block
// of every weight row.  Within a step the LDS reads of 16-wide k step s + 1 (x
// fragments and level lookups) are issued before the MFMAs of k step s, so
// their latency is spent while the matrix cores run.
//
// Work units: the persistent workgroups take 256-row tiles round by round.
// When the last round would leave compute units idle (its tiles number at
// most half the workgroups), each of its tiles is cut into two 128-row halves
// (MI = 4) taken by two workgroups: a half costs more than half a tile (its
// weight tile is expanded for half as many rows) but the round ends sooner.
//
// Operands:
//  - x: the (32 MI) x 64 tile is staged in LDS (two stages of 128-byte rows) by
//    direct global-to-LDS loads (global_load_lds_dwordx4: each wave
//    instruction fills 1 KB, lane l at byte 16 l), issued at the top of the
//    previous step.  16-byte piece p of row r sits at slot p ^ ((r / 2) % 8),
//    so the fragment reads of 16 consecutive rows hit distinct banks.
//  - W: never staged.  Each lane loads the 16 bytes of codes it needs
//    (32 consecutive k of one row) and expands them straight into its MFMA
//    B fragments: a byte (two codes) indexes a 256-entry table of float32
//    level pairs in LDS (kCopies interleaved copies, lane slot
//    lane % kCopies, so the lanes served together hit distinct banks), each
//    level is multiplied by the block scale and the pair rounded once to bf16
//    -- the same value nf4_dequantize writes.  The next step's codes are
//    loaded one step ahead.
//  - The k index of a lane's fragment is a permutation of the step's 64
//    columns (lane half h takes columns 32 h .. 32 h + 31, eight per 16-wide
//    k step); A and B fragments use the same one, so the sum is unchanged.
//
// LoRA: the low-rank term is folded in as extra K columns,
//   [x | s T_hi | s T_lo] . [deq(W) | B | B]^T  with T = x . A^T,
// where s T is split into two bf16 parts (hi = bf16(sT), lo = bf16(sT - hi))
// by the LoRA prep kernel, so the adapter product keeps about 16 significant
// bits.  Those columns (2 r rounded up to a multiple of 64) run as one or two
// more K steps: the x side through the same staged tile, the W side
// [B | B | 0] (laid out row by row in the workspace by k_lora_bx) loaded
// straight into fragments.
#include "gemm_tiles.h"

namespace nf4i {
namespace {

using gt::bf16_pair;
using gt::bf16x8;
using gt::floatx16;
using gt::kThreads;
using gt::lds_frag;
using gt::u32x4;

constexpr int kBN = gt::kTileN, kBK = gt::kStep;
// The configuration the launcher uses: 256-row tiles and 32 copies of the
// pair table (x stages 64 KB + table 64 KB), one workgroup per compute unit.
// (128-row tiles with two workgroups per compute unit measured slower: each
// weight tile is then expanded for half as many rows.)
constexpr int kMI = 8;
constexpr int kCopies = 32;
constexpr int kWgPerCu = 1;
constexpr int kBM = 32 * kMI;
constexpr int kStageBytes = gt::act_stage_bytes<kBM>();

struct GemmArgs {
  const uint8_t* packed;
  int64_t rows, cols;    // W [rows][cols]; y has `rows` columns
  Scales sc;
  const uint16_t* x;     // [m][cols]
  int64_t m;
  uint16_t* y;           // [m][rows]
  const uint16_t* u;     // LoRA columns of x: [m][kl] (s T hi | s T lo | 0), or null
  const uint16_t* bx;    // LoRA columns of W: [rows][kl] (B | B | 0)
  int kl;                // extra K (multiple of 64), 0 without LoRA
  int64_t whole;         // work units 0 .. whole - 1: tile u, all 256 rows
  int64_t units;         // units whole .. units - 1: tile whole + (u - whole) / 2, half (u - whole) % 2
  Codebook cb;
};

// The 256 level pairs (element 2j = high nibble first), C interleaved copies:
// entry e of copy c at byte e * 8 C + c * 8.  Ends with a barrier.
template <int C>
__device__ __forceinline__ void fill_level_pairs(float2* tab, const Codebook& cb) {
  if (threadIdx.x < 256) {
    const int e = threadIdx.x;
    const float2 v = make_float2(cb.level[e >> 4], cb.level[e & 15]);
#pragma unroll
    for (int c = 0; c < C; ++c) tab[e * C + c] = v;
  }
  __syncthreads();
}

// The codes a lane expands in one K step: for its two W rows (j = 0, 1) the
// 16 bytes of columns 32 h .. 32 h + 31, and the rows' block scale inputs.
struct WRegs {
  u32x4 w[2];
  float am[2];   // absmax (plain scales)
  int q[2];      // int8 scale code (double quant)
  float s2[2];
};

struct WPtrs {
  const uint8_t* c[2];    // codes of row j at step 0, lane half's 16 bytes
  int64_t blk[2];         // block index of row j at step 0
};

template <bool kDQ>
__device__ __forceinline__ void load_w(WRegs& r, const WPtrs& p, const GemmArgs& a, int64_t ks) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    r.w[j] = *reinterpret_cast<const u32x4*>(p.c[j] + ks * (kBK / 2));
    const int64_t blk = p.blk[j] + ks;
    if constexpr (kDQ) {
      r.q[j] = a.sc.q[blk];
      r.s2[j] = a.sc.absmax2[blk >> 8];
    } else {
      r.am[j] = a.sc.absmax[blk];
    }
  }
}

// Level pairs of code bytes 4 s .. 4 s + 3 of a lane's 16 bytes (one k step
// of one W row): four LDS reads.  The byte permute puts the code byte at
// bits 8..15 next to the lane's slot; a shift scales it to the entry size
// 8 C (slot = (lane % C) << (8 - log2 C)).
struct Lookups {
  float2 l[2][4];
};

template <int C>
__device__ __forceinline__ void lookup_step(Lookups& lk, const u32x4 (&w)[2], int s, const char* tab,
                                            uint32_t slot) {
  constexpr int kShift = C == 32 ? 0 : C == 16 ? 1 : 2;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t addr = __builtin_amdgcn_perm(w[j][s], slot, 0x0C0C0000u | ((4u + b) << 8)) >> kShift;
      lk.l[j][b] = *reinterpret_cast<const float2*>(tab + addr);
    }
}

// Each level times the block scale, each pair rounded once to bf16.
__device__ __forceinline__ bf16x8 expand_frag(const float2 (&l)[4], float sa) {
  const u32x4 v = {bf16_pair(l[0].x * sa, l[0].y * sa), bf16_pair(l[1].x * sa, l[1].y * sa),
                   bf16_pair(l[2].x * sa, l[2].y * sa), bf16_pair(l[3].x * sa, l[3].y * sa)};
  return __builtin_bit_cast(bf16x8, v);
}

// Spreads the work issued next to the MFMAs of one 16-wide k step between
// them: per MFMA V VALU operations and L LDS accesses.
template <int N, int V, int L>
__device__ __forceinline__ void mfma_interleave() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x080, L, 0);  // LDS read or write
  }
}

// The scale form is a template parameter (plain, int8, float8): a runtime
// choice would put a global-memory table load behind a branch, and the wait
// the compiler places after it would also wait for the next step's loads.
template <bool kDQ, bool kF8>
__device__ __forceinline__ void block_scales(const WRegs& wr, float mean, float (&sa)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if constexpr (kDQ) sa[j] = (code_ratio(wr.q[j], kF8 ? 1 : 0) * wr.s2[j]) + mean;  // a_hat, three roundings
    else sa[j] = wr.am[j];
  }
}

// One work unit: the (32 MI) x 256 tile of y at rows m0.., columns n0..
// (MI = 8: a whole tile; MI = 4: half of one).  Every LDS stage read here is
// read before a barrier that all waves pass before the unit returns.
template <int MI, bool kDQ, bool kF8>
__device__ __forceinline__ void gemm_unit(const GemmArgs& a, int64_t m0, int64_t n0, char* xs0, char* xs1,
                                          const char* tabc, uint32_t slot, float mean, int wave, int lane) {
  // Per MFMA: the expansion and lookups of the next 16-wide k step are the
  // same for both tile heights, spread over 2 MI MFMAs.
  constexpr int kV = MI == 8 ? 3 : 6, kL = MI == 8 ? 1 : 2;
  const int64_t nk = a.cols / kBK;
  const gt::ActPtrs<MI> xp = gt::make_act_ptrs<MI, 32 * MI>(a.x, a.cols, a.m, m0, wave, lane);
  WPtrs wp;
  int64_t nrow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wave * 64 + j * 32 + (lane & 31);
    nrow[j] = n < a.rows ? n : a.rows - 1;  // rows past the end: never stored
    wp.c[j] = a.packed + nrow[j] * (a.cols / 2) + (lane >> 5) * 16;
    wp.blk[j] = nrow[j] * (a.cols / 64);
  }

  floatx16 acc[MI][2];
  gt::zero_acc(acc);

  // K step k: MFMAs from x stage k % 2 and the codes of step k (wc), in
  // four 16-wide k steps s.  Software pipeline: while the MFMAs of s run,
  // the wave expands the B fragments of s + 1 (looked up one k step
  // earlier) and issues the LDS reads of s + 2; during s = 3 it expands
  // the next step's s = 0, so that after the barrier the MFMAs can start at
  // once.  The global loads of step k + 1 (clamped on the last step: x to
  // the other stage, codes to registers) go out at the top of step k.
  WRegs wc, wnx;
  gt::dma_act(xp, 0, xs0, wave);
  load_w<kDQ>(wc, wp, a, 0);
  float sa[2];
  bf16x8 bf[2][2];
  Lookups lk[3];
  bf16x8 af[3][MI];
  const uint32_t sw = ((lane & 31) >> 1) & 7, h4 = (lane >> 5) * 4;
  block_scales<kDQ, kF8>(wc, mean, sa);
  lookup_step<kCopies>(lk[0], wc.w, 0, tabc, slot);
  bf[0][0] = expand_frag(lk[0].l[0], sa[0]);
  bf[0][1] = expand_frag(lk[0].l[1], sa[1]);
  gt::wait_vmem();
  __syncthreads();
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int64_t kn = ks + 1 < nk ? ks + 1 : ks;
    gt::dma_act(xp, kn, (ks & 1) ? xs0 : xs1, wave);  // the other stage was last read before the previous barrier
    load_w<kDQ>(wnx, wp, a, kn);
    __builtin_amdgcn_sched_barrier(0);
    const char* xa = ((ks & 1) ? xs1 : xs0) + (lane & 31) * gt::kActRowBytes;
    gt::read_act(xa, 0, sw, h4, af[0]);
    gt::read_act(xa, 1, sw, h4, af[1]);
    lookup_step<kCopies>(lk[1], wc.w, 1, tabc, slot);
    __builtin_amdgcn_sched_barrier(0);
    // s = 0
    gt::mfma16(af[0], bf[0], acc);
    bf[1][0] = expand_frag(lk[1].l[0], sa[0]);
    bf[1][1] = expand_frag(lk[1].l[1], sa[1]);
    gt::read_act(xa, 2, sw, h4, af[2]);
    lookup_step<kCopies>(lk[2], wc.w, 2, tabc, slot);
    mfma_interleave<2 * MI, kV, kL>();
    __builtin_amdgcn_sched_barrier(0);
    // s = 1
    gt::mfma16(af[1], bf[1], acc);
    bf[0][0] = expand_frag(lk[2].l[0], sa[0]);
    bf[0][1] = expand_frag(lk[2].l[1], sa[1]);
    gt::read_act(xa, 3, sw, h4, af[0]);
    lookup_step<kCopies>(lk[0], wc.w, 3, tabc, slot);
    mfma_interleave<2 * MI, kV, kL>();
    __builtin_amdgcn_sched_barrier(0);
    // s = 2
    gt::mfma16(af[2], bf[0], acc);
    bf[1][0] = expand_frag(lk[0].l[0], sa[0]);
    bf[1][1] = expand_frag(lk[0].l[1], sa[1]);
    mfma_interleave<2 * MI, kV, kL>();
    __builtin_amdgcn_sched_barrier(0);
    // s = 3, with the next step's s = 0 expansion
    gt::mfma16(af[0], bf[1], acc);
    block_scales<kDQ, kF8>(wnx, mean, sa);
    lookup_step<kCopies>(lk[1], wnx.w, 0, tabc, slot);
    bf[0][0] = expand_frag(lk[1].l[0], sa[0]);
    bf[0][1] = expand_frag(lk[1].l[1], sa[1]);
    mfma_interleave<2 * MI, kV, kL>();
    __builtin_amdgcn_sched_barrier(0);
    gt::wait_vmem();
    __syncthreads();
    wc = wnx;
  }
  if (a.kl > 0) {
    // LoRA K steps: u through the x stage, [B | B | 0] rows straight into fragments
    const gt::ActPtrs<MI> up = gt::make_act_ptrs<MI, 32 * MI>(a.u, a.kl, a.m, m0, wave, lane);
    for (int64_t k0 = 0; k0 < a.kl; k0 += kBK) {
      gt::dma_act(up, k0 / kBK, xs0, wave);  // xs0 was last read before the previous barrier
      bf16x8 bl[4][2];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bl[s4][j] = *reinterpret_cast<const bf16x8*>(a.bx + nrow[j] * a.kl + k0 + h4 * 8 + 8 * s4);
      gt::wait_vmem();
      __syncthreads();
      const char* xa = xs0 + (lane & 31) * gt::kActRowBytes;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        gt::read_act(xa, s4, sw, h4, af[0]);
        gt::mfma16(af[0], bl[s4], acc);
      }
      __syncthreads();
    }
  }

  gt::store_acc(acc, a.y, a.m, a.rows, m0, n0, wave, lane);
}

template <bool kDQ, bool kF8>
__global__ __launch_bounds__(kThreads, kWgPerCu) void k_gemm(GemmArgs a) {
  __shared__ __align__(16) char xs0[kStageBytes], xs1[kStageBytes];
  __shared__ __align__(16) float2 tab[256 * kCopies];
  const char* tabc = reinterpret_cast<const char*>(tab);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  constexpr int kShift = kCopies == 32 ? 0 : kCopies == 16 ? 1 : 2;
  const uint32_t slot = static_cast<uint32_t>(lane & (kCopies - 1)) << (3 + kShift);

  fill_level_pairs<kCopies>(tab, a.cb);  // once per workgroup; ends with a barrier
  const float mean = kDQ ? *a.sc.mean : 0.0f;
  const int64_t tiles_n = (a.rows + kBN - 1) / kBN;
  const int64_t tiles = tiles_n * ((a.m + kBM - 1) / kBM);

  // Persistent: the grid holds the resident workgroups and each takes units
  // blockIdx.x, blockIdx.x + gridDim.x, ...  Tile order: dispatch deals
  // workgroups round-robin over the 8 XCDs, so the workgroups of one XCD
  // that run at the same time get neighbouring tiles along N and share x rows.
  for (int64_t u = blockIdx.x; u < a.units; u += gridDim.x) {
    const bool half = u >= a.whole;
    const int64_t tile = half ? a.whole + (u - a.whole) / 2 : u;
    int64_t tid = tile;
    if (tiles % 8 == 0) tid = (tile % 8) * (tiles / 8) + tile / 8;
    const int64_t m0 = (tid / tiles_n) * kBM;
    const int64_t n0 = (tid % tiles_n) * kBN;
    if (!half) {
      gemm_unit<kMI, kDQ, kF8>(a, m0, n0, xs0, xs1, tabc, slot, mean, wave, lane);
    } else {
      const int64_t mh = m0 + ((u - a.whole) & 1) * (kBM / 2);
      if (mh < a.m) gemm_unit<kMI / 2, kDQ, kF8>(a, mh, n0, xs0, xs1, tabc, slot, mean, wave, lane);
    }
  }
}

// bx[n][c] = (B | B | 0)[n][c] for c < kl: B[n][c] for c < r, B[n][c - r_pad]
// for r_pad <= c < r_pad + r, zero elsewhere.
__global__ __launch_bounds__(256) void k_lora_bx(const uint16_t* __restrict__ lb, int64_t rows, int r, int r_pad,
                                                 int kl, uint16_t* __restrict__ bx) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * kl) return;
  const int64_t n = i / kl;
  const int c = static_cast<int>(i - n * kl);
  const int j = c < r_pad ? c : c - r_pad;
  const bool live = c < 2 * r_pad && j < r;
  bx[i] = live ? lb[n * r + j] : static_cast<uint16_t>(0);
}

}  // namespace

size_t gemm_lora_cols(int r) {
  if (r <= 0) return 0;
  const int r_pad = (r + 15) / 16 * 16;
  return static_cast<size_t>((2 * r_pad + kBK - 1) / kBK * kBK);
}

size_t gemm_workspace(int64_t m, int64_t rows, int r) {
  if (r <= 0) return 0;
  const size_t kl = gemm_lora_cols(r);
  const size_t ub = (static_cast<size_t>(m) * kl * sizeof(uint16_t) + 255) & ~size_t(255);
  return ub + static_cast<size_t>(rows) * kl * sizeof(uint16_t);
}

hipError_t launch_gemm(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* x,
                       int64_t m, uint16_t* y, const uint16_t* lora_a, const uint16_t* lora_b, int r,
                       float lora_scale, uint16_t* u_ws, hipStream_t s) {
  GemmArgs a{};
  a.packed = packed; a.rows = rows; a.cols = cols; a.sc = sc; a.x = x; a.m = m; a.y = y;
  a.cb = codebook(sc.fp4);
  if (r > 0) {
    const int r_pad = (r + 15) / 16 * 16;
    a.kl = static_cast<int>(gemm_lora_cols(r));
    a.u = u_ws;
    uint16_t* bx = u_ws + ((static_cast<size_t>(m) * a.kl * sizeof(uint16_t) + 255) & ~size_t(255)) / sizeof(uint16_t);
    a.bx = bx;
    const int64_t nb = rows * a.kl;
    if ((nb + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_lora_bx, dim3(static_cast<unsigned>((nb + 255) / 256)), dim3(256), 0, s, lora_b, rows, r,
                       r_pad, a.kl, bx);
    if (hipError_t e = launch_lora_u(x, lora_a, m, cols, r, lora_scale, u_ws, s)) return e;
  }
  const int64_t tiles = ((rows + kBN - 1) / kBN) * ((m + kBM - 1) / kBM);
  const int64_t slots = kWgPerCu * device_cus();  // resident workgroups
  // Tiles of the last round (all of them when they fill less than one): cut
  // into halves when those fit in one round and the tiles have more than 128 rows.
  const int64_t last = tiles - tiles / slots * slots;
  const bool halve = last > 0 && 2 * last <= slots && m > kBM / 2;
  a.whole = halve ? tiles - last : tiles;
  a.units = halve ? tiles + last : tiles;
  const unsigned grid = static_cast<unsigned>(a.units < slots ? a.units : slots);
  if (sc.absmax) hipLaunchKernelGGL((k_gemm<false, false>), dim3(grid), dim3(kThreads), 0, s, a);
  else if (sc.f8) hipLaunchKernelGGL((k_gemm<true, true>), dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((k_gemm<true, false>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace nf4i
