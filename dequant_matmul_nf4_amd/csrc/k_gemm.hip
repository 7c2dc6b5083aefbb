// Dequantize-and-multiply bf16 matrix-core GEMM with an optional fused LoRA
// term:
//   y = x . deq(W)^T + s . (x . A^T) . B^T
// (bitsandbytes tool page, "How it works", Step 5: matrix hardware works best
// on 16-bit numbers, so each block is expanded to 16-bit and multiplied; the
// tutorial page, "QLoRA: Fine-Tuning a 4-bit Model": low-rank adapters on the
// frozen 4-bit base, their output multiplied by a scale factor.)
//
// Tiling: a workgroup of 4 waves (one per SIMD) computes a 256 x 256 tile of
// y.  Wave w owns the 64 output columns [64 w, 64 w + 64) for all 256 rows:
// 8 x 2 tiles of v_mfma_f32_32x32x16_bf16 per 16-wide k step, 256 fp32
// accumulators per lane.  A K step covers 64 columns, exactly one NF4 block
// of every weight row.  Within a step the LDS reads of 16-wide k step s + 1
// (x fragments and level lookups) are issued before the MFMAs of k step s,
// so their latency is spent while the matrix cores run.
//
// Operands:
//  - x: the 256 x 64 tile is staged in LDS (two stages of 128-byte rows) by
//    direct global-to-LDS loads (global_load_lds_dwordx4: each wave
//    instruction fills 1 KB, lane l at byte 16 l), issued at the top of the
//    previous step.  16-byte piece p of row r sits at slot p ^ ((r / 2) % 8),
//    so the fragment reads of 16 consecutive rows hit distinct banks.
//  - W: never staged.  Each lane loads the 16 bytes of codes it needs
//    (32 consecutive k of one row) and expands them straight into its MFMA
//    B fragments: a byte (two codes) indexes a 256-entry table of float32
//    level pairs in LDS (32 copies, lane slot (lane % 32) * 8, so the lanes
//    served together hit distinct banks; address = one byte permute), each
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
// bits.
// Those columns (2 r rounded up to a multiple of 64) run as one or two more
// K steps with both operands staged in LDS.
#include "gemm_tiles.h"

namespace nf4i {
namespace {

using gt::bf16_pair;
using gt::bf16x8;
using gt::floatx16;
using gt::kThreads;
using gt::lds_frag;
using gt::u32x4;

constexpr int kBM = gt::kTileM, kBN = gt::kTileN, kBK = gt::kStep;
constexpr int kRowBytes = 144;                  // 64 bf16 + 16 bytes of padding
constexpr int kTileBytes = 256 * kRowBytes;     // one operand tile in LDS
constexpr int kPairSlots = 32;                  // copies of the level-pair table
constexpr int kXPieces = gt::kActPieces;        // 16-byte x pieces per thread and step (8)

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

// The 256 level pairs (element 2j = high nibble first), kPairSlots copies;
// entry e of slot c at byte e * 256 + c * 8.  Two phases so that each wave
// writes consecutive addresses.  Ends with a barrier.
__device__ __forceinline__ void fill_level_pairs(float2* tab, float2* base, const Codebook& cb) {
  if (threadIdx.x < 256) {
    const int e = threadIdx.x;
    float l0 = cb.level[0], l1 = cb.level[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      l0 = ((e >> 4) == i) ? cb.level[i] : l0;
      l1 = ((e & 15) == i) ? cb.level[i] : l1;
    }
    base[e] = make_float2(l0, l1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 256 * kPairSlots; i += blockDim.x) tab[i] = base[i / kPairSlots];
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
// of one W row): four LDS reads, addresses from one byte permute each.
struct Lookups {
  float2 l[2][4];
};

__device__ __forceinline__ void lookup_step(Lookups& lk, const u32x4 (&w)[2], int s, const char* tab,
                                            uint32_t slot) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t addr = __builtin_amdgcn_perm(w[j][s], slot, 0x0C0C0000u | ((4u + b) << 8));
      lk.l[j][b] = *reinterpret_cast<const float2*>(tab + addr);
    }
}

// Each level times the block scale, each pair rounded once to bf16.
__device__ __forceinline__ bf16x8 expand_frag(const float2 (&l)[4], float sa) {
  const u32x4 v = {bf16_pair(l[0].x * sa, l[0].y * sa), bf16_pair(l[1].x * sa, l[1].y * sa),
                   bf16_pair(l[2].x * sa, l[2].y * sa), bf16_pair(l[3].x * sa, l[3].y * sa)};
  return __builtin_bit_cast(bf16x8, v);
}

// Spreads the work issued next to 16 MFMAs between them: per MFMA three
// VALU operations and one LDS access.
__device__ __forceinline__ void mfma_interleave() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);  // LDS read or write
  }
}

template <bool kDQ>
__device__ __forceinline__ void block_scales(const WRegs& wr, float mean, float (&sa)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if constexpr (kDQ) sa[j] = (div127(wr.q[j]) * wr.s2[j]) + mean;  // a_hat, three roundings
    else sa[j] = wr.am[j];
  }
}

// One LoRA step (64 extra K columns): the x side from u into xs, the W side
// [B | B] (zero past the rank) into ws as rows of output columns; both then
// feed the MFMAs as fragments.
__device__ __forceinline__ void lora_step_to_lds(char* xs, char* ws, const GemmArgs& a, int64_t m0, int64_t n0,
                                                 int64_t k0) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kXPieces; ++i) {
    const int64_t row = m0 + (t >> 3) + 32 * i;
    const int64_t rc = row < a.m ? row : a.m - 1;
    const u32x4 v = *reinterpret_cast<const u32x4*>(a.u + rc * a.kl + k0 + (t & 7) * 8);
    *reinterpret_cast<u32x4*>(xs + ((t >> 3) + 32 * i) * kRowBytes + (t & 7) * 16) = v;
  }
  // W side: thread t fills output row t
  const int64_t n = n0 + t;
  const int64_t nc = n < a.rows ? n : a.rows - 1;
  const uint16_t* bp = a.lb + nc * a.r;
  char* wrow = ws + t * kRowBytes;
  for (int c = 0; c < kBK; ++c) {
    const int64_t col = k0 + c;
    const int64_t j = col < a.r_pad ? col : col - a.r_pad;
    const bool live = col < 2 * a.r_pad && j < a.r;
    reinterpret_cast<uint16_t*>(wrow)[c] = live ? bp[j] : static_cast<uint16_t>(0);
  }
}

__device__ __forceinline__ void mfma_lora(const char* xs, const char* ws, floatx16 (&acc)[8][2], int wave,
                                          int lane) {
  const char* xa = xs + (lane & 31) * kRowBytes + (lane >> 5) * 64;
  const char* wb = ws + (wave * 64 + (lane & 31)) * kRowBytes + (lane >> 5) * 64;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 bfr[2], af[8];
#pragma unroll
    for (int j = 0; j < 2; ++j) bfr[j] = lds_frag(wb + j * 32 * kRowBytes + s * 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = lds_frag(xa + i * 32 * kRowBytes + s * 16);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
  }
}

template <bool kDQ>
__global__ __launch_bounds__(kThreads) void k_gemm(GemmArgs a) {
  __shared__ __align__(16) char xs0[kTileBytes], xs1[kTileBytes];
  __shared__ float2 tab[256 * kPairSlots];
  __shared__ float2 tab_base[256];
  const char* tabc = reinterpret_cast<const char*>(tab);
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const uint32_t slot = static_cast<uint32_t>(lane & 31) << 3;

  fill_level_pairs(tab, tab_base, a.cb);  // once per workgroup; ends with a barrier
  const float mean = kDQ ? *a.sc.mean : 0.0f;
  const int64_t tiles_n = (a.rows + kBN - 1) / kBN;
  const int64_t tiles = tiles_n * ((a.m + kBM - 1) / kBM);
  const int64_t nk = a.cols / kBK;

  // Persistent: the grid holds one workgroup per CU and each takes tiles
  // blockIdx.x, blockIdx.x + gridDim.x, ...  Tile order: dispatch deals
  // workgroups round-robin over the 8 XCDs, so the workgroups of one XCD
  // that run at the same time get neighbouring tiles along N and share x rows.
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    int64_t tid = tile;
    if (tiles % 8 == 0) tid = (tile % 8) * (tiles / 8) + tile / 8;
    const int64_t m0 = (tid / tiles_n) * kBM;
    const int64_t n0 = (tid % tiles_n) * kBN;

    const gt::ActPtrs xp = gt::make_act_ptrs(a.x, a.cols, a.m, m0, wave, lane);
    WPtrs wp;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wave * 64 + j * 32 + (lane & 31);
      const int64_t nc = n < a.rows ? n : a.rows - 1;  // rows past the end: never stored
      wp.c[j] = a.packed + nc * (a.cols / 2) + (lane >> 5) * 16;
      wp.blk[j] = nc * (a.cols / 64);
    }

    floatx16 acc[8][2];
    gt::zero_acc(acc);

    // K step k: MFMAs from x stage k % 2 and the codes of step k (wc), in
    // four 16-wide k steps s.  Software pipeline: while the MFMAs of s run,
    // the wave expands the B fragments of s + 1 (looked up one k step
    // earlier) and issues the LDS reads of s + 2; during s = 3 it writes the
    // next step's x tile to the other stage and expands the next step's
    // s = 0, so that after the barrier the MFMAs can start at once.  The
    // global loads of step k + 1 (clamped on the last step) go out at the top
    // of step k.
    WRegs wc, wnx;
    gt::dma_act(xp, 0, xs0, wave);
    load_w<kDQ>(wc, wp, a, 0);
    float sa[2];
    bf16x8 bf[2][2];
    Lookups lk[3];
    bf16x8 af[3][8];
    const uint32_t sw = ((lane & 31) >> 1) & 7, h4 = (lane >> 5) * 4;
    block_scales<kDQ>(wc, mean, sa);
    lookup_step(lk[0], wc.w, 0, tabc, slot);
    bf[0][0] = expand_frag(lk[0].l[0], sa[0]);
    bf[0][1] = expand_frag(lk[0].l[1], sa[1]);
    gt::wait_vmem();
    __syncthreads();
    for (int64_t ks = 0; ks < nk; ++ks) {
      const int64_t kn = ks + 1 < nk ? ks + 1 : ks;
      // the next step's x tile goes straight to the other stage (last read
      // before the previous barrier) and its codes to registers
      gt::dma_act(xp, kn, (ks & 1) ? xs0 : xs1, wave);
      load_w<kDQ>(wnx, wp, a, kn);
      __builtin_amdgcn_sched_barrier(0);
      const char* xa = ((ks & 1) ? xs1 : xs0) + (lane & 31) * gt::kActRowBytes;
      gt::read_act(xa, 0, sw, h4, af[0]);
      gt::read_act(xa, 1, sw, h4, af[1]);
      lookup_step(lk[1], wc.w, 1, tabc, slot);
      __builtin_amdgcn_sched_barrier(0);
      // s = 0
      gt::mfma16(af[0], bf[0], acc);
      bf[1][0] = expand_frag(lk[1].l[0], sa[0]);
      bf[1][1] = expand_frag(lk[1].l[1], sa[1]);
      gt::read_act(xa, 2, sw, h4, af[2]);
      lookup_step(lk[2], wc.w, 2, tabc, slot);
      mfma_interleave();
      __builtin_amdgcn_sched_barrier(0);
      // s = 1
      gt::mfma16(af[1], bf[1], acc);
      bf[0][0] = expand_frag(lk[2].l[0], sa[0]);
      bf[0][1] = expand_frag(lk[2].l[1], sa[1]);
      gt::read_act(xa, 3, sw, h4, af[0]);
      lookup_step(lk[0], wc.w, 3, tabc, slot);
      mfma_interleave();
      __builtin_amdgcn_sched_barrier(0);
      // s = 2
      gt::mfma16(af[2], bf[0], acc);
      bf[1][0] = expand_frag(lk[0].l[0], sa[0]);
      bf[1][1] = expand_frag(lk[0].l[1], sa[1]);
      mfma_interleave();
      __builtin_amdgcn_sched_barrier(0);
      // s = 3, with the next step's s = 0 expansion
      gt::mfma16(af[0], bf[1], acc);
      block_scales<kDQ>(wnx, mean, sa);
      lookup_step(lk[1], wnx.w, 0, tabc, slot);
      bf[0][0] = expand_frag(lk[1].l[0], sa[0]);
      bf[0][1] = expand_frag(lk[1].l[1], sa[1]);
      mfma_interleave();
      __builtin_amdgcn_sched_barrier(0);
      gt::wait_vmem();
      __syncthreads();
      wc = wnx;
    }
    for (int64_t k0 = 0; k0 < a.kl; k0 += kBK) {
      lora_step_to_lds(xs0, xs1, a, m0, n0, k0);
      __syncthreads();
      mfma_lora(xs0, xs1, acc, wave, lane);
      __syncthreads();
    }

    gt::store_acc(acc, a.y, a.m, a.rows, m0, n0, wave, lane);
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
  GemmArgs a{};
  a.packed = packed; a.rows = rows; a.cols = cols; a.sc = sc; a.x = x; a.m = m; a.y = y;
  a.cb = codebook();
  if (r > 0) {
    a.r = r;
    a.r_pad = (r + 15) / 16 * 16;
    a.kl = static_cast<int>(gemm_lora_cols(r));
    a.u = u_ws;
    a.lb = lora_b;
    if (hipError_t e = launch_lora_u(x, lora_a, m, cols, r, lora_scale, u_ws, s)) return e;
  }
  const int64_t tiles = ((rows + kBN - 1) / kBN) * ((m + kBM - 1) / kBM);
  const int64_t cus = device_cus();
  const unsigned grid = static_cast<unsigned>(tiles < cus ? tiles : cus);  // persistent: one per CU
  if (sc.absmax) hipLaunchKernelGGL(k_gemm<false>, dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(k_gemm<true>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace nf4i
