// Input gradient through the frozen 4-bit base, for QLoRA training (tutorial
// page "bitsandbytes quantization tutorial: 4-bit and 8-bit models", section
// "QLoRA: Fine-Tuning a 4-bit Model": the base stays frozen while gradients
// pass through it to the adapters):
//
//   dX = dY . deq(W) + s . (dY . B) . A          dY [m][rows], dX [m][cols]
//
// The reduction runs over the weight's rows, so W enters in the other
// orientation than in the forward GEMM and has to be transposed on chip.
//
// Tiling: a workgroup of 8 waves (two per SIMD) computes a 256 (m) x 256
// (col) tile of dX.  Wave (h, w) = (wave / 4, wave % 4) owns columns
// [64 w, 64 w + 64) for rows [128 h, 128 h + 128): 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16, transposed so that a lane holds 4 consecutive
// output columns.  A step covers 64 weight rows:
//  - dY: the 256 x 64 tile goes to LDS by direct global-to-LDS loads (two
//    stages, swizzled rows), issued one step ahead;
//  - W: column quarter w is expanded into a Wt tile in LDS, Wt[col][row] (two
//    buffers per quarter), shared by the two waves (0, w) and (1, w): wave
//    (h, w) expands weight rows 32 h .. 32 h + 31 of the step.  Lane
//    (g, q) = (lane % 4, lane / 4) holds the codes of rows 32 h + 8 g .. + 7 at
//    columns 4 q .. 4 q + 3 (one 2-byte load per row), looks up the level
//    pair of each code byte (a 256-entry table in LDS, read half a step ahead
//    of use), multiplies by the row's block scale and rounds once to bf16 --
//    the value nf4_dequantize writes -- and stores each column's 8 values as
//    one 16-byte run.  Runs of a Wt row are swizzled (run c of column k at
//    slot c ^ ((k / 16) % 8), rows padded to 144 bytes), which keeps both
//    these stores and the fragment reads free of bank conflicts.
//  - Software pipeline: while the MFMAs of step s run, the wave expands its
//    half of step s + 1 (codes loaded during step s - 1) and loads the codes
//    of step s + 2; the one barrier per step guards the dY stages and the
//    shared Wt buffers.  The step's body is kept free of branches so that
//    the expansion can be interleaved with the MFMAs, and the second wave on
//    each SIMD fills the gaps of the first.
// A last partial step (rows % 64 != 0) loads its dY tile through registers,
// zero past the end.
//
// The LoRA term is folded in as extra reduction indices,
//   [dY | U_hi | U_lo] . [deq(W) ; A ; A]  with U = s . dY . B,
// U split into two bf16 parts (hi = bf16(U), lo = bf16(U - hi)) by the LoRA
// prep kernel (run on dY and B transposed), so the adapter product keeps
// about 16 significant bits.
#include "gemm_tiles.h"

namespace nf4i {
namespace {

using gt::bf16x8;
using gt::floatx16;
using gt::u32x4;

constexpr int kDxThreads = 512;           // 8 waves
constexpr int kMI = 4;                    // 32 x 32 tiles per wave along m (128 rows)
constexpr int kP = 4;                     // dY pieces per thread and step
constexpr int kTm = 256, kTk = gt::kTileN, kStep = gt::kStep;
constexpr int kStageBytes = gt::act_stage_bytes<kTm>();
constexpr int kWtRowB = 144;              // 64 bf16 + 16 bytes of padding
constexpr int kWtBytes = 64 * kWtRowB;    // one quarter's Wt tile: 64 columns x 64 rows
constexpr int kPairCopies = 8;

struct DxArgs {
  const uint8_t* packed;
  int64_t rows, cols;  // W [rows][cols]
  Scales sc;
  const uint16_t* dy;  // [m][rows]
  int64_t m;
  uint16_t* dx;        // [m][cols]
  const uint16_t* u;   // [m][kl]: (s U hi | s U lo | 0), or null
  const uint16_t* la;  // LoRA A [r][cols]
  int r, r_pad, kl;
  Codebook cb;
};

// Byte offset of run c (reduction indices 8 c .. 8 c + 7) of Wt row k.
__device__ __forceinline__ uint32_t wt_off(int k, int c) {
  return static_cast<uint32_t>(k * kWtRowB + 16 * (c ^ ((k >> 4) & 7)));
}

// What a lane loads for one step: the codes of its 8 rows (2 bytes each,
// columns 4 q .. 4 q + 3) and the scale inputs of row 32 h + lane % 32 of the
// step (block of the wave's 64 columns).
struct CodeRegs {
  uint32_t w[8];
  float am;
  int q;
  float s2;
};

struct CodePtrs {
  const uint8_t* c;    // the wave's first code byte in weight row 0 (the same in every lane)
  uint32_t off;        // the lane's 2 bytes in row 32 h + 8 g: (32 h + 8 g) row_bytes + 2 q
  uint32_t row_bytes;  // cols / 2
  int r0;              // 32 h + 8 g: the lane's first row within a step
  int rs;              // 32 h + lane % 32: the row whose scale the lane loads
  int64_t kb;          // the wave's column block
  int64_t nbr;         // blocks per row
};

template <bool kDQ>
__device__ __forceinline__ void load_codes(CodeRegs& r, const CodePtrs& p, const DxArgs& a, int64_t ks, int q) {
  const int64_t n0 = ks * kStep;
  if (n0 + kStep <= a.rows) {  // a whole step: no clamping
    const uint8_t* b = p.c + n0 * p.row_bytes;
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) r.w[r8] = *reinterpret_cast<const uint16_t*>(b + p.off + r8 * p.row_bytes);
  } else {  // rows past the end re-read the last one (they meet zero dY)
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      const int64_t n = n0 + p.r0 + r8 < a.rows ? n0 + p.r0 + r8 : a.rows - 1;
      r.w[r8] = *reinterpret_cast<const uint16_t*>(p.c + n * p.row_bytes + 2 * q);
    }
  }
  const int64_t nl = n0 + p.rs < a.rows ? n0 + p.rs : a.rows - 1;
  const int64_t b = nl * p.nbr + p.kb;
  if constexpr (kDQ) {
    r.q = a.sc.q[b];
    r.s2 = a.sc.absmax2[b >> 8];
  } else {
    r.am = a.sc.absmax[b];
  }
}

// The scale form is a template parameter (see the forward GEMM).
template <bool kDQ, bool kF8>
__device__ __forceinline__ float row_scale(const CodeRegs& r, float mean) {
  if constexpr (kDQ) return code_ratio(r.q, kF8 ? 1 : 0) * r.s2 + mean;  // a_hat: three roundings (contraction is off)
  else return r.am;
}

// The 256 level pairs of a code byte (element 2 j = high nibble first), in
// kPairCopies interleaved copies: entry e of copy c at byte e * 64 + c * 8.
// A lane reads copy lane % 8, which spreads the lookups of 8 lanes over all
// 64 banks.  Ends with a barrier.
__device__ __forceinline__ void fill_pairs(float2* tab, const Codebook& cb) {
  if (threadIdx.x < 256) {
    const int e = threadIdx.x;
    const float2 v = make_float2(cb.level[e >> 4], cb.level[e & 15]);
#pragma unroll
    for (int c = 0; c < kPairCopies; ++c) tab[e * kPairCopies + c] = v;
  }
  __syncthreads();
}

// Level pairs of code byte b (columns 4 q + 2 b, 4 q + 2 b + 1) of the lane's 8 rows.
__device__ __forceinline__ void lookup_half(float2 (&l)[8], const uint32_t (&w)[8], const char* tab, int b,
                                            uint32_t slot) {
#pragma unroll
  for (int r8 = 0; r8 < 8; ++r8) {
    const uint32_t e = __builtin_amdgcn_ubfe(w[r8], 8 * b, 8);
    l[r8] = *reinterpret_cast<const float2*>(tab + ((e << 6) | slot));
  }
}

// Column 4 q + 2 b + c (c = 0: first of the pair) of the lane's 8 rows into Wt.
__device__ __forceinline__ void expand_col(char* wt, const float2 (&l)[8], const float (&ah)[8], int b, int c,
                                           int run, int q) {
  u32x4 o;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // fl32(level * a_hat), rounded once to bf16
    const float v0 = (c == 0 ? l[2 * p].x : l[2 * p].y) * ah[2 * p];
    const float v1 = (c == 0 ? l[2 * p + 1].x : l[2 * p + 1].y) * ah[2 * p + 1];
    o[p] = gt::bf16_pair(v0, v1);
  }
  *reinterpret_cast<u32x4*>(wt + wt_off(4 * q + 2 * b + c, run)) = o;
}

// Wt fragments of 16-wide step s for lane half h2: logical run 4 h2 + s (the
// activation fragments' order).
__device__ __forceinline__ void read_wt(const char* wt, int s, int lane, bf16x8 (&f)[2]) {
  const int h4 = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) f[j] = gt::lds_frag(wt + wt_off(32 * j + (lane & 31), h4 + s));
}

// Spreads the work issued next to the 8 MFMAs of one 16-wide step between them.
__device__ __forceinline__ void mfma_interleave() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);  // LDS read or write
  }
}

// dY tile of the last step when it is partial: loads through registers,
// zero past rows (rows % 8 == 0, so a 16-byte piece is all in or all out),
// stored where the direct loads would have put them.
__device__ __forceinline__ void act_tail(const gt::ActPtrs<kP>& p, int64_t ks, int64_t rows, char* stage, int wave,
                                         int lane) {
  const uint8_t* b = p.base + ks * (kStep * 2);
#pragma unroll
  for (int i = 0; i < kP; ++i) {
    const int64_t n = ks * kStep + 8 * gt::act_piece(i, lane);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < rows) v = *reinterpret_cast<const u32x4*>(b + p.off[i]);
    *reinterpret_cast<u32x4*>(stage + (kP * wave + i) * 1024 + 16 * lane) = v;
  }
}

template <bool kDQ, bool kF8>
__global__ __launch_bounds__(kDxThreads) void k_gemm_dx(DxArgs a) {
  __shared__ __align__(16) char stage0[kStageBytes], stage1[kStageBytes];
  __shared__ __align__(16) char wts[4][2][kWtBytes];
  __shared__ __align__(16) float scl[8][32];  // per wave: a_hat of its 32 rows of the step
  __shared__ __align__(16) float2 pairs[256 * kPairCopies];  // 16 KB
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wh = wave >> 2, wq = wave & 3;  // row half, column quarter
  const int g = lane & 3, q = lane >> 2;
  const uint32_t slot = static_cast<uint32_t>(lane & 7) << 3;
  const char* tab = reinterpret_cast<const char*>(pairs);
  const float mean = kDQ ? *a.sc.mean : 0.0f;

  const int64_t tiles_k = (a.cols + kTk - 1) / kTk;
  const int64_t tiles = tiles_k * ((a.m + kTm - 1) / kTm);
  int64_t tid = blockIdx.x;
  // consecutive tiles (one dY row strip) on one XCD: dispatch deals workgroups round-robin over 8
  if (tiles % 8 == 0) tid = (tid % 8) * (tiles / 8) + tid / 8;
  const int64_t m0 = (tid / tiles_k) * kTm;
  const int64_t k0 = (tid % tiles_k) * kTk;
  const int64_t nsteps = (a.rows + kStep - 1) / kStep;
  const bool ragged = (a.rows % kStep) != 0;

  const gt::ActPtrs<kP> ap = gt::make_act_ptrs<kP, kTm>(a.dy, a.rows, a.m, m0, wave, lane);
  CodePtrs cp;
  {
    const int64_t wc = k0 + 64 * wq;                        // the wave's first column
    const int64_t wcc = wc < a.cols ? wc : a.cols - 64;     // columns past the end: never stored
    cp.row_bytes = static_cast<uint32_t>(a.cols / 2);
    cp.c = a.packed + wcc / 2;
    cp.r0 = 32 * wh + 8 * g;
    cp.rs = 32 * wh + (lane & 31);
    cp.off = static_cast<uint32_t>(cp.r0) * cp.row_bytes + 2 * q;
    cp.nbr = a.cols / 64;
    cp.kb = wcc / 64;
  }
  char* wt0 = wts[wq][0];
  char* wt1 = wts[wq][1];
  float* scw = scl[wave];
  const int run = 4 * wh + g;  // the lane's 8-row group within a step: its Wt run

  floatx16 acc[kMI][2];
  gt::zero_acc(acc);
  const uint32_t sw = ((lane & 31) >> 1) & 7, h4 = (lane >> 5) * 4;
  const int xrow = 128 * wh + (lane & 31);  // the wave's first fragment row in a stage

  // a_hat of the lane's 8 rows from the wave's scale buffer (written just before, same wave)
  auto scales_of = [&](const CodeRegs& c, float (&ah)[8]) {
    scw[lane & 31] = row_scale<kDQ, kF8>(c, mean);
    const float4 a0 = *reinterpret_cast<const float4*>(scw + 8 * g);
    const float4 a1 = *reinterpret_cast<const float4*>(scw + 8 * g + 4);
    ah[0] = a0.x; ah[1] = a0.y; ah[2] = a0.z; ah[3] = a0.w; ah[4] = a1.x; ah[5] = a1.y; ah[6] = a1.z; ah[7] = a1.w;
  };

  // prologue: dY of step 0, Wt of step 0, codes of step 1
  CodeRegs c1, c2;
  if (ragged && nsteps == 1) act_tail(ap, 0, a.rows, stage0, wave, lane);
  else gt::dma_act_buf(ap, 0, stage0, wave);
  load_codes<kDQ>(c1, cp, a, 0, q);
  load_codes<kDQ>(c2, cp, a, nsteps > 1 ? 1 : 0, q);
  fill_pairs(pairs, a.cb);
  {
    float ah[8];
    scales_of(c1, ah);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float2 l[8];
      lookup_half(l, c1.w, tab, b, slot);
      expand_col(wt0, l, ah, b, 0, run, q);
      expand_col(wt0, l, ah, b, 1, run, q);
    }
  }
  c1 = c2;
  gt::wait_vmem();
  __syncthreads();
  // level pairs of byte 0 of the next expansion, half a step ahead of use
  float2 lk[2][8];
  lookup_half(lk[0], c1.w, tab, 0, slot);

  for (int64_t ks = 0; ks < nsteps; ++ks) {
    const int64_t kn = ks + 1 < nsteps ? ks + 1 : ks;
    char* st_cur = (ks & 1) ? stage1 : stage0;
    char* st_nxt = (ks & 1) ? stage0 : stage1;
    char* wt_cur = (ks & 1) ? wt1 : wt0;
    char* wt_nxt = (ks & 1) ? wt0 : wt1;
    // the next step's dY tile (the stage was last read before the previous
    // barrier); on the last step a harmless reload, so that the code below
    // stays one basic block for the scheduler
    if (ragged && kn == nsteps - 1) act_tail(ap, kn, a.rows, st_nxt, wave, lane);
    else gt::dma_act_buf(ap, kn, st_nxt, wave);
    load_codes<kDQ>(c2, cp, a, ks + 2 < nsteps ? ks + 2 : kn, q);
    float ah[8];
    scales_of(c1, ah);
    __builtin_amdgcn_sched_barrier(0);
    const char* xa = st_cur + xrow * gt::kActRowBytes;
    bf16x8 af[2][kMI], bw[2][2];
    gt::read_act(xa, 0, sw, h4, af[0]);
    read_wt(wt_cur, 0, lane, bw[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
        if (s == 0) lookup_half(lk[1], c1.w, tab, 1, slot);
        gt::read_act(xa, s + 1, sw, h4, af[(s + 1) & 1]);
        read_wt(wt_cur, s + 1, lane, bw[(s + 1) & 1]);
      }
      gt::mfma16(af[s & 1], bw[s & 1], acc);
      // byte s / 2, column s % 2 of it; on the last step into a buffer never read
      expand_col(wt_nxt, lk[s >> 1], ah, s >> 1, s & 1, run, q);
      mfma_interleave();
      __builtin_amdgcn_sched_barrier(0);
    }
    c1 = c2;
    gt::wait_vmem();
    __syncthreads();
    lookup_half(lk[0], c1.w, tab, 0, slot);
  }

  // LoRA: reduction indices of [U_hi | U_lo | 0] against [A ; A ; 0]
  if (a.kl > 0) {
    const gt::ActPtrs<kP> up = gt::make_act_ptrs<kP, kTm>(a.u, a.kl, a.m, m0, wave, lane);
    for (int64_t j0 = 0; j0 < a.kl; j0 += kStep) {
      gt::dma_act_buf(up, j0 / kStep, stage0, wave);
      // quarter wq's Wt: column k0 + 64 wq + 4 q + c, run 4 wh + g holds A[j0 + 8 run + e][column]
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t col = k0 + 64 * wq + 4 * q + c;
        const int64_t cc = col < a.cols ? col : a.cols - 1;
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t jj = j0 + 8 * run + e;
          const int64_t ja = jj < a.r_pad ? jj : jj - a.r_pad;
          const bool live = jj < 2 * a.r_pad && ja < a.r;
          h[e] = live ? a.la[ja * a.cols + cc] : 0u;
        }
        const u32x4 o = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        *reinterpret_cast<u32x4*>(wt0 + wt_off(4 * q + c, run)) = o;
      }
      gt::wait_vmem();
      __syncthreads();
      const char* xa = stage0 + xrow * gt::kActRowBytes;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 af[kMI], bw[2];
        gt::read_act(xa, s, sw, h4, af);
        read_wt(wt0, s, lane, bw);
        gt::mfma16(af, bw, acc);
      }
      __syncthreads();
    }
  }

  gt::store_acc(acc, a.dx, a.m, a.cols, m0 + 128 * wh, k0, wq, lane);
}

// Elements of u before Bt in the workspace, rounded up to 256 bytes.
int64_t u_elems(int64_t m, int r) {
  return (m * static_cast<int64_t>(gemm_lora_cols(r)) + 127) / 128 * 128;
}

}  // namespace

// Bt[j][n] = B[n][j], so that the prep reads both of its operands along n.
static __global__ __launch_bounds__(256) void k_transpose_b(const uint16_t* __restrict__ lb, int64_t rows, int r,
                                                            uint16_t* __restrict__ bt) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * r) return;
  const int64_t n = i / r, j = i - n * r;
  bt[j * rows + n] = lb[i];
}

hipError_t launch_transpose_b(const uint16_t* b, int64_t rows, int r, uint16_t* bt, hipStream_t s) {
  const int64_t nt = rows * r;
  if ((nt + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_transpose_b, dim3(static_cast<unsigned>((nt + 255) / 256)), dim3(256), 0, s, b, rows, r, bt);
  return hipSuccess;
}

size_t gemm_dx_workspace(int64_t m, int64_t rows, int r) {
  if (r <= 0) return 0;
  return static_cast<size_t>(u_elems(m, r) + rows * r) * sizeof(uint16_t);
}

hipError_t launch_gemm_dx(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* dy,
                          int64_t m, uint16_t* dx, const uint16_t* lora_a, const uint16_t* lora_b, int r,
                          float lora_scale, uint16_t* ws, hipStream_t s) {
  DxArgs a{};
  a.packed = packed; a.rows = rows; a.cols = cols; a.sc = sc; a.dy = dy; a.m = m; a.dx = dx;
  a.cb = codebook(sc.fp4);
  const int64_t tiles = ((m + kTm - 1) / kTm) * ((cols + kTk - 1) / kTk);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (r > 0) {
    a.r = r;
    a.r_pad = (r + 15) / 16 * 16;
    a.kl = static_cast<int>(gemm_lora_cols(r));
    a.la = lora_a;
    a.u = ws;
    uint16_t* bt = ws + u_elems(m, r);
    if (hipError_t e = launch_transpose_b(lora_b, rows, r, bt, s)) return e;
    if (hipError_t e = launch_lora_u(dy, bt, m, rows, r, lora_scale, ws, s)) return e;
  }
  const dim3 gd(static_cast<unsigned>(tiles)), bd(kDxThreads);
  if (sc.absmax) hipLaunchKernelGGL((k_gemm_dx<false, false>), gd, bd, 0, s, a);
  else if (sc.f8) hipLaunchKernelGGL((k_gemm_dx<true, true>), gd, bd, 0, s, a);
  else hipLaunchKernelGGL((k_gemm_dx<true, false>), gd, bd, 0, s, a);
  return hipGetLastError();
}

}  // namespace nf4i
