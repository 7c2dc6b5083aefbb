// Input gradient through the frozen 4-bit base, for QLoRA training (tutorial
// page "bitsandbytes quantization tutorial: 4-bit and 8-bit models", section
// "QLoRA: Fine-Tuning a 4-bit Model": the base stays frozen while gradients
// pass through it to the adapters):
//
//   dX = dY . deq(W) + s . (dY . B) . A          dY [m][rows], dX [m][cols]
//
// The reduction runs over the weight's rows, so W enters in the other
// orientation than in the forward GEMM: its NF4 codes are expanded into LDS
// transposed, as Wt[col][row], and both MFMA operands are then read as
// 16-byte runs along the reduction index.
//
// Tiling: a workgroup of 4 waves computes a 256 (m) x 256 (col) tile of dX;
// wave w owns columns [64 w, 64 w + 64) for all 256 rows of dY, 8 x 2 tiles
// of v_mfma_f32_32x32x16_bf16 per 16-wide reduction step, computed transposed
// (Wt fragment as A, dY fragment as B) so that each lane ends up with 4
// consecutive output columns.  One step covers 64 weight rows:
//  1. the dY tile (256 x 64 bf16), the raw codes (64 weight rows x 256
//     columns, 8 KB) and the 64 x 4 block scales are written to LDS from
//     registers (their global loads were issued during the previous step);
//  2. each thread expands 8 weight rows x 8 columns: level x block scale,
//     rounded once to bf16 -- the value nf4_dequantize writes -- and stores
//     each column's 8 values as one 16-byte run of Wt;
//  3. the MFMAs read dY and Wt fragments from LDS.
// LDS rows are 144 bytes (64 bf16 + 16 bytes of padding), so fragment reads
// of consecutive rows fall in distinct banks; in Wt the 16-byte run c of row
// k sits at slot c ^ ((k / 16) % 8), which also spreads the expansion's
// stores (lanes write rows 8 apart) over the banks without moving the
// fragment reads of any 16 consecutive rows.
//
// The LoRA term is folded in as extra reduction indices,
//   [dY | U_hi | U_lo] . [deq(W) ; A ; A]  with U = s . dY . B,
// U split into two bf16 parts (hi = bf16(U), lo = bf16(U - hi)) by the same
// prep kernel as the forward GEMM's (run on dY and B transposed), so the
// adapter product keeps about 16 significant bits.
#include "nf4_device.h"

namespace nf4i {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kTm = 256, kTk = 256, kStep = 64;
constexpr int kRowB = 144;  // 64 bf16 (128 bytes) + 16 bytes of padding per LDS row
constexpr int kThr = 256;

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

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const bf16x2_t p = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // round to nearest even
  return __builtin_bit_cast(uint32_t, p);
}

// Byte offset of the 16-byte run c (reduction indices 8 c .. 8 c + 7) of Wt row k.
__device__ __forceinline__ int wt_off(int k, int c) { return k * kRowB + 16 * (c ^ ((k >> 4) & 7)); }

// Global loads of one reduction step, held in registers until the LDS is free.
struct StepRegs {
  uint4 dy[8];    // piece t + 256 i: dY tile row (t + 256 i) / 8, 16-byte run (t + 256 i) % 8
  uint4 code[2];  // piece t + 256 i: weight row (t + 256 i) / 8 of the step, 16 bytes (t + 256 i) % 8
  float am;       // plain scale of (weight row t / 4, tile block t % 4)
  int q;
  float s2;
};

template <bool kDQ>
__device__ __forceinline__ void load_step(StepRegs& g, const DxArgs& a, int64_t m0, int64_t k0, int64_t n0) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = t + kThr * i;
    const int64_t row = m0 + (p >> 3);
    const int64_t rc = row < a.m ? row : a.m - 1;  // rows past the end: never stored
    const int64_t n = n0 + 8 * (p & 7);           // rows % 8 == 0: a run is all in or all out
    g.dy[i] = n < a.rows ? *reinterpret_cast<const uint4*>(a.dy + rc * a.rows + n) : make_uint4(0, 0, 0, 0);
  }
  const int64_t half_cols = a.cols / 2;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = t + kThr * i;
    int64_t wrow = n0 + (p >> 3);
    wrow = wrow < a.rows ? wrow : a.rows - 1;     // meets zero dY: adds nothing
    int64_t off = k0 / 2 + 16 * (p & 7);          // byte within the weight row
    off = off + 16 <= half_cols ? off : half_cols - 16;  // columns past the end: never stored
    g.code[i] = *reinterpret_cast<const uint4*>(a.packed + wrow * half_cols + off);
  }
  int64_t wrow = n0 + (t >> 2);
  wrow = wrow < a.rows ? wrow : a.rows - 1;
  const int64_t nbr = a.cols / 64;
  int64_t kb = k0 / 64 + (t & 3);
  kb = kb < nbr ? kb : nbr - 1;
  const int64_t b = wrow * nbr + kb;
  if constexpr (kDQ) {
    g.q = a.sc.q[b];
    g.s2 = a.sc.absmax2[b >> 8];
  } else {
    g.am = a.sc.absmax[b];
  }
}

template <bool kDQ>
__global__ __launch_bounds__(kThr) void k_gemm_dx(DxArgs a) {
  __shared__ __align__(16) char dyt[kTm * kRowB];      // dY tile [m][64 reduction]
  __shared__ __align__(16) char wt[kTk * kRowB];       // Wt tile [col][64 reduction], runs swizzled
  __shared__ __align__(16) char codes[kStep * kRowB];  // raw codes [64 weight rows][128 bytes]
  __shared__ float scl[kStep * 4];                     // scale of (weight row, tile block)
  __shared__ float lv[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t < 16) lv[t] = a.cb.level[t];
  const float mean = kDQ ? *a.sc.mean : 0.0f;
  const int64_t tiles_k = (a.cols + kTk - 1) / kTk;
  const int64_t m0 = (static_cast<int64_t>(blockIdx.x) / tiles_k) * kTm;
  const int64_t k0 = (static_cast<int64_t>(blockIdx.x) % tiles_k) * kTk;
  const int64_t nsteps = (a.rows + kStep - 1) / kStep;

  floatx16_t acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Fragments of 16-wide step s: Wt rows 64 w + 32 j + lane % 32 and dY rows
  // 32 i + lane % 32, each at reduction indices 16 s + 8 (lane / 32) .. + 7.
  auto mfma_step = [&]() {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 2 * s + (lane >> 5);
      bf16x8_t af[2], bfr[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        af[j] = *reinterpret_cast<const bf16x8_t*>(wt + wt_off(wave * 64 + j * 32 + (lane & 31), c));
#pragma unroll
      for (int i = 0; i < 8; ++i)
        bfr[i] = *reinterpret_cast<const bf16x8_t*>(dyt + (i * 32 + (lane & 31)) * kRowB + 16 * c);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j], bfr[i], acc[i][j], 0, 0, 0);
    }
  };

  StepRegs g;
  if (nsteps > 0) load_step<kDQ>(g, a, m0, k0, 0);
  for (int64_t ns = 0; ns < nsteps; ++ns) {
    __syncthreads();  // the previous step's MFMAs are done with dyt and wt
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = t + kThr * i;
      *reinterpret_cast<uint4*>(dyt + (p >> 3) * kRowB + 16 * (p & 7)) = g.dy[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = t + kThr * i;
      *reinterpret_cast<uint4*>(codes + (p >> 3) * kRowB + 16 * (p & 7)) = g.code[i];
    }
    if constexpr (kDQ) scl[t] = div127(g.q) * g.s2 + mean;  // a_hat: three roundings (contraction is off)
    else scl[t] = g.am;
    __syncthreads();
    // the next step's loads go out now and land while this step expands and multiplies
    const int64_t nn = ns + 1 < nsteps ? ns + 1 : ns;
    load_step<kDQ>(g, a, m0, k0, nn * kStep);
    {
      // weight rows 8 g8 .. 8 g8 + 7 of the step, tile columns 8 kg .. 8 kg + 7
      const int g8 = t >> 5, kg = t & 31;
      float v[8][8];
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8) {
        const int wr = 8 * g8 + r8;
        const uint32_t word = *reinterpret_cast<const uint32_t*>(codes + wr * kRowB + 4 * kg);
        const float ah = scl[wr * 4 + (kg >> 3)];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t code = (word >> (8 * (c >> 1) + ((c & 1) ? 0 : 4))) & 0xFu;  // high nibble first
          v[r8][c] = lv[code] * ah;  // fl32(level * a_hat)
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 o = make_uint4(bf16_pair(v[0][c], v[1][c]), bf16_pair(v[2][c], v[3][c]),
                                   bf16_pair(v[4][c], v[5][c]), bf16_pair(v[6][c], v[7][c]));
        *reinterpret_cast<uint4*>(wt + wt_off(8 * kg + c, g8)) = o;
      }
    }
    __syncthreads();
    mfma_step();
  }

  // LoRA: reduction indices of [U_hi | U_lo | 0] against [A ; A ; 0]
  for (int64_t j0 = 0; j0 < a.kl; j0 += kStep) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = t + kThr * i;
      const int64_t row = m0 + (p >> 3);
      const int64_t rc = row < a.m ? row : a.m - 1;
      *reinterpret_cast<uint4*>(dyt + (p >> 3) * kRowB + 16 * (p & 7)) =
          *reinterpret_cast<const uint4*>(a.u + rc * a.kl + j0 + 8 * (p & 7));
    }
    {
      // thread t fills Wt row t (tile column k0 + t) with A[j][col] for the step's 64 indices
      const int64_t col = k0 + t;
      const int64_t cc = col < a.cols ? col : a.cols - 1;
#pragma unroll
      for (int jg = 0; jg < 8; ++jg) {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t jj = j0 + 8 * jg + e;
          const int64_t ja = jj < a.r_pad ? jj : jj - a.r_pad;
          const bool live = jj < 2 * a.r_pad && ja < a.r;
          h[e] = live ? a.la[ja * a.cols + cc] : 0u;
        }
        *reinterpret_cast<uint4*>(wt + wt_off(t, jg)) =
            make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      }
    }
    __syncthreads();
    mfma_step();
  }

  // epilogue: of each 32 x 32 tile of dX^T the lane holds element e at output
  // column (e % 4) + 4 (lane / 32) + 8 (e / 4) and output row lane % 32
  const bool vec = (a.cols & 3) == 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = m0 + i * 32 + (lane & 31);
    if (row >= a.m) continue;
    uint16_t* dr = a.dx + row * a.cols;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int64_t col = k0 + wave * 64 + j * 32 + 4 * (lane >> 5) + 8 * gq;
        const uint32_t p0 = bf16_pair(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]);
        const uint32_t p1 = bf16_pair(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
        if (vec && col + 3 < a.cols) {
          *reinterpret_cast<uint2*>(dr + col) = make_uint2(p0, p1);
        } else {
          const uint16_t vv[4] = {static_cast<uint16_t>(p0), static_cast<uint16_t>(p0 >> 16),
                                  static_cast<uint16_t>(p1), static_cast<uint16_t>(p1 >> 16)};
          for (int e = 0; e < 4; ++e)
            if (col + e < a.cols) dr[col + e] = vv[e];
        }
      }
    }
  }
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
  a.cb = codebook();
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
  if (sc.absmax) hipLaunchKernelGGL(k_gemm_dx<false>, dim3(static_cast<unsigned>(tiles)), dim3(kThr), 0, s, a);
  else hipLaunchKernelGGL(k_gemm_dx<true>, dim3(static_cast<unsigned>(tiles)), dim3(kThr), 0, s, a);
  return hipGetLastError();
}

}  // namespace nf4i
