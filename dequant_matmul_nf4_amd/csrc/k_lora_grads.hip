// Gradients of the low-rank adapters on the frozen 4-bit base (tutorial page
// "bitsandbytes quantization tutorial: 4-bit and 8-bit models", section
// "QLoRA: Fine-Tuning a 4-bit Model": only the adapters train).  For
// y = x . deq(W)^T + s . (x . A^T) . B^T:
//
//   dA = s . (dY . B)^T . X     [r][cols]
//   dB = s . dY^T . (X . A^T)   [rows][r]
//
// Both are C[j][n] = sum_i P[i][j] Q[i][n] with a thin float32 P [m][r] and a
// wide bf16 Q [m][N]: P = s dY B and Q = X for dA; P = s X A^T and Q = dY for
// dB (written transposed).  The thin factors come from the LoRA prep kernel in
// float32.  The wide one is read once: a wave owns 512 consecutive columns
// (8 per lane, one 16-byte load per row) and 16 rank entries, and walks rows
// of Q; the 16 values P[i][j0 .. j0 + 15] of a row are the same for the whole
// wave, staged in LDS and read as broadcasts, and feed 128 fused
// multiply-adds per lane.  Rows are split over the four waves of a workgroup (summed in LDS)
// and over workgroups (grid y, summed by k_grad_reduce in a fixed order, so
// results are deterministic).  float32 accumulation throughout.
#include "nf4_device.h"

namespace nf4i {
namespace {

constexpr int kGW = 4;              // waves per workgroup
constexpr int kGCols = 8 * kWave;   // columns per workgroup
constexpr int kGJ = 16;             // rank entries per pass
constexpr int kGU = 4;              // rows of Q per wave per iteration
constexpr int kGChunk = 256;        // rows of P staged in LDS at a time
constexpr int kGTargetWg = 512;     // workgroups to aim for (two per compute unit)

struct GradPlan {
  int64_t chunks, splits, rows_per_split;
  int passes;
};

GradPlan grad_plan(int64_t m, int64_t n, int r) {
  GradPlan p;
  p.chunks = (n + kGCols - 1) / kGCols;
  p.passes = (r + kGJ - 1) / kGJ;
  const int64_t want = (kGTargetWg + p.chunks * p.passes - 1) / (p.chunks * p.passes);
  const int64_t most = (m + 4 * kGW - 1) / (4 * kGW);  // at least 4 rows per wave
  p.splits = want < most ? want : most;
  if (p.splits < 1) p.splits = 1;
  if (p.splits > 65535) p.splits = 65535;
  p.rows_per_split = (m + p.splits - 1) / p.splits;
  p.splits = (m + p.rows_per_split - 1) / p.rows_per_split;
  return p;
}

// part[split][j][n] = sum over the split's rows i of p[i][j] q[i][n], for
// j in [16 z, 16 z + 16) (p rows hold r_pad floats, zero past r).  The split's
// rows go in chunks of kGChunk: their P values are staged in LDS, then each
// wave takes rows c0 + wave + kGW k of the chunk, kGU at a time with the next
// kGU rows of Q already loading.
__global__ __launch_bounds__(kGW * kWave) void k_grad_partial(const float* __restrict__ p, int r_pad,
                                                              const uint16_t* __restrict__ q, int64_t m, int64_t n,
                                                              int64_t rows_per_split, float* __restrict__ part) {
  __shared__ float red[kGJ * kGCols];     // 32 KB
  __shared__ float4 pl[kGChunk * kGJ / 4];  // 16 KB
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t col = static_cast<int64_t>(blockIdx.x) * kGCols + 8 * lane;
  const int j0 = blockIdx.z * kGJ;
  const int64_t i0 = static_cast<int64_t>(blockIdx.y) * rows_per_split;
  const int64_t i1 = i0 + rows_per_split < m ? i0 + rows_per_split : m;
  const bool live = col < n;  // n % 8 == 0: a lane's 8 columns are all in or all out
  const uint16_t* qc = q + (live ? col : 0);

  float acc[kGJ][8];
#pragma unroll
  for (int j = 0; j < kGJ; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[j][c] = 0.0f;

  auto fma_row = [&](const uint4& v, int pr) {  // pr: row within the chunk
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
    float pj[kGJ];
#pragma unroll
    for (int j4 = 0; j4 < kGJ / 4; ++j4) {
      const float4 f = pl[pr * (kGJ / 4) + j4];  // the same address in every lane
      pj[4 * j4] = f.x; pj[4 * j4 + 1] = f.y; pj[4 * j4 + 2] = f.z; pj[4 * j4 + 3] = f.w;
    }
#pragma unroll
    for (int j = 0; j < kGJ; ++j)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[j][c] = fmaf(pj[j], x[c], acc[j][c]);
  };

  for (int64_t c0 = i0; c0 < i1; c0 += kGChunk) {
    const int rows = static_cast<int>(i1 - c0 < kGChunk ? i1 - c0 : kGChunk);
    __syncthreads();  // the previous chunk's reads of pl are done
    for (int t = threadIdx.x; t < rows * (kGJ / 4); t += kGW * kWave)
      pl[t] = *reinterpret_cast<const float4*>(p + (c0 + t / (kGJ / 4)) * r_pad + j0 + 4 * (t % (kGJ / 4)));
    __syncthreads();
    const int nr = rows - wave > 0 ? (rows - wave + kGW - 1) / kGW : 0;  // this wave's rows
    const int last = nr > 0 ? wave + (nr - 1) * kGW : 0;
    auto row_of = [&](int k) { return k < nr ? wave + k * kGW : last; };  // clamped: stays in bounds
    uint4 nxt[kGU];
#pragma unroll
    for (int u = 0; u < kGU; ++u) nxt[u] = *reinterpret_cast<const uint4*>(qc + (c0 + row_of(u)) * n);
    int k0 = 0;
    for (; k0 + kGU <= nr; k0 += kGU) {  // whole groups
      uint4 cur[kGU];
#pragma unroll
      for (int u = 0; u < kGU; ++u) {
        cur[u] = nxt[u];
        nxt[u] = *reinterpret_cast<const uint4*>(qc + (c0 + row_of(k0 + kGU + u)) * n);
      }
#pragma unroll
      for (int u = 0; u < kGU; ++u) fma_row(cur[u], row_of(k0 + u));
    }
#pragma unroll
    for (int u = 0; u < kGU - 1; ++u)  // the last partial group, already loaded
      if (k0 + u < nr) fma_row(nxt[u], row_of(k0 + u));
  }

  // waves 1..3 add their sums into LDS in turn; wave 0 adds the total to its own
  for (int w = 1; w < kGW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int j = 0; j < kGJ; ++j)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float* d = &red[j * kGCols + 8 * lane + c];
          *d = (w == 1 ? 0.0f : *d) + acc[j][c];
        }
    }
    __syncthreads();
  }
  if (wave != 0 || !live) return;
  float* out = part + (static_cast<int64_t>(blockIdx.y) * r_pad + j0) * n + col;
#pragma unroll
  for (int j = 0; j < kGJ; ++j) {
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = acc[j][c] + red[j * kGCols + 8 * lane + c];
    *reinterpret_cast<float4*>(out + j * n) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(out + j * n + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
}

// out = sum over splits of part (split ascending); a thread sums 4
// consecutive columns of one rank entry, eight splits per iteration.
// transposed: out[n][j] (rows of r floats), else out[j][n].
__global__ __launch_bounds__(256) void k_grad_reduce(const float* __restrict__ part, int64_t splits, int r, int r_pad,
                                                     int64_t n, int transposed, float* __restrict__ out) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n4 = n / 4;  // n % 8 == 0
  if (e >= n4 * r) return;
  const int64_t j = e / n4, col = 4 * (e - j * n4);
  const float* pp = part + j * n + col;
  const int64_t stride = static_cast<int64_t>(r_pad) * n;
  float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  int64_t sp = 0;
  for (; sp + 8 <= splits; sp += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(pp + (sp + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
    }
  }
  for (; sp < splits; ++sp) {
    const float4 v = *reinterpret_cast<const float4*>(pp + sp * stride);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if (transposed) {
    out[col * r + j] = s.x;
    out[(col + 1) * r + j] = s.y;
    out[(col + 2) * r + j] = s.z;
    out[(col + 3) * r + j] = s.w;
  } else {
    *reinterpret_cast<float4*>(out + j * n + col) = s;
  }
}

hipError_t grad_tn(const float* p, int r, const uint16_t* q, int64_t m, int64_t n, float* part, int transposed,
                   float* out, hipStream_t s) {
  const GradPlan pl = grad_plan(m, n, r);
  const int r_pad = (r + 15) / 16 * 16;
  if (pl.chunks > 0x7FFFFFFF || (n / 4 * r + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_grad_partial, dim3(static_cast<unsigned>(pl.chunks), static_cast<unsigned>(pl.splits),
                                          static_cast<unsigned>(pl.passes)),
                     dim3(kGW * kWave), 0, s, p, r_pad, q, m, n, pl.rows_per_split, part);
  hipLaunchKernelGGL(k_grad_reduce, dim3(static_cast<unsigned>((n / 4 * r + 255) / 256)), dim3(256), 0, s, part,
                     pl.splits, r, r_pad, n, transposed, out);
  return hipSuccess;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct GradLayout {
  size_t bt, pu, pt, part, total;  // byte offsets
};

GradLayout grad_layout(int64_t m, int64_t rows, int64_t cols, int r) {
  const int r_pad = (r + 15) / 16 * 16;
  const GradPlan pa = grad_plan(m, cols, r), pb = grad_plan(m, rows, r);
  const size_t part_a = static_cast<size_t>(pa.splits) * r_pad * cols * sizeof(float);
  const size_t part_b = static_cast<size_t>(pb.splits) * r_pad * rows * sizeof(float);
  GradLayout l;
  l.bt = 0;
  l.pu = align256(static_cast<size_t>(rows) * r * sizeof(uint16_t));
  l.pt = l.pu + align256(static_cast<size_t>(m) * r_pad * sizeof(float));
  l.part = l.pt + align256(static_cast<size_t>(m) * r_pad * sizeof(float));
  l.total = l.part + align256(part_a > part_b ? part_a : part_b);
  return l;
}

}  // namespace

size_t lora_grads_workspace(int64_t m, int64_t rows, int64_t cols, int r) {
  if (m < 1 || rows < 1 || cols < 1 || r < 1) return 0;
  return grad_layout(m, rows, cols, r).total;
}

hipError_t launch_lora_grads(const uint16_t* x, const uint16_t* dy, int64_t m, int64_t rows, int64_t cols,
                             const uint16_t* lora_a, const uint16_t* lora_b, int r, float scale, float* da,
                             float* db, void* ws, hipStream_t s) {
  const GradLayout l = grad_layout(m, rows, cols, r);
  char* base = static_cast<char*>(ws);
  uint16_t* bt = reinterpret_cast<uint16_t*>(base + l.bt);
  float* pu = reinterpret_cast<float*>(base + l.pu);
  float* pt = reinterpret_cast<float*>(base + l.pt);
  float* part = reinterpret_cast<float*>(base + l.part);
  if (da) {
    // U = s dY B: the prep reads dY and B transposed along the rows of W
    if (hipError_t e = launch_transpose_b(lora_b, rows, r, bt, s)) return e;
    if (hipError_t e = launch_lora_t32(dy, bt, m, rows, r, scale, pu, s)) return e;
    if (hipError_t e = grad_tn(pu, r, x, m, cols, part, 0, da, s)) return e;
  }
  if (db) {
    // T = s X A^T
    if (hipError_t e = launch_lora_t32(x, lora_a, m, cols, r, scale, pt, s)) return e;
    if (hipError_t e = grad_tn(pt, r, dy, m, rows, part, 1, db, s)) return e;
  }
  return hipGetLastError();
}

}  // namespace nf4i
