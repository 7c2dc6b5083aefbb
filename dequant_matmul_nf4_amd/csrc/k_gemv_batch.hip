// Decode GEMV over several weights in one launch: y_i = x_i . deq(W_i)^T at
// m = 1 for up to kGemvBatchMax weights (bitsandbytes tool page, "How it
// works", Step 5: each block is expanded with its scale and multiplied; the
// expanded copy never leaves the registers).
//
// A decode step multiplies one token's activations by every weight of a
// layer; several of those products share their input (the attention
// projections, the two MLP input projections).  Launched one by one, each
// small product pays the launch, the level-table fill and the first memory
// round trip again, and the chip idles in every tail.  Here one persistent
// grid streams all of them:
//  - weights that share x (same pointer and width) form a group whose rows
//    are concatenated into one virtual row range;
//  - each group is cut as the single-weight streaming kernel cuts a weight
//    (column segments of up to 64 blocks, the rows in parts interleaved over
//    the whole grid, so the chip reads one contiguous window at a time);
//  - a wave walks its rows of group 0, then of group 1, ..., and requests
//    the next row one step ahead across the group boundaries, so the memory
//    pipe does not drain between weights;
//  - a wave keeps the x values of its column segment in registers as fp16
//    (each 64-value block scaled by a power of two chosen from its largest
//    |x|); the x of its next group is requested together with that group's
//    first row, one step before the wave needs it;
//  - partial sums of every (row, segment) stay in LDS until the end, when
//    each row's segments are added in a fixed order (results do not depend
//    on timing) and written to that weight's y.
#include "gemv_rows.h"

namespace nf4i {
namespace {

constexpr int kBWaves = 16;
constexpr int kAhead = 1;          // rows requested ahead of the one in use
constexpr int kSlots = kAhead + 1; // register slots of the row ring
constexpr int kBPartMax = 2048;    // partial sums per workgroup (floats)

struct BMat {
  const uint8_t* packed;
  const float* absmax;   // plain scales, or
  const int8_t* q;       // double-quantized scales
  const float* absmax2;
  const float* mean;
  void* y;
  int64_t vrow0;         // first virtual row within its group
  int64_t rows;
};

struct BGroup {
  const uint16_t* x;
  int64_t vrows;         // rows of all its weights
  int64_t nblk;          // blocks per row
  int nseg, seg_blocks, wpr, kmax;
  int mat0, mat1;        // its weights
  int part0;             // first partial-sum slot (per workgroup)
};

struct BArgs {
  BMat mat[kGemvBatchMax];
  BGroup grp[kGemvBatchMax];
  int ngroups;
  Codebook cb;
};

// The lane's piece offsets in a row segment of group G (as k_gemv_rows).
__device__ __forceinline__ void lane_offsets(const BGroup& G, int seg, int lane, LaneOffs& lo, bool (&on)[2],
                                             int (&blk)[2]) {
  const int seg_end = static_cast<int>(G.nblk - seg * G.seg_blocks < G.seg_blocks ? G.nblk - seg * G.seg_blocks
                                                                                  : G.seg_blocks);
  make_lane_offs(seg * G.seg_blocks, seg_end, lane, lo, on, blk);
}

// A wave's walk over its rows (wave-uniform state, kept in scalar
// registers): group g, rows left in it, the current virtual row v (rows v,
// v + np, ... of the group), the weight m that holds v (rows before mend),
// and v's first block within that weight.  Group and weight parameters are
// read from the kernel arguments only when the walk enters a new group or
// weight, not per row.
struct Walk {
  int g, m, seg, prt;
  int64_t left, i, v, np, mend, blk0, nblk;
};

__device__ __forceinline__ void walk_weight(Walk& w, const BArgs& a) {
  // the weight holding w.v (weights of a group are consecutive in v)
  while (w.m + 1 < a.grp[w.g].mat1 && w.v >= a.mat[w.m + 1].vrow0) ++w.m;
  w.mend = w.m + 1 < a.grp[w.g].mat1 ? a.mat[w.m + 1].vrow0 : a.grp[w.g].vrows;
  w.blk0 = (w.v - a.mat[w.m].vrow0) * w.nblk;
}

// Enters the first group at or after w.g in which the wave has rows
// (w.left = 0 when there is none).
__device__ __forceinline__ void walk_enter(Walk& w, const BArgs& a, int wave) {
  for (; w.g < a.ngroups; ++w.g) {
    const BGroup& G = a.grp[w.g];
    w.seg = wave % G.nseg;
    w.prt = wave / G.nseg;
    w.np = static_cast<int64_t>(gridDim.x) * G.wpr;
    const int64_t gp = static_cast<int64_t>(blockIdx.x) * G.wpr + w.prt;
    w.left = (w.prt < G.wpr && gp < G.vrows) ? (G.vrows - gp + w.np - 1) / w.np : 0;
    if (w.left > 0) {
      w.i = 0;
      w.v = gp;
      w.nblk = G.nblk;
      w.m = G.mat0;
      walk_weight(w, a);
      return;
    }
  }
  w.left = 0;
}

// Next row of the walk; returns true when it entered another group.  A walk
// past its last row stays on that row (its loads are then repeated, never
// branched around).
__device__ __forceinline__ bool walk_next(Walk& w, const BArgs& a, int wave) {
  if (w.left <= 1) {
    if (w.left == 1) {
      const Walk keep = w;
      ++w.g;
      walk_enter(w, a, wave);
      if (w.left == 0) {
        w = keep;
        w.left = 0;
        return false;
      }
      return true;
    }
    return false;
  }
  --w.left;
  ++w.i;
  w.v += w.np;
  w.blk0 += w.np * w.nblk;
  if (w.v >= w.mend) walk_weight(w, a);
  return false;
}

template <bool kDQ>
__device__ __forceinline__ Scales mat_scales(const BMat& M) {
  Scales sc{};
  if constexpr (kDQ) {
    sc.q = M.q;
    sc.absmax2 = M.absmax2;
  } else {
    sc.absmax = M.absmax;
  }
  return sc;
}

template <bool kDQ, bool kF8, bool kBf16Out>
__global__ __launch_bounds__(kBWaves * 64) void k_gemv_batch(BArgs a) {
  __shared__ uint32_t tab[256 * 64];
  __shared__ float part[kBPartMax];
  __shared__ float rtab[kDQ ? 256 : 1];
  __shared__ float means[kGemvBatchMax];
  const char* smem = reinterpret_cast<const char*>(tab);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t slot = static_cast<uint32_t>(lane) << 2;

  // load walk (one row ahead) and compute walk
  Walk wl{};
  walk_enter(wl, a, wave);
  Walk wc = wl;
  const bool any = wl.left > 0;

  // lane offsets of the load walk's group
  LaneOffs lol;
  {
    bool on_[2];
    int blk_[2];
    if (any) lane_offsets(a.grp[wl.g], wl.seg, lane, lol, on_, blk_);
  }
  const uint8_t* packed_l = any ? a.mat[wl.m].packed : nullptr;
  Scales sc_l = any ? mat_scales<kDQ>(a.mat[wl.m]) : Scales{};
  int m_l = wl.m;

  // raw (bf16) x of the lane's two half blocks of a group's segment; xr_g is
  // the group whose x it holds and that the compute walk has not entered yet
  // (-1: none)
  uint4 xr[2][4];
  int xr_g = -1;
  auto load_x = [&](uint4 (&dst)[2][4], int g, int seg) {
    const BGroup& G = a.grp[g];
    LaneOffs lo_;
    bool on_[2];
    int blk_[2];
    lane_offsets(G, seg, lane, lo_, on_, blk_);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4* xp = reinterpret_cast<const uint4*>(G.x + static_cast<int64_t>(blk_[j]) * 64 + 32 * (lane & 1));
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[j][i] = xp[i];
    }
  };

  // advances the load walk and requests its row into `dst` (past the wave's
  // last row the last row is requested again: loads are never branched
  // around); on entering a group it also requests that group's x, unless the
  // x of an earlier group is still waiting to be used
  auto load_next = [&](RowItem& dst) {
    if (walk_next(wl, a, wave)) {
      bool on_[2];
      int blk_[2];
      lane_offsets(a.grp[wl.g], wl.seg, lane, lol, on_, blk_);
      if (xr_g < 0) {
        load_x(xr, wl.g, wl.seg);
        xr_g = wl.g;
      }
    }
    if (wl.m != m_l) {
      m_l = wl.m;
      packed_l = a.mat[m_l].packed;
      sc_l = mat_scales<kDQ>(a.mat[m_l]);
    }
    row_load<kDQ>(dst, packed_l, wl.blk0, lol, sc_l);
  };

  // the wave's first kAhead rows and its first x are requested before the
  // tables are built
  RowItem it[kSlots];
  if (any) {
    row_load<kDQ>(it[0], packed_l, wl.blk0, lol, sc_l);
    load_x(xr, wl.g, wl.seg);
    xr_g = wl.g;
#pragma unroll
    for (int r = 1; r < kAhead; ++r) load_next(it[r]);
  }

  if (kDQ && static_cast<int>(threadIdx.x) < a.grp[a.ngroups - 1].mat1) means[threadIdx.x] = *a.mat[threadIdx.x].mean;
  if constexpr (kDQ) fill_ratio_table<kF8>(rtab, kBWaves * 64);
  fill_half_table<kBWaves * 64>(tab, a.cb);  // ends with a barrier

  // state of the compute walk's group: x in registers, segment flags, slots
  uint32_t xh[1][2][16];
  float xinv[1][2];
  float xsel[1];
  bool on[2];
  int part_row = 0, nseg_c = 1;  // part index of the current row, stride per row
  float mean_c = 0.0f;
  int m_c = -1;
  auto enter_compute_group = [&]() {
    const BGroup& G = a.grp[wc.g];
    LaneOffs lo_;
    int blk[2];
    lane_offsets(G, wc.seg, lane, lo_, on, blk);
    if (xr_g != wc.g) {
      // this group's x was not requested ahead (the wave's rows of the group
      // before it were too few): request it now
      uint4 xn[2][4];
      load_x(xn, wc.g, wc.seg);
#pragma unroll
      for (int j = 0; j < 2; ++j) x_half_block_to_half(xn[j], xh[0][j], xinv[0][j]);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) x_half_block_to_half(xr[j], xh[0][j], xinv[0][j]);
      xr_g = -1;
    }
    lane_x_scales<1>(xinv, on, xsel);
    nseg_c = G.nseg;
    part_row = G.part0 + (wc.prt * G.kmax) * G.nseg + wc.seg;
  };
  if (any) enter_compute_group();

  // step: request the row kAhead ahead into the slot the previous step
  // used, then use this step's slot; unrolled by the slots so every slot
  // keeps its registers (a wave without rows skips to the final barrier)
  bool done = !any;
  while (!done) {
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      if (!done) {  // wave-uniform
        load_next(it[(u + kAhead) % kSlots]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kDQ) {
          if (wc.m != m_c) {
            m_c = wc.m;
            mean_c = means[m_c];
          }
        }
        float v[1];
        row_dot<1, kDQ>(it[u], xh, smem, slot, mean_c, rtab, xsel, v);
        const float t = wave_sum_to_last(v[0]);
        if (lane == 63) part[part_row] = t;
        part_row += nseg_c;
        if (wc.left <= 1) {
          const Walk keep = wc;
          ++wc.g;
          walk_enter(wc, a, wave);
          if (wc.left == 0) {
            wc = keep;
            done = true;
          } else {
            enter_compute_group();
          }
        } else {
          walk_next(wc, a, wave);
        }
      }
    }
  }
  __syncthreads();

  // each row's segments in a fixed order, into its weight's y
  for (int g = 0; g < a.ngroups; ++g) {
    const BGroup& G = a.grp[g];
    const int64_t np = static_cast<int64_t>(gridDim.x) * G.wpr;
    for (int t = threadIdx.x; t < G.wpr * G.kmax; t += kBWaves * 64) {
      const int prt = t / G.kmax, i = t % G.kmax;
      const int64_t v = static_cast<int64_t>(blockIdx.x) * G.wpr + prt + i * np;
      if (v >= G.vrows) continue;
      float s = part[G.part0 + t * G.nseg];
      for (int k = 1; k < G.nseg; ++k) s += part[G.part0 + t * G.nseg + k];
      int m = G.mat0;
      while (m + 1 < G.mat1 && v >= a.mat[m + 1].vrow0) ++m;
      const int64_t r = v - a.mat[m].vrow0;
      if constexpr (kBf16Out) static_cast<uint16_t*>(a.mat[m].y)[r] = static_cast<uint16_t>(f32_to_bf16(s));
      else static_cast<float*>(a.mat[m].y)[r] = s;
    }
  }
}

// Groups the jobs by their x (same pointer and width), plans the groups for
// a grid of one workgroup per compute unit (more if the partial sums would
// not fit), and fills the kernel arguments.
bool plan_batch(const GemvJob* jobs, int count, BArgs& a, int& grid) {
  a = BArgs{};
  int order[kGemvBatchMax];
  int n = 0, ng = 0;
  int gof[kGemvBatchMax];
  for (int i = 0; i < count; ++i) {
    int g = -1;
    for (int k = 0; k < ng; ++k)
      if (a.grp[k].x == jobs[i].x && a.grp[k].nblk == jobs[i].cols / 64) g = k;
    if (g < 0) {
      g = ng++;
      a.grp[g].x = jobs[i].x;
      a.grp[g].nblk = jobs[i].cols / 64;
    }
    gof[i] = g;
  }
  // weights ordered by group, in the caller's order within a group
  for (int g = 0; g < ng; ++g) {
    a.grp[g].mat0 = n;
    int64_t v = 0;
    for (int i = 0; i < count; ++i) {
      if (gof[i] != g) continue;
      order[n] = i;
      BMat& M = a.mat[n++];
      M.packed = jobs[i].packed;
      M.absmax = jobs[i].sc.absmax;
      M.q = jobs[i].sc.q;
      M.absmax2 = jobs[i].sc.absmax2;
      M.mean = jobs[i].sc.mean;
      M.y = jobs[i].y;
      M.vrow0 = v;
      M.rows = jobs[i].rows;
      v += jobs[i].rows;
    }
    a.grp[g].mat1 = n;
    a.grp[g].vrows = v;
  }
  (void)order;
  a.ngroups = ng;
  for (int g = 0; g < ng; ++g) {
    BGroup& G = a.grp[g];
    G.nseg = static_cast<int>((G.nblk + 63) / 64);
    G.seg_blocks = static_cast<int>((G.nblk + G.nseg - 1) / G.nseg);
    G.wpr = kBWaves / G.nseg;
  }
  int64_t g = device_cus();
  for (;; ++g) {
    int64_t slots = 0;
    for (int k = 0; k < ng; ++k) {
      BGroup& G = a.grp[k];
      G.kmax = static_cast<int>((G.vrows + g * G.wpr - 1) / (g * G.wpr));
      G.part0 = static_cast<int>(slots);
      slots += static_cast<int64_t>(G.wpr) * G.kmax * G.nseg;
    }
    if (slots <= kBPartMax) break;
  }
  grid = static_cast<int>(g);
  return true;
}

template <bool kDQ, bool kF8>
hipError_t launch_batch_sc(const BArgs& a, int grid, int y_bf16, hipStream_t s) {
  if (y_bf16) hipLaunchKernelGGL((k_gemv_batch<kDQ, kF8, true>), dim3(grid), dim3(kBWaves * 64), 0, s, a);
  else hipLaunchKernelGGL((k_gemv_batch<kDQ, kF8, false>), dim3(grid), dim3(kBWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_batch(const GemvJob* jobs, int count, int y_bf16, hipStream_t s) {
  if (count < 1 || count > kGemvBatchMax) return hipErrorInvalidValue;
  BArgs a;
  int grid = 0;
  if (!plan_batch(jobs, count, a, grid)) return hipErrorInvalidValue;
  a.cb = codebook(jobs[0].sc.fp4);
  if (jobs[0].sc.absmax) return launch_batch_sc<false, false>(a, grid, y_bf16, s);
  if (jobs[0].sc.f8) return launch_batch_sc<true, true>(a, grid, y_bf16, s);
  return launch_batch_sc<true, false>(a, grid, y_bf16, s);
}

}  // namespace nf4i
