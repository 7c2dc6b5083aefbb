// Plain streaming read of a device buffer: the calibration of what the memory
// system gives a read-only kernel on this GPU, against which the HBM-bound
// NF4 kernels are also reported.  Measurement only; not part of libnf4.
//
// Every lane reads 16-byte chunks (plain or non-temporal loads) with kUnroll
// loads in flight: chunk
// i + u * stride for u < kUnroll, stride = all threads of the grid, so at any
// moment the grid reads kUnroll contiguous windows.  The data are folded with
// xor into one word per lane, written only if it equals a value the data
// cannot produce here (the buffer is filled by the caller), which keeps every
// load alive without a store per lane.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool kNT>
__device__ __forceinline__ u32x4_t load16(const u32x4_t* p) {
  if constexpr (kNT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int kUnroll, bool kNT>
__global__ __launch_bounds__(512) void k_stream_read(const u32x4_t* __restrict__ p, int64_t n16, uint32_t never,
                                                     uint32_t* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load16<kNT>(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = load16<kNT>(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == never) out[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, buffer 16-byte aligned) with `grid`
// workgroups of 512 threads and `unroll` (4 or 8) loads in flight per lane,
// non-temporal loads when `nontemporal` is nonzero.
// `out` holds `grid` words and is written only when a lane's xor of its data
// equals `never`.  Returns 0, or 1 for invalid arguments, 2 for a launch error.
int nf4_calib_stream_read(const void* buf, int64_t bytes, int grid, int unroll, int nontemporal, uint32_t never,
                          uint32_t* out, void* stream) {
  if (!buf || !out || bytes < 16 || bytes % 16 || grid < 1 || (unroll != 4 && unroll != 8)) return 1;
  if (reinterpret_cast<uintptr_t>(buf) % 16) return 1;
  const int64_t n16 = bytes / 16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const u32x4_t* p = static_cast<const u32x4_t*>(buf);
  if (unroll == 4 && nontemporal)
    hipLaunchKernelGGL((k_stream_read<4, true>), dim3(grid), dim3(512), 0, s, p, n16, never, out);
  else if (unroll == 4)
    hipLaunchKernelGGL((k_stream_read<4, false>), dim3(grid), dim3(512), 0, s, p, n16, never, out);
  else if (nontemporal)
    hipLaunchKernelGGL((k_stream_read<8, true>), dim3(grid), dim3(512), 0, s, p, n16, never, out);
  else
    hipLaunchKernelGGL((k_stream_read<8, false>), dim3(grid), dim3(512), 0, s, p, n16, never, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
