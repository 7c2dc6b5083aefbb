// Plain streaming read of a device buffer: the calibration of what the memory
// system gives a read-only kernel on this GPU, against which the HBM-bound
// NF4 kernels are also reported.  Measurement only; not part of libnf4.
//
// Every lane reads 16-byte chunks with kUnroll loads in flight: chunk
// i + u * stride for u < kUnroll, stride = all threads of the grid, so at any
// moment the grid reads kUnroll contiguous windows.  The data are folded with
// xor into one word per lane, written only if it equals a value the data
// cannot produce here (the buffer is filled by the caller), which keeps every
// load alive without a store per lane.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

template <int kUnroll>
__global__ __launch_bounds__(512) void k_stream_read(const uint4* __restrict__ p, int64_t n16, uint32_t never,
                                                     uint32_t* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == never) out[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, buffer 16-byte aligned) with `grid`
// workgroups of 512 threads and `unroll` (4 or 8) loads in flight per lane.
// `out` holds `grid` words and is written only when a lane's xor of its data
// equals `never`.  Returns 0, or 1 for invalid arguments, 2 for a launch error.
int nf4_calib_stream_read(const void* buf, int64_t bytes, int grid, int unroll, uint32_t never, uint32_t* out,
                          void* stream) {
  if (!buf || !out || bytes < 16 || bytes % 16 || grid < 1 || (unroll != 4 && unroll != 8)) return 1;
  if (reinterpret_cast<uintptr_t>(buf) % 16) return 1;
  const int64_t n16 = bytes / 16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (unroll == 4)
    hipLaunchKernelGGL(k_stream_read<4>, dim3(grid), dim3(512), 0, s, static_cast<const uint4*>(buf), n16, never, out);
  else
    hipLaunchKernelGGL(k_stream_read<8>, dim3(grid), dim3(512), 0, s, static_cast<const uint4*>(buf), n16, never, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
