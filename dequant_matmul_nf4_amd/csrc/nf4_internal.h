// Internal interface between the C-ABI front end (api.cpp) and the HIP
// kernels.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace nf4i {

// The 16 NF4 levels (ascending) and the 15 decision thresholds of the
// nearest-level search: the code of a normalized value v is the number of
// thresholds t_i with v >= t_i.  Passed to kernels by value.
struct Codebook {
  float level[16];
  float thresh[16];  // thresh[15] = +inf, never reached by |v| <= 1
};

// Host derivation, computed once (thread-safe) at first use.
const Codebook& codebook();

// Scale description shared by the consumers of a quantized weight.
struct Scales {
  const float* absmax;   // non-null: plain scales
  const int8_t* q;       // double-quantized scales when absmax is null
  const float* absmax2;
  const float* mean;
};

// Workspace layout of the double-quant kernels (device, 16 x u64).
constexpr int kDqDigits = 12;      // 32-bit digits of the exact scale sum
constexpr int kDqDoneSlot = 12;    // arrival counter of the summing blocks
constexpr size_t kDqWorkspaceBytes = 16 * sizeof(unsigned long long);

hipError_t launch_quantize(const void* x, int x_bf16, int64_t n, uint8_t* packed,
                           float* absmax, hipStream_t s);
hipError_t launch_double_quant(const float* absmax, int64_t nb, int8_t* q, float* absmax2,
                               float* mean, unsigned long long* ws, hipStream_t s);
hipError_t launch_dequantize(const uint8_t* packed, int64_t n, Scales sc, void* out,
                             int out_bf16, hipStream_t s);
hipError_t launch_gemv(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc,
                       const uint16_t* x, int64_t m, void* y, int y_bf16, hipStream_t s);
hipError_t launch_gemm(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc,
                       const uint16_t* x, int64_t m, uint16_t* y, const uint16_t* lora_a,
                       const uint16_t* lora_b, int r, float lora_scale, float* t_ws,
                       hipStream_t s);

}  // namespace nf4i
