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

// Host derivation, computed once (thread-safe) at first use.  fp4 = 1
// selects the FP4 code book (levels by 4-bit E2M1 pattern).
const Codebook& codebook(int fp4 = 0);

// Bucket table of the quantizer's nearest-level search.  A normalized value
// v in [-1, 1] falls in bucket (bits(v) >> 21): its sign, exponent and two
// leading significand bits.  Each bucket holds at most one decision
// threshold, so code(v) = base[bucket] + (v >= thr[bucket]).  Buckets with
// |v| < 2^-5 all give code 7; only the 48 buckets with exponent 2^-5 .. 2^0
// differ, and those are listed here (order: sign, exponent, bits).
constexpr int kLutBuckets = 2048;
constexpr int kLutSpecial = 48;
constexpr int kLutFirstExp = 122;  // 2^-5
struct QuantLut {
  float thr[kLutSpecial];
  uint32_t base[kLutSpecial];
};
// The quantizer's bucket table.  For FP4 it is built on the 15 producible
// levels in ascending order (zero at index 7, like NF4); the kernel maps the
// ascending index c to the E2M1 pattern (c >= 7 ? c - 7 : 15 - c).  Built and
// self-checked once; returns nullptr (and the reason in *err) if the check
// failed, in which case nothing may be quantized.
const QuantLut* quant_lut(int fp4 = 0, const char** err = nullptr);
// The construction behind quant_lut for any ascending code book: false (with
// the reason in err) when some bucket holds two decision thresholds, a bucket
// below 2^-5 is not the zero level, or a needed bucket has no table slot.
bool build_lut(const Codebook& cb, QuantLut* out, char* err, size_t err_len);

__host__ __device__ inline int lut_special_index(int t) {
  const int sign = t / 24, e = kLutFirstExp + (t % 24) / 4, m2 = t % 4;
  return (sign << 10) | (e << 2) | m2;
}

// The float8 reading of the second level (tutorial page "bitsandbytes
// quantization tutorial: 4-bit and 8-bit models", section "How NF4 Works":
// the scales go from float32 to float8): E4M3 codes as the Open Compute
// Project's 8-bit floating point specification defines them (bias 7, three
// mantissa bits, subnormals, largest finite 448).  Where the int8 reading
// divides the code by 127, this one takes fl32(e4m3(q) / 448) from a table.
// The double quotient is rounded once more to float32; it is either exact or
// has a repeating binary expansion ((8 + m) / 7 times a power of two), so it
// never falls on a float32 tie and the two roundings give the correctly
// rounded quotient.
constexpr double e4m3_value(int c) {
  const double sign = (c & 0x80) ? -1.0 : 1.0;
  const int e = (c >> 3) & 0xF, m = c & 7;
  if (e == 0xF && m == 7) return 0.0;  // the NaN codes, never written
  double p = 1.0;
  for (int i = 0; i < (e == 0 ? 9 : (e < 7 ? 7 - e : 0)); ++i) p *= 0.5;
  for (int i = 0; i < (e > 7 ? e - 7 : 0); ++i) p *= 2.0;
  return e == 0 ? sign * m * p : sign * (1.0 + m / 8.0) * p;
}
struct E4m3Ratio {
  float v[256];
};
constexpr E4m3Ratio make_e4m3_ratio() {
  E4m3Ratio t{};
  for (int c = 0; c < 256; ++c) t.v[c] = static_cast<float>(e4m3_value(c) / 448.0);
  return t;
}
// Compute units of the current device (set by the front end's device check
// before any launch; used to size persistent grids).
int device_cus();

// Scale description shared by the consumers of a quantized weight.
struct Scales {
  const float* absmax;   // non-null: plain scales
  const int8_t* q;       // double-quantized scales when absmax is null
  const float* absmax2;
  const float* mean;
  int f8;                // second level: 0 = int8 codes, 1 = float8 (E4M3) codes
  int fp4;               // code book: 0 = NF4, 1 = FP4
};

// Workspace of the double-quant kernels: one row of partial digit sums per
// summing workgroup (at most kDqMaxGroups rows of kDqDigits u64).
constexpr int kDqDigits = 12;      // 32-bit digits of the exact scale sum
constexpr int kDqMaxGroups = 256;
constexpr size_t kDqWorkspaceBytes = kDqMaxGroups * kDqDigits * sizeof(unsigned long long);

hipError_t launch_quantize(const void* x, int x_bf16, int64_t n, uint8_t* packed,
                           float* absmax, const QuantLut& tab, int fp4, hipStream_t s);
// Several tensors (at most kQuantMaxJobs, one input dtype and code book) in
// one launch; each tensor's codes and absmax are those of launch_quantize.
constexpr int kQuantMaxJobs = 8;
struct QuantJob {
  const void* x;
  int64_t n;
  uint8_t* packed;
  float* absmax;
};
hipError_t launch_quantize_batch(const QuantJob* jobs, int count, int x_bf16, const QuantLut& tab, int fp4,
                                 hipStream_t s);
hipError_t launch_double_quant(const float* absmax, int64_t nb, int8_t* q, float* absmax2,
                               float* mean, unsigned long long* ws, int f8, hipStream_t s);
// Several scale arrays (at most kDqMaxJobs) in one pair of launches; ws holds
// kDqWorkspaceBytes per array.  Each array's results are those of
// launch_double_quant on it alone (its mean is an exact sum, whatever the
// split of the work).
constexpr int kDqMaxJobs = 8;
struct DqJob {
  const float* absmax;
  int64_t nblocks;
  int8_t* q;
  float* absmax2;
  float* mean;
};
hipError_t launch_double_quant_batch(const DqJob* jobs, int count, unsigned long long* ws, int f8, hipStream_t s);
// Device address of the double quantization's static scratch on the current
// device (kDqWorkspaceBytes or more, 256-byte aligned), for callers that
// cannot allocate.  Looked up once per device.
constexpr size_t kDqScratchBytes = kDqWorkspaceBytes;
hipError_t dq_scratch(unsigned long long** out);
hipError_t launch_dequantize(const uint8_t* packed, int64_t n, Scales sc, void* out,
                             int out_bf16, hipStream_t s);
hipError_t launch_gemv(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc,
                       const uint16_t* x, int64_t m, void* y, int y_bf16, hipStream_t s);
// One decode product of a batched launch: y = x . deq(W)^T at m = 1.
constexpr int kGemvBatchMax = 8;
struct GemvJob {
  const uint8_t* packed;
  int64_t rows, cols;
  Scales sc;
  const uint16_t* x;
  void* y;
};
// Decode GEMV of up to kGemvBatchMax weights (all with the same scale form
// and code book, cols % 64 == 0, cols <= 65536) in one launch.
hipError_t launch_gemv_batch(const GemvJob* jobs, int count, int y_bf16, hipStream_t s);
// Extra K columns the GEMM uses for a LoRA term of rank r (0 without one);
// the workspace holds m rows of that many bf16 values.
size_t gemm_lora_cols(int r);
// Workspace bytes of the forward GEMM with LoRA rank r: u (m rows of
// gemm_lora_cols(r) bf16, rounded up to 256 bytes), then (B | B | 0) as rows
// rows of the same width.
size_t gemm_workspace(int64_t m, int64_t rows, int r);
// u[i][.] = (bf16(s T[i][j]) for j < r | bf16(s T - hi) at r_pad + j | 0) with
// T[i][j] = sum_k x[i][k] a[j][k] formed in float32, for the m rows of
// x [m][len] and the r rows of a [r][len] (len % 8 == 0); each row of u holds
// gemm_lora_cols(r) bf16 values, r_pad = r rounded up to 16.
hipError_t launch_lora_u(const uint16_t* x, const uint16_t* a, int64_t m, int64_t len, int r, float scale,
                         uint16_t* u, hipStream_t s);
// The same product kept in float32: t[i][j] = fl32(s T[i][j]) in rows of
// r_pad floats, zero for j >= r.
hipError_t launch_lora_t32(const uint16_t* x, const uint16_t* a, int64_t m, int64_t len, int r, float scale,
                           float* t, hipStream_t s);
// bt[j][n] = b[n][j] for b [rows][r] bf16.
hipError_t launch_transpose_b(const uint16_t* b, int64_t rows, int r, uint16_t* bt, hipStream_t s);
hipError_t launch_gemm(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc,
                       const uint16_t* x, int64_t m, uint16_t* y, const uint16_t* lora_a,
                       const uint16_t* lora_b, int r, float lora_scale, uint16_t* u_ws,
                       hipStream_t s);
// Extra reduction indices and workspace of the input-gradient GEMM.
size_t gemm_dx_workspace(int64_t m, int64_t rows, int r);
hipError_t launch_gemm_dx(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* dy,
                          int64_t m, uint16_t* dx, const uint16_t* lora_a, const uint16_t* lora_b, int r,
                          float lora_scale, uint16_t* ws, hipStream_t s);
// LoRA gradients (float32 out): da [r][cols], db [rows][r].
size_t lora_grads_workspace(int64_t m, int64_t rows, int64_t cols, int r);
hipError_t launch_lora_grads(const uint16_t* x, const uint16_t* dy, int64_t m, int64_t rows, int64_t cols,
                             const uint16_t* lora_a, const uint16_t* lora_b, int r, float scale, float* da,
                             float* db, void* ws, hipStream_t s);
hipError_t launch_lora_merge(const uint8_t* packed, int64_t rows, int64_t cols, Scales sc, const uint16_t* lora_a,
                             const uint16_t* lora_b, int r, float scale, uint16_t* out, int out_f16,
                             hipStream_t s);

}  // namespace nf4i
