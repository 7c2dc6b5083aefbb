// C-ABI front end: argument checks, device check and dispatch to the kernels.
// Every check runs on the host before any HIP call, so a rejected call
// touches no device state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "nf4.h"
#include "nf4_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return NF4_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxN = int64_t(1) << 40;

// gfx950 check, cached per device id.
std::mutex g_dev_mu;
int g_dev_state[64];  // 0 unknown, 1 gfx950, 2 other
int g_dev_cus[64];
thread_local int t_cus = 256;

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NF4_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(NF4_ERR_DEVICE, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(NF4_ERR_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_cus[dev] = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  }
  if (g_dev_state[dev] != 1) return fail(NF4_ERR_DEVICE, "device %d is not a gfx950 (MI355X)", dev);
  t_cus = g_dev_cus[dev];
  return NF4_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(NF4_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Validates a weight descriptor; fills `sc` and the element count.
int check_weight(const nf4_weight* w, nf4i::Scales* sc, int64_t* n_out, const char* who) {
  if (!w) return fail(NF4_ERR_NULL, "%s: weight descriptor is NULL", who);
  if (!w->packed) return fail(NF4_ERR_NULL, "%s: weight packed pointer is NULL", who);
  if (w->blocksize != NF4_BLOCKSIZE)
    return fail(NF4_ERR_BLOCKSIZE, "%s: blocksize %d unsupported (only 64)", who, (int)w->blocksize);
  if (w->rows < 1 || w->cols < 1 || w->rows > kMaxN || w->cols > kMaxN || w->rows > kMaxN / w->cols)
    return fail(NF4_ERR_SIZE, "%s: bad shape %lld x %lld", who, (long long)w->rows, (long long)w->cols);
  if (!aligned(w->packed, 16)) return fail(NF4_ERR_ALIGN, "%s: packed must be 16-byte aligned", who);
  const int64_t n = w->rows * w->cols;
  const int64_t nb = (n + 63) / 64;
  if (w->absmax) {
    if (!aligned(w->absmax, 4)) return fail(NF4_ERR_ALIGN, "%s: absmax must be 4-byte aligned", who);
    *sc = nf4i::Scales{w->absmax, nullptr, nullptr, nullptr, 0, 0};
  } else {
    if (!w->qabsmax || !w->absmax2 || !w->mean)
      return fail(NF4_ERR_NULL, "%s: absmax is NULL, so qabsmax, absmax2 and mean are required", who);
    if (w->blocksize2 != NF4_BLOCKSIZE2)
      return fail(NF4_ERR_BLOCKSIZE, "%s: blocksize2 %d unsupported (only 256)", who, (int)w->blocksize2);
    if (nb >= (int64_t(1) << 31)) return fail(NF4_ERR_SIZE, "%s: too many blocks for double quant", who);
    if (!aligned(w->absmax2, 4) || !aligned(w->mean, 4))
      return fail(NF4_ERR_ALIGN, "%s: absmax2 and mean must be 4-byte aligned", who);
    if (w->dq_type != NF4_DQ_INT8 && w->dq_type != NF4_DQ_FP8)
      return fail(NF4_ERR_DTYPE, "%s: dq_type %d unknown", who, (int)w->dq_type);
    *sc = nf4i::Scales{nullptr, w->qabsmax, w->absmax2, w->mean, w->dq_type == NF4_DQ_FP8 ? 1 : 0, 0};
  }
  if (w->quant_type != NF4_QT_NF4 && w->quant_type != NF4_QT_FP4)
    return fail(NF4_ERR_DTYPE, "%s: quant_type %d unknown", who, (int)w->quant_type);
  sc->fp4 = w->quant_type == NF4_QT_FP4 ? 1 : 0;
  *n_out = n;
  return NF4_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

const uint8_t* w_packed(const nf4_weight& w) { return w.packed; }

}  // namespace

int nf4i::device_cus() { return t_cus; }

namespace {

int double_quant(const float* absmax, int64_t nblocks, int32_t blocksize2, int8_t* qabsmax, float* absmax2,
                 float* mean, void* workspace, size_t workspace_bytes, void* stream, int f8, const char* who) {
  if (!absmax || !qabsmax || !absmax2 || !mean)
    return fail(NF4_ERR_NULL, "%s: absmax, qabsmax, absmax2 and mean are required", who);
  if (nblocks < 1 || nblocks >= (int64_t(1) << 31))
    return fail(NF4_ERR_SIZE, "%s: nblocks = %lld out of range", who, (long long)nblocks);
  if (blocksize2 != NF4_BLOCKSIZE2)
    return fail(NF4_ERR_BLOCKSIZE, "%s: blocksize2 %d unsupported (only 256)", who, (int)blocksize2);
  if (!workspace || workspace_bytes < nf4i::kDqWorkspaceBytes)
    return fail(NF4_ERR_WORKSPACE, "%s: workspace needs %zu bytes", who, nf4i::kDqWorkspaceBytes);
  if (!aligned(absmax, 16) || !aligned(qabsmax, 16) || !aligned(workspace, 16))
    return fail(NF4_ERR_ALIGN, "%s: absmax, qabsmax and workspace must be 16-byte aligned", who);
  if (!aligned(absmax2, 4) || !aligned(mean, 4))
    return fail(NF4_ERR_ALIGN, "%s: absmax2 and mean must be 4-byte aligned", who);
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_double_quant(absmax, nblocks, qabsmax, absmax2, mean,
                                            static_cast<unsigned long long*>(workspace), f8, as_stream(stream)),
                  who);
}

}  // namespace

namespace {

int quantize(const void* x, int x_dtype, int64_t n, int32_t blocksize, uint8_t* packed, float* absmax,
             void* stream, int fp4, const char* who) {
  if (!x || !packed || !absmax) return fail(NF4_ERR_NULL, "%s: x, packed and absmax are required", who);
  if (x_dtype != NF4_F32 && x_dtype != NF4_BF16) return fail(NF4_ERR_DTYPE, "%s: x_dtype %d unknown", who, x_dtype);
  if (n < 1 || n >= kMaxN) return fail(NF4_ERR_SIZE, "%s: n = %lld out of range", who, (long long)n);
  if (blocksize != NF4_BLOCKSIZE) return fail(NF4_ERR_BLOCKSIZE, "%s: blocksize %d unsupported (only 64)", who, (int)blocksize);
  if (!aligned(x, 16) || !aligned(packed, 16)) return fail(NF4_ERR_ALIGN, "%s: x and packed must be 16-byte aligned", who);
  if (!aligned(absmax, 4)) return fail(NF4_ERR_ALIGN, "%s: absmax must be 4-byte aligned", who);
  const char* lut_err = "";
  const nf4i::QuantLut* lut = nf4i::quant_lut(fp4, &lut_err);
  if (!lut) return fail(NF4_ERR_INTERNAL, "%s: %s", who, lut_err);
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_quantize(x, x_dtype == NF4_BF16, n, packed, absmax, *lut, fp4, as_stream(stream)),
                  who);
}

}  // namespace

extern "C" {

const char* nf4_last_error(void) { return g_err; }

int nf4_codebook(float out[16]) {
  if (!out) return fail(NF4_ERR_NULL, "nf4_codebook: out is NULL");
  std::memcpy(out, nf4i::codebook().level, 16 * sizeof(float));
  return ok();
}

int nf4_codebook_fp4(float out[16]) {
  if (!out) return fail(NF4_ERR_NULL, "nf4_codebook_fp4: out is NULL");
  std::memcpy(out, nf4i::codebook(1).level, 16 * sizeof(float));
  return ok();
}

int nf4_quantize(const void* x, int x_dtype, int64_t n, int32_t blocksize, uint8_t* packed,
                 float* absmax, void* stream) {
  return quantize(x, x_dtype, n, blocksize, packed, absmax, stream, 0, "nf4_quantize");
}

int nf4_quantize_fp4(const void* x, int x_dtype, int64_t n, int32_t blocksize, uint8_t* packed,
                     float* absmax, void* stream) {
  return quantize(x, x_dtype, n, blocksize, packed, absmax, stream, 1, "nf4_quantize_fp4");
}

int nf4_quantize_batched(const nf4_quantize_job* jobs, int32_t count, int x_dtype, int32_t blocksize,
                         int32_t quant_type, void* stream) {
  const char* who = "nf4_quantize_batched";
  if (!jobs) return fail(NF4_ERR_NULL, "%s: jobs is NULL", who);
  if (count < 1 || count > nf4i::kQuantMaxJobs)
    return fail(NF4_ERR_SIZE, "%s: count = %d out of range 1..%d", who, (int)count, nf4i::kQuantMaxJobs);
  if (x_dtype != NF4_F32 && x_dtype != NF4_BF16) return fail(NF4_ERR_DTYPE, "%s: x_dtype %d unknown", who, x_dtype);
  if (blocksize != NF4_BLOCKSIZE) return fail(NF4_ERR_BLOCKSIZE, "%s: blocksize %d unsupported (only 64)", who, (int)blocksize);
  if (quant_type != NF4_QT_NF4 && quant_type != NF4_QT_FP4)
    return fail(NF4_ERR_DTYPE, "%s: quant_type %d unknown", who, (int)quant_type);
  nf4i::QuantJob qj[nf4i::kQuantMaxJobs];
  for (int i = 0; i < count; ++i) {
    const nf4_quantize_job& j = jobs[i];
    if (!j.x || !j.packed || !j.absmax) return fail(NF4_ERR_NULL, "%s: tensor %d: x, packed and absmax are required", who, i);
    if (j.n < 1 || j.n >= kMaxN) return fail(NF4_ERR_SIZE, "%s: tensor %d: n = %lld out of range", who, i, (long long)j.n);
    if (!aligned(j.x, 16) || !aligned(j.packed, 16))
      return fail(NF4_ERR_ALIGN, "%s: tensor %d: x and packed must be 16-byte aligned", who, i);
    if (!aligned(j.absmax, 4)) return fail(NF4_ERR_ALIGN, "%s: tensor %d: absmax must be 4-byte aligned", who, i);
    qj[i] = nf4i::QuantJob{j.x, j.n, j.packed, j.absmax};
  }
  const int fp4 = quant_type == NF4_QT_FP4 ? 1 : 0;
  const char* lut_err = "";
  const nf4i::QuantLut* lut = nf4i::quant_lut(fp4, &lut_err);
  if (!lut) return fail(NF4_ERR_INTERNAL, "%s: %s", who, lut_err);
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_quantize_batch(qj, count, x_dtype == NF4_BF16, *lut, fp4, as_stream(stream)), who);
}

size_t nf4_double_quant_workspace(int64_t nblocks) {
  (void)nblocks;
  return nf4i::kDqWorkspaceBytes;
}

int nf4_e4m3_ratio(float out[256]) {
  if (!out) return fail(NF4_ERR_NULL, "nf4_e4m3_ratio: out is NULL");
  constexpr nf4i::E4m3Ratio t = nf4i::make_e4m3_ratio();
  for (int c = 0; c < 256; ++c) out[c] = t.v[c];
  return ok();
}

int nf4_double_quant(const float* absmax, int64_t nblocks, int32_t blocksize2, int8_t* qabsmax,
                     float* absmax2, float* mean, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return double_quant(absmax, nblocks, blocksize2, qabsmax, absmax2, mean, workspace, workspace_bytes, stream, 0,
                      "nf4_double_quant");
}

int nf4_double_quant_noalloc(const float* absmax, int64_t nblocks, int32_t blocksize2, int8_t* qabsmax,
                             float* absmax2, float* mean, void* stream) {
  const char* who = "nf4_double_quant_noalloc";
  if (!absmax || !qabsmax || !absmax2 || !mean)
    return fail(NF4_ERR_NULL, "%s: absmax, qabsmax, absmax2 and mean are required", who);
  if (nblocks < 1 || nblocks >= (int64_t(1) << 31))
    return fail(NF4_ERR_SIZE, "%s: nblocks = %lld out of range 1..2^31-1", who, (long long)nblocks);
  if (blocksize2 != NF4_BLOCKSIZE2)
    return fail(NF4_ERR_BLOCKSIZE, "%s: blocksize2 %d unsupported (only 256)", who, (int)blocksize2);
  if (nf4_double_quant_workspace(nblocks) > nf4i::kDqScratchBytes)
    return fail(NF4_ERR_SIZE, "%s: %lld scales need %zu bytes of scratch, more than the %zu held", who,
                (long long)nblocks, nf4_double_quant_workspace(nblocks), nf4i::kDqScratchBytes);
  if (!aligned(absmax, 16) || !aligned(qabsmax, 16))
    return fail(NF4_ERR_ALIGN, "%s: absmax and qabsmax must be 16-byte aligned", who);
  if (!aligned(absmax2, 4) || !aligned(mean, 4))
    return fail(NF4_ERR_ALIGN, "%s: absmax2 and mean must be 4-byte aligned", who);
  if (int rc = check_device()) return rc;
  unsigned long long* ws = nullptr;
  if (hipError_t e = nf4i::dq_scratch(&ws); e != hipSuccess)
    return fail(NF4_ERR_DEVICE, "%s: scratch address lookup failed: %s", who, hipGetErrorString(e));
  return launched(nf4i::launch_double_quant(absmax, nblocks, qabsmax, absmax2, mean, ws, 0, as_stream(stream)), who);
}

int nf4_double_quant_f8(const float* absmax, int64_t nblocks, int32_t blocksize2, uint8_t* qabsmax,
                        float* absmax2, float* mean, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return double_quant(absmax, nblocks, blocksize2, reinterpret_cast<int8_t*>(qabsmax), absmax2, mean, workspace,
                      workspace_bytes, stream, 1, "nf4_double_quant_f8");
}

size_t nf4_double_quant_batched_workspace(int32_t count) {
  if (count < 1 || count > nf4i::kDqMaxJobs) return 0;
  return static_cast<size_t>(count) * nf4i::kDqWorkspaceBytes;
}

int nf4_double_quant_batched(const nf4_dq_job* jobs, int32_t count, int32_t blocksize2, int32_t dq_type,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "nf4_double_quant_batched";
  if (!jobs) return fail(NF4_ERR_NULL, "%s: jobs is NULL", who);
  if (count < 1 || count > nf4i::kDqMaxJobs)
    return fail(NF4_ERR_SIZE, "%s: count = %d out of range 1..%d", who, (int)count, nf4i::kDqMaxJobs);
  if (blocksize2 != NF4_BLOCKSIZE2)
    return fail(NF4_ERR_BLOCKSIZE, "%s: blocksize2 %d unsupported (only 256)", who, (int)blocksize2);
  if (dq_type != NF4_DQ_INT8 && dq_type != NF4_DQ_FP8)
    return fail(NF4_ERR_DTYPE, "%s: dq_type %d unknown", who, (int)dq_type);
  const size_t need = nf4_double_quant_batched_workspace(count);
  if (!workspace || workspace_bytes < need) return fail(NF4_ERR_WORKSPACE, "%s: workspace needs %zu bytes", who, need);
  if (!aligned(workspace, 16)) return fail(NF4_ERR_ALIGN, "%s: workspace must be 16-byte aligned", who);
  nf4i::DqJob dj[nf4i::kDqMaxJobs];
  for (int i = 0; i < count; ++i) {
    const nf4_dq_job& j = jobs[i];
    if (!j.absmax || !j.qabsmax || !j.absmax2 || !j.mean)
      return fail(NF4_ERR_NULL, "%s: array %d: absmax, qabsmax, absmax2 and mean are required", who, i);
    if (j.nblocks < 1 || j.nblocks >= (int64_t(1) << 31))
      return fail(NF4_ERR_SIZE, "%s: array %d: nblocks = %lld out of range", who, i, (long long)j.nblocks);
    if (!aligned(j.absmax, 16) || !aligned(j.qabsmax, 16))
      return fail(NF4_ERR_ALIGN, "%s: array %d: absmax and qabsmax must be 16-byte aligned", who, i);
    if (!aligned(j.absmax2, 4) || !aligned(j.mean, 4))
      return fail(NF4_ERR_ALIGN, "%s: array %d: absmax2 and mean must be 4-byte aligned", who, i);
    dj[i] = nf4i::DqJob{j.absmax, j.nblocks, static_cast<int8_t*>(j.qabsmax), j.absmax2, j.mean};
  }
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_double_quant_batch(dj, count, static_cast<unsigned long long*>(workspace),
                                                  dq_type == NF4_DQ_FP8 ? 1 : 0, as_stream(stream)),
                  who);
}

int nf4_dequantize(const nf4_weight* w, void* out, int out_dtype, void* stream) {
  nf4i::Scales sc{};
  int64_t n = 0;
  if (int rc = check_weight(w, &sc, &n, "nf4_dequantize")) return rc;
  if (!out) return fail(NF4_ERR_NULL, "nf4_dequantize: out is NULL");
  if (out_dtype != NF4_F32 && out_dtype != NF4_BF16) return fail(NF4_ERR_DTYPE, "nf4_dequantize: out_dtype %d unknown", out_dtype);
  if (!aligned(out, 16)) return fail(NF4_ERR_ALIGN, "nf4_dequantize: out must be 16-byte aligned");
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_dequantize(w->packed, n, sc, out, out_dtype == NF4_BF16, as_stream(stream)), "nf4_dequantize");
}

int nf4_gemv(const nf4_weight* w, const void* x, int64_t m, void* y, int y_dtype, void* stream) {
  nf4i::Scales sc{};
  int64_t n = 0;
  if (int rc = check_weight(w, &sc, &n, "nf4_gemv")) return rc;
  if (!x || !y) return fail(NF4_ERR_NULL, "nf4_gemv: x and y are required");
  if (w->cols % 64) return fail(NF4_ERR_SIZE, "nf4_gemv: cols = %lld is not a multiple of 64", (long long)w->cols);
  if (m < 1 || m > 16) return fail(NF4_ERR_SIZE, "nf4_gemv: m = %lld out of range 1..16", (long long)m);
  if (y_dtype != NF4_F32 && y_dtype != NF4_BF16) return fail(NF4_ERR_DTYPE, "nf4_gemv: y_dtype %d unknown", y_dtype);
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(NF4_ERR_ALIGN, "nf4_gemv: x and y must be 16-byte aligned");
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_gemv(w->packed, w->rows, w->cols, sc, static_cast<const uint16_t*>(x), m, y,
                                    y_dtype == NF4_BF16, as_stream(stream)),
                  "nf4_gemv");
}

int nf4_gemv_batched(const nf4_weight* ws, int32_t count, const void* const* xs, void* const* ys, int y_dtype,
                     void* stream) {
  const char* who = "nf4_gemv_batched";
  if (!ws || !xs || !ys) return fail(NF4_ERR_NULL, "%s: ws, xs and ys are required", who);
  if (count < 1 || count > nf4i::kGemvBatchMax)
    return fail(NF4_ERR_SIZE, "%s: count = %d out of range 1..%d", who, (int)count, nf4i::kGemvBatchMax);
  if (y_dtype != NF4_F32 && y_dtype != NF4_BF16) return fail(NF4_ERR_DTYPE, "%s: y_dtype %d unknown", who, y_dtype);
  nf4i::GemvJob jobs[nf4i::kGemvBatchMax];
  for (int i = 0; i < count; ++i) {
    nf4i::Scales sc{};
    int64_t n = 0;
    if (int rc = check_weight(&ws[i], &sc, &n, who)) return rc;
    if (!xs[i] || !ys[i]) return fail(NF4_ERR_NULL, "%s: x and y of weight %d are required", who, i);
    if (ws[i].cols % 64 || ws[i].cols > 65536)
      return fail(NF4_ERR_SIZE, "%s: weight %d has cols = %lld (a multiple of 64 up to 65536 is required)", who, i,
                  (long long)ws[i].cols);
    if (!aligned(xs[i], 16) || !aligned(ys[i], 16))
      return fail(NF4_ERR_ALIGN, "%s: x and y of weight %d must be 16-byte aligned", who, i);
    if (i > 0 && ((sc.absmax == nullptr) != (jobs[0].sc.absmax == nullptr) || sc.f8 != jobs[0].sc.f8 ||
                  sc.fp4 != jobs[0].sc.fp4))
      return fail(NF4_ERR_DTYPE, "%s: weight %d has another scale form or code book than weight 0", who, i);
    jobs[i] = nf4i::GemvJob{w_packed(ws[i]), ws[i].rows, ws[i].cols, sc, static_cast<const uint16_t*>(xs[i]), ys[i]};
  }
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_gemv_batch(jobs, count, y_dtype == NF4_BF16, as_stream(stream)), who);
}

size_t nf4_gemm_workspace(int64_t m, int64_t rows, int32_t r) {
  if (m < 1 || rows < 1 || r < 1 || r > 64) return 0;
  return (nf4i::gemm_workspace(m, rows, r) + 255) & ~size_t(255);
}

int nf4_gemm(const nf4_weight* w, const void* x, int64_t m, void* y, const void* lora_a,
             const void* lora_b, int32_t r, float lora_scale, void* workspace,
             size_t workspace_bytes, void* stream) {
  nf4i::Scales sc{};
  int64_t n = 0;
  if (int rc = check_weight(w, &sc, &n, "nf4_gemm")) return rc;
  if (!x || !y) return fail(NF4_ERR_NULL, "nf4_gemm: x and y are required");
  if (w->cols % 64) return fail(NF4_ERR_SIZE, "nf4_gemm: cols = %lld is not a multiple of 64", (long long)w->cols);
  if (w->cols >= (int64_t(1) << 23)) return fail(NF4_ERR_SIZE, "nf4_gemm: cols = %lld out of range", (long long)w->cols);
  if (m < 1 || m > (int64_t(1) << 31)) return fail(NF4_ERR_SIZE, "nf4_gemm: m = %lld out of range", (long long)m);
  if ((lora_a == nullptr) != (lora_b == nullptr))
    return fail(NF4_ERR_NULL, "nf4_gemm: lora_a and lora_b must both be NULL or both be set");
  if (lora_a) {
    if (r < 1 || r > 64) return fail(NF4_ERR_SIZE, "nf4_gemm: LoRA rank r = %d out of range 1..64", (int)r);
    if (!std::isfinite(lora_scale)) return fail(NF4_ERR_SIZE, "nf4_gemm: lora_scale is not finite");
    if (!aligned(lora_a, 16) || !aligned(lora_b, 16))
      return fail(NF4_ERR_ALIGN, "nf4_gemm: lora_a and lora_b must be 16-byte aligned");
    const size_t need = nf4_gemm_workspace(m, w->rows, r);
    if (!workspace || workspace_bytes < need)
      return fail(NF4_ERR_WORKSPACE, "nf4_gemm: workspace needs %zu bytes", need);
    if (!aligned(workspace, 16)) return fail(NF4_ERR_ALIGN, "nf4_gemm: workspace must be 16-byte aligned");
  } else if (r != 0) {
    return fail(NF4_ERR_SIZE, "nf4_gemm: r must be 0 without LoRA matrices");
  }
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(NF4_ERR_ALIGN, "nf4_gemm: x and y must be 16-byte aligned");
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_gemm(w->packed, w->rows, w->cols, sc, static_cast<const uint16_t*>(x), m,
                                    static_cast<uint16_t*>(y), static_cast<const uint16_t*>(lora_a),
                                    static_cast<const uint16_t*>(lora_b), lora_a ? r : 0, lora_scale,
                                    static_cast<uint16_t*>(workspace), as_stream(stream)),
                  "nf4_gemm");
}

size_t nf4_gemm_dx_workspace(int64_t m, int64_t rows, int32_t r) {
  if (m < 1 || rows < 1 || r < 1 || r > 64) return 0;
  const size_t bytes = nf4i::gemm_dx_workspace(m, rows, r);
  return (bytes + 255) & ~size_t(255);
}

int nf4_gemm_dx(const nf4_weight* w, const void* dy, int64_t m, void* dx, const void* lora_a,
                const void* lora_b, int32_t r, float lora_scale, void* workspace, size_t workspace_bytes,
                void* stream) {
  nf4i::Scales sc{};
  int64_t n = 0;
  if (int rc = check_weight(w, &sc, &n, "nf4_gemm_dx")) return rc;
  if (!dy || !dx) return fail(NF4_ERR_NULL, "nf4_gemm_dx: dy and dx are required");
  if (w->cols % 64)
    return fail(NF4_ERR_SIZE, "nf4_gemm_dx: cols = %lld is not a multiple of 64", (long long)w->cols);
  if (w->rows % 8) return fail(NF4_ERR_SIZE, "nf4_gemm_dx: rows = %lld is not a multiple of 8", (long long)w->rows);
  if (w->rows >= (int64_t(1) << 23) || w->cols >= (int64_t(1) << 23))
    return fail(NF4_ERR_SIZE, "nf4_gemm_dx: rows = %lld, cols = %lld out of range", (long long)w->rows,
                (long long)w->cols);
  if (m < 1 || m > (int64_t(1) << 31)) return fail(NF4_ERR_SIZE, "nf4_gemm_dx: m = %lld out of range", (long long)m);
  if ((lora_a == nullptr) != (lora_b == nullptr))
    return fail(NF4_ERR_NULL, "nf4_gemm_dx: lora_a and lora_b must both be NULL or both be set");
  if (lora_a) {
    if (r < 1 || r > 64) return fail(NF4_ERR_SIZE, "nf4_gemm_dx: LoRA rank r = %d out of range 1..64", (int)r);
    if (!std::isfinite(lora_scale)) return fail(NF4_ERR_SIZE, "nf4_gemm_dx: lora_scale is not finite");
    if (!aligned(lora_a, 16) || !aligned(lora_b, 16))
      return fail(NF4_ERR_ALIGN, "nf4_gemm_dx: lora_a and lora_b must be 16-byte aligned");
    const size_t need = nf4_gemm_dx_workspace(m, w->rows, r);
    if (!workspace || workspace_bytes < need)
      return fail(NF4_ERR_WORKSPACE, "nf4_gemm_dx: workspace needs %zu bytes", need);
    if (!aligned(workspace, 256)) return fail(NF4_ERR_ALIGN, "nf4_gemm_dx: workspace must be 256-byte aligned");
  } else if (r != 0) {
    return fail(NF4_ERR_SIZE, "nf4_gemm_dx: r must be 0 without LoRA matrices");
  }
  if (!aligned(dy, 16) || !aligned(dx, 16))
    return fail(NF4_ERR_ALIGN, "nf4_gemm_dx: dy and dx must be 16-byte aligned");
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_gemm_dx(w->packed, w->rows, w->cols, sc, static_cast<const uint16_t*>(dy), m,
                                       static_cast<uint16_t*>(dx), static_cast<const uint16_t*>(lora_a),
                                       static_cast<const uint16_t*>(lora_b), lora_a ? r : 0, lora_scale,
                                       static_cast<uint16_t*>(workspace), as_stream(stream)),
                  "nf4_gemm_dx");
}

size_t nf4_lora_grads_workspace(int64_t m, int64_t rows, int64_t cols, int32_t r) {
  if (m < 1 || rows < 1 || cols < 1 || r < 1 || r > 64) return 0;
  return nf4i::lora_grads_workspace(m, rows, cols, r);
}

int nf4_lora_grads(const void* x, const void* dy, int64_t m, int64_t rows, int64_t cols, const void* lora_a,
                   const void* lora_b, int32_t r, float lora_scale, float* da, float* db, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!x || !dy || !lora_a || !lora_b)
    return fail(NF4_ERR_NULL, "nf4_lora_grads: x, dy, lora_a and lora_b are required");
  if (!da && !db) return fail(NF4_ERR_NULL, "nf4_lora_grads: at least one of da and db is required");
  if (m < 1 || m > (int64_t(1) << 31)) return fail(NF4_ERR_SIZE, "nf4_lora_grads: m = %lld out of range", (long long)m);
  if (rows < 8 || rows > kMaxN || rows % 8 || cols < 8 || cols > kMaxN || cols % 8)
    return fail(NF4_ERR_SIZE, "nf4_lora_grads: rows = %lld and cols = %lld must be positive multiples of 8",
                (long long)rows, (long long)cols);
  if (r < 1 || r > 64) return fail(NF4_ERR_SIZE, "nf4_lora_grads: LoRA rank r = %d out of range 1..64", (int)r);
  if (!std::isfinite(lora_scale)) return fail(NF4_ERR_SIZE, "nf4_lora_grads: lora_scale is not finite");
  if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(lora_a, 16) || !aligned(lora_b, 16) || !aligned(da, 16) ||
      !aligned(db, 16))
    return fail(NF4_ERR_ALIGN, "nf4_lora_grads: x, dy, lora_a, lora_b, da and db must be 16-byte aligned");
  const size_t need = nf4_lora_grads_workspace(m, rows, cols, r);
  if (!workspace || workspace_bytes < need)
    return fail(NF4_ERR_WORKSPACE, "nf4_lora_grads: workspace needs %zu bytes", need);
  if (!aligned(workspace, 256)) return fail(NF4_ERR_ALIGN, "nf4_lora_grads: workspace must be 256-byte aligned");
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_lora_grads(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dy), m, rows,
                                          cols, static_cast<const uint16_t*>(lora_a),
                                          static_cast<const uint16_t*>(lora_b), r, lora_scale, da, db, workspace,
                                          as_stream(stream)),
                  "nf4_lora_grads");
}

int nf4_lora_merge(const nf4_weight* w, const void* lora_a, const void* lora_b, int32_t r, float lora_scale,
                   void* out, int out_dtype, void* stream) {
  nf4i::Scales sc{};
  int64_t n = 0;
  if (int rc = check_weight(w, &sc, &n, "nf4_lora_merge")) return rc;
  if (!lora_a || !lora_b || !out) return fail(NF4_ERR_NULL, "nf4_lora_merge: lora_a, lora_b and out are required");
  if (w->cols % 8) return fail(NF4_ERR_SIZE, "nf4_lora_merge: cols = %lld is not a multiple of 8", (long long)w->cols);
  if (w->rows > (int64_t(1) << 24)) return fail(NF4_ERR_SIZE, "nf4_lora_merge: rows = %lld out of range", (long long)w->rows);
  if (w->cols > int64_t(65535) * 2048)
    return fail(NF4_ERR_SIZE, "nf4_lora_merge: cols = %lld out of range", (long long)w->cols);
  if (r < 1 || r > 64) return fail(NF4_ERR_SIZE, "nf4_lora_merge: LoRA rank r = %d out of range 1..64", (int)r);
  if (!std::isfinite(lora_scale)) return fail(NF4_ERR_SIZE, "nf4_lora_merge: lora_scale is not finite");
  if (out_dtype != NF4_BF16 && out_dtype != NF4_F16)
    return fail(NF4_ERR_DTYPE, "nf4_lora_merge: out_dtype %d is not NF4_BF16 or NF4_F16", out_dtype);
  if (!aligned(lora_a, 16) || !aligned(lora_b, 16) || !aligned(out, 16))
    return fail(NF4_ERR_ALIGN, "nf4_lora_merge: lora_a, lora_b and out must be 16-byte aligned");
  if (int rc = check_device()) return rc;
  return launched(nf4i::launch_lora_merge(w->packed, w->rows, w->cols, sc, static_cast<const uint16_t*>(lora_a),
                                          static_cast<const uint16_t*>(lora_b), r, lora_scale,
                                          static_cast<uint16_t*>(out), out_dtype == NF4_F16, as_stream(stream)),
                  "nf4_lora_merge");
}

}  // extern "C"
