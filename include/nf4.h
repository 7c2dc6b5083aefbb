/*
 * nf4.h -- C ABI of the NF4 (4-bit NormalFloat) weight library for AMD
 * Instinct MI355X (gfx950).
 *
 * What the calls compute is stated on the bitsandbytes tool page
 * (ozercemkelahmet.com/tools/bitsandbytes), section "How it works", Steps 1-5:
 * weights are cut into blocks of 64, each block is divided by its largest
 * absolute value, each value is replaced by the index of the nearest entry of
 * a 16-entry code book spaced to a bell curve ("How NF4 works"), two indices
 * are packed per byte with the scales stored beside them, and at run time a
 * block is expanded back to 16-bit with its scale and multiplied.  The scales
 * themselves can be quantized again ("Double quantization"; the tutorial page
 * "bitsandbytes quantization tutorial: 4-bit and 8-bit models", section
 * "4-bit Loading with NF4").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Array arguments are DEVICE pointers unless marked [host].
 *  - The caller allocates, sizes and owns every buffer.  The library never
 *    allocates or frees memory, never synchronizes, and keeps no per-call
 *    state; the only state it keeps is a per-device record of whether the
 *    device is a gfx950.
 *  - Every call checks its arguments on the host first.  On failure it
 *    returns a non-zero nf4_status, launches nothing and writes nothing; the
 *    reason is available from nf4_last_error().  On success the work is
 *    enqueued on `stream` (a hipStream_t passed as void*; NULL = the null
 *    stream of the current device) and the call returns NF4_OK.  Faults inside
 *    a kernel surface at the caller's next synchronization.
 *  - Calls are thread-safe.  Calls on different streams may overlap; they
 *    share nothing except caller-provided buffers.
 *  - bf16 buffers are passed as void* and hold IEEE bfloat16 bit patterns.
 *  - Inputs must be finite; results for NaN or infinite inputs are undefined.
 */
#ifndef NF4_H
#define NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nf4_status {
  NF4_OK = 0,
  NF4_ERR_NULL = 1,       /* a required pointer is NULL                           */
  NF4_ERR_SIZE = 2,       /* a size or count is out of range                      */
  NF4_ERR_BLOCKSIZE = 3,  /* blocksize != 64 or blocksize2 != 256                 */
  NF4_ERR_ALIGN = 4,      /* a pointer is not aligned as documented               */
  NF4_ERR_DTYPE = 5,      /* unknown nf4_dtype, or a dtype the call does not take */
  NF4_ERR_WORKSPACE = 6,  /* workspace missing or smaller than the *_workspace()  */
  NF4_ERR_DEVICE = 7,     /* the device is not gfx950, or a HIP call failed       */
  NF4_ERR_INTERNAL = 8    /* a self-check of the library's own host tables failed */
} nf4_status;

typedef enum nf4_dtype { NF4_F32 = 0, NF4_BF16 = 1, NF4_F16 = 2 } nf4_dtype;

/* Type of the double-quantized scale codes (nf4_weight.dq_type). */
typedef enum nf4_dq_type { NF4_DQ_INT8 = 0, NF4_DQ_FP8 = 1 } nf4_dq_type;

/* Code book of the 4-bit codes (nf4_weight.quant_type): NF4, or FP4 (tool
 * page "What it is": 4-bit FP4 and NF4 formats; "Glossary": FP4 is a 4-bit
 * floating-point type).  A zero-initialised weight descriptor means NF4. */
typedef enum nf4_quant_type { NF4_QT_NF4 = 0, NF4_QT_FP4 = 1 } nf4_quant_type;

#define NF4_BLOCKSIZE 64
#define NF4_BLOCKSIZE2 256

/* [host] Text describing the last failure on the calling thread ("" if none). */
const char* nf4_last_error(void);

/* [host] The 16 NF4 levels as float32, ascending: out[0] = -1, out[7] = 0,
 * out[15] = +1.  Tool page, "How NF4 works": the 16 code values each cover an
 * equal share of the bell curve.  They are the normal quantiles at 8 (positive
 * side) and 7 (negative side) evenly spaced probabilities between
 * delta = 1 - (1/30 + 1/32)/2 and 1/2 (1/2 excluded), plus 0, divided by the
 * quantile at delta.  Derived on the host in extended precision at first use.
 * Needs no GPU.  Returns NF4_ERR_NULL if out is NULL. */
int nf4_codebook(float out[16]);

/* [host] The 16 FP4 levels as float32, by code (the 4-bit pattern).  The pages
 * name FP4 without values; the reading used is the E2M1 element type of the
 * Open Compute Project microscaling formats specification (sign in bit 3, two
 * exponent bits with bias 1, one mantissa bit, exponent field 0 subnormal:
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), divided by 6 so that the block
 * absmax maps to +-1: out[c] = e2m1(c) / 6, out[7] = 1, out[15] = -1,
 * out[8] = -0.  Needs no GPU.  Returns NF4_ERR_NULL if out is NULL. */
int nf4_codebook_fp4(float out[16]);

/* Blockwise NF4 quantization -- tool page "How it works", Steps 1-4.
 *   x       : n input values, x_dtype NF4_F32 or NF4_BF16; 16-byte aligned.
 *   n       : number of values, 1 <= n < 2^40.  Blocks run along x in order;
 *             the last block may be partial and its absmax covers only the
 *             values that exist.
 *   blocksize: must be 64.
 *   packed  : out, ceil(n/2) bytes, 16-byte aligned.  Byte j holds the code of
 *             element 2j in bits 7..4 and of element 2j+1 in bits 3..0; when n
 *             is odd the final low nibble is 7 (the zero level).
 *   absmax  : out, ceil(n/64) float32, 4-byte aligned: the largest |x| of each
 *             block (exact).
 * Each code is the index of the level nearest to fl32(x / absmax) (an IEEE
 * float32 division), an exact tie going to the level farther from zero; a
 * block whose absmax is 0 gets code 7 throughout. */
int nf4_quantize(const void* x, int x_dtype, int64_t n, int32_t blocksize,
                 uint8_t* packed, float* absmax, void* stream);

/* FP4 quantization: nf4_quantize's steps with the FP4 code book (see
 * nf4_codebook_fp4).  Each code is the pattern of the FP4 level nearest to
 * fl32(x / absmax) among the 15 patterns other than 1000 (negative zero),
 * an exact tie going to the level farther from zero; zero is 0000, so an odd
 * n ends in a low nibble 0 and a block whose absmax is 0 gets code 0
 * throughout.  Arguments, layout and errors as nf4_quantize. */
int nf4_quantize_fp4(const void* x, int x_dtype, int64_t n, int32_t blocksize,
                     uint8_t* packed, float* absmax, void* stream);

/* One tensor of a batched quantization (device pointers). */
typedef struct nf4_quantize_job {
  const void* x;    /* n values (x_dtype of the call), 16-byte aligned      */
  int64_t n;        /* 1 <= n < 2^40                                         */
  uint8_t* packed;  /* out: ceil(n/2) bytes, 16-byte aligned                 */
  float* absmax;    /* out: ceil(n/64) float32, 4-byte aligned               */
} nf4_quantize_job;

/* The blockwise quantization of the tool page's "How it works", Steps 1-4,
 * for 1 to 8 tensors (for instance the seven weights of one transformer
 * layer) in one launch instead of one per tensor.  All tensors share
 * x_dtype and the code book: quant_type NF4_QT_NF4 gives each tensor exactly
 * the outputs of nf4_quantize on it alone, NF4_QT_FP4 those of
 * nf4_quantize_fp4.  jobs: count host structs.  Outputs of different
 * tensors must not overlap.  Errors as nf4_quantize, checked for every
 * tensor before anything is launched; NF4_ERR_SIZE for count outside 1..8,
 * NF4_ERR_DTYPE for another quant_type. */
int nf4_quantize_batched(const nf4_quantize_job* jobs, int32_t count, int x_dtype, int32_t blocksize,
                         int32_t quant_type, void* stream);

/* Bytes of device workspace nf4_double_quant needs (a small constant). */
size_t nf4_double_quant_workspace(int64_t nblocks);

/* Double quantization of the block scales -- tool page "Double quantization"
 * with the int8 scheme of its section "A worked example".
 *   absmax  : nblocks float32 scales from nf4_quantize, 16-byte aligned,
 *             1 <= nblocks < 2^31.
 *   blocksize2: must be 256.
 *   qabsmax : out, nblocks int8, 16-byte aligned.
 *   absmax2 : out, ceil(nblocks/256) float32, 4-byte aligned.
 *   mean    : out, one float32 (device).
 *   workspace: at least nf4_double_quant_workspace(nblocks) bytes, 16-byte
 *             aligned; its contents on entry do not matter.
 * mean = fl32(fl64(S) / nblocks) where S is the exact sum of the scales (the
 * sum is accumulated exactly in a wide integer, so mean does not depend on
 * summation order).  With c = fl32(absmax - mean) and, per group of 256,
 * s2 = max |c|: t = fl32(fl32(c / s2) * 127) and q = sign(t) floor(|t| + 1/2)
 * (half away from zero); q = 0 in a group whose s2 is 0. */
int nf4_double_quant(const float* absmax, int64_t nblocks, int32_t blocksize2,
                     int8_t* qabsmax, float* absmax2, float* mean,
                     void* workspace, size_t workspace_bytes, void* stream);

/* nf4_double_quant for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, hosts that forbid
 * allocation): the same arguments, results and errors without the
 * workspace.  The partial sums live in a static 24 KiB device array that the
 * library holds on every device it runs on until the process ends; its
 * address is looked up on the first call on a device.  Allocates nothing.
 * nblocks is limited to 1 <= nblocks < 2^31 as for nf4_double_quant (the
 * scratch needed does not grow with nblocks); a size outside that range is
 * rejected with NF4_ERR_SIZE.  Every call on one device shares that array:
 * calls that may overlap on one device (different streams with no ordering
 * between them) race and must not be made; calls ordered on one stream are
 * fine.  The array's contents on entry do not matter. */
int nf4_double_quant_noalloc(const float* absmax, int64_t nblocks, int32_t blocksize2,
                             int8_t* qabsmax, float* absmax2, float* mean, void* stream);

/* The float8 reading of the second level -- tutorial page "How NF4 Works":
 * the scales go from float32 to float8.  Same arguments and mean as
 * nf4_double_quant; qabsmax receives E4M3 codes (Open Compute Project 8-bit
 * floating point: bias 7, 3 mantissa bits, subnormals, largest finite 448):
 * t = fl32(fl32(c / s2) * 448) and q = the E4M3 code nearest to t, ties to the
 * even mantissa; q = 0 in a group whose s2 is 0.  A weight using these codes
 * sets dq_type = NF4_DQ_FP8, and its scales are
 * a_hat = fl32(fl32(fl32(e4m3(q) / 448) * s2) + mean). */
/* [host] The 256 values fl32(e4m3(q) / 448) the float8 second level uses in
 * place of q / 127 (0 for the two NaN codes, which are never written).
 * Needs no GPU.  Returns NF4_ERR_NULL for a NULL out. */
int nf4_e4m3_ratio(float out[256]);

int nf4_double_quant_f8(const float* absmax, int64_t nblocks, int32_t blocksize2,
                        uint8_t* qabsmax, float* absmax2, float* mean,
                        void* workspace, size_t workspace_bytes, void* stream);

/* One scale array of a batched double quantization (device pointers). */
typedef struct nf4_dq_job {
  const float* absmax;  /* nblocks float32 scales, 16-byte aligned            */
  int64_t nblocks;      /* 1 <= nblocks < 2^31                                 */
  void* qabsmax;        /* out: nblocks int8 (or E4M3) codes, 16-byte aligned  */
  float* absmax2;       /* out: ceil(nblocks / 256) float32, 4-byte aligned    */
  float* mean;          /* out: one float32                                    */
} nf4_dq_job;

/* Bytes of device workspace nf4_double_quant_batched needs for `count`
 * arrays (24 KiB per array; 0 for count outside 1..8). */
size_t nf4_double_quant_batched_workspace(int32_t count);

/* The double quantization of the tool page's "Double quantization" section
 * for 1 to 8 scale arrays at once (for instance the seven weights of one
 * transformer layer), in one pair of launches instead of one pair per
 * array.  dq_type NF4_DQ_INT8 gives each array exactly the outputs of
 * nf4_double_quant on it alone, NF4_DQ_FP8 those of nf4_double_quant_f8:
 * each array has its own exact mean and its own groups of 256.
 *   jobs     : count host structs (the struct itself is read on the host).
 *   workspace: at least nf4_double_quant_batched_workspace(count) bytes,
 *              16-byte aligned; its contents on entry do not matter.
 * Outputs of different arrays must not overlap.  Errors as
 * nf4_double_quant, checked for every array before anything is launched;
 * NF4_ERR_SIZE for count outside 1..8, NF4_ERR_DTYPE for another dq_type. */
int nf4_double_quant_batched(const nf4_dq_job* jobs, int32_t count, int32_t blocksize2, int32_t dq_type,
                             void* workspace, size_t workspace_bytes, void* stream);

/* [host] A quantized weight: a struct holding device pointers.  The logical
 * matrix W[rows][cols] is row-major, element i = r*cols + c, and blocks of 64
 * run along that order.  Exactly one scale form is given:
 *   absmax != NULL                      : plain fp32 scales (no double quant);
 *   absmax == NULL, qabsmax/absmax2/mean: double-quantized scales, and each
 *     block's scale is a_hat = fl32(fl32(fl32(q / 127) * s2) + mean) for
 *     dq_type NF4_DQ_INT8, or fl32(fl32(fl32(e4m3(q) / 448) * s2) + mean) for
 *     NF4_DQ_FP8 (codes from nf4_double_quant_f8).  dq_type is ignored for
 *     plain scales; a zero-initialised struct means int8. */
typedef struct nf4_weight {
  const uint8_t* packed;    /* ceil(rows*cols/2) bytes, 16-byte aligned          */
  int64_t rows, cols;       /* rows >= 1, cols >= 1                              */
  int32_t blocksize;        /* 64                                                */
  const float* absmax;      /* ceil(rows*cols/64) float32, or NULL               */
  const int8_t* qabsmax;    /* ceil(rows*cols/64) int8 when absmax == NULL       */
  const float* absmax2;     /* ceil(nblocks/256) float32 when absmax == NULL     */
  const float* mean;        /* one float32 when absmax == NULL                   */
  int32_t blocksize2;       /* 256 when absmax == NULL                           */
  int32_t dq_type;          /* nf4_dq_type of qabsmax when absmax == NULL        */
  int32_t quant_type;       /* nf4_quant_type of the codes in packed             */
} nf4_weight;

/* Dequantization -- tool page "How it works", Step 5.
 *   out: rows*cols values of out_dtype (NF4_F32 or NF4_BF16), 16-byte aligned.
 * out[i] = fl32(level[code_i] * a_hat_block(i)); for bf16 that float32 value
 * is rounded once to nearest even. */
int nf4_dequantize(const nf4_weight* w, void* out, int out_dtype, void* stream);

/* Fused dequantize-and-multiply for decode: y = x . deq(W)^T.
 *   x : bf16 [m][cols], 16-byte aligned;  1 <= m <= 16;  cols % 64 == 0.
 *   y : [m][rows] of y_dtype (NF4_F32 or NF4_BF16), 16-byte aligned.
 * Products are accumulated in float32; no dequantized copy of W is written
 * to memory (tool page "How it works", Step 5: the expanded copy is
 * temporary).  What enters the products depends on the path:
 *  - m <= 2, and m <= 4 on matrices of at least 2^27 weights, with
 *    cols <= 65536 (m == 1) or cols <= 32768 (m > 1): the levels rounded to
 *    fp16 (11 significant bits, relative error <= 2^-11) and x exactly
 *    (scaled by a power of two per 64-block); the block scale is applied
 *    once per block in float32; wider rows take the float32 levels (m > 1),
 *    or each level as a pair of bf16 parts (16 significant bits, m == 1);
 *  - any other m <= 16 (the matrix cores): the weight rounded once to bf16
 *    after scaling, bf16(fl32(level * a_hat)), exactly as nf4_gemm takes it,
 *    and x exactly. */
int nf4_gemv(const nf4_weight* w, const void* x, int64_t m, void* y, int y_dtype,
             void* stream);

/* Decode GEMV of several weights in one launch: ys[i] = xs[i] . deq(ws[i])^T
 * for i < count, each at m = 1 (tool page "How it works", Step 5, as
 * nf4_gemv).  One decode step multiplies the same token by every weight of a
 * layer, and several of those products share their input (the attention
 * projections, the MLP input projections); one launch streams all of them
 * back to back with no drain of the chip between weights.
 *   ws    : [host] array of count weight descriptors, 1 <= count <= 8, each
 *           with cols % 64 == 0 and cols <= 65536, all with the same scale
 *           form (plain, int8 or float8 second level) and code book.
 *   xs    : [host] array of count device pointers, xs[i] bf16 [1][ws[i].cols],
 *           16-byte aligned.  Weights whose x is the same pointer (and
 *           width) are streamed as one group of rows.
 *   ys    : [host] array of count device pointers, ys[i] [1][ws[i].rows] of
 *           y_dtype (NF4_F32 or NF4_BF16), 16-byte aligned, not overlapping
 *           each other or any input.
 * Each ys[i] holds exactly the bits nf4_gemv(&ws[i], xs[i], 1, ys[i], ...)
 * writes for cols <= 65536: the same levels rounded to fp16, the same x
 * scaling, the same per-lane sums and the same fixed order of the segment
 * sums.  One launch. */
int nf4_gemv_batched(const nf4_weight* ws, int32_t count, const void* const* xs, void* const* ys, int y_dtype,
                     void* stream);

/* Bytes of device workspace nf4_gemm needs for m rows of x, a weight of
 * `rows` rows and LoRA rank r (0 when r == 0): m + rows rows of 2 r (rounded
 * up to 64) bf16 values. */
size_t nf4_gemm_workspace(int64_t m, int64_t rows, int32_t r);

/* Dequantize-and-multiply bf16 matrix-core GEMM for prefill and training
 * (the codes are expanded to bf16 straight into the matrix-core operands; no
 * dequantized copy of W is written to memory), with an optional fused LoRA
 * term (tutorial page "QLoRA: Fine-Tuning a 4-bit Model"
 * and tool page "Fine-tuning with adapters on a 4-bit model": a frozen 4-bit
 * base plus low-rank adapters whose output is multiplied by a scale factor):
 *   y = x . deq(W)^T + lora_scale . (x . A^T) . B^T
 *   x      : bf16 [m][cols], 16-byte aligned, m >= 1, cols % 64 == 0,
 *            cols < 2^23.
 *   y      : bf16 [m][rows], 16-byte aligned.
 *   lora_a : bf16 [r][cols] and lora_b : bf16 [rows][r], both NULL (then r
 *            must be 0) or both set with 1 <= r <= 64; 16-byte aligned.
 *   workspace: at least nf4_gemm_workspace(m, rows, r) bytes, 16-byte aligned
 *            (may be NULL when that is 0).
 * W is dequantized to bf16 exactly as nf4_dequantize does; products are
 * accumulated in float32 and y is rounded once to bf16. */
int nf4_gemm(const nf4_weight* w, const void* x, int64_t m, void* y,
             const void* lora_a, const void* lora_b, int32_t r, float lora_scale,
             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace nf4_gemm_dx needs for m rows of dy, a weight of
 * `rows` rows and LoRA rank r (0 when r == 0). */
size_t nf4_gemm_dx_workspace(int64_t m, int64_t rows, int32_t r);

/* Input gradient through the frozen 4-bit base for QLoRA training (tutorial
 * page "QLoRA: Fine-Tuning a 4-bit Model": the base stays frozen and the
 * gradients pass through it to the low-rank adapters; tool page "How it
 * works", Step 5: blocks are expanded to 16-bit for the matrix hardware):
 *   dx = dy . deq(W) + lora_scale . (dy . B) . A
 * the backward of nf4_gemm's y = x . deq(W)^T + lora_scale . (x . A^T) . B^T
 * with respect to x.
 *   w      : the NF4 weight [rows][cols] (either scale form); cols % 64 == 0,
 *            rows % 8 == 0, rows and cols < 2^23.
 *   dy     : bf16 [m][rows], 16-byte aligned, 1 <= m <= 2^31.
 *   dx     : bf16 [m][cols], 16-byte aligned, not overlapping dy.
 *   lora_a : bf16 [r][cols] and lora_b : bf16 [rows][r], both NULL (then r
 *            must be 0) or both set with 1 <= r <= 64; 16-byte aligned.
 *   workspace: at least nf4_gemm_dx_workspace(m, rows, r) bytes, 256-byte
 *            aligned (may be NULL when that is 0); overwritten.
 * W is dequantized to bf16 exactly as nf4_dequantize does; products are
 * accumulated in float32 and dx is rounded once to bf16.  The adapter term
 * forms U = lora_scale . dy . B in float32 and carries it as two bf16 parts. */
int nf4_gemm_dx(const nf4_weight* w, const void* dy, int64_t m, void* dx,
                const void* lora_a, const void* lora_b, int32_t r, float lora_scale,
                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace nf4_lora_grads needs (0 for invalid sizes). */
size_t nf4_lora_grads_workspace(int64_t m, int64_t rows, int64_t cols, int32_t r);

/* Gradients of the low-rank adapters on the frozen base (tutorial page
 * "QLoRA: Fine-Tuning a 4-bit Model": only the adapters train and their
 * output is multiplied by a scale factor).  For nf4_gemm's
 * y = x . deq(W)^T + lora_scale . (x . A^T) . B^T:
 *   da = lora_scale . (dy . B)^T . x        float32 [r][cols]
 *   db = lora_scale . dy^T . (x . A^T)      float32 [rows][r]
 *   x      : bf16 [m][cols], dy : bf16 [m][rows], 1 <= m <= 2^31;
 *            rows and cols positive multiples of 8.
 *   lora_a : bf16 [r][cols], lora_b : bf16 [rows][r], 1 <= r <= 64.
 *   da, db : outputs; either may be NULL to skip it, not both.  Overwritten.
 *   All arrays 16-byte aligned; workspace at least
 *   nf4_lora_grads_workspace(m, rows, cols, r) bytes, 256-byte aligned.
 * The thin products (dy . B and x . A^T) and every sum are formed in float32;
 * results are deterministic (fixed summation order). */
int nf4_lora_grads(const void* x, const void* dy, int64_t m, int64_t rows, int64_t cols,
                   const void* lora_a, const void* lora_b, int32_t r, float lora_scale,
                   float* da, float* db, void* workspace, size_t workspace_bytes, void* stream);

/* LoRA merge -- tutorial page, "Merging LoRA Adapters After Fine-Tuning":
 * after training the adapters are folded into one dense 16-bit copy of the
 * base, which needs the base dequantized first (tool page, "Practical
 * guidance and best practices": merging adds a rounding step).
 *   out[n][k] = round( deq[n][k] + lora_scale * sum_j B[n][j] * A[j][k] )
 *   w      : the NF4 weight [rows][cols] (either scale form); cols % 8 == 0.
 *   lora_a : bf16 [r][cols], lora_b : bf16 [rows][r], 1 <= r <= 64, both
 *            16-byte aligned.  lora_scale is finite (alpha / r).
 *   out    : [rows][cols] of out_dtype (NF4_BF16 or NF4_F16), 16-byte
 *            aligned, not overlapping any input.
 * deq[n][k] is the float32 value nf4_dequantize writes.  The sum is formed in
 * float64 with j ascending (exact for bf16 adapters unless its terms span
 * more than about 37 binary orders), multiplied by lora_scale and added to
 * deq[n][k] in float64, and the result is rounded once to nearest even into
 * out_dtype (fp16 subnormals kept). */
int nf4_lora_merge(const nf4_weight* w, const void* lora_a, const void* lora_b, int32_t r,
                   float lora_scale, void* out, int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NF4_H */
