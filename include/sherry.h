/*
 * sherry.h - C ABI of libsherry.so: Sherry 1.25-bit (3:4-sparse ternary)
 * weights on AMD Instinct MI355X (gfx950).
 *
 * The format ("Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via
 * Fine-grained Sparsification", Abstract; Figure 2 caption): weights are
 * ternary, {-1, 0, +1}; every block of four consecutive weights holds exactly
 * one zero (3:4 fine-grained sparsity), so a block has 4 * 2^3 = 32 states and
 * packs into a 5-bit code, 1.25 bits per weight.  The layout below is this
 * library's reading of that format (the pages give no bit layout):
 *
 *   block j of row r   = W[r, 4j .. 4j+3] (along the reduction axis K)
 *   code               = z | n0 << 2 | n1 << 3 | n2 << 4
 *                        z  = slot of the zero (0..3)
 *                        n0..n2 = sign bits of the three nonzero slots in
 *                        ascending slot order, 1 = -1, 0 = +1
 *   group              = 32 codes (128 weights) in 5 little-endian uint32
 *                        words, one LSB-first 160-bit stream: code j at bits
 *                        [5j, 5j+5) of d0 + d1*2^32 + ... + d4*2^128
 *   row                = 5 * K/128 words: words 0-3 of every group first
 *                        (group g at word 4g, 16 bytes), then word 4 of
 *                        every group (group g at word 4*K/128 + g)
 *   matrix             = n rows one after another, K % 128 == 0
 *   scales             = one per output row (fp32 or fp16)
 *
 * Products (all accumulate exactly in int32 for int8 activations):
 *   acc[r]    = sum_k T[r, k] * x[k]
 *   y[r]      = ydt( (fp32(acc[r]) * fp32(s_w[r])) * s_x )     int8 x
 *   y[r]      = fp32 accumulation of T[r, k] * x[k], then * fp32(s_w[r])  bf16 x
 *   Y[m, r]   = ydt( (fp32(acc[m, r]) * fp32(s_w[r])) * s_x[m] )  int8 X
 * Every multiply is a separate IEEE fp32 round-to-nearest-even step; the
 * final conversion to fp16 is round-to-nearest-even.
 *
 * Conventions for every entry point:
 *   - Buffers are DEVICE pointers owned by the caller (except where a
 *     parameter says HOST).  The library allocates no device memory and keeps
 *     no per-call state (its one setting, sherry_set_prefill_kernel, is
 *     process-wide); calls are thread-safe.
 *   - All argument checks run on the host before any HIP call.  On an error
 *     the call returns a status and enqueues nothing.
 *   - Work is enqueued on `stream` (asynchronous, no implicit sync).  Errors
 *     that happen on the device are not reported by the call.
 *   - Input and output buffers must not overlap.
 */
#ifndef SHERRY_H
#define SHERRY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SHERRY_OK = 0,
  SHERRY_EINVAL = 1,  /* null pointer where one is required, n/k/m <= 0, bad enum */
  SHERRY_ESHAPE = 2,  /* k % 128 != 0, leading dimension too small, size overflow; for the
                         products also one matrix's codes (or a GEMM's x, m * ldx bytes)
                         above 4 GiB - 1 bytes, the reach of the kernels' 32-bit offsets */
  SHERRY_EDTYPE = 3,  /* unsupported dtype combination */
  SHERRY_EALIGN = 4,  /* a pointer or leading dimension breaks the stated alignment */
  SHERRY_EDEVICE = 5, /* no HIP device, or the current device is not gfx950 */
  SHERRY_ELAUNCH = 6, /* the kernel launch failed (hipGetLastError) */
  SHERRY_ESCRATCH = 7 /* sherry_gemv_grouped_noalloc: plan above its 1 MiB static memory */
} sherry_status;

typedef enum {
  SHERRY_I8 = 0,
  SHERRY_I32 = 1,
  SHERRY_F16 = 2,
  SHERRY_BF16 = 3,
  SHERRY_F32 = 4
} sherry_dtype;

/* Library version, e.g. "0.1.0". */
const char* sherry_version(void);

/* Human-readable name of a status code (never NULL). */
const char* sherry_status_str(sherry_status s);

/* Bytes of packed codes for an n x k matrix: n * (k / 128) * 20, i.e. exactly
 * 5 bits per 4 weights.  Returns 0 if n <= 0, k <= 0, k % 128 != 0 or the size
 * overflows. */
size_t sherry_packed_bytes(int64_t n, int64_t k);

/* Pack real weights into codes and per-row scales (Sherry Abstract: ternary
 * weights under 3:4 sparsity, four weights in five bits).  Rule per block:
 * the zero goes to the slot of smallest |w| (lowest slot on ties); each other
 * slot keeps the sign of w (negative iff w < 0, so -0.0 is +1).  Per row,
 * scale = (sum of kept |w|) / (3k/4), the least-squares scale for that
 * pattern, accumulated in fp64 (double-double) and rounded once, RNE, to s_dt.
 *   w      : n x k weights, element (r, c) at w[r * ldw + c]; w_dt F32|F16|BF16
 *   ldw    : row stride in elements, ldw >= k
 *   codes  : out, sherry_packed_bytes(n, k) bytes, 4-byte aligned
 *   scales : out, n elements of s_dt (F32|F16), aligned to its size
 * Non-finite weights are a caller error (codes and scales then unspecified).
 * Alignment: w aligned to 4 * element size and ldw a multiple of 4. */
sherry_status sherry_pack(const void* w, sherry_dtype w_dt, int64_t n, int64_t k, int64_t ldw,
                          uint32_t* codes, void* scales, sherry_dtype s_dt, hipStream_t stream);

/* Expand packed codes to the dense ternary matrix: t[r * ldt + c] = T[r, c]
 * as int8 (-1, 0, +1), the inverse of the layout above (every 5-bit pattern is
 * a valid block, so any code words decode).
 *   t : out, n x k int8, row stride ldt >= k, ldt % 16 == 0, 16-byte aligned */
sherry_status sherry_decode(const uint32_t* codes, int64_t n, int64_t k, int8_t* t, int64_t ldt,
                            hipStream_t stream);

/* Per-token int8 quantization of activations, the input of the int8
 * products (x_scale / x_scales arguments).  The Sherry paper quantizes the
 * weights only; the activations follow the symmetric absmax rule, in fp32:
 *   scales[t] = max_j |x[t, j]| / 127  (one IEEE division; 1.0 for an
 *               all-zero token)
 *   xq[t, j]  = clip(rint(x[t, j] / scales[t]), -127, 127)  (one IEEE
 *               division per element, then round half to even)
 *   x      : m x k values of x_dt (F32|F16|BF16), row stride ldx >= k
 *            elements, aligned to its element size; DEVICE
 *   xq     : out, m x k int8, row stride ldq >= k bytes; DEVICE
 *   scales : out, m fp32, 4-byte aligned; DEVICE
 * Non-finite inputs are a caller error (outputs then unspecified).
 * Errors: EINVAL null pointer or m, k <= 0; EDTYPE other x_dt; ESHAPE
 * ld < k or m above 2^31 - 1; EALIGN misaligned x or scales. */
sherry_status sherry_act_quant(const void* x, sherry_dtype x_dt, int64_t m, int64_t k, int64_t ldx, int8_t* xq,
                               int64_t ldq, float* scales, hipStream_t stream);

/* Batch-1 product of fp activations: x is quantized per token inside the
 * kernel (the rule of sherry_act_quant, bit for bit), then the int8 product
 * and epilogue of sherry_gemv with that scale -- one launch instead of
 * sherry_act_quant followed by sherry_gemv, for decode steps.
 *   x           : k values of x_dt (F32|F16|BF16), aligned to its size; DEVICE
 *   x_scale_out : nullable; receives the token's scale (4-byte aligned)
 *   k           : at most 8192 (the quantized x is held in LDS)
 * Everything else as sherry_gemv with int8 x.  Errors: as sherry_gemv, plus
 * ESHAPE for k > 8192 and EDTYPE for another x_dt. */
sherry_status sherry_gemv_quant(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n, int64_t k,
                                const void* x, sherry_dtype x_dt, float* x_scale_out, int32_t* acc, void* y,
                                sherry_dtype y_dt, hipStream_t stream);

/* Batch-1 product y = diag(s_w) * T * x (the decode-phase GEMV).  The Sherry
 * paper packs 3:4 ternary blocks into five bits for SIMD-friendly,
 * table-based inference (TL;DR; Abstract); this product reads those codes
 * and expands each through a small table.  One scale per row is the
 * library's reading of the scale (format block above).
 *   codes    : n x k packed codes (layout above), 4-byte aligned
 *   w_scales : n scales of s_dt (F32|F16)
 *   x        : k activations, x_dt I8 (int8) or BF16; 16-byte aligned
 *   x_scale  : I8 only: pointer to ONE device float s_x, or NULL for 1.0;
 *              must be NULL for BF16
 *   acc      : optional out, n int32 exact sums (I8 only, else must be NULL)
 *   y        : optional out, n values of y_dt: F32 or F16 for I8; F32 for BF16
 * At least one of acc / y must be non-NULL. */
sherry_status sherry_gemv(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n,
                          int64_t k, const void* x, sherry_dtype x_dt, const float* x_scale,
                          int32_t* acc, void* y, sherry_dtype y_dt, hipStream_t stream);

/* One problem of a grouped GEMV: same meaning as the sherry_gemv arguments. */
typedef struct {
  const uint32_t* codes;
  const void* w_scales;
  int64_t n;
  int64_t k;
  const void* x;
  const float* x_scale;
  int32_t* acc;
  void* y;
} sherry_gemv_problem;

/* Bytes of the launch plan for these problems (the plan holds one 64-byte
 * record per problem plus one 8-byte record per workgroup tile).  Returns 0
 * if probs is NULL, count <= 0 or a problem has an invalid shape. */
size_t sherry_gemv_plan_bytes(const sherry_gemv_problem* probs /* HOST */, int32_t count);

/* Build the launch plan of a grouped GEMV (many independent batch-1 products,
 * one kernel launch) into `plan`, a HOST buffer of at least
 * sherry_gemv_plan_bytes(probs, count) bytes, 8-byte aligned.  Every problem
 * is validated as in sherry_gemv, with the dtypes shared by all problems.
 * Pure host code: no HIP call.  The caller then copies the plan bytes
 * unchanged to a device buffer (8-byte aligned) and launches it. */
sherry_status sherry_gemv_plan(const sherry_gemv_problem* probs /* HOST */, int32_t count,
                               sherry_dtype s_dt, sherry_dtype x_dt, sherry_dtype y_dt, void* plan,
                               size_t plan_bytes);

/* The same plan for bf16 x, run on the matrix cores (v_mfma_f32_16x16x32_bf16)
 * instead of v_dot2_f32_bf16: each lane's 8 weights and 8 x values per
 * product sit on the diagonal of the 16 x 16 result, and the four lanes of a
 * column (one row) add there.  At batch 1 only 16 of a product's 256 results
 * are distinct, so its useful rate equals v_dot2's; it is an alternative
 * kernel, not the faster default (sherry_gemv_plan is).  Same arguments,
 * buffer size and launch as sherry_gemv_plan; x_dt must be BF16
 * (SHERRY_EDTYPE) and every k <= 8192 (SHERRY_ESHAPE).  fp32 outputs within
 * the bf16 tolerance of sherry_gemv; the per-row sum order is fixed, so
 * results repeat bit for bit.  (The Sherry paper's kernel is a CPU LUT
 * design, TL;DR and Abstract; this is a GPU counterpart.) */
sherry_status sherry_gemv_plan_mfma(const sherry_gemv_problem* probs /* HOST */, int32_t count,
                                    sherry_dtype s_dt, sherry_dtype x_dt, sherry_dtype y_dt, void* plan,
                                    size_t plan_bytes);

/* Launch a planned grouped GEMV (a plan from sherry_gemv_plan or
 * tern2_gemv_plan or tern3_gemv_plan): `plan_host` is the host plan, `plan_dev` a device copy of
 * the same bytes.  Returns SHERRY_EINVAL if the host plan header is malformed.
 * The device copy and every buffer named by the plan must stay alive until
 * the kernel completes. */
sherry_status sherry_gemv_grouped(const void* plan_host, const void* plan_dev, hipStream_t stream);

/* For callers that cannot allocate device memory or hold a device copy of the
 * plan (code under stream capture, tight serving loops, harnesses that forbid
 * hipMalloc): sherry_gemv_grouped without plan_dev.  The call copies the
 * plan's bytes (its header's byte count) from `plan_host` (a plan from
 * sherry_gemv_plan, sherry_gemv_plan_mfma, tern2_gemv_plan or tern3_gemv_plan,
 * 8-byte aligned) into plan memory that the library holds in a static device
 * array of 1 MiB on each GPU, with a copy ordered on `stream`, then launches
 * the same kernels on it; results are those of sherry_gemv_grouped bit for bit.
 * It calls no hipMalloc / hipFree and no allocating routine.
 *   - SHERRY_ESCRATCH if the plan is larger than 1 MiB (about 120,000 tiles;
 *     the 784 problems of 112 one-billion-parameter decoder layers take
 *     104 KB), SHERRY_EINVAL for a malformed header, as sherry_gemv_grouped.
 *   - The plan memory is shared by every call on one GPU and keeps the last
 *     call's plan.  Calls on one stream are ordered; calls on the same GPU
 *     that overlap (other streams, other threads without ordering) race on it
 *     and may run with each other's plans.
 *   - `plan_host` must stay unchanged until the copy has completed on
 *     `stream` (from pinned memory the copy is asynchronous).
 * The first call on a device looks up the device address of its plan memory. */
sherry_status sherry_gemv_grouped_noalloc(const void* plan_host, hipStream_t stream);

/* Matrix product for M tokens: Y[m, r] = s_x[m] * s_w[r] * sum_k X[m, k] T[r, k]
 * (sherry_gemv's product for every token row of X, on the same codes: Sherry
 * TL;DR and Abstract for the packing; the pages time single-token inference,
 * and the M-token form is this library's extension of it).
 * M <= 2 with k in {1024, 2048, 3072, 4096, 8192} runs the batch-1 walk with
 * both tokens' x in registers (each decoded code feeds one v_dot4 per token);
 * other small M (<= 16) decode codes in registers into int8 MFMA operands;
 * larger M decode tiles of codes once per tile and feed int8 MFMA.  All give
 * the same bits.
 *   X        : m x k int8, row-major with row stride ldx bytes (ldx >= k,
 *              ldx % 16 == 0, X 16-byte aligned); x_dt must be I8
 *   x_scales : m floats (per-token scale), or NULL for 1.0
 *   acc      : optional out, m x n int32, row stride n
 *   y        : optional out, m x n of y_dt (F16|F32), row stride ldy >= n
 * At least one of acc / y must be non-NULL. */
sherry_status sherry_gemm(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n,
                          int64_t k, const void* x, sherry_dtype x_dt, int64_t m, int64_t ldx,
                          const float* x_scales, int32_t* acc, void* y, sherry_dtype y_dt, int64_t ldy,
                          hipStream_t stream);

/* One product of a grouped GEMM (HOST struct; the pointers are device
 * pointers with the meaning, layout and alignment of sherry_gemm's arguments). */
typedef struct sherry_gemm_problem {
  const uint32_t* codes;
  const void* w_scales;
  int64_t n;
  int64_t k;
  const void* x;
  int64_t m;
  int64_t ldx;
  const float* x_scales; /* may be NULL */
  int32_t* acc;          /* may be NULL */
  void* y;               /* may be NULL (not both acc and y) */
  int64_t ldy;
} sherry_gemm_problem;

/* Bytes of the launch plan of a grouped GEMM (a 64-byte header, one 80-byte
 * record per problem, one 16-byte record per workgroup tile).  Returns 0 if
 * probs is NULL, count <= 0 or a problem has an invalid shape. */
size_t sherry_gemm_plan_bytes(const sherry_gemm_problem* probs /* HOST */, int32_t count);

/* Build the plan of a grouped GEMM: many independent products for M tokens
 * (each as in sherry_gemm, dtypes shared by all problems) in one kernel
 * launch, e.g. the seven matrices of a decoder layer during prefill.  The
 * kernel is chosen for the whole plan as in sherry_gemm (the two-token walk
 * only if every problem qualifies).  The tiles of the problems with the
 * longest rows come first.  Pure host code, no
 * HIP call; `plan` is a HOST buffer of at least sherry_gemm_plan_bytes bytes,
 * 8-byte aligned.  The caller copies the bytes unchanged to a device buffer
 * (8-byte aligned) and passes both to sherry_gemm_grouped. */
sherry_status sherry_gemm_plan(const sherry_gemm_problem* probs /* HOST */, int32_t count, sherry_dtype s_dt,
                               sherry_dtype x_dt, sherry_dtype y_dt, void* plan, size_t plan_bytes);

/* Launch a planned grouped GEMM (from sherry_gemm_plan or tern2_gemm_plan).
 * Returns SHERRY_EINVAL if the host plan header is malformed.  The device copy
 * and every buffer named by the plan must stay alive until the kernel
 * completes. */
sherry_status sherry_gemm_grouped(const void* plan_host, const void* plan_dev, hipStream_t stream);

/* Kernel of the int8 products for many tokens (sherry_gemm, tern2_gemm and
 * grouped plans that take the 256 x 128 tiles):
 *   SHERRY_PREFILL_TILED (default): waves expand the codes they multiply,
 *     straight from a staged copy in LDS into 16 x 16 x 64 matrix-core
 *     operands (4 waves of 64 rows x 128 tokens, two workgroups per CU);
 *   SHERRY_PREFILL_DECODE_ONCE: on 3:4 codes, each group of a tile's codes is
 *     decoded once per workgroup into an int8 weight tile in LDS that the
 *     waves multiply (Sherry Abstract: 3:4 blocks of four weights in five
 *     bits), for k a multiple of 1024 (other k and 2-bit codes keep the tiled
 *     kernel);
 *   SHERRY_PREFILL_TILED32: the tiled kernel on 32 x 32 x 32 matrix-core
 *     operands, same waves and tiles.
 * All give identical results.  The setting is process-wide and applies to
 * launches issued after the call.  Errors: SHERRY_EINVAL for another kind. */
typedef enum sherry_prefill_kernel {
  SHERRY_PREFILL_TILED = 0,
  SHERRY_PREFILL_DECODE_ONCE = 1,
  SHERRY_PREFILL_TILED32 = 2
} sherry_prefill_kernel;
sherry_status sherry_set_prefill_kernel(sherry_prefill_kernel kind);

/* ---- 2-bit dense-ternary comparator (Sherry Abstract and Figure 2: the
 * 2-bit aligned packing that keeps alignment by wasting bits) ----
 * Layout (a reading; the pages give none): 16 weights per little-endian
 * uint32 word, field value 00 = 0, 01 = +1, 11 = -1 (10 never written);
 * weight 4q + p of a word (q, p in 0..3) sits at bits [8p + 2q, 8p + 2q + 2),
 * so one shift and mask put four consecutive weights in the low bits of the
 * four bytes.  Row-major, k / 16 words per row, k % 128 == 0.  Scales and
 * epilogues are exactly those of the Sherry entry points. */
size_t tern2_packed_bytes(int64_t n, int64_t k); /* n * k / 4, 0 if invalid */

/* Pack real weights into 2-bit words with the decisions and scales of
 * sherry_pack: per block of four the zero at the smallest |w|, the other
 * three by sign, one least-squares scale per row.  The two formats then hold
 * the same ternary matrix (a reading: the pages compare packings of ternary
 * weights, Abstract and Figure 2, and give no separate quantizer for the
 * 2-bit one).  Arguments, alignment and errors as in sherry_pack; codes
 * receives tern2_packed_bytes(n, k) bytes (4-byte aligned). */
sherry_status tern2_pack(const void* w, sherry_dtype w_dt, int64_t n, int64_t k, int64_t ldw, uint32_t* codes,
                         void* scales, sherry_dtype s_dt, hipStream_t stream);

/* Encode a dense ternary int8 matrix t (values -1, 0, +1; row stride ldt
 * elements, ldt >= k, ldt % 16 == 0, t 16-byte aligned) into 2-bit words.
 * Values outside {-1, 0, +1} are a caller error (output unspecified). */
sherry_status tern2_encode(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint32_t* codes,
                           hipStream_t stream);

/* Same contract as sherry_gemv with I8 x, on 2-bit codes. */
sherry_status tern2_gemv(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n,
                         int64_t k, const void* x, sherry_dtype x_dt, const float* x_scale,
                         int32_t* acc, void* y, sherry_dtype y_dt, hipStream_t stream);

/* Same contract as sherry_gemv_plan, on 2-bit codes (x_dt must be I8); the
 * plan is launched with sherry_gemv_grouped. */
sherry_status tern2_gemv_plan(const sherry_gemv_problem* probs /* HOST */, int32_t count,
                              sherry_dtype s_dt, sherry_dtype x_dt, sherry_dtype y_dt, void* plan,
                              size_t plan_bytes);

/* Same contract as sherry_gemm_plan, on 2-bit codes. */
sherry_status tern2_gemm_plan(const sherry_gemm_problem* probs /* HOST */, int32_t count, sherry_dtype s_dt,
                              sherry_dtype x_dt, sherry_dtype y_dt, void* plan, size_t plan_bytes);

/* Same contract as sherry_gemm, on 2-bit codes. */
sherry_status tern2_gemm(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n,
                         int64_t k, const void* x, sherry_dtype x_dt, int64_t m, int64_t ldx,
                         const float* x_scales, int32_t* acc, void* y, sherry_dtype y_dt, int64_t ldy,
                         hipStream_t stream);

/* ---- 1.67-bit comparator (same paper, Figure 2 caption, middle: three
 * ternary weights packed into five bits, in patterns of three; Abstract: the
 * irregular 1.67-bit packing) ----
 * Layout (a reading; the pages give none): a code holds three consecutive
 * weights of a row, c = (t0 + 1) + 3 (t1 + 1) + 9 (t2 + 1) (0..26); 32 codes
 * (96 weights) form a group of 5 words in the LSB-first stream of the Sherry
 * layout above, rows are zero-padded to G3 = ceil(k / 96) groups and stored
 * in its two-part row layout (words 0-3 of group g at 4g, word 4 at
 * 4 G3 + g).  k % 128 == 0.  Scales and epilogues as the Sherry entry points. */
size_t tern3_packed_bytes(int64_t n, int64_t k); /* n * ceil(k / 96) * 20, 0 if invalid */

/* Encode a dense int8 matrix t into 1.67-bit codes (values taken by sign:
 * negative -1, zero 0, positive +1).  Same argument rules as tern2_encode. */
sherry_status tern3_encode(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint32_t* codes,
                           hipStream_t stream);

/* Same contract as sherry_gemv with I8 x, on 1.67-bit codes. */
sherry_status tern3_gemv(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n,
                         int64_t k, const void* x, sherry_dtype x_dt, const float* x_scale,
                         int32_t* acc, void* y, sherry_dtype y_dt, hipStream_t stream);

/* Plan size and plan for a grouped 1.67-bit GEMV (x_dt I8), launched with
 * sherry_gemv_grouped; same contract as sherry_gemv_plan_bytes /
 * sherry_gemv_plan (tile rows follow this format's row length). */
size_t tern3_gemv_plan_bytes(const sherry_gemv_problem* probs /* HOST */, int32_t count);
sherry_status tern3_gemv_plan(const sherry_gemv_problem* probs /* HOST */, int32_t count,
                              sherry_dtype s_dt, sherry_dtype x_dt, sherry_dtype y_dt, void* plan,
                              size_t plan_bytes);

#ifdef __cplusplus
}
#endif

#endif /* SHERRY_H */
