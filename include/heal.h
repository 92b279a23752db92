/*
 * heal.h -- C ABI of the HEAL hot path on AMD Instinct MI355X (gfx950).
 *
 * HEAL gets near-FP32 results out of 16-bit matrix units and keeps the attention inputs at 16 bits:
 *   - an FP32 operand is split into a 16-bit leading part and a 16-bit remainder, and the 16-bit products are
 *     summed into one FP32 accumulator (the "algebraic error compensation" GEMM);
 *   - Q, K and V are stored as INT16, and each INT16 value is unpacked into two exactly representable
 *     FP16 halves ("Dual-FP16") for the QK^T and PV products, with FP32 softmax.
 *
 * Sources (cited by page and section):
 *   [TS]  gist.science explainer "Demystifying Numerical Instability in LLM Inference: Achieving
 *         Reproducible Inference for Mission-Critical Tasks with HEAL", section "Technical Summary";
 *         [TS 2A] "Mitigating Attention Truncation via INT16 Quantization" (Solution, Mechanism, Benefit);
 *         [TS 2B] "Mitigating GEMM Truncation via Algebraic Error Compensation" (Solution, Mechanism,
 *         Overflow Handling).
 *   [ABS] the authors' abstract, arXiv 2606.21023 v2.
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library never allocates, frees or
 *     synchronises; work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and the call
 *     returns at once.
 *   - Arguments are validated before anything is launched; on any error nothing is enqueued and the
 *     status says why.  A launch failure reported by the runtime gives HEAL_ERR_LAUNCH.
 *   - Matrices are row-major.  Leading dimensions are in ELEMENTS.  Base pointers must be 16-byte aligned
 *     and leading dimensions must be multiples of 8 elements (16 bytes for 16-bit data); otherwise
 *     HEAL_ERR_ALIGN.  There is no slow fallback path.
 *   - NaN or infinite inputs are outside the contract: they are not detected and the result is
 *     unspecified.  Zero-sized problems are valid and enqueue nothing (or only the zero fill they imply).
 *   - Results are bitwise deterministic: no floating-point atomics, fixed reduction orders.
 *   - Calls are stateless and may be made from several host threads at once.
 */
#ifndef HEAL_H
#define HEAL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HEAL_ABI_VERSION 7

#if defined(__GNUC__) || defined(__clang__)
#define HEAL_API __attribute__((visibility("default")))
#else
#define HEAL_API
#endif

typedef enum {
  HEAL_OK = 0,
  HEAL_ERR_NULL = 1,        /* a required pointer is NULL */
  HEAL_ERR_SHAPE = 2,       /* a size is negative or inconsistent */
  HEAL_ERR_STRIDE = 3,      /* a leading dimension / stride is smaller than the row it must hold */
  HEAL_ERR_ALIGN = 4,       /* pointer not 16-byte aligned, or leading dimension not a multiple of 8 */
  HEAL_ERR_DTYPE = 5,       /* a dtype code that the call does not accept */
  HEAL_ERR_UNSUPPORTED = 6, /* a valid request this library does not implement (e.g. head_dim != 128), or
                               one whose launch grid would exceed HIP's 2^32 work-items per dimension */
  HEAL_ERR_LAUNCH = 7,      /* the HIP runtime refused a launch */
  HEAL_ERR_WORKSPACE = 8    /* workspace missing or smaller than heal_attn_workspace_bytes() */
} heal_status;

typedef enum { HEAL_F32 = 0, HEAL_BF16 = 1, HEAL_F16 = 2, HEAL_I16 = 3 } heal_dtype;

/*
 * Readings of the Dual-FP16 pair of an INT16 value q ([TS 2A Mechanism] writes the pair as
 * X_hi + X_lo / 2^10 without fixing how the bits are divided).  Each is exact: q is recovered from the
 * two FP16 values without rounding.
 *   HEAL_DUAL_BYTE     hi = q >> 8 (floor), lo = q & 0xFF;           q = 256 hi + lo.  The default.
 *   HEAL_DUAL_SHIFT10  hi = q >> 10 (floor), lo = q & 0x3FF;         q = 1024 hi + lo.
 *   HEAL_DUAL_FLOAT    hi = fp16_rn(q), lo = 2^10 (q - hi);           q = hi + lo / 2^10 (|lo| <= 2^14).
 */
typedef enum { HEAL_DUAL_BYTE = 0, HEAL_DUAL_SHIFT10 = 1, HEAL_DUAL_FLOAT = 2 } heal_dual_split;

/* Human-readable name of a status code (static storage; never NULL). */
HEAL_API const char* heal_status_str(int status);
/* HEAL_ABI_VERSION of the loaded library. */
HEAL_API int heal_abi_version(void);

/*
 * heal_split -- the operand decomposition of [TS 2B Mechanism] (FP32/bf16 in) and the Dual-FP16 unpack
 * of [TS 2A Mechanism] (INT16 in).
 *
 * x_type = HEAL_F32 or HEAL_BF16 (x is [rows, cols], leading dimension ld_x):
 *   per row r:  e_r = 14 - ilogb(max_c |x_rc|)  (0 for an all-zero row; 0 for every row if exps == NULL)
 *               x'  = fl32(x * 2^e_r)                      (exact unless x' falls below the fp32 normals)
 *               hi  = round16(x'),  lo = round16(x' - hi)  (x' - hi is exact in fp32)
 *   round16 is IEEE round-to-nearest-even into part_type (HEAL_F16, the graded mode, or HEAL_BF16, the
 *   contrast mode), gradual underflow, overflow to infinity.  The prescale is the exact power-of-two form
 *   of the "targeted rescaling" of [TS 2B Overflow Handling]: each row's maximum lands in [2^14, 2^15), so
 *   no FP16 part overflows and the residual keeps 11 more bits.  exps[r] receives e_r (int32) when
 *   exps != NULL.  lo == NULL drops the residual (used for weights that are exact in 16 bits).
 * x_type = HEAL_I16 (x is int16 [rows, cols]): the byte split hi = x >> 8 (floor), lo = x & 0xFF, written
 *   as FP16 values with x = 256*hi + lo exactly.  part_type must be HEAL_F16, lo must be non-NULL and
 *   exps must be NULL.
 * (heal_unpack_i16 below offers the other readings of the pair.)
 * hi and lo are [rows, cols] 16-bit, leading dimension ld_part.  Rows are independent; hi/lo must not
 * overlap x.  Alignment: x needs only its element alignment and any ld_x >= cols (rows that start on a
 * 16-byte boundary are read with 16-byte loads, others element by element); hi and lo must be 16-byte
 * aligned with ld_part a multiple of 8.
 * Errors: HEAL_ERR_NULL (x or hi NULL with rows*cols > 0; lo NULL for I16), HEAL_ERR_SHAPE (negative
 * sizes), HEAL_ERR_STRIDE (ld < cols), HEAL_ERR_ALIGN, HEAL_ERR_DTYPE (bad x_type/part_type pairing).
 */
HEAL_API heal_status heal_split(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ld_x, int part_type,
                       void* hi, void* lo, int64_t ld_part, int32_t* exps, void* stream);

/*
 * heal_unpack_i16 -- the Dual-FP16 unpack of [TS 2A Mechanism] under any of the three readings of
 * heal_dual_split: x is int16 [rows, cols] (leading dimension ld_x); hi and lo receive the FP16 bit
 * patterns of the reading's two values, [rows, cols] with leading dimension ld_part.  HEAL_DUAL_BYTE gives
 * the same output as heal_split with x_type HEAL_I16.  Alignment and errors as heal_split (x_type HEAL_I16),
 * plus HEAL_ERR_DTYPE for a dual_split code outside heal_dual_split.
 */
HEAL_API heal_status heal_unpack_i16(const int16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int dual_split,
                            void* hi, void* lo, int64_t ld_part, void* stream);

/*
 * Calibrated outlier channels -- the "targeted rescaling of rare outlier channels" of [TS 2B Overflow
 * Handling] as an exact power-of-two scale per input channel (column of the activations X [M, K], column
 * of the weights W [N, K]): X' = X diag(2^c), W' = W diag(2^-c), so X' W'^T = X W^T exactly while the
 * large channels no longer set the row prescale of the ordinary values beside them.
 *
 * heal_channel_exponents: from a calibration batch x [rows, cols] FP32 (leading dimension ld_x), per column
 *   m_c = max_r |x[r, c]|  and  col_exps[c] = threshold_log2 - ilogb(m_c) where ilogb(m_c) > threshold_log2,
 *   else 0 (all-zero columns: 0).  So every column's maximum ends up below 2^(threshold_log2 + 1).
 *   col_exps is int32 [cols], 16-byte aligned.  Errors: HEAL_ERR_NULL, HEAL_ERR_SHAPE (negative sizes,
 *   threshold_log2 outside [-126, 127]), HEAL_ERR_STRIDE (ld_x < cols), HEAL_ERR_ALIGN (x not 4-byte aligned,
 *   col_exps not 16-byte aligned).
 * heal_split_scaled: heal_split (x_type HEAL_F32 or HEAL_BF16) applied to x'[r, c] = fl32(x[r, c] *
 *   2^(col_sign * col_exps[c])) (exact unless x' leaves the fp32 normal range); col_sign = +1 for the
 *   activations, -1 for the weights.  Errors: as heal_split, HEAL_ERR_NULL (col_exps NULL), HEAL_ERR_SHAPE
 *   (col_sign not +-1), HEAL_ERR_DTYPE (x_type HEAL_I16), HEAL_ERR_ALIGN (col_exps not 16-byte aligned).
 */
HEAL_API heal_status heal_channel_exponents(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   int32_t threshold_log2, int32_t* col_exps, void* stream);
HEAL_API heal_status heal_split_scaled(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ld_x,
                              int part_type, void* hi, void* lo, int64_t ld_part, int32_t* exps,
                              const int32_t* col_exps, int32_t col_sign, void* stream);

/*
 * heal_gemm_comp -- the error-compensated GEMM of [TS 2B Solution/Mechanism]:
 *   C[i, j] = 2^-(ea_i + eb_j) * sum_k ( ah*bh + [b_lo] ah*bl + [a_lo] al*bh )[i, k, j]
 * with A [M, K] given as parts a_hi / a_lo (leading dimension lda) and B given TRANSPOSED as parts
 * b_hi / b_lo of B^T [N, K] (leading dimension ldb): both operands are K-contiguous.  Parts are what
 * heal_split writes (16-bit, part_type HEAL_F16 or HEAL_BF16).  A NULL a_lo / b_lo drops the products
 * that need it: P = 1 + (a_lo != NULL) + (b_lo != NULL) products of 16-bit inputs, all accumulated in
 * ONE FP32 accumulator per output; lo*lo is never formed.  a_exp / b_exp are the int32 row exponents of
 * heal_split (NULL means 0).  C is FP32 [M, N] (leading dimension ldc, a multiple of 4 elements): the
 * accumulator scaled by the exact power of two is the only rounding at the kernel boundary.
 * Each part buffer holds its rows x ld elements (the padding columns K .. ld-1 may hold anything; they are
 * read as whole 16-byte chunks and never contribute).  K = 0 writes zeros.
 * Errors: HEAL_ERR_NULL (a_hi, b_hi or c NULL with M*N > 0), HEAL_ERR_SHAPE (a negative size, or M, N or
 * K above 2^31), HEAL_ERR_STRIDE (lda, ldb < K or ldc < N), HEAL_ERR_ALIGN, HEAL_ERR_DTYPE.
 */
HEAL_API heal_status heal_gemm_comp(int64_t M, int64_t N, int64_t K, const void* a_hi, const void* a_lo,
                           const int32_t* a_exp, int64_t lda, const void* b_hi, const void* b_lo,
                           const int32_t* b_exp, int64_t ldb, int part_type, float* c, int64_t ldc,
                           void* stream);

/*
 * Split in the GEMM's prologue ([TS 2B Mechanism]: A's primary 16-bit value and residual are formed where
 * they are multiplied, so the 16-bit parts of A never travel through memory).  heal_row_exponents followed
 * by heal_gemm_comp_f32a computes what heal_split (FP32 x, HEAL_F16 parts, prescale, residual) followed by
 * heal_gemm_comp computes, bit for bit, reading A once in each call instead of writing and re-reading its
 * parts.
 *
 * heal_row_exponents: exps[r] = 14 - ilogb(max_c |x[r, c]|) (0 for an all-zero or empty row): the
 *   exponents heal_split writes.  x FP32 [rows, cols] with leading dimension ld_x (4-byte alignment only);
 *   exps int32 [rows], 4-byte aligned.
 *   Errors: HEAL_ERR_NULL (exps NULL, or x NULL with cols > 0), HEAL_ERR_SHAPE, HEAL_ERR_STRIDE
 *   (ld_x < cols), HEAL_ERR_ALIGN.
 * heal_gemm_comp_f32a: heal_gemm_comp with A given as FP32 a [M, K] (leading dimension lda, in floats) and
 *   its row exponents a_exp: each A value is split as heal_split splits it, xs = fl32(a * 2^e),
 *   hi = fp16_rn(xs), lo = fp16_rn(xs - hi), inside the kernel.  B as in heal_gemm_comp with FP16 parts
 *   (b_lo NULL: P = 2 products, else 3).  With the exponents of heal_row_exponents every |xs| < 2^15;
 *   other exponents are accepted, with the parts heal_split would form from them.  a must be 16-byte
 *   aligned and lda a multiple of 4; a row needs to hold only its K values (the last partial step of K is
 *   read element by element).  For M <= 16, a_exp may be NULL: the kernel then derives the exponents of
 *   heal_row_exponents itself (the same values, so the same C bits), saving that launch at the cost of one
 *   more read of A per workgroup from L2 (cheap for a few rows; at 16 rows and K = 14336 it is 0.9 MB).
 *   Errors: HEAL_ERR_NULL (c NULL with M*N > 0; a_exp NULL with M > 16 and M*N > 0; a or b_hi NULL with
 *   M*N*K > 0), HEAL_ERR_SHAPE,
 *   HEAL_ERR_STRIDE (lda, ldb < K or ldc < N), HEAL_ERR_ALIGN.
 */
HEAL_API heal_status heal_row_exponents(const float* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t* exps,
                               void* stream);
HEAL_API heal_status heal_gemm_comp_f32a(int64_t M, int64_t N, int64_t K, const float* a, int64_t lda,
                                const int32_t* a_exp, const void* b_hi, const void* b_lo, const int32_t* b_exp,
                                int64_t ldb, float* c, int64_t ldc, void* stream);

/*
 * heal_gemm_comp_quant_i16 -- the compensated GEMM of heal_gemm_comp with the INT16 quantisation of
 * heal_qkv_quant_i16 applied in its epilogue ([TS 2A Solution]: the attention inputs are stored as INT16), so
 * a Q/K/V projection writes its INT16 codes and scales straight into a cache without an FP32 round trip.
 * C (never stored) is split into heads of 128 consecutive columns; for each row i and head h:
 *   s[i, h] = fl32(max_c |C[i, c]| / 32767),  q[i, c] = clamp(rint(fl32(C[i, c] / s[i, h])), -32767, 32767)
 *   (q = 0 where s = 0), with C[i, c] the value heal_gemm_comp stores.
 * For M > 64 the codes and scales equal heal_gemm_comp followed by heal_qkv_quant_i16 (tokens = M,
 * heads = N / 128) bit for bit.  For M <= 64 heal_gemm_comp uses a skinny kernel whose summation order
 * differs: both are within the FP32 accumulation bound of the exact sum, and a code may differ by one step.
 * q is int16 [M, N] (leading dimension ldq, a multiple of 8), scale fp32 [M, N / 128] (leading dimension
 * ld_s >= N / 128); q may point into a larger cache.  Only part_type HEAL_F16.
 * Errors: as heal_gemm_comp (q and scale take the place of c), HEAL_ERR_SHAPE (N not a multiple of 128),
 * HEAL_ERR_STRIDE (ldq < N, ld_s < N / 128), HEAL_ERR_DTYPE (part_type other than HEAL_F16).
 */
HEAL_API heal_status heal_gemm_comp_quant_i16(int64_t M, int64_t N, int64_t K, const void* a_hi, const void* a_lo,
                                     const int32_t* a_exp, int64_t lda, const void* b_hi, const void* b_lo,
                                     const int32_t* b_exp, int64_t ldb, int part_type, int16_t* q, int64_t ldq,
                                     float* scale, int64_t ld_s, void* stream);

/*
 * heal_gemm_comp_variant -- the name of the kernel instantiation heal_gemm_comp launches for an M x N x K
 * problem with `products` (1..3) 16-bit products, e.g. "gemm_comp_kernel 128x256 P2" (static storage;
 * "none" for an empty problem).  products = 2 names the case where A has a low part and B has none (an
 * activation times a 16-bit weight).  For profiling: it lets a caller attribute a profiler's per-kernel times
 * to problem shapes.  Host function, no device work; it reads the current device's compute-unit count (the
 * streamed-B kernel for at most 16 rows is chosen by columns per CU) and assumes 256 when there is no device.
 */
HEAL_API const char* heal_gemm_comp_variant(int64_t M, int64_t N, int64_t K, int products);

/*
 * heal_gemm_comp_splitk -- the error-compensated GEMM of [TS 2B Solution/Mechanism], the operation and
 * arguments of heal_gemm_comp, for problems whose own launch would leave compute units idle: M x N of at
 * most 128 tiles of 128 x 128 (M > 64), or 17..64 rows where every workgroup would re-read more of A than
 * twice its share of B.  There K is cut into S slices (2..16, each a multiple of
 * 64 but the last); each slice's products go into one FP32 accumulator as in heal_gemm_comp, the S FP32
 * partials of an output are added in slice order (0, 1, ..., S-1), and the exponents are applied once, so the
 * result keeps the FP32-accumulation error bound of the exact sum and is the same bits on every run.  It
 * differs from heal_gemm_comp's bits only by the grouping of those additions.  When no split helps (S = 1)
 * the call is heal_gemm_comp itself, bit for bit, and needs no workspace.
 * workspace: device memory of at least heal_gemm_comp_workspace_bytes(M, N, K, P) bytes, 256-byte aligned,
 * owned by the caller, with P = 1 + (a_lo != NULL) + (b_lo != NULL); its contents on entry do not matter and
 * are scratch afterwards.  Calls that share a workspace must not overlap.
 * Errors: as heal_gemm_comp, and HEAL_ERR_WORKSPACE (workspace needed but NULL, too small or misaligned).
 */
HEAL_API heal_status heal_gemm_comp_splitk(int64_t M, int64_t N, int64_t K, const void* a_hi, const void* a_lo,
                                  const int32_t* a_exp, int64_t lda, const void* b_hi, const void* b_lo,
                                  const int32_t* b_exp, int64_t ldb, int part_type, float* c, int64_t ldc,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * heal_gemm_comp_workspace_bytes -- the workspace heal_gemm_comp_splitk needs for an M x N x K problem with
 * `products` (1..3) 16-bit products (products = 2: A has a low part, B none, as in heal_gemm_comp_variant);
 * 0 when it does not split.  heal_gemm_comp_splitk_slices -- its slice count S (1 = no split).  Pure host
 * functions; sizes out of range give 0 bytes and 1 slice.
 */
HEAL_API size_t heal_gemm_comp_workspace_bytes(int64_t M, int64_t N, int64_t K, int products);
HEAL_API int heal_gemm_comp_splitk_slices(int64_t M, int64_t N, int64_t K, int products);

/*
 * heal_gemm_comp_f32a_splitk -- heal_gemm_comp_f32a (A given as FP32 and split in the kernel, [TS 2B Mechanism])
 * with K cut into slices as heal_gemm_comp_splitk cuts it, for 8..16 rows with K >= 8192 (a decode batch
 * through a down projection), where each workgroup of the unsplit launch would re-read and re-split all of A
 * for its 16 columns.  The slices, their kernel and the fixed-order reduction are those of
 * heal_gemm_comp_splitk, so the result equals heal_split (FP32 A, HEAL_F16 parts, prescale, residual)
 * followed by heal_gemm_comp_splitk bit for bit.  It splits only with row exponents given (a_exp non-NULL,
 * e.g. from heal_row_exponents): with a_exp NULL, or where no split helps, the call is heal_gemm_comp_f32a
 * itself, bit for bit, and needs no workspace.  Arguments as heal_gemm_comp_f32a.
 * workspace: device memory of at least heal_gemm_comp_f32a_workspace_bytes(M, N, K, P) bytes (P = 2 with
 * b_lo NULL, else 3), 256-byte aligned, owned by the caller, scratch on return.  Calls that share a workspace
 * must not overlap.
 * Errors: as heal_gemm_comp_f32a, and HEAL_ERR_WORKSPACE (workspace needed but NULL, too small or misaligned).
 * heal_gemm_comp_f32a_workspace_bytes / heal_gemm_comp_f32a_splitk_slices: the workspace (0 when it does not
 * split) and slice count (1 = no split) of a call with a_exp given; pure host functions; P outside 2..3 or
 * sizes out of range give 0 bytes and 1 slice.
 */
HEAL_API heal_status heal_gemm_comp_f32a_splitk(int64_t M, int64_t N, int64_t K, const float* a, int64_t lda,
                                       const int32_t* a_exp, const void* b_hi, const void* b_lo,
                                       const int32_t* b_exp, int64_t ldb, float* c, int64_t ldc,
                                       void* workspace, size_t workspace_bytes, void* stream);
HEAL_API size_t heal_gemm_comp_f32a_workspace_bytes(int64_t M, int64_t N, int64_t K, int products);
HEAL_API int heal_gemm_comp_f32a_splitk_slices(int64_t M, int64_t N, int64_t K, int products);

/*
 * heal_qkv_quant_i16 -- INT16 quantisation of Q, K or V per (token, head) ([TS 2A Solution]; [ABS]):
 *   a = max_d |x|;  s = fl32(a / 32767);  q = clamp(rint(fl32(x / s)), -32767, 32767)   (IEEE division,
 *   ties-to-even rint, symmetric, no zero point);  s = 0 (an all-zero row, or one so small that s
 *   underflows) gives q = 0.
 * x is fp32 [tokens, heads, head_dim] with token stride ld_x (elements; heads packed at head_dim).
 * q is int16 with token stride ld_q and heads packed; scale is fp32 with token stride ld_s and heads
 * packed.  The strides let a caller quantise new tokens straight into a larger KV cache (fold the batch
 * into `tokens` with the cache's per-sequence stride).  head_dim must be a multiple of 4 and at most 1024.
 * Errors: HEAL_ERR_NULL, HEAL_ERR_SHAPE, HEAL_ERR_STRIDE (ld_x or ld_q < heads*head_dim, ld_s < heads),
 * HEAL_ERR_ALIGN (x 16-byte and q 8-byte aligned; ld_x, ld_q multiples of 4; scale 4-byte aligned),
 * HEAL_ERR_UNSUPPORTED (head_dim).
 */
HEAL_API heal_status heal_qkv_quant_i16(const float* x, int64_t tokens, int64_t heads, int64_t head_dim,
                               int64_t ld_x, int16_t* q, int64_t ld_q, float* scale, int64_t ld_s,
                               void* stream);

/*
 * Arguments of heal_attn_dual_fp16.  Strides are in elements; the last (head_dim) axis is contiguous.
 *   q        int16 [batch, q_len, n_q_heads, head_dim]     strides q_strides  = {batch, token, head}
 *   k, v     int16 [batch, kv_len, n_kv_heads, head_dim]   strides kv_strides (shared by k and v)
 *   q_scale  fp32  [batch, q_len, n_q_heads]               strides qs_strides
 *   k_scale, v_scale fp32 [batch, kv_len, n_kv_heads]      strides kvs_strides
 *   out      fp32  [batch, q_len, n_q_heads, head_dim]     strides o_strides
 * causal != 0 masks key j for query i unless j <= i + (kv_len - q_len) (bottom-right alignment, so a
 * decode step with q_len = 1 sees the whole cache).  softmax_scale = 0 means 1/sqrt(head_dim).
 * Query head h reads key/value head h / (n_q_heads / n_kv_heads) (grouped-query attention).
 * workspace: device scratch of at least heal_attn_workspace_bytes(args) bytes (may be NULL when that is
 * 0), 256-byte aligned, owned by the caller, not shared by calls that may run concurrently.
 */
typedef struct {
  int64_t batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim;
  const int16_t* q;
  const int16_t* k;
  const int16_t* v;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  int64_t q_strides[3];
  int64_t kv_strides[3];
  int64_t qs_strides[3];
  int64_t kvs_strides[3];
  int64_t o_strides[3];
  int32_t causal;
  float softmax_scale;
  int32_t dual_split; /* heal_dual_split; 0 (a zero-initialised struct) is the byte split */
  float* out;
  void* workspace;
  size_t workspace_bytes;
} heal_attn_args;

/* Workspace bytes heal_attn_dual_fp16 needs for these arguments (0 when none). */
HEAL_API size_t heal_attn_workspace_bytes(const heal_attn_args* args);

/*
 * heal_attn_dual_fp16 -- attention over INT16 Q/K/V with Dual-FP16 products ([TS 2A Mechanism, Benefit]):
 *   x^ = s * q  (per-(token, head) scale);  S = softmax_scale * Q^ K^T;  P = softmax(S) over the visible
 *   keys (FP32, running maximum and sum);  O = P V^.
 * Each INT16 operand is unpacked in registers into FP16 halves (hi = q >> 8, lo = q & 0xFF), QK^T is the
 * sum of the four 16-bit products of the halves, and PV is formed from P * s_v (renormalised by an exact
 * power of two and split into FP16 hi + lo) against the halves of V: 4 + 4 16-bit matrix products,
 * FP32 accumulation, FP32 output.  args->dual_split selects the reading of the pair: HEAL_DUAL_SHIFT10
 * (also 4 + 4 products, q.k still exact) or HEAL_DUAL_FLOAT (3 + 3 products: the lo.lo terms are dropped,
 * and the FP32 sum of the hi.hi products rounds, about 2^-24 of sum |hi hi| per logit).  q_len = 1 takes the decode path (split over the keys, partial results
 * merged in a fixed order); q_len > 1 the prefill path.
 * Errors: HEAL_ERR_NULL, HEAL_ERR_SHAPE (sizes, n_q_heads % n_kv_heads != 0), HEAL_ERR_STRIDE,
 * HEAL_ERR_ALIGN (q/k/v/out 16-byte aligned, strides multiples of 8), HEAL_ERR_UNSUPPORTED
 * (head_dim != 128), HEAL_ERR_WORKSPACE, HEAL_ERR_DTYPE (dual_split outside heal_dual_split).
 */
HEAL_API heal_status heal_attn_dual_fp16(const heal_attn_args* args, void* stream);

/*
 * heal_attn_dual_fp16_noalloc -- heal_attn_dual_fp16 for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same operation, the
 * same kernels and the same output bits, with the decode partials kept in a scratch array the library
 * holds in device memory (one per GPU it runs on, HEAL_ATTN_NOALLOC_MAX_WORKSPACE bytes, kept until the
 * process ends) instead of a caller workspace.  args->workspace and args->workspace_bytes are ignored.
 * The call allocates nothing: no hipMalloc, hipFree or allocating library routine.  Its first call on a
 * device looks up that device's scratch address once.  Every call on one GPU shares that GPU's scratch, so
 * calls that may overlap on one GPU (several streams, several host threads) race and must be ordered by
 * the caller.  The scratch needs no clearing: the decode kernels write every partial they later read.
 * Errors: as heal_attn_dual_fp16; HEAL_ERR_WORKSPACE when heal_attn_workspace_bytes(args) exceeds
 * HEAL_ATTN_NOALLOC_MAX_WORKSPACE (checked on the host before any device call); HEAL_ERR_LAUNCH when the
 * runtime cannot give the scratch address.
 */
#define HEAL_ATTN_NOALLOC_MAX_WORKSPACE ((size_t)8 << 20)
HEAL_API heal_status heal_attn_dual_fp16_noalloc(const heal_attn_args* args, void* stream);

/*
 * Paged, variable-length INT16 KV cache for decode (one query token per sequence): the attention of
 * heal_attn_dual_fp16 with q_len = 1, the same Dual-FP16 arithmetic ([TS 2A Mechanism]) and the same
 * 16-bit cache footprint ([TS 2A Benefit]), with the keys of each sequence held in fixed-size pages of a
 * shared pool instead of one contiguous run.
 *
 * Layout (all device memory, owned by the caller):
 *   q        int16 [batch, n_q_heads, 128]            element (b, h, d) at q[b*q_strides[0] + h*q_strides[1] + d]
 *   q_scale  fp32  [batch, n_q_heads]                 at q_scale[b*qs_strides[0] + h*qs_strides[1]]
 *   k_pages, v_pages  int16 [num_pages, page_size, n_kv_heads, 128]
 *                                                     (p, t, h, d) at [p*kv_strides[0] + t*kv_strides[1] + h*kv_strides[2] + d]
 *   k_scale, v_scale  fp32 [num_pages, page_size, n_kv_heads]
 *                                                     (p, t, h) at [p*kvs_strides[0] + t*kvs_strides[1] + h*kvs_strides[2]]
 *   block_table int32 [batch, max_pages_per_seq]: key j of sequence b lives in page
 *            block_table[b*bt_stride + j / page_size], slot j % page_size
 *   seq_lens int32 [batch]: keys of each sequence (0 gives an all-zero output row)
 *   out      fp32  [batch, n_q_heads, 128]            at out[b*o_strides[0] + h*o_strides[1] + d]
 * Query head h reads kv head h / (n_q_heads / n_kv_heads).  Every key of a sequence is visible.
 * page_size must be a power of two >= 32 (HEAL_ERR_UNSUPPORTED otherwise); head_dim must be 128.
 * max_kv_len bounds seq_lens and sizes the launch (no device read on the host): a length outside
 * [0, max_kv_len] is clamped into it, and a page id outside [0, num_pages) is clamped into it, so no
 * access leaves the pool whatever the table holds; the result for such entries is unspecified.
 * The workspace (heal_attn_paged_workspace_bytes) holds the partial results of the key splits.
 * Errors: HEAL_ERR_NULL, HEAL_ERR_SHAPE (sizes, n_q_heads % n_kv_heads != 0, max_pages_per_seq *
 * page_size < max_kv_len), HEAL_ERR_STRIDE, HEAL_ERR_ALIGN (q/pages/out 16-byte aligned, q/kv/o strides
 * multiples of 8), HEAL_ERR_UNSUPPORTED (head_dim, page_size, n_q_heads / n_kv_heads > 16),
 * HEAL_ERR_WORKSPACE, HEAL_ERR_DTYPE (dual_split outside heal_dual_split).
 */
typedef struct {
  int64_t batch, n_q_heads, n_kv_heads, head_dim;
  int64_t page_size, num_pages, max_pages_per_seq, max_kv_len;
  const int16_t* q;
  const float* q_scale;
  const int16_t* k_pages;
  const int16_t* v_pages;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int64_t q_strides[2];
  int64_t qs_strides[2];
  int64_t kv_strides[3];
  int64_t kvs_strides[3];
  int64_t o_strides[2];
  int64_t bt_stride;
  float softmax_scale; /* 0 selects 1/sqrt(head_dim) */
  int32_t dual_split;  /* heal_dual_split, as in heal_attn_args */
  float* out;
  void* workspace;
  size_t workspace_bytes;
} heal_paged_decode_args;

/* Workspace bytes heal_attn_decode_paged needs for these arguments. */
HEAL_API size_t heal_attn_paged_workspace_bytes(const heal_paged_decode_args* args);
HEAL_API heal_status heal_attn_decode_paged(const heal_paged_decode_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HEAL_H */
