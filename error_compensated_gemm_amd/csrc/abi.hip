// abi.hip -- the extern "C" entry points of libheal: argument validation, then the kernel launches.
// Every check runs on the host before anything is enqueued; the library never allocates, frees or
// synchronises.  The operations themselves are defined in include/heal.h.
#include <math.h>

#include "heal_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// the launchers answer hipErrorInvalidConfiguration, before any runtime call, for a grid beyond HIP's limits
heal_status launched(hipError_t e) {
  return e == hipSuccess ? HEAL_OK : (e == hipErrorInvalidConfiguration ? HEAL_ERR_UNSUPPORTED : HEAL_ERR_LAUNCH);
}

}  // namespace

extern "C" {

const char* heal_status_str(int status) {
  switch (status) {
    case HEAL_OK: return "HEAL_OK";
    case HEAL_ERR_NULL: return "HEAL_ERR_NULL: a required pointer is NULL";
    case HEAL_ERR_SHAPE: return "HEAL_ERR_SHAPE: a size is negative or inconsistent";
    case HEAL_ERR_STRIDE: return "HEAL_ERR_STRIDE: a leading dimension or stride is too small";
    case HEAL_ERR_ALIGN: return "HEAL_ERR_ALIGN: pointer not 16-byte aligned or leading dimension not a multiple of 8";
    case HEAL_ERR_DTYPE: return "HEAL_ERR_DTYPE: dtype not accepted by this call";
    case HEAL_ERR_UNSUPPORTED: return "HEAL_ERR_UNSUPPORTED: valid request not implemented by this library";
    case HEAL_ERR_LAUNCH: return "HEAL_ERR_LAUNCH: the HIP runtime refused a kernel launch";
    case HEAL_ERR_WORKSPACE: return "HEAL_ERR_WORKSPACE: workspace missing or too small";
    default: return "HEAL: unknown status";
  }
}

int heal_abi_version(void) { return HEAL_ABI_VERSION; }

heal_status heal_split(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ld_x, int part_type,
                       void* hi, void* lo, int64_t ld_part, int32_t* exps, void* stream) {
  if (rows < 0 || cols < 0) return HEAL_ERR_SHAPE;
  if (x_type != HEAL_F32 && x_type != HEAL_BF16 && x_type != HEAL_I16) return HEAL_ERR_DTYPE;
  if (part_type != HEAL_F16 && part_type != HEAL_BF16) return HEAL_ERR_DTYPE;
  if (x_type == HEAL_I16 && (part_type != HEAL_F16 || exps != nullptr)) return HEAL_ERR_DTYPE;
  if (rows == 0) return HEAL_OK;
  if (cols > 0 && (!x || !hi)) return HEAL_ERR_NULL;
  if (x_type == HEAL_I16 && cols > 0 && !lo) return HEAL_ERR_NULL;
  if (ld_x < cols || ld_part < cols) return HEAL_ERR_STRIDE;
  // x: element alignment only (rows that start 16-byte aligned take vector loads); parts: 16-byte rows
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
  if ((x_type == HEAL_F32 ? (xa & 3u) : (xa & 1u)) || (hi && !aligned16(hi)) || (lo && !aligned16(lo)) ||
      (exps && !aligned4(exps)) || (ld_part & 7))
    return HEAL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  switch (x_type) {
    case HEAL_F32:
      return launched(heal::launch_split_f32((const float*)x, rows, cols, ld_x, part_type, hi, lo, ld_part,
                                             exps, s));
    case HEAL_BF16:
      return launched(heal::launch_split_bf16((const uint16_t*)x, rows, cols, ld_x, part_type, hi, lo,
                                              ld_part, exps, s));
    default:
      return launched(heal::launch_unpack_i16((const int16_t*)x, rows, cols, ld_x, HEAL_DUAL_BYTE, hi, lo, ld_part,
                                              s));
  }
}

static bool valid_dual_split(int d) {
  return d == HEAL_DUAL_BYTE || d == HEAL_DUAL_SHIFT10 || d == HEAL_DUAL_FLOAT;
}

heal_status heal_unpack_i16(const int16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int dual_split, void* hi,
                            void* lo, int64_t ld_part, void* stream) {
  if (rows < 0 || cols < 0) return HEAL_ERR_SHAPE;
  if (!valid_dual_split(dual_split)) return HEAL_ERR_DTYPE;
  if (rows == 0 || cols == 0) return HEAL_OK;
  if (!x || !hi || !lo) return HEAL_ERR_NULL;
  if (ld_x < cols || ld_part < cols) return HEAL_ERR_STRIDE;
  if ((reinterpret_cast<uintptr_t>(x) & 1u) || !aligned16(hi) || !aligned16(lo) || (ld_part & 7))
    return HEAL_ERR_ALIGN;
  return launched(
      heal::launch_unpack_i16(x, rows, cols, ld_x, dual_split, hi, lo, ld_part, (hipStream_t)stream));
}

heal_status heal_channel_exponents(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   int32_t threshold_log2, int32_t* col_exps, void* stream) {
  if (rows < 0 || cols < 0 || threshold_log2 < -126 || threshold_log2 > 127) return HEAL_ERR_SHAPE;
  if (cols == 0) return HEAL_OK;
  if (!col_exps || (rows > 0 && !x)) return HEAL_ERR_NULL;
  if (ld_x < cols) return HEAL_ERR_STRIDE;
  if (!aligned4(x) || !aligned16(col_exps)) return HEAL_ERR_ALIGN;
  return launched(heal::launch_channel_exps(x, rows, cols, ld_x, threshold_log2, col_exps, (hipStream_t)stream));
}

heal_status heal_split_scaled(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ld_x,
                              int part_type, void* hi, void* lo, int64_t ld_part, int32_t* exps,
                              const int32_t* col_exps, int32_t col_sign, void* stream) {
  if (rows < 0 || cols < 0) return HEAL_ERR_SHAPE;
  if (x_type != HEAL_F32 && x_type != HEAL_BF16) return HEAL_ERR_DTYPE;
  if (part_type != HEAL_F16 && part_type != HEAL_BF16) return HEAL_ERR_DTYPE;
  if (col_sign != 1 && col_sign != -1) return HEAL_ERR_SHAPE;
  if (rows == 0) return HEAL_OK;
  if (cols > 0 && (!x || !hi || !col_exps)) return HEAL_ERR_NULL;
  if (ld_x < cols || ld_part < cols) return HEAL_ERR_STRIDE;
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
  if ((x_type == HEAL_F32 ? (xa & 3u) : (xa & 1u)) || (hi && !aligned16(hi)) || (lo && !aligned16(lo)) ||
      (exps && !aligned4(exps)) || (col_exps && !aligned16(col_exps)) || (ld_part & 7))
    return HEAL_ERR_ALIGN;
  return launched(heal::launch_split_scaled(x, x_type, rows, cols, ld_x, part_type, hi, lo, ld_part, exps, col_exps,
                                            col_sign, (hipStream_t)stream));
}

heal_status heal_gemm_comp(int64_t M, int64_t N, int64_t K, const void* a_hi, const void* a_lo,
                           const int32_t* a_exp, int64_t lda, const void* b_hi, const void* b_lo,
                           const int32_t* b_exp, int64_t ldb, int part_type, float* c, int64_t ldc,
                           void* stream) {
  if (M < 0 || N < 0 || K < 0) return HEAL_ERR_SHAPE;
  if (M > (int64_t)1 << 31 || N > (int64_t)1 << 31 || K > (int64_t)1 << 31) return HEAL_ERR_SHAPE;
  if (part_type != HEAL_F16 && part_type != HEAL_BF16) return HEAL_ERR_DTYPE;
  if (M == 0 || N == 0) return HEAL_OK;
  if (!c || (K > 0 && (!a_hi || !b_hi))) return HEAL_ERR_NULL;
  if (lda < K || ldb < K || ldc < N) return HEAL_ERR_STRIDE;
  if ((a_hi && !aligned16(a_hi)) || (a_lo && !aligned16(a_lo)) || (b_hi && !aligned16(b_hi)) ||
      (b_lo && !aligned16(b_lo)) || !aligned16(c) || (a_exp && !aligned4(a_exp)) ||
      (b_exp && !aligned4(b_exp)) || (lda & 7) || (ldb & 7) || (ldc & 3))
    return HEAL_ERR_ALIGN;
  return launched(heal::launch_gemm_comp(M, N, K, (const uint16_t*)a_hi, (const uint16_t*)a_lo, a_exp, lda,
                                         (const uint16_t*)b_hi, (const uint16_t*)b_lo, b_exp, ldb, part_type,
                                         c, ldc, (hipStream_t)stream));
}

heal_status heal_row_exponents(const float* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t* exps,
                               void* stream) {
  if (rows < 0 || cols < 0) return HEAL_ERR_SHAPE;
  if (rows == 0) return HEAL_OK;
  if (!exps || (cols > 0 && !x)) return HEAL_ERR_NULL;
  if (ld_x < cols) return HEAL_ERR_STRIDE;
  if ((x && !aligned4(x)) || !aligned4(exps)) return HEAL_ERR_ALIGN;
  return launched(heal::launch_row_exps(x, rows, cols, ld_x, exps, (hipStream_t)stream));
}

heal_status heal_gemm_comp_f32a(int64_t M, int64_t N, int64_t K, const float* a, int64_t lda, const int32_t* a_exp,
                                const void* b_hi, const void* b_lo, const int32_t* b_exp, int64_t ldb, float* c,
                                int64_t ldc, void* stream) {
  if (M < 0 || N < 0 || K < 0) return HEAL_ERR_SHAPE;
  if (M > (int64_t)1 << 31 || N > (int64_t)1 << 31 || K > (int64_t)1 << 31) return HEAL_ERR_SHAPE;
  if (M == 0 || N == 0) return HEAL_OK;
  if (!c || (!a_exp && M > 16) || (K > 0 && (!a || !b_hi))) return HEAL_ERR_NULL;
  if (lda < K || ldb < K || ldc < N) return HEAL_ERR_STRIDE;
  if ((a && !aligned16(a)) || (b_hi && !aligned16(b_hi)) || (b_lo && !aligned16(b_lo)) || !aligned16(c) ||
      (a_exp && !aligned4(a_exp)) || (b_exp && !aligned4(b_exp)) || (lda & 3) || (ldb & 7) || (ldc & 3))
    return HEAL_ERR_ALIGN;
  return launched(heal::launch_gemm_comp_f32a(M, N, K, a, lda, a_exp, (const uint16_t*)b_hi, (const uint16_t*)b_lo,
                                              b_exp, ldb, c, ldc, (hipStream_t)stream));
}

heal_status heal_gemm_comp_quant_i16(int64_t M, int64_t N, int64_t K, const void* a_hi, const void* a_lo,
                                     const int32_t* a_exp, int64_t lda, const void* b_hi, const void* b_lo,
                                     const int32_t* b_exp, int64_t ldb, int part_type, int16_t* q, int64_t ldq,
                                     float* scale, int64_t ld_s, void* stream) {
  if (M < 0 || N < 0 || K < 0) return HEAL_ERR_SHAPE;
  if (M > (int64_t)1 << 31 || N > (int64_t)1 << 31 || K > (int64_t)1 << 31) return HEAL_ERR_SHAPE;
  if (N % 128 != 0) return HEAL_ERR_SHAPE;
  if (part_type != HEAL_F16) return HEAL_ERR_DTYPE;
  if (M == 0 || N == 0) return HEAL_OK;
  if (!q || !scale || (K > 0 && (!a_hi || !b_hi))) return HEAL_ERR_NULL;
  if (lda < K || ldb < K || ldq < N || ld_s < N / 128) return HEAL_ERR_STRIDE;
  if ((a_hi && !aligned16(a_hi)) || (a_lo && !aligned16(a_lo)) || (b_hi && !aligned16(b_hi)) ||
      (b_lo && !aligned16(b_lo)) || !aligned16(q) || !aligned4(scale) || (a_exp && !aligned4(a_exp)) ||
      (b_exp && !aligned4(b_exp)) || (lda & 7) || (ldb & 7) || (ldq & 7))
    return HEAL_ERR_ALIGN;
  return launched(heal::launch_gemm_comp_quant(M, N, K, (const uint16_t*)a_hi, (const uint16_t*)a_lo, a_exp, lda,
                                               (const uint16_t*)b_hi, (const uint16_t*)b_lo, b_exp, ldb, q, ldq,
                                               scale, ld_s, (hipStream_t)stream));
}

const char* heal_gemm_comp_variant(int64_t M, int64_t N, int64_t K, int products) {
  return heal::gemm_comp_variant(M, N, K, products);
}

static bool gemm_sizes_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 0 && N >= 0 && K >= 0 && M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31 && K <= (int64_t)1 << 31;
}

size_t heal_gemm_comp_workspace_bytes(int64_t M, int64_t N, int64_t K, int products) {
  if (!gemm_sizes_ok(M, N, K) || products < 1 || products > 3) return 0;
  return heal::gemm_comp_workspace(M, N, K, products >= 2, products == 3);
}

int heal_gemm_comp_splitk_slices(int64_t M, int64_t N, int64_t K, int products) {
  if (!gemm_sizes_ok(M, N, K) || products < 1 || products > 3) return 1;
  return heal::gemm_comp_slices(M, N, K, products >= 2, products == 3);
}

heal_status heal_gemm_comp_splitk(int64_t M, int64_t N, int64_t K, const void* a_hi, const void* a_lo,
                                  const int32_t* a_exp, int64_t lda, const void* b_hi, const void* b_lo,
                                  const int32_t* b_exp, int64_t ldb, int part_type, float* c, int64_t ldc,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!gemm_sizes_ok(M, N, K)) return HEAL_ERR_SHAPE;
  if (part_type != HEAL_F16 && part_type != HEAL_BF16) return HEAL_ERR_DTYPE;
  if (M == 0 || N == 0) return HEAL_OK;
  if (!c || (K > 0 && (!a_hi || !b_hi))) return HEAL_ERR_NULL;
  if (lda < K || ldb < K || ldc < N) return HEAL_ERR_STRIDE;
  if ((a_hi && !aligned16(a_hi)) || (a_lo && !aligned16(a_lo)) || (b_hi && !aligned16(b_hi)) ||
      (b_lo && !aligned16(b_lo)) || !aligned16(c) || (a_exp && !aligned4(a_exp)) ||
      (b_exp && !aligned4(b_exp)) || (lda & 7) || (ldb & 7) || (ldc & 3))
    return HEAL_ERR_ALIGN;
  const size_t need = heal::gemm_comp_workspace(M, N, K, a_lo != nullptr, b_lo != nullptr);
  if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return HEAL_ERR_WORKSPACE;
  return launched(heal::launch_gemm_comp_splitk(M, N, K, (const uint16_t*)a_hi, (const uint16_t*)a_lo, a_exp, lda,
                                                (const uint16_t*)b_hi, (const uint16_t*)b_lo, b_exp, ldb, part_type,
                                                c, ldc, workspace, (hipStream_t)stream));
}

size_t heal_gemm_comp_f32a_workspace_bytes(int64_t M, int64_t N, int64_t K, int products) {
  if (!gemm_sizes_ok(M, N, K) || products < 2 || products > 3) return 0;
  return heal::gemm_comp_f32a_workspace(M, N, K, products == 3);
}

int heal_gemm_comp_f32a_splitk_slices(int64_t M, int64_t N, int64_t K, int products) {
  if (!gemm_sizes_ok(M, N, K) || products < 2 || products > 3) return 1;
  return heal::gemm_comp_f32a_slices(M, N, K, products == 3);
}

heal_status heal_gemm_comp_f32a_splitk(int64_t M, int64_t N, int64_t K, const float* a, int64_t lda,
                                       const int32_t* a_exp, const void* b_hi, const void* b_lo,
                                       const int32_t* b_exp, int64_t ldb, float* c, int64_t ldc, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (!gemm_sizes_ok(M, N, K)) return HEAL_ERR_SHAPE;
  if (M == 0 || N == 0) return HEAL_OK;
  if (!c || (!a_exp && M > 16) || (K > 0 && (!a || !b_hi))) return HEAL_ERR_NULL;
  if (lda < K || ldb < K || ldc < N) return HEAL_ERR_STRIDE;
  if ((a && !aligned16(a)) || (b_hi && !aligned16(b_hi)) || (b_lo && !aligned16(b_lo)) || !aligned16(c) ||
      (a_exp && !aligned4(a_exp)) || (b_exp && !aligned4(b_exp)) || (lda & 3) || (ldb & 7) || (ldc & 3))
    return HEAL_ERR_ALIGN;
  // without row exponents the call is heal_gemm_comp_f32a (exponents derived in the kernel), unsplit
  const size_t need = a_exp ? heal::gemm_comp_f32a_workspace(M, N, K, b_lo != nullptr) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return HEAL_ERR_WORKSPACE;
  return launched(heal::launch_gemm_comp_f32a_splitk(M, N, K, a, lda, a_exp, (const uint16_t*)b_hi,
                                                     (const uint16_t*)b_lo, b_exp, ldb, c, ldc, workspace,
                                                     (hipStream_t)stream));
}

heal_status heal_qkv_quant_i16(const float* x, int64_t tokens, int64_t heads, int64_t head_dim,
                               int64_t ld_x, int16_t* q, int64_t ld_q, float* scale, int64_t ld_s,
                               void* stream) {
  if (tokens < 0 || heads < 0 || head_dim < 0) return HEAL_ERR_SHAPE;
  if (head_dim % 4 != 0 || head_dim > 1024) return HEAL_ERR_UNSUPPORTED;
  if (tokens == 0 || heads == 0 || head_dim == 0) return HEAL_OK;
  if (!x || !q || !scale) return HEAL_ERR_NULL;
  if (ld_x < heal::mul_sat(heads, head_dim) || ld_q < heal::mul_sat(heads, head_dim) || ld_s < heads)
    return HEAL_ERR_STRIDE;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u) || !aligned4(scale) || (ld_x & 3) || (ld_q & 3))
    return HEAL_ERR_ALIGN;
  return launched(heal::launch_quant_i16(x, tokens, heads, head_dim, ld_x, q, ld_q, scale, ld_s,
                                         (hipStream_t)stream));
}

size_t heal_attn_workspace_bytes(const heal_attn_args* a) {
  if (!a) return 0;
  return heal::attn_workspace_bytes(*a);
}

}  // extern "C"

namespace {

// The argument checks of heal_attn_dual_fp16 other than the workspace.  HEAL_OK with *empty set means a
// valid problem with nothing to compute.
heal_status check_attn(const heal_attn_args* a, bool* empty) {
  *empty = false;
  if (!a) return HEAL_ERR_NULL;
  if (!valid_dual_split(a->dual_split)) return HEAL_ERR_DTYPE;
  if (a->batch < 0 || a->q_len < 0 || a->kv_len < 0 || a->n_q_heads < 0 || a->n_kv_heads < 0 ||
      a->head_dim < 0)
    return HEAL_ERR_SHAPE;
  if (a->head_dim != 128) return HEAL_ERR_UNSUPPORTED;
  if (a->n_kv_heads == 0 || a->n_q_heads % a->n_kv_heads != 0) return HEAL_ERR_SHAPE;
  if (a->batch == 0 || a->q_len == 0 || a->n_q_heads == 0) {
    *empty = true;
    return HEAL_OK;
  }
  if (!a->q || !a->q_scale || !a->out) return HEAL_ERR_NULL;
  if (a->kv_len > 0 && (!a->k || !a->v || !a->k_scale || !a->v_scale)) return HEAL_ERR_NULL;
  if (!(a->softmax_scale >= 0.0f) || isinf(a->softmax_scale)) return HEAL_ERR_SHAPE;
  const int64_t D = a->head_dim;
  for (int i = 0; i < 3; ++i)
    if (a->q_strides[i] < 0 || a->kv_strides[i] < 0 || a->qs_strides[i] < 0 || a->kvs_strides[i] < 0 ||
        a->o_strides[i] < 0)
      return HEAL_ERR_STRIDE;
  if (a->q_strides[2] < D || a->kv_strides[2] < D || a->o_strides[2] < D) return HEAL_ERR_STRIDE;
  const int64_t* st[3] = {a->q_strides, a->kv_strides, a->o_strides};
  for (int t = 0; t < 3; ++t)
    for (int i = 0; i < 3; ++i)
      if (st[t][i] & 7) return HEAL_ERR_ALIGN;
  if (!aligned16(a->q) || !aligned16(a->out) || (a->k && !aligned16(a->k)) || (a->v && !aligned16(a->v)) ||
      !aligned4(a->q_scale) || (a->k_scale && !aligned4(a->k_scale)) || (a->v_scale && !aligned4(a->v_scale)))
    return HEAL_ERR_ALIGN;
  return HEAL_OK;
}

}  // namespace

extern "C" {

heal_status heal_attn_dual_fp16(const heal_attn_args* a, void* stream) {
  bool empty = false;
  const heal_status st = check_attn(a, &empty);
  if (st != HEAL_OK || empty) return st;
  const size_t need = heal::attn_workspace_bytes(*a);
  if (need > 0 && (!a->workspace || a->workspace_bytes < need || (reinterpret_cast<uintptr_t>(a->workspace) & 255u)))
    return HEAL_ERR_WORKSPACE;
  return launched(heal::launch_attn(*a, (hipStream_t)stream));
}

heal_status heal_attn_dual_fp16_noalloc(const heal_attn_args* a, void* stream) {
  bool empty = false;
  const heal_status st = check_attn(a, &empty);
  if (st != HEAL_OK || empty) return st;
  if (heal::attn_workspace_bytes(*a) > HEAL_ATTN_NOALLOC_MAX_WORKSPACE) return HEAL_ERR_WORKSPACE;
  return launched(heal::launch_attn_noalloc(*a, (hipStream_t)stream));
}

size_t heal_attn_paged_workspace_bytes(const heal_paged_decode_args* a) {
  if (!a) return 0;
  return heal::paged_workspace_bytes(*a);
}

heal_status heal_attn_decode_paged(const heal_paged_decode_args* a, void* stream) {
  if (!a) return HEAL_ERR_NULL;
  if (!valid_dual_split(a->dual_split)) return HEAL_ERR_DTYPE;
  if (a->batch < 0 || a->n_q_heads < 0 || a->n_kv_heads < 0 || a->head_dim < 0 || a->page_size < 0 ||
      a->num_pages < 0 || a->max_pages_per_seq < 0 || a->max_kv_len < 0)
    return HEAL_ERR_SHAPE;
  if (a->head_dim != 128) return HEAL_ERR_UNSUPPORTED;
  if (a->page_size < 32 || (a->page_size & (a->page_size - 1)) || a->page_size > (int64_t(1) << 30))
    return HEAL_ERR_UNSUPPORTED;
  if (a->n_kv_heads == 0 || a->n_q_heads % a->n_kv_heads != 0) return HEAL_ERR_SHAPE;
  if (a->n_q_heads / a->n_kv_heads > 16) return HEAL_ERR_UNSUPPORTED;
  // the table must be able to hold max_kv_len keys (checked without overflow)
  if (a->max_kv_len > 0 && (a->max_pages_per_seq == 0 || a->max_pages_per_seq < (a->max_kv_len + a->page_size - 1) / a->page_size))
    return HEAL_ERR_SHAPE;
  if (a->max_kv_len > 0 && a->num_pages == 0) return HEAL_ERR_SHAPE;
  if (a->batch == 0 || a->n_q_heads == 0) return HEAL_OK;
  if (!a->q || !a->q_scale || !a->out || !a->seq_lens) return HEAL_ERR_NULL;
  if (a->max_kv_len > 0 && (!a->k_pages || !a->v_pages || !a->k_scale || !a->v_scale || !a->block_table))
    return HEAL_ERR_NULL;
  if (!(a->softmax_scale >= 0.0f) || isinf(a->softmax_scale)) return HEAL_ERR_SHAPE;
  const int64_t D = a->head_dim;
  for (int i = 0; i < 2; ++i)
    if (a->q_strides[i] < 0 || a->qs_strides[i] < 0 || a->o_strides[i] < 0) return HEAL_ERR_STRIDE;
  for (int i = 0; i < 3; ++i)
    if (a->kv_strides[i] < 0 || a->kvs_strides[i] < 0) return HEAL_ERR_STRIDE;
  if (a->q_strides[1] < D || a->o_strides[1] < D || a->kv_strides[2] < D || a->bt_stride < a->max_pages_per_seq)
    return HEAL_ERR_STRIDE;
  for (int i = 0; i < 2; ++i)
    if ((a->q_strides[i] & 7) || (a->o_strides[i] & 7)) return HEAL_ERR_ALIGN;
  for (int i = 0; i < 3; ++i)
    if (a->kv_strides[i] & 7) return HEAL_ERR_ALIGN;
  if (!aligned16(a->q) || !aligned16(a->out) || (a->k_pages && !aligned16(a->k_pages)) ||
      (a->v_pages && !aligned16(a->v_pages)) || !aligned4(a->q_scale) || !aligned4(a->seq_lens) ||
      (a->k_scale && !aligned4(a->k_scale)) || (a->v_scale && !aligned4(a->v_scale)) ||
      (a->block_table && !aligned4(a->block_table)))
    return HEAL_ERR_ALIGN;
  const size_t need = heal::paged_workspace_bytes(*a);
  if (need > 0 && (!a->workspace || a->workspace_bytes < need || (reinterpret_cast<uintptr_t>(a->workspace) & 255u)))
    return HEAL_ERR_WORKSPACE;
  return launched(heal::launch_attn_paged(*a, (hipStream_t)stream));
}

}  // extern "C"
