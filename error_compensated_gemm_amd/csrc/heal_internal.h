// heal_internal.h -- declarations shared by the HIP translation units of libheal (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/heal.h"

namespace heal {

// HIP runs fewer than 2^32 work-items per grid dimension.  Every launcher checks its grid with this before
// any runtime call and answers hipErrorInvalidConfiguration, which the C ABI reports as
// HEAL_ERR_UNSUPPORTED; a 64-bit block count is never truncated into a smaller grid.
inline bool grid_fits(int64_t blocks, int64_t threads) {
  return blocks >= 0 && blocks <= ((((int64_t)1) << 32) - 1) / threads;
}
// a * b for non-negative sizes, saturating at INT64_MAX instead of wrapping
inline int64_t mul_sat(int64_t a, int64_t b) {
  if (a <= 0 || b <= 0) return 0;
  return a > INT64_MAX / b ? INT64_MAX : a * b;
}

// Launchers (host side).  Each enqueues its kernels on `stream` and returns hipGetLastError().
hipError_t launch_split_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x, int part, void* hi,
                            void* lo, int64_t ld_part, int32_t* exps, hipStream_t stream);
hipError_t launch_split_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int part, void* hi,
                             void* lo, int64_t ld_part, int32_t* exps, hipStream_t stream);
hipError_t launch_split_scaled(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ld_x, int part,
                               void* hi, void* lo, int64_t ld_part, int32_t* exps, const int32_t* col_e,
                               int col_sign, hipStream_t stream);
hipError_t launch_row_exps(const float* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t* exps,
                           hipStream_t stream);
hipError_t launch_channel_exps(const float* x, int64_t rows, int64_t cols, int64_t ld_x, int threshold_log2,
                               int32_t* col_e, hipStream_t stream);
hipError_t launch_unpack_i16(const int16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int dual_split, void* hi,
                             void* lo, int64_t ld_part, hipStream_t stream);
hipError_t launch_quant_i16(const float* x, int64_t tokens, int64_t heads, int64_t head_dim, int64_t ld_x,
                            int16_t* q, int64_t ld_q, float* scale, int64_t ld_s, hipStream_t stream);
hipError_t launch_gemm_comp(int64_t M, int64_t N, int64_t K, const uint16_t* a_hi, const uint16_t* a_lo,
                            const int32_t* a_exp, int64_t lda, const uint16_t* b_hi, const uint16_t* b_lo,
                            const int32_t* b_exp, int64_t ldb, int part, float* c, int64_t ldc,
                            hipStream_t stream);
const char* gemm_comp_variant(int64_t M, int64_t N, int64_t K, int products);
hipError_t launch_gemm_comp_quant(int64_t M, int64_t N, int64_t K, const uint16_t* a_hi, const uint16_t* a_lo,
                                  const int32_t* a_exp, int64_t lda, const uint16_t* b_hi, const uint16_t* b_lo,
                                  const int32_t* b_exp, int64_t ldb, int16_t* q, int64_t ldq, float* s,
                                  int64_t ld_s, hipStream_t stream);
hipError_t launch_gemm_comp_f32a(int64_t M, int64_t N, int64_t K, const float* a, int64_t lda, const int32_t* a_exp,
                                 const uint16_t* b_hi, const uint16_t* b_lo, const int32_t* b_exp, int64_t ldb,
                                 float* c, int64_t ldc, hipStream_t stream);
size_t gemm_comp_workspace(int64_t M, int64_t N, int64_t K, bool a_lo, bool b_lo);
size_t gemm_comp_f32a_workspace(int64_t M, int64_t N, int64_t K, bool b_lo);
int gemm_comp_f32a_slices(int64_t M, int64_t N, int64_t K, bool b_lo);
hipError_t launch_gemm_comp_f32a_splitk(int64_t M, int64_t N, int64_t K, const float* a, int64_t lda,
                                        const int32_t* a_exp, const uint16_t* b_hi, const uint16_t* b_lo,
                                        const int32_t* b_exp, int64_t ldb, float* c, int64_t ldc, void* workspace,
                                        hipStream_t stream);
int gemm_comp_slices(int64_t M, int64_t N, int64_t K, bool a_lo, bool b_lo);
hipError_t launch_gemm_comp_splitk(int64_t M, int64_t N, int64_t K, const uint16_t* a_hi, const uint16_t* a_lo,
                                   const int32_t* a_exp, int64_t lda, const uint16_t* b_hi, const uint16_t* b_lo,
                                   const int32_t* b_exp, int64_t ldb, int part, float* c, int64_t ldc, void* workspace,
                                   hipStream_t stream);
size_t attn_workspace_bytes(const heal_attn_args& a);
hipError_t launch_attn(const heal_attn_args& a, hipStream_t stream);
// launch_attn with the decode partials in the library's own device scratch (HEAL_ATTN_NOALLOC_MAX_WORKSPACE
// bytes per device); the caller has checked that attn_workspace_bytes(a) fits
hipError_t launch_attn_noalloc(const heal_attn_args& a, hipStream_t stream);
size_t paged_workspace_bytes(const heal_paged_decode_args& a);
hipError_t launch_attn_paged(const heal_paged_decode_args& a, hipStream_t stream);

}  // namespace heal
