/*
 * heal_glue.h -- the non-GEMM, non-attention steps of a Llama-style decoder block (embedding gather, RMSNorm,
 * rotary embedding, SwiGLU, residual add, argmax), used to run a random-initialised decoder stack on the
 * HEAL path for the model-level check (argmax agreement with an FP64 forward).  Harness code, not part of
 * the HEAL boundary of heal.h; built into libheal_glue.so.
 *
 * All pointers are device memory owned by the caller; all arithmetic is FP32 with fixed-order reductions;
 * each call enqueues on `stream` (a hipStream_t, NULL = the default stream) and returns 0, 6 when a size
 * would need a launch grid beyond HIP's 2^32 work-items per dimension (or, for argmax, n above INT32_MAX),
 * checked before any runtime call, or 7 when the HIP runtime refused the launch.  Sizes <= 0 do nothing.
 */
#ifndef HEAL_GLUE_H
#define HEAL_GLUE_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define GLUE_API __attribute__((visibility("default")))
#else
#define GLUE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* out[t, :] = emb[ids[t], :] as FP32 (emb: bf16 bit patterns [vocab, d]; out [T, d]) */
GLUE_API int glue_embed(const uint16_t* emb, const int32_t* ids, int64_t T, int64_t d, float* out, void* stream);
/* y[t, :] = x[t, :] / sqrt(mean_c x[t, c]^2 + eps)  (unit weight; x, y [T, d], may alias) */
GLUE_API int glue_rmsnorm(const float* x, int64_t T, int64_t d, float eps, float* y, void* stream);
/* x[T, d] += r[T, d] in place, then y = rmsnorm(x) (the bits of glue_add followed by glue_rmsnorm), one launch */
GLUE_API int glue_add_rmsnorm(float* x, const float* r, int64_t T, int64_t d, float eps, float* y, void* stream);
/* rotary embedding in place on H heads of 128 per token (row stride ld_t floats): for i < 64, the pair
 * (v[i], v[i + 64]) of the token at position pos0 + t is rotated by the angle whose cosine and sine are
 * cs[((pos0 + t) * 64 + i) * 2 + {0, 1}] */
GLUE_API int glue_rope(float* x, int64_t T, int64_t H, int64_t ld_t, int64_t pos0, const float* cs, void* stream);
/* out[i] = g[i] / (1 + exp(-g[i])) * u[i], i < n */
GLUE_API int glue_swiglu(const float* g, const float* u, int64_t n, float* out, void* stream);
/* x[i] += y[i], i < n */
GLUE_API int glue_add(float* x, const float* y, int64_t n, void* stream);
/* out[0] = the index of the largest of x[0..n) (the lowest index among equal maxima) */
GLUE_API int glue_argmax(const float* x, int64_t n, int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HEAL_GLUE_H */
