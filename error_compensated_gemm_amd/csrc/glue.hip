// glue.hip -- the non-GEMM, non-attention steps of a Llama-style decoder block, for the model-level check of
// the HEAL path (a random-initialised stack run with HEAL's GEMM and attention).  Harness code: these kernels
// are not part of HEAL's boundary (include/heal.h); include/heal_glue.h declares them.  All arithmetic is
// FP32, every reduction has a fixed order, and nothing here rounds to 16 bits.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/heal_glue.h"

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// out[t, :] = embedding row ids[t] (bf16 -> fp32, exact)
__global__ void embed_kernel(const uint16_t* __restrict__ emb, const int32_t* __restrict__ ids, int64_t d,
                             float* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const uint16_t* row = emb + (int64_t)ids[t] * d;
  for (int64_t c = threadIdx.x; c < d; c += blockDim.x)
    out[t * d + c] = __builtin_bit_cast(float, (uint32_t)row[c] << 16);
}

// y = x / sqrt(mean(x^2) + eps), one 256-thread workgroup per row; the sum of squares is formed per lane in
// column order, then across lanes and wavefronts in a fixed tree
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int64_t d, float eps,
                                                      float* __restrict__ y) {
  __shared__ float part[4];
  const int64_t t = blockIdx.x;
  const float* xr = x + t * d;
  float s = 0.0f;
  for (int64_t c = threadIdx.x; c < d; c += 256) s = fmaf(xr[c], xr[c], s);
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);  // IEEE division and square root
  for (int64_t c = threadIdx.x; c < d; c += 256) y[t * d + c] = xr[c] * inv;
}

// x += r, then y = rmsnorm(x) as rmsnorm_kernel forms it: each thread adds and squares the columns it later
// scales, so the values and the order of every sum are those of add_kernel followed by rmsnorm_kernel
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(float* __restrict__ x, const float* __restrict__ r,
                                                          int64_t d, float eps, float* __restrict__ y) {
  __shared__ float part[4];
  const int64_t t = blockIdx.x;
  float* xr = x + t * d;
  const float* rr = r + t * d;
  float s = 0.0f;
  for (int64_t c = threadIdx.x; c < d; c += 256) {
    const float v = xr[c] + rr[c];
    xr[c] = v;
    s = fmaf(v, v, s);
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  for (int64_t c = threadIdx.x; c < d; c += 256) y[t * d + c] = xr[c] * inv;
}

// rotary embedding on heads of 128 (pairs (i, i + 64)), in place; cs holds cos and sin per (position, i) as
// [positions][64][2], computed by the caller
__global__ void rope_kernel(float* __restrict__ x, int64_t T, int64_t H, int64_t ld_t, int64_t pos0,
                            const float* __restrict__ cs) {
  const int64_t t = blockIdx.x, h = blockIdx.y;
  const int i = threadIdx.x;  // 0..63
  float* v = x + t * ld_t + h * 128;
  const float c = cs[((pos0 + t) * 64 + i) * 2], s = cs[((pos0 + t) * 64 + i) * 2 + 1];
  const float a = v[i], b = v[i + 64];
  v[i] = a * c - b * s;
  v[i + 64] = b * c + a * s;
}

// out = silu(g) * u with silu(g) = g / (1 + exp(-g))
__global__ void swiglu_kernel(const float* __restrict__ g, const float* __restrict__ u, int64_t n,
                              float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float gv = g[i];
  out[i] = gv / (1.0f + expf(-gv)) * u[i];
}

__global__ void add_kernel(float* __restrict__ x, const float* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] += y[i];
}

// index of the largest value (the lowest index among equal maxima), one 1024-thread workgroup
__global__ __launch_bounds__(1024) void argmax_kernel(const float* __restrict__ x, int64_t n,
                                                      int32_t* __restrict__ out) {
  __shared__ float bv[1024];
  __shared__ int64_t bi[1024];
  float best = -INFINITY;
  int64_t idx = n;  // stays n only when every value is NaN or -inf
  for (int64_t i = threadIdx.x; i < n; i += 1024)
    if (x[i] > best) {
      best = x[i];
      idx = i;
    }
  bv[threadIdx.x] = best;
  bi[threadIdx.x] = idx;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) {
      const float ov = bv[threadIdx.x + w];
      const int64_t oi = bi[threadIdx.x + w];
      if (ov > bv[threadIdx.x] || (ov == bv[threadIdx.x] && oi < bi[threadIdx.x])) {
        bv[threadIdx.x] = ov;
        bi[threadIdx.x] = oi;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = (int32_t)(bi[0] < n ? bi[0] : 0);
}

int status(hipError_t e) { return e == hipSuccess ? 0 : 7; }

// fewer than 2^32 work-items per grid dimension, checked before the launch (6 otherwise)
bool fits(int64_t blocks, int64_t threads) { return blocks <= ((((int64_t)1) << 32) - 1) / threads; }

}  // namespace

extern "C" {

int glue_embed(const uint16_t* emb, const int32_t* ids, int64_t T, int64_t d, float* out, void* stream) {
  if (T <= 0 || d <= 0) return 0;
  if (!fits(T, 256)) return 6;
  hipLaunchKernelGGL(embed_kernel, dim3((unsigned)T), dim3(256), 0, (hipStream_t)stream, emb, ids, d, out);
  return status(hipGetLastError());
}

int glue_rmsnorm(const float* x, int64_t T, int64_t d, float eps, float* y, void* stream) {
  if (T <= 0 || d <= 0) return 0;
  if (!fits(T, 256)) return 6;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)T), dim3(256), 0, (hipStream_t)stream, x, d, eps, y);
  return status(hipGetLastError());
}

int glue_add_rmsnorm(float* x, const float* r, int64_t T, int64_t d, float eps, float* y, void* stream) {
  if (T <= 0 || d <= 0) return 0;
  if (!fits(T, 256)) return 6;
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3((unsigned)T), dim3(256), 0, (hipStream_t)stream, x, r, d, eps, y);
  return status(hipGetLastError());
}

int glue_rope(float* x, int64_t T, int64_t H, int64_t ld_t, int64_t pos0, const float* cs, void* stream) {
  if (T <= 0 || H <= 0) return 0;
  if (!fits(T, 64) || !fits(H, 1)) return 6;
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)T, (unsigned)H), dim3(64), 0, (hipStream_t)stream, x, T, H, ld_t,
                     pos0, cs);
  return status(hipGetLastError());
}

int glue_swiglu(const float* g, const float* u, int64_t n, float* out, void* stream) {
  if (n <= 0) return 0;
  if (!fits((n + 255) / 256, 256)) return 6;
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, g, u, n,
                     out);
  return status(hipGetLastError());
}

int glue_add(float* x, const float* y, int64_t n, void* stream) {
  if (n <= 0) return 0;
  if (!fits((n + 255) / 256, 256)) return 6;
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, x, y, n);
  return status(hipGetLastError());
}

int glue_argmax(const float* x, int64_t n, int32_t* out, void* stream) {
  if (n <= 0) return 0;
  if (n > INT32_MAX) return 6;  // the index is returned as int32
  hipLaunchKernelGGL(argmax_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, x, n, out);
  return status(hipGetLastError());
}

}  // extern "C"
