// split_quant.hip -- the HBM-bound passes of the HEAL hot path on gfx950:
//   * the split of an FP32 / bf16 matrix into a 16-bit primary value and a 16-bit residual, with an exact
//     power-of-two row prescale ([TS 2B Mechanism, Overflow Handling]);
//   * the same split's row exponents alone, for a GEMM that splits its FP32 operand itself;
//   * the outlier-channel calibration (per-column exponents) and the column-scaled split ([TS 2B Overflow
//     Handling]);
//   * the Dual-FP16 unpack of an INT16 matrix under the byte, shift-10 or float-float reading ([TS 2A
//     Mechanism]);
//   * the INT16 quantisation of Q/K/V per (token, head) ([TS 2A Solution]).
// [TS] = gist.science explainer "Demystifying Numerical Instability in LLM Inference: Achieving
// Reproducible Inference for Mission-Critical Tasks with HEAL", Technical Summary.
//
// Layout of the work: one 64-lane wavefront per matrix row (split) or one 32-lane half-wave per
// (token, head) row (quantise), 16-byte vector loads and stores, the row maximum reduced with cross-lane
// shuffles, no atomics (only the column calibration meets its wavefronts in LDS).  Rows of 2049 to 16384 FP32
// values are split by one workgroup per row with the row held in registers, so every input byte is read once;
// narrower rows take the two-pass wavefront-per-row kernel, whose second read of a row hits L2.  Every output
// byte is written once.
#include "heal_internal.h"

namespace heal {
namespace {

constexpr int kPartF16 = HEAL_F16;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float halfwave_max(float v) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 32));
  return v;
}

// Nontemporal (streaming) stores for outputs that this kernel never reads back.  On the INT16 quantiser they
// took one launch over 4096 tokens x 96 heads x 128 from 69 to 60 us, the plain device-copy rate; the same
// hint on the loads gained nothing and, combined with it, lost the gain.
__device__ __forceinline__ void store_nt(uint2* p, uint2 v) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  u32x2 t;
  t.x = v.x;
  t.y = v.y;
  __builtin_nontemporal_store(t, reinterpret_cast<u32x2*>(p));
}

// ilogb of a positive finite float (subnormals included): v_frexp_exp gives e with x = m * 2^e,
// m in [0.5, 1).
__device__ __forceinline__ int ilogb_pos(float x) { return __builtin_amdgcn_frexp_expf(x) - 1; }

// round-to-nearest-even into the 16-bit part type; returns the bit pattern and the value back in fp32
template <int PART>
__device__ __forceinline__ uint16_t round16(float x, float* back) {
  if constexpr (PART == kPartF16) {
    const _Float16 h = (_Float16)x;
    *back = (float)h;
    return __builtin_bit_cast(uint16_t, h);
  } else {
    const __bf16 h = (__bf16)x;
    *back = (float)h;
    return __builtin_bit_cast(uint16_t, h);
  }
}

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float v[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float v[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) {
  return __builtin_bit_cast(float, (uint32_t)(*p) << 16);
}

// One wavefront per row.  PRESCALE: e = 14 - ilogb(rowmax) (else 0).  RESID: write lo.
// vec: every row of x starts 16-byte aligned (else every element takes the scalar path).
// COLS: every element is first scaled by its column's power of two, x' = fl32(x * 2^(col_sign * col_e[c]))
// (exact unless it leaves the normal range), and the row is then split as x'.
// PARTS = false: only the row exponents are written (for a GEMM that splits its operand itself).
template <typename TIn, int PART, bool PRESCALE, bool RESID, bool COLS = false, bool PARTS = true>
__global__ __launch_bounds__(256) void split_rows_kernel(const TIn* __restrict__ x, int64_t rows,
                                                         int64_t cols, int64_t ld_x, int vec,
                                                         uint16_t* __restrict__ hi,
                                                         uint16_t* __restrict__ lo, int64_t ld_part,
                                                         int32_t* __restrict__ exps,
                                                         const int32_t* __restrict__ col_e = nullptr,
                                                         int col_sign = 0) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // the whole wave leaves together
  const TIn* xr = x + row * ld_x;
  const int64_t nvec = vec ? cols >> 3 : 0;
  const int64_t tail0 = nvec << 3;
  // the column scaling of 8 consecutive values starting at column c0 (col_e is 16-byte aligned)
  auto colscale8 = [&](float v[8], int64_t c0) {
    if constexpr (COLS) {
      const int4 a = *reinterpret_cast<const int4*>(col_e + c0);
      const int4 b = *reinterpret_cast<const int4*>(col_e + c0 + 4);
      const int ce[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __builtin_amdgcn_ldexpf(v[i], col_sign * ce[i]);
    }
  };
  auto colscale1 = [&](float v, int64_t c) {
    if constexpr (COLS) return __builtin_amdgcn_ldexpf(v, col_sign * col_e[c]);
    return v;
  };

  int e = 0;
  if constexpr (PRESCALE) {
    float amax = 0.0f;
#pragma unroll 4
    for (int64_t c = lane; c < nvec; c += 64) {
      float v[8];
      load8(xr + (c << 3), v);
      colscale8(v, c << 3);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    for (int64_t c = tail0 + lane; c < cols; c += 64) amax = fmaxf(amax, fabsf(colscale1(load1(xr + c), c)));
    amax = wave_max(amax);
    e = amax > 0.0f ? 14 - ilogb_pos(amax) : 0;
    if (lane == 0) exps[row] = e;
  }
  if constexpr (!PARTS) return;

  uint16_t* hr = hi + row * ld_part;
  uint16_t* lr = RESID ? lo + row * ld_part : nullptr;
#pragma unroll 2
  for (int64_t c = lane; c < nvec; c += 64) {
    float v[8];
    load8(xr + (c << 3), v);
    colscale8(v, c << 3);
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t h2[2], l2[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float xs = PRESCALE ? __builtin_amdgcn_ldexpf(v[2 * i + j], e) : v[2 * i + j];
        float hb;
        h2[j] = round16<PART>(xs, &hb);
        if constexpr (RESID) {
          float lb;
          l2[j] = round16<PART>(xs - hb, &lb);
        }
      }
      hw[i] = (uint32_t)h2[0] | ((uint32_t)h2[1] << 16);
      if constexpr (RESID) lw[i] = (uint32_t)l2[0] | ((uint32_t)l2[1] << 16);
    }
    *reinterpret_cast<uint4*>(hr + (c << 3)) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    if constexpr (RESID) *reinterpret_cast<uint4*>(lr + (c << 3)) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  for (int64_t c = tail0 + lane; c < cols; c += 64) {
    const float xv = colscale1(load1(xr + c), c);
    const float xs = PRESCALE ? __builtin_amdgcn_ldexpf(xv, e) : xv;
    float hb;
    hr[c] = round16<PART>(xs, &hb);
    if constexpr (RESID) {
      float lb;
      lr[c] = round16<PART>(xs - hb, &lb);
    }
  }
}

// The same split with each row held in registers: one workgroup of 256 threads per row of 2048 < cols <= 2048 NCH
// FP32 values (16-byte aligned rows, prescale on), each thread holding NCH chunks of 8.  The row is read once:
// with many rows in flight the two-pass kernel's second read of a long row misses L2 (its FETCH_SIZE is twice
// the input at 8192 and 14336 columns).  The operations per element are the two-pass kernel's, so the bits are.
// COLS: every value is first scaled by its column's power of two, x' = fl32(x * 2^(col_sign * col_e[c])), with
// the two-pass kernel's operation, and the row is split as x' (col_e 16-byte aligned).
template <int PART, bool RESID, int NCH, bool COLS = false>
__global__ __launch_bounds__(256) void split_row_regs_kernel(const float* __restrict__ x, int64_t cols, int64_t ld_x,
                                                             uint16_t* __restrict__ hi, uint16_t* __restrict__ lo,
                                                             int64_t ld_part, int32_t* __restrict__ exps,
                                                             const int32_t* __restrict__ col_e = nullptr,
                                                             int col_sign = 0) {
  __shared__ float wmax[4];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * ld_x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nvec = cols >> 3;
  float v[NCH][8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int64_t c = tid + 256 * j;
    if (c < nvec) {
      load8(xr + (c << 3), v[j]);
      if constexpr (COLS) {
        const int4 a = *reinterpret_cast<const int4*>(col_e + (c << 3));
        const int4 b = *reinterpret_cast<const int4*>(col_e + (c << 3) + 4);
        const int ce[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][i] = __builtin_amdgcn_ldexpf(v[j][i], col_sign * ce[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
  }
  const int64_t tc = (nvec << 3) + tid;  // the last cols % 8 values, one per thread
  float tv = tc < cols ? xr[tc] : 0.0f;
  if constexpr (COLS) {
    if (tc < cols) tv = __builtin_amdgcn_ldexpf(tv, col_sign * col_e[tc]);
  }
  amax = fmaxf(amax, fabsf(tv));
  amax = wave_max(amax);
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e = amax > 0.0f ? 14 - ilogb_pos(amax) : 0;
  if (tid == 0) exps[row] = e;
  uint16_t* hr = hi + row * ld_part;
  uint16_t* lr = RESID ? lo + row * ld_part : nullptr;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int64_t c = tid + 256 * j;
    if (c < nvec) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t h2[2], l2[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float xs = __builtin_amdgcn_ldexpf(v[j][2 * i + k], e);
          float hb;
          h2[k] = round16<PART>(xs, &hb);
          if constexpr (RESID) {
            float lb;
            l2[k] = round16<PART>(xs - hb, &lb);
          }
        }
        hw[i] = (uint32_t)h2[0] | ((uint32_t)h2[1] << 16);
        if constexpr (RESID) lw[i] = (uint32_t)l2[0] | ((uint32_t)l2[1] << 16);
      }
      *reinterpret_cast<uint4*>(hr + (c << 3)) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      if constexpr (RESID) *reinterpret_cast<uint4*>(lr + (c << 3)) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  }
  if (tc < cols) {
    const float xs = __builtin_amdgcn_ldexpf(tv, e);
    float hb;
    hr[tc] = round16<PART>(xs, &hb);
    if constexpr (RESID) {
      float lb;
      lr[tc] = round16<PART>(xs - hb, &lb);
    }
  }
}

// Dual-FP16 pair of one INT16 value under each reading; every value is an integer (or an integer times
// 2^10) of at most 11 significant bits, so each conversion to FP16 is exact except the one that defines the
// float-float hi (round to nearest even).
//   byte:     hi = q >> 8 (arithmetic shift = floor), lo = q & 0xFF
//   shift-10: hi = q >> 10, lo = q & 0x3FF
//   float:    hi = fp16_rn(q), lo = 2^10 (q - hi)  (q - hi is an integer of magnitude <= 16)
template <int SPLIT>
__device__ __forceinline__ void dual_pair(int q, _Float16& h, _Float16& l) {
  if constexpr (SPLIT == HEAL_DUAL_BYTE) {
    h = (_Float16)(float)(q >> 8);
    l = (_Float16)(float)(q & 0xFF);
  } else if constexpr (SPLIT == HEAL_DUAL_SHIFT10) {
    h = (_Float16)(float)(q >> 10);
    l = (_Float16)(float)(q & 0x3FF);
  } else {
    const float f = (float)q;
    h = (_Float16)f;
    l = (_Float16)(1024.0f * (f - (float)h));
  }
}

template <int SPLIT>
__global__ __launch_bounds__(256) void unpack_i16_kernel(const int16_t* __restrict__ x, int64_t rows,
                                                         int64_t cols, int64_t ld_x, int vec,
                                                         uint16_t* __restrict__ hi,
                                                         uint16_t* __restrict__ lo, int64_t ld_part) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int16_t* xr = x + row * ld_x;
  uint16_t* hr = hi + row * ld_part;
  uint16_t* lr = lo + row * ld_part;
  const int64_t nvec = vec ? cols >> 3 : 0;
  for (int64_t c = lane; c < nvec; c += 64) {
    const uint4 raw = *reinterpret_cast<const uint4*>(xr + (c << 3));
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      _Float16 h0, l0, h1, l1;
      dual_pair<SPLIT>((int)(int16_t)(w[i] & 0xFFFFu), h0, l0);
      dual_pair<SPLIT>((int)(int16_t)(w[i] >> 16), h1, l1);
      hw[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      lw[i] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
    *reinterpret_cast<uint4*>(hr + (c << 3)) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *reinterpret_cast<uint4*>(lr + (c << 3)) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  for (int64_t c = (nvec << 3) + lane; c < cols; c += 64) {
    _Float16 h, l;
    dual_pair<SPLIT>(xr[c], h, l);
    hr[c] = __builtin_bit_cast(uint16_t, h);
    lr[c] = __builtin_bit_cast(uint16_t, l);
  }
}

// INT16 quantisation, one 32-lane half-wave per (token, head) row of head_dim elements; each lane owns
// NV float4 groups of the row (head_dim <= 128 * NV).
template <int NV>
__global__ __launch_bounds__(256) void quant_i16_kernel(const float* __restrict__ x, int64_t tokens,
                                                        int64_t heads, int64_t D, int64_t ld_x,
                                                        int16_t* __restrict__ q, int64_t ld_q,
                                                        float* __restrict__ s, int64_t ld_s) {
  const int sub = threadIdx.x & 31;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 5;
  if (row >= tokens * heads) return;  // both halves of a wave test their own row; shuffles stay in-half
  const int64_t t = row / heads, h = row - t * heads;
  const float* xr = x + t * ld_x + h * D;
  float4 v[NV];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t d = (int64_t)(sub + 32 * i) * 4;
    if (d < D) {
      v[i] = *reinterpret_cast<const float4*>(xr + d);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    } else {
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  amax = halfwave_max(amax);
  const float sc = amax / 32767.0f;  // IEEE fp32 division (correctly rounded build flag)
  if (sub == 0) s[t * ld_s + h] = sc;
  int16_t* qr = q + t * ld_q + h * D;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t d = (int64_t)(sub + 32 * i) * 4;
    if (d < D) {
      const float in[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      uint32_t packed[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        int16_t o[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float r = 0.0f;
          if (sc > 0.0f) {
            r = rintf(in[2 * j + u] / sc);
            r = fminf(fmaxf(r, -32767.0f), 32767.0f);
          }
          o[u] = (int16_t)r;
        }
        packed[j] = (uint32_t)(uint16_t)o[0] | ((uint32_t)(uint16_t)o[1] << 16);
      }
      store_nt(reinterpret_cast<uint2*>(qr + d), make_uint2(packed[0], packed[1]));
    }
  }
}

// Outlier-channel calibration: per column c, m = max_r |x[r, c]| and col_e[c] = T - ilogb(m) where
// ilogb(m) > T (0 otherwise, and for an all-zero column).  A workgroup owns 64 columns of one block of rows; its 4
// wavefronts split the block's rows (each reads 256 consecutive bytes per row, 8 rows requested at a time) and
// meet in LDS.  The row blocks of a column combine through an integer atomicMin on the exponent itself:
// min(0, T - ilogb(m)) only falls as m grows, so the minimum over the blocks is the exponent of the column's
// maximum, in any order (col_e is zeroed by zero_i32_kernel first).  A whole column in one workgroup read at
// 0.62 TB/s (64 workgroups at 4096 columns).
__global__ __launch_bounds__(256) void channel_exps_kernel(const float* __restrict__ x, int64_t rows,
                                                           int64_t cols, int64_t ld_x, int T,
                                                           int32_t* __restrict__ col_e, int64_t rows_per_block) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;  // r0 < r1 (grid of row blocks)
  float m = 0.0f;
  if (c < cols) {
    for (int64_t r = r0 + wave; r < r1; r += 32) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t rr = r + 4 * u < r1 ? r + 4 * u : r1 - 1;  // a repeated row leaves the maximum unchanged
        v[u] = fabsf(x[rr * ld_x + c]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) m = fmaxf(m, v[u]);
    }
  }
  red[wave][lane] = m;
  __syncthreads();
  if (wave == 0 && c < cols) {
    m = fmaxf(fmaxf(red[0][lane], red[1][lane]), fmaxf(red[2][lane], red[3][lane]));
    if (m > 0.0f) {
      const int il = ilogb_pos(m);
      if (il > T) atomicMin(&col_e[c], T - il);
    }
  }
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

inline unsigned blocks_for_rows(int64_t rows, int64_t per_block) {
  return (unsigned)((rows + per_block - 1) / per_block);
}

inline int rows_vectorisable(const void* x, int64_t ld_x, int64_t elem_bytes) {
  return ((reinterpret_cast<uintptr_t>(x) & 15u) == 0 && ((ld_x * elem_bytes) & 15) == 0) ? 1 : 0;
}

template <typename TIn>
hipError_t launch_split_cols(const TIn* x, int64_t rows, int64_t cols, int64_t ld_x, int part, void* hi,
                             void* lo, int64_t ld_part, int32_t* exps, const int32_t* col_e, int col_sign,
                             hipStream_t stream) {
  if (!grid_fits((rows + 3) / 4, 256)) return hipErrorInvalidConfiguration;
  const int vec = rows_vectorisable(x, ld_x, (int64_t)sizeof(TIn));
  const dim3 grid(blocks_for_rows(rows, 4)), block(256);
  uint16_t* h = (uint16_t*)hi;
  uint16_t* l = (uint16_t*)lo;
  const bool pre = exps != nullptr, res = lo != nullptr;
  if constexpr (sizeof(TIn) == 4) {  // FP32 rows of 2049 .. 16384 values: one read, the row in registers
    if (vec && pre && cols > 2048 && cols <= 16384 && grid_fits(rows, 256)) {
      const int nch = (int)(((cols >> 3) + 255) / 256);
#define HEAL_SPLIT_REGS(PART, RES, NCH)                                                                      \
  if (part == PART && res == RES && nch <= NCH) {                                                             \
    hipLaunchKernelGGL((split_row_regs_kernel<PART, RES, NCH, true>), dim3((unsigned)rows), block, 0, stream, \
                       (const float*)x, cols, ld_x, h, l, ld_part, exps, col_e, col_sign);                    \
    return hipGetLastError();                                                                                 \
  }
      HEAL_SPLIT_REGS(HEAL_F16, true, 4)
      HEAL_SPLIT_REGS(HEAL_F16, true, 8)
      HEAL_SPLIT_REGS(HEAL_F16, false, 4)
      HEAL_SPLIT_REGS(HEAL_F16, false, 8)
      HEAL_SPLIT_REGS(HEAL_BF16, true, 4)
      HEAL_SPLIT_REGS(HEAL_BF16, true, 8)
      HEAL_SPLIT_REGS(HEAL_BF16, false, 4)
      HEAL_SPLIT_REGS(HEAL_BF16, false, 8)
#undef HEAL_SPLIT_REGS
    }
  }
#define HEAL_SPLIT_CASE(PART, PRE, RES)                                                                      \
  if (part == PART && pre == PRE && res == RES) {                                                             \
    hipLaunchKernelGGL((split_rows_kernel<TIn, PART, PRE, RES, true>), grid, block, 0, stream, x, rows, cols, \
                       ld_x, vec, h, l, ld_part, exps, col_e, col_sign);                                      \
    return hipGetLastError();                                                                                 \
  }
  HEAL_SPLIT_CASE(HEAL_F16, true, true)
  HEAL_SPLIT_CASE(HEAL_F16, true, false)
  HEAL_SPLIT_CASE(HEAL_F16, false, true)
  HEAL_SPLIT_CASE(HEAL_F16, false, false)
  HEAL_SPLIT_CASE(HEAL_BF16, true, true)
  HEAL_SPLIT_CASE(HEAL_BF16, true, false)
  HEAL_SPLIT_CASE(HEAL_BF16, false, true)
  HEAL_SPLIT_CASE(HEAL_BF16, false, false)
#undef HEAL_SPLIT_CASE
  return hipErrorInvalidValue;
}

template <typename TIn>
hipError_t launch_split_any(const TIn* x, int64_t rows, int64_t cols, int64_t ld_x, int part, void* hi,
                            void* lo, int64_t ld_part, int32_t* exps, hipStream_t stream) {
  if (!grid_fits((rows + 3) / 4, 256)) return hipErrorInvalidConfiguration;
  const int vec = rows_vectorisable(x, ld_x, (int64_t)sizeof(TIn));
  if (rows == 0 || cols == 0) {
    // an empty row still has a defined exponent (0); set it with a one-wave launch of the kernel
    if (rows > 0 && exps) {
      hipLaunchKernelGGL((split_rows_kernel<TIn, kPartF16, true, false>), dim3(blocks_for_rows(rows, 4)),
                         dim3(256), 0, stream, x, rows, (int64_t)0, ld_x, vec, (uint16_t*)hi,
                         (uint16_t*)lo, ld_part, exps);
    }
    return hipGetLastError();
  }
  const dim3 grid(blocks_for_rows(rows, 4)), block(256);
  uint16_t* h = (uint16_t*)hi;
  uint16_t* l = (uint16_t*)lo;
  const bool pre = exps != nullptr, res = lo != nullptr;
  if constexpr (sizeof(TIn) == 4) {  // FP32 rows of 2049 .. 16384 values: one read, the row in registers
    if (vec && pre && cols > 2048 && cols <= 16384 && grid_fits(rows, 256)) {
      const int nch = (int)(((cols >> 3) + 255) / 256);
#define HEAL_SPLIT_REGS(PART, RES, NCH)                                                                      \
  if (part == PART && res == RES && nch <= NCH) {                                                             \
    hipLaunchKernelGGL((split_row_regs_kernel<PART, RES, NCH>), dim3((unsigned)rows), block, 0, stream,       \
                       (const float*)x, cols, ld_x, h, l, ld_part, exps);                                     \
    return hipGetLastError();                                                                                 \
  }
      HEAL_SPLIT_REGS(HEAL_F16, true, 4)
      HEAL_SPLIT_REGS(HEAL_F16, true, 8)
      HEAL_SPLIT_REGS(HEAL_F16, false, 4)
      HEAL_SPLIT_REGS(HEAL_F16, false, 8)
      HEAL_SPLIT_REGS(HEAL_BF16, true, 4)
      HEAL_SPLIT_REGS(HEAL_BF16, true, 8)
      HEAL_SPLIT_REGS(HEAL_BF16, false, 4)
      HEAL_SPLIT_REGS(HEAL_BF16, false, 8)
#undef HEAL_SPLIT_REGS
    }
  }
#define HEAL_SPLIT_CASE(PART, PRE, RES)                                                                \
  if (part == PART && pre == PRE && res == RES) {                                                       \
    hipLaunchKernelGGL((split_rows_kernel<TIn, PART, PRE, RES>), grid, block, 0, stream, x, rows, cols, \
                       ld_x, vec, h, l, ld_part, exps);                                                 \
    return hipGetLastError();                                                                           \
  }
  HEAL_SPLIT_CASE(HEAL_F16, true, true)
  HEAL_SPLIT_CASE(HEAL_F16, true, false)
  HEAL_SPLIT_CASE(HEAL_F16, false, true)
  HEAL_SPLIT_CASE(HEAL_F16, false, false)
  HEAL_SPLIT_CASE(HEAL_BF16, true, true)
  HEAL_SPLIT_CASE(HEAL_BF16, true, false)
  HEAL_SPLIT_CASE(HEAL_BF16, false, true)
  HEAL_SPLIT_CASE(HEAL_BF16, false, false)
#undef HEAL_SPLIT_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_split_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x, int part, void* hi,
                            void* lo, int64_t ld_part, int32_t* exps, hipStream_t stream) {
  return launch_split_any<float>(x, rows, cols, ld_x, part, hi, lo, ld_part, exps, stream);
}

hipError_t launch_row_exps(const float* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t* exps,
                           hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (!grid_fits((rows + 3) / 4, 256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((split_rows_kernel<float, kPartF16, true, false, false, false>), dim3(blocks_for_rows(rows, 4)),
                     dim3(256), 0, stream, x, rows, cols, ld_x, rows_vectorisable(x, ld_x, 4), (uint16_t*)nullptr,
                     (uint16_t*)nullptr, (int64_t)0, exps);
  return hipGetLastError();
}

hipError_t launch_split_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int part,
                             void* hi, void* lo, int64_t ld_part, int32_t* exps, hipStream_t stream) {
  return launch_split_any<uint16_t>(x, rows, cols, ld_x, part, hi, lo, ld_part, exps, stream);
}

hipError_t launch_split_scaled(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ld_x, int part,
                               void* hi, void* lo, int64_t ld_part, int32_t* exps, const int32_t* col_e,
                               int col_sign, hipStream_t stream) {
  if (rows == 0 || cols == 0)  // no column scaling to apply: the exponents of empty rows as heal_split sets them
    return x_type == HEAL_F32
               ? launch_split_any<float>((const float*)x, rows, cols, ld_x, part, hi, lo, ld_part, exps, stream)
               : launch_split_any<uint16_t>((const uint16_t*)x, rows, cols, ld_x, part, hi, lo, ld_part, exps,
                                            stream);
  if (x_type == HEAL_F32)
    return launch_split_cols<float>((const float*)x, rows, cols, ld_x, part, hi, lo, ld_part, exps, col_e,
                                    col_sign, stream);
  return launch_split_cols<uint16_t>((const uint16_t*)x, rows, cols, ld_x, part, hi, lo, ld_part, exps, col_e,
                                     col_sign, stream);
}

hipError_t launch_channel_exps(const float* x, int64_t rows, int64_t cols, int64_t ld_x, int threshold_log2,
                               int32_t* col_e, hipStream_t stream) {
  if (cols == 0) return hipSuccess;
  const int64_t groups = (cols + 63) / 64;
  if (!grid_fits(groups, 256) || !grid_fits((cols + 255) / 256, 256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, stream, col_e, cols);
  if (rows == 0) return hipGetLastError();
  // about 1024 workgroups over the (column group, row block) grid, each row block at least 32 rows
  int64_t blocks = 1024 / groups;
  if (blocks > (rows + 31) / 32) blocks = (rows + 31) / 32;
  if (blocks < 1) blocks = 1;
  const int64_t per = (rows + blocks - 1) / blocks;
  blocks = (rows + per - 1) / per;
  hipLaunchKernelGGL(channel_exps_kernel, dim3((unsigned)groups, (unsigned)blocks), dim3(256), 0, stream, x, rows,
                     cols, ld_x, threshold_log2, col_e, per);
  return hipGetLastError();
}

hipError_t launch_unpack_i16(const int16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int dual_split, void* hi,
                             void* lo, int64_t ld_part, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (!grid_fits((rows + 3) / 4, 256)) return hipErrorInvalidConfiguration;
  const dim3 grid(blocks_for_rows(rows, 4)), block(256);
  const int vec = rows_vectorisable(x, ld_x, 2);
  if (dual_split == HEAL_DUAL_SHIFT10)
    hipLaunchKernelGGL(unpack_i16_kernel<HEAL_DUAL_SHIFT10>, grid, block, 0, stream, x, rows, cols, ld_x, vec,
                       (uint16_t*)hi, (uint16_t*)lo, ld_part);
  else if (dual_split == HEAL_DUAL_FLOAT)
    hipLaunchKernelGGL(unpack_i16_kernel<HEAL_DUAL_FLOAT>, grid, block, 0, stream, x, rows, cols, ld_x, vec,
                       (uint16_t*)hi, (uint16_t*)lo, ld_part);
  else
    hipLaunchKernelGGL(unpack_i16_kernel<HEAL_DUAL_BYTE>, grid, block, 0, stream, x, rows, cols, ld_x, vec,
                       (uint16_t*)hi, (uint16_t*)lo, ld_part);
  return hipGetLastError();
}

hipError_t launch_quant_i16(const float* x, int64_t tokens, int64_t heads, int64_t head_dim, int64_t ld_x,
                            int16_t* q, int64_t ld_q, float* scale, int64_t ld_s, hipStream_t stream) {
  const int64_t rows = mul_sat(tokens, heads);
  if (rows == 0) return hipSuccess;
  if (!grid_fits((rows + 7) / 8, 256)) return hipErrorInvalidConfiguration;
  const dim3 grid(blocks_for_rows(rows, 8)), block(256);
  const int nv = (int)((head_dim + 127) / 128);
  switch (nv) {
    case 0:
    case 1:
      hipLaunchKernelGGL(quant_i16_kernel<1>, grid, block, 0, stream, x, tokens, heads, head_dim, ld_x, q,
                         ld_q, scale, ld_s);
      break;
    case 2:
      hipLaunchKernelGGL(quant_i16_kernel<2>, grid, block, 0, stream, x, tokens, heads, head_dim, ld_x, q,
                         ld_q, scale, ld_s);
      break;
    case 3:
    case 4:
      hipLaunchKernelGGL(quant_i16_kernel<4>, grid, block, 0, stream, x, tokens, heads, head_dim, ld_x, q,
                         ld_q, scale, ld_s);
      break;
    default:
      hipLaunchKernelGGL(quant_i16_kernel<8>, grid, block, 0, stream, x, tokens, heads, head_dim, ld_x, q,
                         ld_q, scale, ld_s);
      break;
  }
  return hipGetLastError();
}

}  // namespace heal
