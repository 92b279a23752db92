// gemm_comp.hip -- the error-compensated GEMM of HEAL on gfx950 matrix cores.
//
// [TS 2B Mechanism]: an FP32 operand is decomposed into a primary 16-bit value and a residual, and the
// 16-bit products are summed so that the truncation error of the primary part is captured.  Here
//   C[i, j] = 2^-(ea_i + eb_j) * sum_k ( ah*bh + ah*bl + al*bh )
// with every product formed by v_mfma_f32_32x32x16_{f16,bf16} from the SAME LDS-staged tiles and summed
// into ONE FP32 accumulator; the only rounding at the kernel boundary is the FP32 store of the scaled
// accumulator ([TS 1 "Microscopic Origin"]: keep the accumulator's precision up to the boundary).
// [TS] = gist.science explainer "Demystifying Numerical Instability in LLM Inference: Achieving
// Reproducible Inference for Mission-Critical Tasks with HEAL", Technical Summary.
//
// Kernel shape (tiled GEMM, both operands K-contiguous, "TN"):
//   * 256 threads = 4 wavefronts in a 2 x 2 arrangement; a wave owns a (BM/2) x (BN/2) block of C held as
//     32 x 32 MFMA accumulators (256 x 256 block tile: 16 accumulators = 256 accumulation registers).
//   * BK = 32 per stage; the A parts (hi, lo) and B parts (hi, lo) of a stage sit in LDS as 16-byte chunks
//     with an XOR swizzle on the chunk index so that the 32 rows a fragment read touches fall in distinct
//     bank groups; two stages double-buffer the LDS, so one barrier per stage suffices.
//   * the next stage's global loads are issued before the current stage's MFMAs and written to LDS after
//     them, so HBM/L2 latency hides behind the matrix work.
//   * the block -> tile mapping first gives each of the 8 XCDs (workgroups are dealt to XCDs round-robin)
//     a contiguous range of tiles, then walks that range in groups of 4 tile rows, so concurrently
//     running tiles of one XCD share A and B panels in that XCD's L2.
#include "heal_internal.h"

namespace heal {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int PART>
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  if constexpr (PART == HEAL_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

constexpr int kBK = 32;          // K per stage
constexpr int kCPR = kBK / 8;    // 16-byte chunks per row of a stage
constexpr int kThreads = 256;

// chunk c of tile row r lives at r * kCPR + (c ^ swz(r)): rows that one fragment read touches together
// land in distinct 16-byte bank groups for both 8- and 16-lane read phases.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & (kCPR - 1); }

// 8 consecutive 16-bit values of one row starting at column k (k a multiple of 8); zeros past K
__device__ __forceinline__ uint4 load_chunk(const uint16_t* __restrict__ row, int64_t k, int64_t K) {
  if (k + 8 <= K) return *reinterpret_cast<const uint4*>(row + k);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (k + i < K) w[i >> 1] |= (uint32_t)row[k + i] << (16 * (i & 1));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int PART, int BM, int BN, bool ALO, bool BLO>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_comp_kernel(
    int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ ah, const uint16_t* __restrict__ al,
    const int32_t* __restrict__ ea, int64_t lda, const uint16_t* __restrict__ bh,
    const uint16_t* __restrict__ bl, const int32_t* __restrict__ eb, int64_t ldb, float* __restrict__ C,
    int64_t ldc) {
  constexpr int NA = ALO ? 2 : 1, NB = BLO ? 2 : 1;
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int A_PER_T = BM * kCPR / kThreads, B_PER_T = BN * kCPR / kThreads;
  constexpr int STAGE = (NA * BM + NB * BN) * kCPR;  // uint4 chunks per stage
  static_assert(A_PER_T >= 1 && B_PER_T >= 1, "tile too small for the loader");
  __shared__ uint4 lds[2 * STAGE];

  // ---- tile of this workgroup (XCD-contiguous, then grouped by 4 tile rows) ----
  const int ntm = (int)((M + BM - 1) / BM), ntn = (int)((N + BN - 1) / BN);
  const int total = ntm * ntn;
  int pid = blockIdx.x;
  {
    const int xcd = pid & 7, idx = pid >> 3, per = total >> 3, rem = total & 7;
    pid = xcd * per + (xcd < rem ? xcd : rem) + idx;
  }
  constexpr int GROUP_M = 4;
  const int group = pid / (GROUP_M * ntn);
  const int first_m = group * GROUP_M;
  const int gm = (ntm - first_m) < GROUP_M ? (ntm - first_m) : GROUP_M;
  const int within = pid - group * GROUP_M * ntn;
  const int64_t m0 = (int64_t)(first_m + within % gm) * BM;
  const int64_t n0 = (int64_t)(within / gm) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- loader: per thread, A_PER_T chunks of each A part and B_PER_T of each B part ----
  const uint16_t* a_rows[A_PER_T];
  const uint16_t* al_rows[A_PER_T];
  int a_slot[A_PER_T];
  int a_col[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int id = tid + kThreads * i, r = id / kCPR, c = id % kCPR;
    int64_t gr = m0 + r;
    if (gr > M - 1) gr = M - 1;  // rows past M only feed outputs that are never stored
    a_rows[i] = ah + gr * lda;
    al_rows[i] = ALO ? al + gr * lda : nullptr;
    a_slot[i] = r * kCPR + (c ^ swz(r));
    a_col[i] = c * 8;
  }
  const uint16_t* b_rows[B_PER_T];
  const uint16_t* bl_rows[B_PER_T];
  int b_slot[B_PER_T];
  int b_col[B_PER_T];
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int id = tid + kThreads * i, r = id / kCPR, c = id % kCPR;
    int64_t gr = n0 + r;
    if (gr > N - 1) gr = N - 1;
    b_rows[i] = bh + gr * ldb;
    bl_rows[i] = BLO ? bl + gr * ldb : nullptr;
    b_slot[i] = r * kCPR + (c ^ swz(r));
    b_col[i] = c * 8;
  }

  uint4 ra[NA][A_PER_T], rb[NB][B_PER_T];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      ra[0][i] = load_chunk(a_rows[i], k0 + a_col[i], K);
      if constexpr (ALO) ra[NA - 1][i] = load_chunk(al_rows[i], k0 + a_col[i], K);
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      rb[0][i] = load_chunk(b_rows[i], k0 + b_col[i], K);
      if constexpr (BLO) rb[NB - 1][i] = load_chunk(bl_rows[i], k0 + b_col[i], K);
    }
  };
  auto lstore = [&](int buf) {
    uint4* s = lds + buf * STAGE;
#pragma unroll
    for (int p = 0; p < NA; ++p)
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) s[p * BM * kCPR + a_slot[i]] = ra[p][i];
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) s[NA * BM * kCPR + p * BN * kCPR + b_slot[i]] = rb[p][i];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)((K + kBK - 1) / kBK);
  if (nk > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  const int frow = lane & 31, fhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((int64_t)(kt + 1) * kBK);
    const uint4* s = lds + buf * STAGE;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int c = 2 * ks + fhalf;
      uint4 fa[NA][TM], fb[NB][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 32 + frow;
#pragma unroll
        for (int p = 0; p < NA; ++p) fa[p][i] = s[p * BM * kCPR + r * kCPR + (c ^ swz(r))];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WN + j * 32 + frow;
#pragma unroll
        for (int p = 0; p < NB; ++p) fb[p][j] = s[NA * BM * kCPR + p * BN * kCPR + r * kCPR + (c ^ swz(r))];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = mfma32<PART>(fa[0][i], fb[0][j], acc[i][j]);
          if constexpr (BLO) acc[i][j] = mfma32<PART>(fa[0][i], fb[NB - 1][j], acc[i][j]);
          if constexpr (ALO) acc[i][j] = mfma32<PART>(fa[NA - 1][i], fb[0][j], acc[i][j]);
        }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: C = acc * 2^-(ea_i + eb_j), one rounding (exact unless the result is subnormal) ----
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t col = n0 + wn * WN + j * 32 + (lane & 31);
    if (col >= N) continue;
    const int ebj = eb ? eb[col] : 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) {
          const int e = (ea ? ea[row] : 0) + ebj;
          C[row * ldc + col] = __builtin_amdgcn_ldexpf(acc[i][j][r], -e);
        }
      }
    }
  }
}

template <int PART, int BM, int BN>
hipError_t launch_tile(int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al,
                       const int32_t* ea, int64_t lda, const uint16_t* bh, const uint16_t* bl,
                       const int32_t* eb, int64_t ldb, float* c, int64_t ldc, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(kThreads);
  if (al && bl)
    hipLaunchKernelGGL((gemm_comp_kernel<PART, BM, BN, true, true>), grid, block, 0, stream, M, N, K, ah, al,
                       ea, lda, bh, bl, eb, ldb, c, ldc);
  else if (al)
    hipLaunchKernelGGL((gemm_comp_kernel<PART, BM, BN, true, false>), grid, block, 0, stream, M, N, K, ah, al,
                       ea, lda, bh, bl, eb, ldb, c, ldc);
  else if (bl)
    hipLaunchKernelGGL((gemm_comp_kernel<PART, BM, BN, false, true>), grid, block, 0, stream, M, N, K, ah, al,
                       ea, lda, bh, bl, eb, ldb, c, ldc);
  else
    hipLaunchKernelGGL((gemm_comp_kernel<PART, BM, BN, false, false>), grid, block, 0, stream, M, N, K, ah,
                       al, ea, lda, bh, bl, eb, ldb, c, ldc);
  return hipGetLastError();
}

template <int PART>
hipError_t launch_part(int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al,
                       const int32_t* ea, int64_t lda, const uint16_t* bh, const uint16_t* bl,
                       const int32_t* eb, int64_t ldb, float* c, int64_t ldc, hipStream_t stream) {
  // the largest tile that still gives every CU a workgroup
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t128 = ((M + 255) / 256) * ((N + 127) / 128);
  if (t256 >= 256)
    return launch_tile<PART, 256, 256>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  if (t128 >= 256)
    return launch_tile<PART, 256, 128>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  return launch_tile<PART, 128, 128>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
}

}  // namespace

hipError_t launch_gemm_comp(int64_t M, int64_t N, int64_t K, const uint16_t* a_hi, const uint16_t* a_lo,
                            const int32_t* a_exp, int64_t lda, const uint16_t* b_hi, const uint16_t* b_lo,
                            const int32_t* b_exp, int64_t ldb, int part, float* c, int64_t ldc,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (part == HEAL_F16)
    return launch_part<HEAL_F16>(M, N, K, a_hi, a_lo, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream);
  return launch_part<HEAL_BF16>(M, N, K, a_hi, a_lo, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream);
}

}  // namespace heal
