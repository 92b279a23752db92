// gemm_comp.hip -- the error-compensated GEMM of HEAL on gfx950 matrix cores.
//
// [TS 2B Mechanism]: an FP32 operand becomes a 16-bit leading part plus a 16-bit remainder (what the leading
// part could not hold), and the 16-bit products are summed so that the leading part's rounding error is
// recovered.  Here
//   C[i, j] = 2^-(ea_i + eb_j) * sum_k ( ah*bh + ah*bl + al*bh )
// with every product formed by v_mfma_f32_32x32x16_{f16,bf16} from the SAME LDS-staged tiles and summed
// into ONE FP32 accumulator; the only rounding at the kernel boundary is the FP32 store of the scaled
// accumulator ([TS 1 "Microscopic Origin"]: keep the accumulator's precision up to the boundary).
// [TS] = gist.science explainer "Demystifying Numerical Instability in LLM Inference: Achieving
// Reproducible Inference for Mission-Critical Tasks with HEAL", Technical Summary.
//
// Kernel shapes (both operands K-contiguous, "TN"):
//   * tile kernel (M > 64): 256 threads = 4 wavefronts in a 2 x 2 arrangement; a wave owns a (BM/2) x (BN/2)
//     block of C held as 32 x 32 MFMA accumulators (256 x 256 block tile: 16 accumulators = 256 accumulation
//     registers).  Block tiles 256 x 256, 128 x 256 (only A has a low part), 256 x 128 and 128 x 128.
//   * BK = 32 per stage; the A parts (hi, lo) and B parts (hi, lo) of a stage sit in LDS as 16-byte chunks
//     with an XOR swizzle on the chunk index so that the 32 rows a fragment read touches fall in distinct
//     bank groups.  Full K tiles arrive by direct global -> LDS transfers into three stages where they fit
//     (two otherwise): the step for tile k issues tile k + 2's transfers, multiplies tile k, and waits only
//     for tile k + 1's, so two stages of MFMAs cover each transfer.  The partial last K tile goes through
//     registers with the columns past K zeroed.
//   * the block -> tile mapping first gives each of the 8 XCDs (workgroups are dealt to XCDs round-robin)
//     a contiguous range of tiles, then walks that range in groups of 4 tile rows, so concurrently
//     running tiles of one XCD share A and B panels in that XCD's L2.
//   * skinny kernel (M <= 64): 8 wavefronts per 16 NC output columns split K, stream B from memory through
//     registers with v_mfma_f32_16x16x32, and meet in a fixed-order LDS reduction.
//   * streamed-B kernel (M <= 16, N of at least three 16-column blocks per CU, A's parts within 60 KB): one
//     persistent workgroup per CU splits A once into LDS and walks its column blocks, B arriving through a
//     ring of direct-to-LDS stages that runs on from one block into the next.
//   * split K (heal_gemm_comp_splitk, and heal_gemm_comp_f32a_splitk for FP32 A at 8..16 rows): the tile or
//     skinny kernel on slices of K into FP32 partials, then an ordered reduction that applies the exponents.
#include <type_traits>

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

// chunk c of tile row r lives at r * kCPR + (c ^ swz(r)).  With 64-byte rows, XOR-ing the chunk index
// with bits 2..3 of the row makes the 32-row x 2-chunk fragment reads (ds_read_b128) conflict-free on
// gfx950: SQ_LDS_BANK_CONFLICT measured 0 for this layout against 4 cycles per read for (r >> 1) & 3 and
// 12 for r & 3 in an LDS probe of the same access pattern.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & (kCPR - 1); }

// Loads stay branch-free: a chunk start k (a multiple of 8) is clamped to klast, the last chunk that
// starts inside the row (every row holds ld >= roundup8(K) elements), and the elements at or past K are
// zeroed afterwards, only for the one partial K tile.  (A per-element tail branch here makes the compiler
// wait for each global load in turn, which serialises the prefetch.)
__device__ __forceinline__ uint4 load_chunk(const uint16_t* __restrict__ row, int64_t k, int64_t klast) {
  return *reinterpret_cast<const uint4*>(row + (k < klast ? k : klast));
}
// keep the first `valid` of the 8 values (valid <= 0 clears the chunk)
__device__ __forceinline__ uint4 mask_chunk(uint4 v, int64_t valid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t m = (2 * d < valid ? 0x0000FFFFu : 0u) | (2 * d + 1 < valid ? 0xFFFF0000u : 0u);
    w[d] &= m;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// The FP16 split of 8 consecutive FP32 values of one row of A (bits in x0, x1) after the row's power-of-two
// prescale, in the same operations as the standalone split ([TS 2B Mechanism, Overflow Handling]):
// xs = fl32(x * 2^e), hi = fp16_rn(xs), lo = fp16_rn(xs - hi), the subtraction exact in FP32.  So a GEMM
// that splits A on the way to its MFMAs multiplies exactly the parts the split pass would have written.
struct Split8 {
  uint4 hi, lo;
};
__device__ __forceinline__ uint32_t split2(uint32_t a, uint32_t b, int e, uint32_t& lo) {
  const float xa = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, a), e);
  const float xb = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, b), e);
  const _Float16 ha = (_Float16)xa, hb = (_Float16)xb;
  const _Float16 la = (_Float16)(xa - (float)ha), lb = (_Float16)(xb - (float)hb);
  lo = (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ Split8 split8(uint4 x0, uint4 x1, int e) {
  Split8 r;
  r.hi.x = split2(x0.x, x0.y, e, r.lo.x);
  r.hi.y = split2(x0.z, x0.w, e, r.lo.y);
  r.hi.z = split2(x1.x, x1.y, e, r.lo.z);
  r.hi.w = split2(x1.z, x1.w, e, r.lo.w);
  return r;
}

// maximum over the 32 lanes of each half-wavefront, with DPP and one swizzle (no LDS traffic): quad
// swaps (lane ^ 1, lane ^ 2), mirrors within 8 and within 16 lanes, then lane ^ 16
__device__ __forceinline__ float halfwave_max32(float m) {
  auto dpp = [](float v, int ctrl) -> float {
    switch (ctrl) {  // the control must be a constant
      case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
      case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
      case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
      default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
    }
  };
  m = fmaxf(m, dpp(m, 0xB1));   // quad_perm [1, 0, 3, 2]
  m = fmaxf(m, dpp(m, 0x4E));   // quad_perm [2, 3, 0, 1]
  m = fmaxf(m, dpp(m, 0x141));  // row_half_mirror: lane i <-> 7 - i within 8
  m = fmaxf(m, dpp(m, 0x140));  // row_mirror: lane i <-> 15 - i within 16
  // ds_swizzle bit mode, and_mask 0x1f, or_mask 0, xor_mask 0x10: lane ^ 16 within each 32 lanes
  return fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, m), 0x401F)));
}

// s_waitcnt immediate: at most N vector-memory operations outstanding, all LDS operations done
template <int N>
constexpr int waitcnt_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4);
}

// one 16-byte direct global -> LDS transfer per lane: lane l's bytes land at lds_wave_base + 16 l
// CPOL: the transfer's cache policy bits (kNT: non-temporal, for a stream read once per launch)
constexpr int kNT = 2;
template <int CPOL = 0>
__device__ __forceinline__ void dma16(const uint16_t* src, uint4* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                   (lds_void_t*)(lds_wave_base), 16, 0, CPOL);
}

// QUANT: instead of storing C, quantise each (row, 128-column head) of it to INT16 exactly as
// heal_qkv_quant_i16 does (s = fl32(max |c| / 32767), q = clamp(rint(fl32(c / s)), +-32767)) and store the
// codes in Qo [M, N] and the scales in So [M, N / 128].
// AF32: A arrives as FP32 rows (af, leading dimension lda in floats) with its row exponents ea; a stage
// holds A as one FP32 plane (the bytes of the hi and lo planes together, chunk c of row r at
// r * 8 + (c ^ (r & 7))), and each wavefront splits its A fragments in registers as it reads them.
// SPLITK: this workgroup multiplies slice blockIdx.y of K ([y * kslice, (y + 1) * kslice) of the parts) and
// writes its FP32 sums unscaled into slice y of the partials C ([gridDim.y][M][ldc]); splitk_reduce_kernel adds
// the slices in order and applies the exponents.
template <int PART, int BM, int BN, bool ALO, bool BLO, bool QUANT = false, bool AF32 = false, bool SPLITK = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_comp_kernel(
    int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ ah, const uint16_t* __restrict__ al,
    const int32_t* __restrict__ ea, int64_t lda, const uint16_t* __restrict__ bh,
    const uint16_t* __restrict__ bl, const int32_t* __restrict__ eb, int64_t ldb, float* __restrict__ C,
    int64_t ldc, int16_t* __restrict__ Qo = nullptr, int64_t ldq = 0, float* __restrict__ So = nullptr,
    int64_t ld_s = 0, const float* __restrict__ af = nullptr, int64_t kslice = 0) {
  static_assert(!AF32 || (ALO && PART == HEAL_F16 && !QUANT), "FP32 A: FP16 parts, both A parts, plain C");
  static_assert(!SPLITK || (!AF32 && !QUANT), "split K: 16-bit parts, FP32 partials");
  if constexpr (SPLITK) {
    const int64_t k0 = (int64_t)blockIdx.y * kslice;
    K = K - k0 < kslice ? K - k0 : kslice;
    ah += k0;
    bh += k0;
    if constexpr (ALO) al += k0;
    if constexpr (BLO) bl += k0;
    C += (int64_t)blockIdx.y * M * ldc;
    ea = nullptr;
    eb = nullptr;
  }
  constexpr int NA = ALO ? 2 : 1, NB = BLO ? 2 : 1;
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int A_PER_T = BM * kCPR / kThreads, B_PER_T = BN * kCPR / kThreads;
  constexpr int APLANE = BM * kCPR, BPLANE = BN * kCPR;  // uint4 chunks per operand plane
  constexpr int STAGE = NA * APLANE + NB * BPLANE;
  static_assert(A_PER_T >= 1 && B_PER_T >= 1, "tile too small for the loader");
  // Stages as distinct objects: the compiler can tell the stage being read from the ones the
  // direct-to-LDS loads are filling, so no wait on those loads is placed before the fragment reads.  Three
  // stages where they fit in the 160 KB of LDS, so each stage's transfers have two stages of MFMAs to land
  // (a transfer's round trip under load is longer than one stage of MFMAs).
  constexpr int NST = (3 * STAGE * 16 + (BM + BN) * 4 <= 160 * 1024) ? 3 : 2;
  __shared__ uint4 lds0[STAGE];
  __shared__ uint4 lds1[STAGE];
  __shared__ uint4 lds2[NST == 3 ? STAGE : 1];
  __shared__ int exps_s[BM + BN];

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

  for (int i = tid; i < BM + BN; i += kThreads) {
    if (i < BM) {
      const int64_t r = (m0 + i < M) ? m0 + i : M - 1;
      exps_s[i] = ea ? ea[r] : 0;
    } else {
      const int64_t r = (n0 + i - BM < N) ? n0 + i - BM : N - 1;
      exps_s[i] = eb ? eb[r] : 0;
    }
  }

  // ---- loader: LDS position p = tid + 256 i of a plane holds row p / kCPR, chunk (p % kCPR) ^ swz(row);
  //      a wavefront's 64 consecutive positions are one direct-to-LDS transfer ----
  const uint16_t* a_src[A_PER_T];
  const uint16_t* al_src[A_PER_T];
  int a_col[A_PER_T];
  if constexpr (!AF32) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int p = tid + kThreads * i, r = p / kCPR, c = (p % kCPR) ^ swz(r);
      int64_t gr = m0 + r;
      if (gr > M - 1) gr = M - 1;  // rows past M only feed outputs that are never stored
      a_col[i] = 8 * c;
      a_src[i] = ah + gr * lda + 8 * c;
      al_src[i] = ALO ? al + gr * lda + 8 * c : nullptr;
    }
  }
  // FP32 A: position p = tid + 256 i of the plane holds row p / 8, chunk (p % 8) ^ (row & 7) of 4 floats
  constexpr int AF_PER_T = AF32 ? 2 * A_PER_T : 1;
  const float* af_src[AF_PER_T];
  int af_col[AF_PER_T];
  if constexpr (AF32) {
#pragma unroll
    for (int i = 0; i < AF_PER_T; ++i) {
      const int p = tid + kThreads * i, r = p >> 3, c = (p & 7) ^ (r & 7);
      int64_t gr = m0 + r;
      if (gr > M - 1) gr = M - 1;
      af_col[i] = 4 * c;
      af_src[i] = af + gr * lda + 4 * c;
    }
  }
  const uint16_t* b_src[B_PER_T];
  const uint16_t* bl_src[B_PER_T];
  int b_col[B_PER_T];
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int p = tid + kThreads * i, r = p / kCPR, c = (p % kCPR) ^ swz(r);
    int64_t gr = n0 + r;
    if (gr > N - 1) gr = N - 1;
    b_col[i] = 8 * c;
    b_src[i] = bh + gr * ldb + 8 * c;
    bl_src[i] = BLO ? bl + gr * ldb + 8 * c : nullptr;
  }
  // full K tiles: direct-to-LDS
  auto dma_stage = [&](uint4* s, int64_t k0) {
    if constexpr (AF32) {
#pragma unroll
      for (int i = 0; i < AF_PER_T; ++i)
        dma16(reinterpret_cast<const uint16_t*>(af_src[i] + k0), s + kThreads * i + 64 * wave);
    } else {
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        uint4* dst = s + kThreads * i + 64 * wave;
        dma16(a_src[i] + k0, dst);
        if constexpr (ALO) dma16(al_src[i] + k0, dst + APLANE);
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      uint4* dst = s + NA * APLANE + kThreads * i + 64 * wave;
      dma16(b_src[i] + k0, dst);
      if constexpr (BLO) dma16(bl_src[i] + k0, dst + BPLANE);
    }
  };
  // the partial last K tile: through registers, zeroing the columns at or past K
  const int64_t klast = ((K + 7) / 8 - 1) * 8;
  auto tail_stage = [&](uint4* s, int64_t k0) {
    if constexpr (AF32) {  // element by element: an FP32 row need not extend past K
#pragma unroll
      for (int i = 0; i < AF_PER_T; ++i) {
        const float* row = af_src[i] - af_col[i];
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t k = k0 + af_col[i] + j;
          const float v = row[k < K ? k : K - 1];
          w[j] = k < K ? __builtin_bit_cast(uint32_t, v) : 0u;
        }
        s[kThreads * i + tid] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        const int64_t k = k0 + a_col[i];
        const int64_t kc = k < klast ? k : klast;
        s[kThreads * i + tid] = mask_chunk(*reinterpret_cast<const uint4*>(a_src[i] - a_col[i] + kc), K - k);
        if constexpr (ALO)
          s[APLANE + kThreads * i + tid] =
              mask_chunk(*reinterpret_cast<const uint4*>(al_src[i] - a_col[i] + kc), K - k);
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int64_t k = k0 + b_col[i];
      const int64_t kc = k < klast ? k : klast;
      s[NA * APLANE + kThreads * i + tid] =
          mask_chunk(*reinterpret_cast<const uint4*>(b_src[i] - b_col[i] + kc), K - k);
      if constexpr (BLO)
        s[NA * APLANE + BPLANE + kThreads * i + tid] =
            mask_chunk(*reinterpret_cast<const uint4*>(bl_src[i] - b_col[i] + kc), K - k);
    }
  };
  const int nk = (int)((K + kBK - 1) / kBK);
  const int nfull = (int)(K / kBK);
  auto fill = [&](uint4* s, int kt) {
    if (kt < nfull) dma_stage(s, (int64_t)kt * kBK);
    else tail_stage(s, (int64_t)kt * kBK);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int frow = lane & 31, fhalf = lane >> 5;
  // the MFMA operand fragments of one 16-wide k step of a stage
  struct Frag {
    uint4 a[NA][TM], b[NB][TN];
  };
  auto read_frags = [&](const uint4* s, int ks, Frag& F) {
    const int c = 2 * ks + fhalf;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * WN + j * 32 + frow;
#pragma unroll
      for (int p = 0; p < NB; ++p) F.b[p][j] = s[NA * APLANE + p * BPLANE + r * kCPR + (c ^ swz(r))];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WM + i * 32 + frow;
      if constexpr (AF32) {
        const int c0 = 4 * ks + 2 * fhalf, sw = r & 7;
        const Split8 sp = split8(s[r * 8 + (c0 ^ sw)], s[r * 8 + ((c0 + 1) ^ sw)], exps_s[r]);
        F.a[0][i] = sp.hi;
        F.a[1][i] = sp.lo;
      } else {
#pragma unroll
        for (int p = 0; p < NA; ++p) F.a[p][i] = s[p * APLANE + r * kCPR + (c ^ swz(r))];
      }
    }
  };
  auto mma = [&](const Frag& F) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc[i][j] = mfma32<PART>(F.a[0][i], F.b[0][j], acc[i][j]);
        if constexpr (BLO) acc[i][j] = mfma32<PART>(F.a[0][i], F.b[NB - 1][j], acc[i][j]);
        if constexpr (ALO) acc[i][j] = mfma32<PART>(F.a[NA - 1][i], F.b[0][j], acc[i][j]);
      }
  };
  auto compute = [&](const uint4* s) {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      Frag F;
      read_frags(s, ks, F);
      mma(F);
    }
  };

  // ---- main loop, unrolled over the stages so each stage is a fixed LDS object.  The steady state (all
  //      prefetched tiles full) is branch-free, so the transfers, fragment reads and MFMAs of a stage
  //      share one scheduling region and are interleaved: reads of the first 16-wide k step, then one
  //      transfer, a few MFMAs and the next k step's reads in turn.  Issuing the transfers ahead of the
  //      MFMAs as a block left the matrix unit idle while they went out (measured: -10 % time). ----
  constexpr int NDMA = NA * A_PER_T + NB * B_PER_T;
  constexpr int KS = kBK / 16;
  constexpr int R0 = TM * NA + TN * NB;             // fragment reads per k step
  constexpr int NMFMA = TM * TN * (1 + (ALO ? 1 : 0) + (BLO ? 1 : 0)) * KS;
  constexpr int MF_PER = NMFMA / (NDMA + 1) > 0 ? NMFMA / (NDMA + 1) : 1;
  constexpr int RD_PER = (R0 * (KS - 1) + NDMA - 1) / NDMA;
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, R0, 0);  // DS reads of the first k step
#pragma unroll
    for (int q = 0; q < NDMA; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, MF_PER, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // one direct-to-LDS transfer
      __builtin_amdgcn_sched_group_barrier(0x100, RD_PER, 0);  // DS reads of the next k step
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMFMA, 0);  // the remaining MFMAs
  };
  if constexpr (NST == 3) {
    // Three stages: the step for tile kt issues tile kt + 2's transfers, multiplies tile kt, then waits
    // only until this thread's transfers of tile kt + 1 have landed (tile kt + 2's may still fly) and
    // meets the other wavefronts at a plain barrier (__syncthreads would also drain tile kt + 2).
    auto wait_then_barrier = [&]() {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm<NDMA>());
      __builtin_amdgcn_s_barrier();
    };
    if (nk > 0) fill(lds0, 0);
    if (nk > 1) fill(lds1, 1);
    __syncthreads();
    int kt = 0;
    for (; kt + 4 < nfull; kt += 3) {
      dma_stage(lds2, (int64_t)(kt + 2) * kBK);
      compute(lds0);
      interleave();
      wait_then_barrier();
      dma_stage(lds0, (int64_t)(kt + 3) * kBK);
      compute(lds1);
      interleave();
      wait_then_barrier();
      dma_stage(lds1, (int64_t)(kt + 4) * kBK);
      compute(lds2);
      interleave();
      wait_then_barrier();
    }
    for (; kt < nk; ++kt) {  // the last tiles (tiles kt and kt + 1 are already in their stages)
      const int si = kt % 3;
      if (kt + 2 < nk) fill(si == 0 ? lds2 : (si == 1 ? lds0 : lds1), kt + 2);
      compute(si == 0 ? lds0 : (si == 1 ? lds1 : lds2));
      __syncthreads();
    }
  } else {
    if (nk > 0) fill(lds0, 0);
    __syncthreads();
    int kt = 0;
    // (measured on 256-wide tiles only; the 256 x 128 tiles ran 5 % slower with it, so they keep the
    // plain loop below)
    for (; BN == 256 && kt + 2 < nfull; kt += 2) {
      dma_stage(lds1, (int64_t)(kt + 1) * kBK);
      compute(lds0);
      interleave();
      __syncthreads();
      dma_stage(lds0, (int64_t)(kt + 2) * kBK);
      compute(lds1);
      interleave();
      __syncthreads();
    }
    for (; kt + 1 < nk; kt += 2) {
      fill(lds1, kt + 1);
      compute(lds0);
      __syncthreads();
      if (kt + 2 < nk) fill(lds0, kt + 2);
      compute(lds1);
      __syncthreads();
    }
    if (kt < nk) compute(lds0);  // odd tile count: the last tile sits in stage 0
  }

  // ---- epilogue: C = acc * 2^-(ea_i + eb_j), one rounding (exact unless the result is subnormal) ----
  if constexpr (!QUANT) {
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int cl = wn * WN + j * 32 + (lane & 31);
      const int64_t col = n0 + cl;
      const int ebj = exps_s[BM + cl];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int64_t row = m0 + rl;
          const float v = __builtin_amdgcn_ldexpf(acc[i][j][r], -(exps_s[rl] + ebj));
          if (interior || (row < M && col < N)) C[row * ldc + col] = v;
        }
      }
    }
  } else {
    // A lane holds rows wm*WM + 32 i + 8 (r/4) + 4 (lane/32) + r%4 at columns wn*WN + 32 j + lane%32, so a
    // row's values inside this wavefront sit in the 32 lanes of one half.  A head (128 columns) is 4
    // column blocks of one wavefront (WN >= 128) or 2 blocks in each of the wavefronts wn = 0, 1 (WN = 64),
    // whose partial maxima meet in LDS.  N is a multiple of 128, so a head is wholly in or out of range.
    static_assert(WN % 128 == 0 || WN == 64, "a head is 128 columns");
    constexpr int HW = WN >= 128 ? WN / 128 : 1;  // heads (or half heads) per wavefront
    constexpr int JH = WN >= 128 ? 4 : TN;        // column blocks per head in this wavefront
    auto cval = [&](int i, int j, int r) {
      const int rl = wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int cl = wn * WN + j * 32 + (lane & 31);
      return __builtin_amdgcn_ldexpf(acc[i][j][r], -(exps_s[rl] + exps_s[BM + cl]));
    };
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
      const int64_t c0h = n0 + wn * WN + hh * 128;  // first column of the head (WN = 64: of its half)
      const int64_t head = c0h / 128;
#pragma unroll
      for (int i = 0; i < TM; ++i) {  // one 32-row block at a time keeps 16 maxima per lane live
        float amax[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float m = 0.0f;
#pragma unroll
          for (int jj = 0; jj < JH; ++jj) m = fmaxf(m, fabsf(cval(i, hh * JH + jj, r)));
          amax[r] = halfwave_max32(m);
        }
        if constexpr (WN < 128) {
          // the other half of the head is in wavefront (wm, wn ^ 1): exchange the row maxima through LDS
          float* hred = reinterpret_cast<float*>(lds0);  // the stages are idle after the main loop
          __syncthreads();
          if ((lane & 31) == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int rl = wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              hred[2 * rl + wn] = amax[r];
            }
          }
          __syncthreads();
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            amax[r] = fmaxf(amax[r], hred[2 * rl + (wn ^ 1)]);
          }
        }
        if (c0h >= N) continue;  // wave-uniform
        const bool all_rows = m0 + wm * WM + i * 32 + 32 <= M;  // wave-uniform: no per-row test needed
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int64_t row = m0 + rl;
          if (!all_rows && row >= M) continue;
          const float sc = amax[r] / 32767.0f;  // IEEE fp32 division (correctly rounded build flag)
          if ((lane & 31) == 0 && (WN >= 128 || wn == 0)) So[row * ld_s + head] = sc;
          int16_t* qrow = Qo + row * ldq + n0 + wn * WN + (lane & 31);
#pragma unroll
          for (int jj = 0; jj < JH; ++jj) {
            const int j = hh * JH + jj;
            // a zero scale (all-zero row) gives zero codes: computed branch-free, then selected
            const float q = fminf(fmaxf(rintf(cval(i, j, r) / sc), -32767.0f), 32767.0f);
            qrow[j * 32] = (int16_t)(sc > 0.0f ? q : 0.0f);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------- skinny M
// M <= 64: the problem is a stream over B (N x K 16-bit values read once from HBM) with a small A that
// stays in L2.  A workgroup of 8 wavefronts owns 16 NC output columns; its wavefronts split K in 32-wide
// steps and each accumulates 16 x 16 blocks (16 rows of A x 16 columns) with v_mfma_f32_16x16x32, so each
// A fragment loaded feeds NC MFMAs and A is re-read from L2 once per workgroup.  The 8 partial blocks are
// added in wavefront order through LDS (fixed order: bitwise reproducible).
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int PART>
__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, const f32x4& c) {
  if constexpr (PART == HEAL_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

constexpr int kSkWaves = 8;

// AF32: A arrives as FP32 rows (af, leading dimension lda in floats) with row exponents ea; a lane's 8
// values of a K step are held as raw FP32 bits (the registers the hi and lo chunks would take) and split
// just before the MFMAs, so the prefetch never waits on them.
// SPLITK: as for gemm_comp_kernel, slice blockIdx.y of K into slice blockIdx.y of the unscaled partials C.
// AEXP (FP32 A, at most 16 rows): A's row exponents are derived in the kernel instead of read from ea.
// ALDS (FP32 A, at most 16 rows, 2 M (ceil(K / 8) + 1) 16-byte chunks of dynamic LDS): the workgroup splits all of
// A once into FP16 hi and lo planes in LDS, with the same operations as split8, and the K loop reads its A
// fragments from there.  The loop then carries no split arithmetic between a wait for B and the next B loads,
// which otherwise leaves the wavefront with one group of B in flight for as long as the split takes.
template <int PART, int MT, int NC, bool ALO, bool BLO, bool AF32 = false, bool SPLITK = false, bool AEXP = false,
          bool ALDS = false>
__global__ __launch_bounds__(64 * kSkWaves) void gemm_skinny_kernel(
    int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ ah, const uint16_t* __restrict__ al,
    const int32_t* __restrict__ ea, int64_t lda, const uint16_t* __restrict__ bh,
    const uint16_t* __restrict__ bl, const int32_t* __restrict__ eb, int64_t ldb, float* __restrict__ C,
    int64_t ldc, const float* __restrict__ af = nullptr, int64_t kslice = 0) {
  static_assert(!AF32 || (ALO && PART == HEAL_F16), "FP32 A: FP16 parts, both A parts");
  static_assert(!SPLITK || !AF32 || (MT == 1 && !AEXP && !ALDS),
                "split K with FP32 A: at most 16 rows, given exponents, A split per step");
  static_assert(!ALDS || (AF32 && MT == 1), "A split into LDS: FP32 A, at most 16 rows");
  // SPLITK: this workgroup's slice [k0, k0 + kslice) of K; the partial goes to slice blockIdx.y of C (rows of
  // ldc floats) without exponents, which the reduction applies.  FP32 A keeps ea: it prescales the split.
  if constexpr (SPLITK) {
    const int64_t k0 = (int64_t)blockIdx.y * kslice;
    K = K - k0 < kslice ? K - k0 : kslice;
    if constexpr (AF32) {
      af += k0;
    } else {
      ah += k0;
      if constexpr (ALO) al += k0;
    }
    bh += k0;
    if constexpr (BLO) bl += k0;
    C += (int64_t)blockIdx.y * M * ldc;
    eb = nullptr;
  }
  __shared__ float red[kSkWaves][MT * NC][4][64];
  extern __shared__ uint4 a_lds[];  // ALDS: hi plane [M][Kc + 1] then lo plane, Kc = ceil(K / 8) chunks
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cl = lane & 15, kg = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * NC;
  // The exponents the epilogue applies (wavefront 0: this workgroup's rows, 1: its columns) are requested now and
  // kept in a register through the main loop, so their latency overlaps it instead of closing the kernel.  The
  // branch is on the wavefront index (uniform), and every lane loads an in-range element.
  __shared__ int exp_s[2][64];
  int exp_pre = 0;
  {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    if (wv == 0) {
      if (!AEXP && !SPLITK && ea) exp_pre = ea[lane < M ? lane : M - 1];
    } else if (wv == 1) {
      if (eb) exp_pre = eb[n0 + lane < N ? n0 + lane : N - 1];
    }
  }
  // AEXP: e = 14 - ilogb(max_k |a[m, k]|) for each row (0 for a row without a nonzero value), the value
  // heal_row_exponents writes (a maximum is exact in any order).  The 512 threads stride over each row in
  // float4 chunks and the wavefront maxima meet in LDS.  Every workgroup reads all of A for this once more
  // (16 KB per row at K = 4096, from L2), in place of a launch of its own before the GEMM.
  __shared__ float amax_s[AEXP ? kSkWaves : 1][16];
  __shared__ int aexp_s[AEXP ? 16 : 1];
  static_assert(!AEXP || (AF32 && MT == 1 && !SPLITK), "derived row exponents: FP32 A, at most 16 rows");
  if constexpr (AEXP && !ALDS) {
    const int64_t nch = K >> 2;
    for (int r = 0; r < M; ++r) {
      const float* xr = af + r * lda;
      float m = 0.0f;
      for (int64_t j = threadIdx.x; j < nch; j += 64 * kSkWaves) {
        const float4 v = *reinterpret_cast<const float4*>(xr + 4 * j);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
      }
      for (int64_t k = 4 * nch + threadIdx.x; k < K; k += 64 * kSkWaves) m = fmaxf(m, fabsf(xr[k]));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      if (lane == 0) amax_s[wave][r] = m;
    }
    __syncthreads();
    if (threadIdx.x < M) {
      float m = 0.0f;
#pragma unroll
      for (int w = 0; w < kSkWaves; ++w) m = fmaxf(m, amax_s[w][threadIdx.x]);
      aexp_s[threadIdx.x] = m > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(m) : 0;  // 14 - ilogb(m)
    }
    __syncthreads();
  }
  const uint16_t* brow[NC];
  const uint16_t* blrow[NC];
#pragma unroll
  for (int nc = 0; nc < NC; ++nc) {
    int64_t n = n0 + 16 * nc + cl;
    if (n > N - 1) n = N - 1;  // columns past N feed outputs that are never stored
    brow[nc] = bh + n * ldb;
    blrow[nc] = BLO ? bl + n * ldb : nullptr;
  }
  const uint16_t* arow[MT];
  const uint16_t* alrow[MT];
  const float* afrow[MT];
  int ea_l[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int64_t m = 16 * mt + cl;
    if (m > M - 1) m = M - 1;
    if constexpr (AF32) {
      afrow[mt] = af + m * lda;
      if constexpr (AEXP)
        ea_l[mt] = aexp_s[m];
      else
        ea_l[mt] = ea[m];
    } else {
      arow[mt] = ah + m * lda;
      alrow[mt] = ALO ? al + m * lda : nullptr;
    }
  }
  const int64_t nsteps = (K + 31) / 32, nfull = K / 32;
  const int64_t klast = ((K + 7) / 8 - 1) * 8;
  const int64_t s0 = nsteps * wave / kSkWaves, s1 = nsteps * (wave + 1) / kSkWaves;
  // ALDS: chunk c (8 values from column 8 c) of row r of A's hi plane at a_lds[r * rs + c], of its lo plane at
  // a_lds[M * rs + r * rs + c], c < Kc; the row stride rs = Kc + 1 chunks puts the 16 rows a fragment read
  // touches in distinct banks.  Columns at or past K in the last chunk hold zeros; the partial last K step
  // reads no chunk at or past Kc.
  const int64_t Kc = (K + 7) / 8, rs = Kc + 1;
  // ALDS: the first group of B is requested before A is touched (it does not depend on A), then A is read
  // once into registers (at most 4 chunks of 8 values per thread: M (Kc + 1) <= 2048), the row maxima meet in
  // LDS by integer max on the magnitudes' bit patterns (order-free, so the same value on every run), and the
  // chunks are split from the registers into the LDS planes.
  constexpr int U0 = (MT * NC) >= 4 ? 1 : 4 / (MT * NC);
  uint4 b_first[U0][NC], bl_first[U0][BLO ? NC : 1];
  const bool first_full = s0 + U0 <= (s1 < nfull ? s1 : nfull);
  if constexpr (ALDS) {
    if (first_full) {
#pragma unroll
      for (int u = 0; u < U0; ++u)
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) {
          const int64_t k = (s0 + u) * 32 + 8 * kg;
          b_first[u][nc] = load_chunk(brow[nc], k, klast);
          if constexpr (BLO) bl_first[u][nc] = load_chunk(blrow[nc], k, klast);
        }
    }
    __shared__ uint32_t amax_u[ALDS && AEXP ? 16 : 1];
    if constexpr (AEXP) {
      if (threadIdx.x < 16) amax_u[threadIdx.x] = 0u;
    }
    constexpr int CPT = 2048 / (64 * kSkWaves);
    uint4 x0[CPT], x1[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t idx = threadIdx.x + 64 * kSkWaves * i;
      x0[i] = x1[i] = make_uint4(0u, 0u, 0u, 0u);
      if (idx < M * Kc) {
        const int64_t r = idx / Kc, k = 8 * (idx - r * Kc);
        const float* xr = af + r * lda;
        if (k + 8 <= K) {
          x0[i] = *reinterpret_cast<const uint4*>(xr + k);
          x1[i] = *reinterpret_cast<const uint4*>(xr + k + 4);
        } else {
          uint32_t w[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = k + j < K ? __builtin_bit_cast(uint32_t, xr[k + j]) : 0u;
          x0[i] = make_uint4(w[0], w[1], w[2], w[3]);
          x1[i] = make_uint4(w[4], w[5], w[6], w[7]);
        }
      }
    }
    if constexpr (AEXP) {
      __syncthreads();  // amax_u cleared
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int64_t idx = threadIdx.x + 64 * kSkWaves * i;
        if (idx < M * Kc) {
          // magnitudes' bit patterns: the integer order of non-negative floats is their numeric order
          const uint32_t w[8] = {x0[i].x, x0[i].y, x0[i].z, x0[i].w, x1[i].x, x1[i].y, x1[i].z, x1[i].w};
          uint32_t m = 0u;
#pragma unroll
          for (int j = 0; j < 8; ++j) m = max(m, w[j] & 0x7FFFFFFFu);
          atomicMax(&amax_u[idx / Kc], m);
        }
      }
      __syncthreads();
      if (threadIdx.x < M) {
        const float m = __builtin_bit_cast(float, amax_u[threadIdx.x]);
        aexp_s[threadIdx.x] = m > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(m) : 0;  // 14 - ilogb(m)
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t idx = threadIdx.x + 64 * kSkWaves * i;
      if (idx < M * Kc) {
        const int64_t r = idx / Kc, c = idx - r * Kc;
        int e;
        if constexpr (AEXP)
          e = aexp_s[r];
        else
          e = ea[r];
        const Split8 sp = split8(x0[i], x1[i], e);
        a_lds[r * rs + c] = sp.hi;
        a_lds[M * rs + r * rs + c] = sp.lo;
      }
    }
    __syncthreads();
  }
  const int64_t a_row_lds = (int64_t)(cl < M ? cl : M - 1) * rs;  // ALDS: this lane's A row
  f32x4 acc[MT][NC];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nc = 0; nc < NC; ++nc) acc[mt][nc] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma1 = [&](const uint4 (&a_in)[MT], const uint4 (&a2_in)[ALO ? MT : 1], const uint4 (&b)[NC],
                  const uint4 (&b2)[BLO ? NC : 1]) {
    uint4 a[MT], a2[ALO ? MT : 1];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (AF32 && !ALDS) {
        const Split8 sp = split8(a_in[mt], a2_in[mt], ea_l[mt]);  // raw FP32 bits -> hi, lo
        a[mt] = sp.hi;
        a2[mt] = sp.lo;
      } else {
        a[mt] = a_in[mt];
        if constexpr (ALO) a2[mt] = a2_in[mt];
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) {
        acc[mt][nc] = mfma16<PART>(a[mt], b[nc], acc[mt][nc]);
        if constexpr (BLO) acc[mt][nc] = mfma16<PART>(a[mt], b2[nc], acc[mt][nc]);
        if constexpr (ALO) acc[mt][nc] = mfma16<PART>(a2[mt], b[nc], acc[mt][nc]);
      }
  };
  // FP32 A: the 8 values of row afrow[mt] from column k, as raw bits (all in bounds for a full step)
  struct Raw8 {
    uint4 x0, x1;
  };
  auto load_af = [&](int mt, int64_t k) -> Raw8 {
    return Raw8{*reinterpret_cast<const uint4*>(afrow[mt] + k), *reinterpret_cast<const uint4*>(afrow[mt] + k + 4)};
  };
  // the same for the partial last step, the columns at or past K cleared (and never read)
  auto load_af_tail = [&](int mt, int64_t k) -> Raw8 {
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t kk = k + j;
      const float v = afrow[mt][kk < K ? kk : K - 1];
      w[j] = kk < K ? __builtin_bit_cast(uint32_t, v) : 0u;
    }
    return Raw8{make_uint4(w[0], w[1], w[2], w[3]), make_uint4(w[4], w[5], w[6], w[7])};
  };
  // one K step with the columns at or past K cleared (the partial last step; padding past K may hold any
  // bits, even NaN patterns, so both operands are cleared)
  auto tail_step = [&](int64_t s) {
    const int64_t k = s * 32 + 8 * kg;
    uint4 a[MT], a2[ALO ? MT : 1], b[NC], b2[BLO ? NC : 1];
#pragma unroll
    for (int nc = 0; nc < NC; ++nc) {
      b[nc] = mask_chunk(load_chunk(brow[nc], k, klast), K - k);
      if constexpr (BLO) b2[nc] = mask_chunk(load_chunk(blrow[nc], k, klast), K - k);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (ALDS) {  // the split parts; a chunk wholly past K reads the last one, cleared like B's
        const int64_t c = (k >> 3) < Kc ? (k >> 3) : Kc - 1;
        a[mt] = mask_chunk(a_lds[a_row_lds + c], K - k);
        a2[mt] = mask_chunk(a_lds[M * rs + a_row_lds + c], K - k);
      } else if constexpr (AF32) {
        const Raw8 r = load_af_tail(mt, k);
        a[mt] = r.x0;
        a2[mt] = r.x1;
      } else {
        a[mt] = mask_chunk(load_chunk(arow[mt], k, klast), K - k);
        if constexpr (ALO) a2[mt] = mask_chunk(load_chunk(alrow[mt], k, klast), K - k);
      }
    }
    mma1(a, a2, b, b2);
  };
  const int64_t s1f = s1 < nfull ? s1 : nfull;
  // Full steps in groups of U, software-pipelined through registers: the next group's loads are issued
  // before the current group's MFMAs, so two groups of B (the HBM stream) are in flight per wavefront.  The
  // prefetch address is clamped to the last full group instead of branching (a conditional load block
  // makes the compiler wait for every outstanding load at its boundary).
  constexpr int U = U0;
  struct Grp {
    uint4 b[U][NC], b2[U][BLO ? NC : 1], a[U][MT], a2[U][ALO ? MT : 1];
  };
  auto load = [&](Grp& g, int64_t s) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (s + u) * 32 + 8 * kg;
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) {
        g.b[u][nc] = load_chunk(brow[nc], k, klast);
        if constexpr (BLO) g.b2[u][nc] = load_chunk(blrow[nc], k, klast);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (ALDS) {
          g.a[u][mt] = a_lds[a_row_lds + (k >> 3)];
          g.a2[u][mt] = a_lds[M * rs + a_row_lds + (k >> 3)];
        } else if constexpr (AF32) {
          const Raw8 r = load_af(mt, k);
          g.a[u][mt] = r.x0;
          g.a2[u][mt] = r.x1;
        } else {
          g.a[u][mt] = load_chunk(arow[mt], k, klast);
          if constexpr (ALO) g.a2[u][mt] = load_chunk(alrow[mt], k, klast);
        }
      }
    }
  };
  auto mma = [&](const Grp& g) {
#pragma unroll
    for (int u = 0; u < U; ++u) mma1(g.a[u], g.a2[u], g.b[u], g.b2[u]);
  };
  // ALDS: the A fragments of a group from the LDS planes (its B already requested)
  auto load_a_lds = [&](Grp& g, int64_t s) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (s + u) * 32 + 8 * kg;
      g.a[u][0] = a_lds[a_row_lds + (k >> 3)];
      g.a2[u][0] = a_lds[M * rs + a_row_lds + (k >> 3)];
    }
  };
  const int64_t ng = s1f > s0 ? (s1f - s0) / U : 0;  // full groups of this wavefront
  const int64_t s_last = s0 + (ng - 1) * U;           // first step of the last full group
  if (ng > 0) {
    Grp g0, g1;
    if constexpr (ALDS) {  // the first group's B was requested before A's split
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) {
          g0.b[u][nc] = b_first[u][nc];
          if constexpr (BLO) g0.b2[u][nc] = bl_first[u][nc];
        }
      load_a_lds(g0, s0);
    } else {
      load(g0, s0);
    }
    int64_t gi = 0;
    for (; gi + 1 < ng; gi += 2) {
      load(g1, s0 + (gi + 1) * U);
      mma(g0);
      const int64_t sn = s0 + (gi + 2) * U;
      load(g0, sn < s_last ? sn : s_last);  // past the end: a re-read of the last group, never used
      mma(g1);
    }
    if (gi < ng) mma(g0);
  }
  for (int64_t s = s0 + ng * U; s < s1f; ++s) {  // fewer than U full steps left
    Grp g;
    load(g, s);
    mma1(g.a[0], g.a2[0], g.b[0], g.b2[0]);
  }
  if (s1 > s1f) tail_step(s1f);  // the one partial step (K % 32 != 0) belongs to the last wavefront
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nc = 0; nc < NC; ++nc)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][mt * NC + nc][i][lane] = acc[mt][nc][i];
  if (wave < 2) exp_s[wave][lane] = exp_pre;
  __syncthreads();
  for (int idx = threadIdx.x; idx < MT * NC * 4 * 64; idx += 64 * kSkWaves) {
    const int blk = idx >> 8, i = (idx >> 6) & 3, l = idx & 63;
    const int mt = blk / NC, nc = blk % NC;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) s += red[w][blk][i][l];
    const int64_t row = 16 * mt + 4 * (l >> 4) + i, col = n0 + 16 * nc + (l & 15);
    if (row < M && col < N) {
      int e = exp_s[1][16 * nc + (l & 15)];
      if constexpr (AEXP)
        e += aexp_s[row];
      else
        e += exp_s[0][row];
      C[row * ldc + col] = __builtin_amdgcn_ldexpf(s, -e);
    }
  }
}

// ------------------------------------------------------------------------------------------- streamed B, M <= 16
// At most 16 rows whose split parts fit in LDS.  A persistent workgroup (one per CU) holds all of A's hi and lo
// planes in LDS (split there from FP32 with the split pass's operations, or copied from the parts) and then walks
// its column blocks of 16 outputs (blocks x, x + G, x + 2 G, ... for a grid of G): it streams the block's 16 rows
// of B through a ring of D stages per wavefront by direct-to-LDS transfers, so D x 4 KB per wavefront are in
// flight with no registers held for them, and the ring runs on from one block into the next.  A stage is 128 of
// K: four 1 KB transfers, each 4 rows x 256 contiguous bytes (whole 128-byte lines, where the register-prefetch
// kernel reads 16 rows x 64 bytes per instruction).  Row r's 16-byte chunk c lands in slot c ^ r of that row, so
// the fragment reads of v_mfma_f32_16x16x32 (16 rows, one chunk each, per group of 16 lanes) hit 16 distinct bank
// groups.  Wavefront w takes the contiguous stages [ns w / W, ns (w + 1) / W) of each block and accumulates them
// in order; the partial blocks are added in wavefront order through LDS.  The same bits on every run.
// ASRC: 0 = 16-bit parts (ah, al; exponents ea or none), 1 = FP32 rows af with exponents ea, 2 = FP32 rows af
// with the exponents derived here (e = 14 - ilogb(max |a|), the value heal_row_exponents writes).
constexpr int kStK = 128;       // K per stage
constexpr int kStACap = 3840;   // 16-byte chunks of A's planes in LDS (60 KB)
constexpr int kStMaxBlk = 8;    // column blocks per workgroup, at most

// LDS row stride of A's planes, in 16-byte chunks: odd, so the 16 rows of a fragment read fall in distinct bank
// groups
__host__ __device__ constexpr int64_t stream_rs(int64_t K) { return ((K + 7) / 8 + 1) | 1; }

template <int PART, int W, int D, int ACAP, bool ALO, bool BLO, int ASRC>
__global__ __launch_bounds__(64 * W) void gemm_stream_kernel(
    int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ ah, const uint16_t* __restrict__ al,
    const float* __restrict__ af, const int32_t* __restrict__ ea, int64_t lda, const uint16_t* __restrict__ bh,
    const uint16_t* __restrict__ bl, const int32_t* __restrict__ eb, int64_t ldb, float* __restrict__ C,
    int64_t ldc) {
  static_assert(D >= 2 && D <= 8, "two to eight stages per wavefront");
  static_assert(W == 4, "the block epilogue gives each of the 256 threads one of the 4 x 64 outputs");
  static_assert(ASRC == 0 || (ALO && PART == HEAL_F16), "FP32 A: FP16 parts, both A parts");
  constexpr int NBP = BLO ? 2 : 1;  // B planes
  constexpr int SLOT = NBP * 256;   // 16-byte chunks of one wavefront's stage
  constexpr int NBI = NBP * 4;      // transfers per stage
  static_assert((D - 1) * NBI < 64, "vmcnt range");
  __shared__ uint4 st0[W * SLOT];
  __shared__ uint4 st1[W * SLOT];
  __shared__ uint4 st2[D > 2 ? W * SLOT : 1];
  __shared__ uint4 st3[D > 3 ? W * SLOT : 1];
  __shared__ uint4 st4[D > 4 ? W * SLOT : 1];
  __shared__ uint4 st5[D > 5 ? W * SLOT : 1];
  __shared__ uint4 st6[D > 6 ? W * SLOT : 1];
  __shared__ uint4 st7[D > 7 ? W * SLOT : 1];
  // the wavefronts' partial blocks, kept until the ring has drained (an LDS read of them while transfers are in
  // flight makes the compiler wait for all of them); the W partials of an output side by side
  __shared__ float4 red[kStMaxBlk][4][64];
  __shared__ uint32_t amax_u[16];
  __shared__ int aexp_s[16];               // A's row exponents
  __shared__ int eb_s[kStMaxBlk * 16];     // B's column exponents of this workgroup's blocks
  // A's hi plane [M][rs], then (ALO) its lo plane.  A static array: the compiler cannot tell dynamic LDS from the
  // stage slots, and would then wait for every transfer in flight before each A fragment read.
  __shared__ uint4 a_pl[ACAP];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
  const int cl = lane & 15, kg = lane >> 4;
  const int64_t nblk = (N + 15) / 16, G = gridDim.x;
  const int Q = (int)((nblk - blockIdx.x + G - 1) / G);  // this workgroup's blocks: blockIdx.x + q G, q < Q
  const int64_t Kc = (K + 7) / 8, rs = stream_rs(K), klast = (Kc - 1) * 8;
  const int64_t ns = (K + kStK - 1) / kStK;  // at least W (the launcher's condition), so T >= 1
  const int sbase = (int)(ns * wave / W), T = (int)(ns * (wave + 1) / W) - sbase;
  const int U = Q * T;  // this wavefront's stages over all its blocks
  auto blk = [&](int q) { return (int64_t)blockIdx.x + q * G; };
  // Every workgroup starts its walks at its own place in K (stage index rotated by ns x / G): at any moment the
  // workgroups read spread-out columns of their rows instead of the same ones.
  const int rot = (int)(ns * (int64_t)blockIdx.x / G);
  // a place in the wavefront's sequence of stages: stage t of its share of block q
  struct Pos {
    int q, t;
  };
  auto advance = [&](Pos& p) {
    if (++p.t == T) {
      p.t = 0;
      ++p.q;
    }
  };
  auto pos_k0 = [&](const Pos& p) -> int64_t {
    int st = sbase + p.t + rot;
    if (st >= (int)ns) st -= (int)ns;
    return (int64_t)st * kStK;
  };

  // transfer i of a stage carries rows 4 i + (lane >> 4) of the block; the lane's chunk is (lane & 15) ^ row
  const uint16_t* ibh[4];
  const uint16_t* ibl[BLO ? 4 : 1];
  int tch[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tch[i] = (lane & 15) ^ (4 * i + (lane >> 4));
  auto set_rows = [&](int q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t n = 16 * blk(q) + 4 * i + (lane >> 4);
      if (n > N - 1) n = N - 1;  // rows past N feed outputs that are never stored
      ibh[i] = bh + n * ldb;
      if constexpr (BLO) ibl[i] = bl + n * ldb;
    }
  };
  Pos pi{0, 0};  // the next stage to request
  auto issue = [&](uint4* slot) {
    if (pi.t == 0) set_rows(pi.q);
    const int64_t k0 = pos_k0(pi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t k = k0 + 8 * tch[i];
      if (k > klast) k = klast;  // a partial last stage: in-row chunks, cleared when read
      dma16<kNT>(ibh[i] + k, slot + wave * SLOT + i * 64);
      if constexpr (BLO) dma16<kNT>(ibl[i] + k, slot + wave * SLOT + 256 + i * 64);
    }
    advance(pi);
  };
  // the first stages do not depend on A: request them before A is split
  if (U > 0) issue(st0);
  if (U > 1) issue(st1);
  if constexpr (D > 2) {
    if (U > 2) issue(st2);
  }
  if constexpr (D > 3) {
    if (U > 3) issue(st3);
  }
  if constexpr (D > 4) {
    if (U > 4) issue(st4);
  }
  if constexpr (D > 5) {
    if (U > 5) issue(st5);
  }
  if constexpr (D > 6) {
    if (U > 6) issue(st6);
  }
  if constexpr (D > 7) {
    if (U > 7) issue(st7);
  }
  // the exponents the block epilogues apply, into LDS (a global load there would wait for the whole ring)
  for (int idx = threadIdx.x; idx < Q * 16; idx += 64 * W) {
    const int64_t col = 16 * blk(idx >> 4) + (idx & 15);
    eb_s[idx] = (eb && col < N) ? eb[col] : 0;
  }
  if constexpr (ASRC != 2) {
    if (threadIdx.x < M) aexp_s[threadIdx.x] = ea ? ea[threadIdx.x] : 0;
  }

  // ---- A into LDS: 8 values (one 16-byte chunk of each plane) per item, M x Kc items ----
  // A thread's items (at most CPT) are all requested before any is used, so the prologue waits for memory once:
  // the loads are branch-free (an item past the end reads item 0, and is dropped), since a load inside a divergent
  // branch makes the compiler wait for it where the branches meet.
  const int64_t items = M * Kc;
  constexpr int CPT = ((ALO ? ACAP / 2 : ACAP) + 64 * W - 1) / (64 * W);
  if constexpr (ASRC == 0) {
    uint4 h[CPT], l[ALO ? CPT : 1];
    if (items > 0) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        int64_t idx = threadIdx.x + 64 * W * i;
        if (idx >= items) idx = 0;
        const int64_t r = idx / Kc, c = idx - r * Kc;
        h[i] = *reinterpret_cast<const uint4*>(ah + r * lda + 8 * c);
        if constexpr (ALO) l[i] = *reinterpret_cast<const uint4*>(al + r * lda + 8 * c);
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t idx = threadIdx.x + 64 * W * i;
      if (idx < items) {
        const int64_t r = idx / Kc, c = idx - r * Kc;
        a_pl[r * rs + c] = mask_chunk(h[i], K - 8 * c);
        if constexpr (ALO) a_pl[M * rs + r * rs + c] = mask_chunk(l[i], K - 8 * c);
      }
    }
  } else {
    uint4 x0[CPT], x1[CPT];
    if (K % 8 == 0) {  // whole 8-value chunks (K >= 8 when there are items)
      if (items > 0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          int64_t idx = threadIdx.x + 64 * W * i;
          if (idx >= items) idx = 0;
          const int64_t r = idx / Kc, k = 8 * (idx - r * Kc);
          x0[i] = *reinterpret_cast<const uint4*>(af + r * lda + k);
          x1[i] = *reinterpret_cast<const uint4*>(af + r * lda + k + 4);
        }
      }
    } else {  // a partial last chunk in every row: value by value, columns clamped into the row, zeros past K
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        int64_t idx = threadIdx.x + 64 * W * i;
        if (idx >= items) idx = 0;
        const int64_t r = idx / Kc, k = 8 * (idx - r * Kc);
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t v = __builtin_bit_cast(uint32_t, af[r * lda + (k + j < K ? k + j : K - 1)]);
          w[j] = k + j < K ? v : 0u;
        }
        x0[i] = make_uint4(w[0], w[1], w[2], w[3]);
        x1[i] = make_uint4(w[4], w[5], w[6], w[7]);
      }
    }
    if constexpr (ASRC == 2) {
      if (threadIdx.x < 16) amax_u[threadIdx.x] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int64_t idx = threadIdx.x + 64 * W * i;
        if (idx < items) {
          // magnitudes' bit patterns: the integer order of non-negative floats is their numeric order, and a
          // maximum is the same in any order
          const uint32_t w[8] = {x0[i].x, x0[i].y, x0[i].z, x0[i].w, x1[i].x, x1[i].y, x1[i].z, x1[i].w};
          uint32_t m = 0u;
#pragma unroll
          for (int j = 0; j < 8; ++j) m = max(m, w[j] & 0x7FFFFFFFu);
          atomicMax(&amax_u[idx / Kc], m);
        }
      }
      __syncthreads();
      if (threadIdx.x < M) {
        const float m = __builtin_bit_cast(float, amax_u[threadIdx.x]);
        aexp_s[threadIdx.x] = m > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(m) : 0;  // 14 - ilogb(m)
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t idx = threadIdx.x + 64 * W * i;
      if (idx < items) {
        const int64_t r = idx / Kc, c = idx - r * Kc;
        const Split8 sp = split8(x0[i], x1[i], ASRC == 2 ? aexp_s[r] : ea[r]);
        a_pl[r * rs + c] = sp.hi;
        a_pl[M * rs + r * rs + c] = sp.lo;
      }
    }
  }
  __syncthreads();

  // ---- the stream: wait for stage u, read its fragments, refill its slot with stage u + D, multiply ----
  const int64_t a_row = (int64_t)(cl < M ? cl : M - 1) * rs;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  // block q done by this wavefront: its partial block into LDS
  auto finish = [&](int q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) reinterpret_cast<float*>(&red[q][i][lane])[wave] = acc[i];
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // LATER: stages issued after this one that may still be in flight (the wait leaves them outstanding); REFILL:
  // request the next stage into the slot.  In the steady state both are fixed (D - 1, true), so the compiler sees
  // the same outstanding transfers on every pass and places no wait of its own before the fragment reads.
  Pos ps{0, 0};  // the stage to multiply
  auto step = [&](uint4* slot, auto later_c, bool refill) {
    constexpr int LATER = decltype(later_c)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm<LATER * NBI>());
    const int64_t k0 = pos_k0(ps);
    const uint4* sb = slot + wave * SLOT + cl * 16;
    uint4 b[4][NBP], a[4], a2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = 4 * j + kg;
#pragma unroll
      for (int p = 0; p < NBP; ++p) b[j][p] = sb[p * 256 + (ch ^ cl)];
      int64_t c = k0 / 8 + ch;
      if (c > Kc - 1) c = Kc - 1;  // wholly past K: cleared below
      a[j] = a_pl[a_row + c];
      if constexpr (ALO) a2[j] = a_pl[M * rs + a_row + c];
    }
    if (k0 + kStK > K) {  // the partial last stage: clear both operands at and past K (padding may hold NaNs)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t valid = K - (k0 + 32 * j + 8 * kg);
#pragma unroll
        for (int p = 0; p < NBP; ++p) b[j][p] = mask_chunk(b[j][p], valid);
        a[j] = mask_chunk(a[j], valid);
        if constexpr (ALO) a2[j] = mask_chunk(a2[j], valid);
      }
    }
    // the fragments are in registers before the slot is refilled (the transfer writes LDS behind the reads)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
    if (refill) issue(slot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = mfma16<PART>(a[j], b[j][0], acc);
      if constexpr (BLO) acc = mfma16<PART>(a[j], b[j][1], acc);
      if constexpr (ALO) acc = mfma16<PART>(a2[j], b[j][0], acc);
    }
    if (ps.t == T - 1) finish(ps.q);
    advance(ps);
  };
  using L0 = std::integral_constant<int, 0>;
  using LD = std::integral_constant<int, D - 1>;
  int u = 0;
  // steady state: every step refills its slot, D - 1 later stages in flight
  for (; u + 2 * D <= U; u += D) {
    step(st0, LD{}, true);
    step(st1, LD{}, true);
    if constexpr (D > 2) step(st2, LD{}, true);
    if constexpr (D > 3) step(st3, LD{}, true);
    if constexpr (D > 4) step(st4, LD{}, true);
    if constexpr (D > 5) step(st5, LD{}, true);
    if constexpr (D > 6) step(st6, LD{}, true);
    if constexpr (D > 7) step(st7, LD{}, true);
  }
  // the last (fewer than 2 D) stages: refill while stages remain, and wait for everything issued (the first of
  // these steps finds the ring's last stages in flight and waits for them together)
  for (; u < U; ++u) {
    const bool refill = u + D < U;
    switch (u % D) {
      case 0: step(st0, L0{}, refill); break;
      case 1: step(st1, L0{}, refill); break;
      case 2: if constexpr (D > 2) step(st2, L0{}, refill); break;
      case 3: if constexpr (D > 3) step(st3, L0{}, refill); break;
      case 4: if constexpr (D > 4) step(st4, L0{}, refill); break;
      case 5: if constexpr (D > 5) step(st5, L0{}, refill); break;
      case 6: if constexpr (D > 6) step(st6, L0{}, refill); break;
      default: if constexpr (D > 7) step(st7, L0{}, refill); break;
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());  // no transfer may still write LDS when the workgroup ends

  // ---- each thread adds one output of every block over the wavefronts, in wavefront order ----
  __syncthreads();
  const int i = threadIdx.x >> 6;
  const int64_t row = 4 * (lane >> 4) + i;
  for (int q = 0; q < Q; ++q) {
    const float4 pw = red[q][i][lane];
    const float sum = (((0.0f + pw.x) + pw.y) + pw.z) + pw.w;
    const int64_t col = 16 * blk(q) + (lane & 15);
    if (row < M && col < N)
      C[row * ldc + col] = __builtin_amdgcn_ldexpf(sum, -(aexp_s[row] + eb_s[q * 16 + (lane & 15)]));
  }
}

// ------------------------------------------------------------------------- streamed B, K in slices, 8..16 rows
// Split K for at most 16 rows: workgroup (x, y) multiplies slice y of K ([y kslice, (y + 1) kslice)) for the
// column blocks x, x + G, ... and writes its FP32 sums unscaled into slice y of the partials (splitk_reduce_kernel
// adds the slices in order and applies the exponents).  The slice's A parts sit in LDS (from the 16-bit parts,
// or split there from FP32 with the split pass's operations and the given row exponents, so both sources give the
// same parts), and B streams through the same non-temporal direct-to-LDS ring as in gemm_stream_kernel.  Unlike
// there, each ring wavefront owns whole blocks (blocks q = w, w + 4, ... of the workgroup) and runs all of the
// slice's stages of one block before the next, keeping each block's sum in its own registers: no cross-wavefront
// reduction, so a workgroup can hold many blocks and the S x G grid stays near one workgroup per CU.
constexpr int kSkACap = 6016;  // 16-byte chunks of A's slice planes in LDS (94 KB)
constexpr int kSkMaxJ = 8;     // blocks per wavefront, at most (32 per workgroup)

template <int PART, int D, bool ALO, bool BLO, int ASRC>
__global__ __launch_bounds__(256) void gemm_stream_sk_kernel(
    int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ ah, const uint16_t* __restrict__ al,
    const float* __restrict__ af, const int32_t* __restrict__ ea, int64_t lda, const uint16_t* __restrict__ bh,
    const uint16_t* __restrict__ bl, int64_t ldb, float* __restrict__ C, int64_t ldc, int64_t kslice) {
  constexpr int W = 4;
  static_assert(D >= 2 && D <= 4, "two to four stages per wavefront");
  static_assert(ASRC == 0 || (ASRC == 1 && ALO && PART == HEAL_F16), "FP32 A: FP16 parts, both A parts");
  constexpr int NBP = BLO ? 2 : 1;
  constexpr int SLOT = NBP * 256;
  constexpr int NBI = NBP * 4;
  static_assert((D - 1) * NBI < 64, "vmcnt range");
  // this workgroup's slice
  {
    const int64_t k0 = (int64_t)blockIdx.y * kslice;
    K = K - k0 < kslice ? K - k0 : kslice;
    if constexpr (ASRC == 0) {
      ah += k0;
      if constexpr (ALO) al += k0;
    } else {
      af += k0;
    }
    bh += k0;
    if constexpr (BLO) bl += k0;
    C += (int64_t)blockIdx.y * M * ldc;
  }
  __shared__ uint4 st0[W * SLOT];
  __shared__ uint4 st1[W * SLOT];
  __shared__ uint4 st2[D > 2 ? W * SLOT : 1];
  __shared__ uint4 st3[D > 3 ? W * SLOT : 1];
  __shared__ uint4 a_pl[kSkACap];  // A's hi plane [M][rs], then (ALO) its lo plane
  __shared__ int aexp_s[16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cl = lane & 15, kg = lane >> 4;
  const int64_t nblk = (N + 15) / 16, G = gridDim.x;
  const int Q = (int)((nblk - blockIdx.x + G - 1) / G);  // this workgroup's blocks: blockIdx.x + q G
  const int Qw = Q > wave ? (Q - wave + W - 1) / W : 0;  // this wavefront's: q = wave + W j, j < Qw
  const int64_t Kc = (K + 7) / 8, rs = stream_rs(K), klast = (Kc - 1) * 8;
  const int ns = (int)((K + kStK - 1) / kStK);
  const int U = Qw * ns;
  auto blk = [&](int j) { return (int64_t)blockIdx.x + (int64_t)(wave + W * j) * G; };
  // every workgroup starts its walk of a block's stages at its own place (spread-out columns at any moment)
  const int rot = (int)((int64_t)ns * blockIdx.x / G);
  struct Pos {
    int j, t;
  };
  auto advance = [&](Pos& p) {
    if (++p.t == ns) {
      p.t = 0;
      ++p.j;
    }
  };
  auto pos_k0 = [&](const Pos& p) -> int64_t {
    int st = p.t + rot;
    if (st >= ns) st -= ns;
    return (int64_t)st * kStK;
  };
  const uint16_t* ibh[4];
  const uint16_t* ibl[BLO ? 4 : 1];
  int tch[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tch[i] = (lane & 15) ^ (4 * i + (lane >> 4));
  Pos pi{0, 0};
  auto issue = [&](uint4* slot) {
    if (pi.t == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t n = 16 * blk(pi.j) + 4 * i + (lane >> 4);
        if (n > N - 1) n = N - 1;  // rows past N feed outputs that are never stored
        ibh[i] = bh + n * ldb;
        if constexpr (BLO) ibl[i] = bl + n * ldb;
      }
    }
    const int64_t k0 = pos_k0(pi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t k = k0 + 8 * tch[i];
      if (k > klast) k = klast;  // a partial last stage: in-row chunks, cleared when read
      dma16<kNT>(ibh[i] + k, slot + wave * SLOT + i * 64);
      if constexpr (BLO) dma16<kNT>(ibl[i] + k, slot + wave * SLOT + 256 + i * 64);
    }
    advance(pi);
  };
  if (U > 0) issue(st0);
  if (U > 1) issue(st1);
  if constexpr (D > 2) {
    if (U > 2) issue(st2);
  }
  if constexpr (D > 3) {
    if (U > 3) issue(st3);
  }
  if constexpr (ASRC == 1) {
    if (threadIdx.x < M) aexp_s[threadIdx.x] = ea[threadIdx.x];
    __syncthreads();
  }

  // ---- the slice of A into LDS: 8 values (one 16-byte chunk of each plane) per item, M x Kc items, every item
  //      of a thread requested before any is used (branch-free: an item past the end reads item 0, dropped) ----
  const int64_t items = M * Kc;
  constexpr int CPT = ((ALO ? kSkACap / 2 : kSkACap) + 64 * W - 1) / (64 * W);
  if constexpr (ASRC == 0) {
    uint4 h[CPT], l[ALO ? CPT : 1];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      int64_t idx = threadIdx.x + 64 * W * i;
      if (idx >= items) idx = 0;
      const int64_t r = idx / Kc, c = idx - r * Kc;
      h[i] = *reinterpret_cast<const uint4*>(ah + r * lda + 8 * c);
      if constexpr (ALO) l[i] = *reinterpret_cast<const uint4*>(al + r * lda + 8 * c);
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t idx = threadIdx.x + 64 * W * i;
      if (idx < items) {
        const int64_t r = idx / Kc, c = idx - r * Kc;
        a_pl[r * rs + c] = mask_chunk(h[i], K - 8 * c);
        if constexpr (ALO) a_pl[M * rs + r * rs + c] = mask_chunk(l[i], K - 8 * c);
      }
    }
  } else {
    uint4 x0[CPT], x1[CPT];
    if (K % 8 == 0) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        int64_t idx = threadIdx.x + 64 * W * i;
        if (idx >= items) idx = 0;
        const int64_t r = idx / Kc, k = 8 * (idx - r * Kc);
        x0[i] = *reinterpret_cast<const uint4*>(af + r * lda + k);
        x1[i] = *reinterpret_cast<const uint4*>(af + r * lda + k + 4);
      }
    } else {  // a partial last chunk in every row: value by value, columns clamped into the slice, zeros past it
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        int64_t idx = threadIdx.x + 64 * W * i;
        if (idx >= items) idx = 0;
        const int64_t r = idx / Kc, k = 8 * (idx - r * Kc);
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t v = __builtin_bit_cast(uint32_t, af[r * lda + (k + j < K ? k + j : K - 1)]);
          w[j] = k + j < K ? v : 0u;
        }
        x0[i] = make_uint4(w[0], w[1], w[2], w[3]);
        x1[i] = make_uint4(w[4], w[5], w[6], w[7]);
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t idx = threadIdx.x + 64 * W * i;
      if (idx < items) {
        const int64_t r = idx / Kc, c = idx - r * Kc;
        const Split8 sp = split8(x0[i], x1[i], aexp_s[r]);
        a_pl[r * rs + c] = sp.hi;
        a_pl[M * rs + r * rs + c] = sp.lo;
      }
    }
  }
  __syncthreads();

  // ---- the ring: wait for stage u, read its fragments, refill its slot with stage u + D, multiply into the
  //      block's accumulator ----
  const int64_t a_row = (int64_t)(cl < M ? cl : M - 1) * rs;
  f32x4 acc[kSkMaxJ];
#pragma unroll
  for (int j = 0; j < kSkMaxJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  Pos ps{0, 0};
  auto step = [&](uint4* slot, auto later_c, bool refill) {
    constexpr int LATER = decltype(later_c)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm<LATER * NBI>());
    const int64_t k0 = pos_k0(ps);
    const uint4* sb = slot + wave * SLOT + cl * 16;
    uint4 b[4][NBP], a[4], a2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = 4 * j + kg;
#pragma unroll
      for (int p = 0; p < NBP; ++p) b[j][p] = sb[p * 256 + (ch ^ cl)];
      int64_t c = k0 / 8 + ch;
      if (c > Kc - 1) c = Kc - 1;  // wholly past K: cleared below
      a[j] = a_pl[a_row + c];
      if constexpr (ALO) a2[j] = a_pl[M * rs + a_row + c];
    }
    if (k0 + kStK > K) {  // the partial last stage: clear both operands at and past K (padding may hold NaNs)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t valid = K - (k0 + 32 * j + 8 * kg);
#pragma unroll
        for (int p = 0; p < NBP; ++p) b[j][p] = mask_chunk(b[j][p], valid);
        a[j] = mask_chunk(a[j], valid);
        if constexpr (ALO) a2[j] = mask_chunk(a2[j], valid);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // the fragments are in registers before the slot is refilled
    if (refill) issue(slot);
    auto mma = [&](f32x4& c) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c = mfma16<PART>(a[j], b[j][0], c);
        if constexpr (BLO) c = mfma16<PART>(a[j], b[j][1], c);
        if constexpr (ALO) c = mfma16<PART>(a2[j], b[j][0], c);
      }
    };
    switch (ps.j) {  // uniform: each block's accumulator stays a fixed set of registers
      case 0: mma(acc[0]); break;
      case 1: mma(acc[1]); break;
      case 2: mma(acc[2]); break;
      case 3: mma(acc[3]); break;
      case 4: mma(acc[4]); break;
      case 5: mma(acc[5]); break;
      case 6: mma(acc[6]); break;
      default: mma(acc[7]); break;
    }
    advance(ps);
  };
  static_assert(kSkMaxJ == 8, "one switch case per block");
  using L0 = std::integral_constant<int, 0>;
  using LD = std::integral_constant<int, D - 1>;
  int u = 0;
  for (; u + 2 * D <= U; u += D) {
    step(st0, LD{}, true);
    step(st1, LD{}, true);
    if constexpr (D > 2) step(st2, LD{}, true);
    if constexpr (D > 3) step(st3, LD{}, true);
  }
  for (; u < U; ++u) {
    const bool refill = u + D < U;
    switch (u % D) {
      case 0: step(st0, L0{}, refill); break;
      case 1: step(st1, L0{}, refill); break;
      case 2: if constexpr (D > 2) step(st2, L0{}, refill); break;
      default: if constexpr (D > 3) step(st3, L0{}, refill); break;
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());  // no transfer may still write LDS when the workgroup ends

  // ---- this wavefront's blocks: the unscaled sums into the slice's partials (row 4 (lane / 16) + i) ----
#pragma unroll
  for (int j = 0; j < kSkMaxJ; ++j) {
    if (j < Qw) {
      const int64_t col = 16 * blk(j) + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = 4 * (lane >> 4) + i;
        if (row < M && col < N) C[row * ldc + col] = acc[j][i];
      }
    }
  }
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || n < 1)
    return 256;
  return n;
}

// Launch shape of the streamed kernel: 4 wavefronts with 4 ring stages of 4 KB each (2 when B has a low part), so
// 64 KB in flight per CU, and one workgroup per CU (at most 8 column blocks each).  The ring's transfers are
// non-temporal (B is read once per launch): a 117 MB stream then takes 24.7 instead of 26.5 us (M = 1, N x K =
// 14336 x 4096), 41.9 instead of 46.0 us at 28672 x 4096.  It serves at most 16 rows where A's planes fit their
// 60 KB, K spans at least one stage per wavefront, every CU gets a column block, and the CUs' stages (column blocks
// x stages of 128 of K) come to at least 64 each: measured on MI355X against the register-prefetch kernel (M = 1,
// weights rotated through HBM, graph-replayed launches), 26.2 against 27.0 us at N x K = 4096 x 14336 (one block
// and 112 stages per CU), 17.2 against 17.6 us at 8192 x 4096 (64 stages), but 11.9 against 10.4 us at 4096 x 4096
// (32 stages: the ring barely fills before the block ends).  Six ring stages instead of four (A's planes in a
// smaller array, plain transfers) did not help (26.9 against 26.2 us at 14336 x 4096).  heal_gemm_comp and
// heal_gemm_comp_f32a take the same decision from (M, N, K, A's low part), so they keep giving the same bits.
constexpr int kStW = 4, kStD = 4, kStDLo = 2;

bool stream_fits(int64_t M, int64_t N, int64_t K, bool a_lo) {
  if (M < 1 || M > 16 || K < (int64_t)kStW * kStK - (kStK - 1)) return false;
  const int64_t nblk = (N + 15) / 16, cus = cu_count(), ns = (K + kStK - 1) / kStK;
  if (nblk < cus || nblk * ns < 64 * cus) return false;
  return (a_lo ? 2 : 1) * M * stream_rs(K) <= kStACap;
}

// ASRC as for gemm_stream_kernel; al / bl select the products
template <int PART, int ASRC>
hipError_t launch_stream(int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al, const float* af,
                         const int32_t* ea, int64_t lda, const uint16_t* bh, const uint16_t* bl, const int32_t* eb,
                         int64_t ldb, float* c, int64_t ldc, hipStream_t stream) {
  const int64_t nblk = (N + 15) / 16;
  int64_t wgs = cu_count();
  if (wgs > nblk) wgs = nblk;
  if (wgs < (nblk + kStMaxBlk - 1) / kStMaxBlk) wgs = (nblk + kStMaxBlk - 1) / kStMaxBlk;
  if (!grid_fits(wgs, 64 * kStW)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)wgs), block(64 * kStW);
  if constexpr (ASRC == 0) {
    if (al && bl)
      hipLaunchKernelGGL((gemm_stream_kernel<PART, kStW, kStDLo, kStACap, true, true, 0>), grid, block, 0, stream, M,
                         N, K, ah, al, af, ea, lda, bh, bl, eb, ldb, c, ldc);
    else if (al)
      hipLaunchKernelGGL((gemm_stream_kernel<PART, kStW, kStD, kStACap, true, false, 0>), grid, block, 0, stream, M,
                         N, K, ah, al, af, ea, lda, bh, bl, eb, ldb, c, ldc);
    else if (bl)
      hipLaunchKernelGGL((gemm_stream_kernel<PART, kStW, kStDLo, kStACap, false, true, 0>), grid, block, 0, stream, M,
                         N, K, ah, al, af, ea, lda, bh, bl, eb, ldb, c, ldc);
    else
      hipLaunchKernelGGL((gemm_stream_kernel<PART, kStW, kStD, kStACap, false, false, 0>), grid, block, 0, stream, M,
                         N, K, ah, al, af, ea, lda, bh, bl, eb, ldb, c, ldc);
  } else {
    if (bl)
      hipLaunchKernelGGL((gemm_stream_kernel<HEAL_F16, kStW, kStDLo, kStACap, true, true, ASRC>), grid, block, 0,
                         stream, M, N, K, ah, al, af, ea, lda, bh, bl, eb, ldb, c, ldc);
    else
      hipLaunchKernelGGL((gemm_stream_kernel<HEAL_F16, kStW, kStD, kStACap, true, false, ASRC>), grid, block, 0,
                         stream, M, N, K, ah, al, af, ea, lda, bh, bl, eb, ldb, c, ldc);
  }
  return hipGetLastError();
}

// Column blocks per skinny workgroup.  Each workgroup re-reads A (M x K) from L2, so more columns per
// workgroup save that traffic, but fewer workgroups keep fewer loads in flight.  Measured on MI355X at
// K = 4096 / 14336 (M = 1 .. 64; weights rotated through four copies, so read from HBM): N = 4096 runs
// best with 1 block (256 workgroups); N = 14336 with 2 blocks for M <= 4 (448 workgroups: M = 1 32.1 ->
// 30.0 us) and 4 above (224 workgroups: M = 16 44.1 -> 38.5 us, M = 32 59.9 -> 45.6 us, M = 64 149.3 ->
// 62.2 us).
int skinny_nc(int64_t M, int64_t N) {
  const int64_t cap = M <= 4 ? 2 : 4;
  int64_t nc = 1;
  while (nc < cap && N / (16 * 2 * nc) >= 224) nc *= 2;
  return (int)nc;
}

template <int PART, int MT, int NC>
hipError_t launch_skinny_nc(int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al,
                            const int32_t* ea, int64_t lda, const uint16_t* bh, const uint16_t* bl,
                            const int32_t* eb, int64_t ldb, float* c, int64_t ldc, hipStream_t stream) {
  if (!grid_fits((N + 16 * NC - 1) / (16 * NC), 64 * kSkWaves)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((N + 16 * NC - 1) / (16 * NC))), block(64 * kSkWaves);
  if (al && bl)
    hipLaunchKernelGGL((gemm_skinny_kernel<PART, MT, NC, true, true>), grid, block, 0, stream, M, N, K, ah, al,
                       ea, lda, bh, bl, eb, ldb, c, ldc);
  else if (al)
    hipLaunchKernelGGL((gemm_skinny_kernel<PART, MT, NC, true, false>), grid, block, 0, stream, M, N, K, ah, al,
                       ea, lda, bh, bl, eb, ldb, c, ldc);
  else if (bl)
    hipLaunchKernelGGL((gemm_skinny_kernel<PART, MT, NC, false, true>), grid, block, 0, stream, M, N, K, ah, al,
                       ea, lda, bh, bl, eb, ldb, c, ldc);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<PART, MT, NC, false, false>), grid, block, 0, stream, M, N, K, ah,
                       al, ea, lda, bh, bl, eb, ldb, c, ldc);
  return hipGetLastError();
}

template <int PART>
hipError_t launch_skinny(int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al,
                         const int32_t* ea, int64_t lda, const uint16_t* bh, const uint16_t* bl,
                         const int32_t* eb, int64_t ldb, float* c, int64_t ldc, hipStream_t stream) {
  if (stream_fits(M, N, K, al != nullptr))
    return launch_stream<PART, 0>(M, N, K, ah, al, nullptr, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  const int nc = skinny_nc(M, N);
  if (M <= 16) {
    if (nc >= 4) return launch_skinny_nc<PART, 1, 4>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    if (nc == 2) return launch_skinny_nc<PART, 1, 2>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    return launch_skinny_nc<PART, 1, 1>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  }
  if (M <= 32) {
    if (nc >= 4) return launch_skinny_nc<PART, 2, 4>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    if (nc == 2) return launch_skinny_nc<PART, 2, 2>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    return launch_skinny_nc<PART, 2, 1>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  }
  if (nc >= 4) return launch_skinny_nc<PART, 4, 4>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  if (nc == 2) return launch_skinny_nc<PART, 4, 2>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  return launch_skinny_nc<PART, 4, 1>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
}

template <int PART, int BM, int BN>
hipError_t launch_tile(int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al,
                       const int32_t* ea, int64_t lda, const uint16_t* bh, const uint16_t* bl,
                       const int32_t* eb, int64_t ldb, float* c, int64_t ldc, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (!grid_fits(tiles, kThreads)) return hipErrorInvalidConfiguration;
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

// Kernel choice: M <= 64 streams B (skinny kernel); otherwise the largest block tile that still gives
// every CU a workgroup.  Where A alone has a low part (two A tiles, one B tile per k step), a 128 x 256 tile
// takes the place of 256 x 128: the same tile count, but each wavefront reads 2 x 2 A and 4 B fragments per
// 16 MFMAs instead of 4 x 2 A and 2 B, so LDS reads fall from 10 to 8 fragments per 16 MFMAs.
constexpr int64_t kSkinnyMaxM = 64;
enum TileKind { kTile256x256 = 0, kTile256x128 = 1, kTile128x128 = 2, kSkinny = 3, kTile128x256 = 4 };
TileKind choose_tile(int64_t M, int64_t N, bool a_lo_only) {
  if (M <= kSkinnyMaxM) return kSkinny;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t128 = ((M + 255) / 256) * ((N + 127) / 128);
  const int64_t t128t = ((M + 127) / 128) * ((N + 255) / 256);
  if (t256 >= 256) return kTile256x256;
  if (a_lo_only && t128t >= 256) return kTile128x256;
  if (t128 >= 256) return kTile256x128;
  return kTile128x128;
}

// The 128 x 256 tile, instantiated for its one use: A with a low part, B without.
template <int PART, bool QUANT>
hipError_t launch_tile_128x256(int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al,
                               const int32_t* ea, int64_t lda, const uint16_t* bh, const int32_t* eb, int64_t ldb,
                               float* c, int64_t ldc, int16_t* q, int64_t ldq, float* s, int64_t ld_s,
                               hipStream_t stream) {
  const int64_t tiles = ((M + 127) / 128) * ((N + 255) / 256);
  if (!grid_fits(tiles, kThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((gemm_comp_kernel<PART, 128, 256, true, false, QUANT>), dim3((unsigned)tiles),
                     dim3(kThreads), 0, stream, M, N, K, ah, al, ea, lda, bh, (const uint16_t*)nullptr, eb, ldb, c,
                     ldc, q, ldq, s, ld_s);
  return hipGetLastError();
}

template <int PART>
hipError_t launch_part(int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al,
                       const int32_t* ea, int64_t lda, const uint16_t* bh, const uint16_t* bl,
                       const int32_t* eb, int64_t ldb, float* c, int64_t ldc, hipStream_t stream) {
  switch (choose_tile(M, N, al && !bl)) {
    case kSkinny:
      return launch_skinny<PART>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    case kTile256x256:
      return launch_tile<PART, 256, 256>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    case kTile128x256:
      return launch_tile_128x256<PART, false>(M, N, K, ah, al, ea, lda, bh, eb, ldb, c, ldc, nullptr, 0, nullptr,
                                              0, stream);
    case kTile256x128:
      return launch_tile<PART, 256, 128>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    default:
      return launch_tile<PART, 128, 128>(M, N, K, ah, al, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  }
}

}  // namespace

const char* gemm_comp_variant(int64_t M, int64_t N, int64_t K, int products) {
  static const char* names[4][3] = {
      {"gemm_comp_kernel 256x256 P1", "gemm_comp_kernel 256x256 P2", "gemm_comp_kernel 256x256 P3"},
      {"gemm_comp_kernel 256x128 P1", "gemm_comp_kernel 256x128 P2", "gemm_comp_kernel 256x128 P3"},
      {"gemm_comp_kernel 128x128 P1", "gemm_comp_kernel 128x128 P2", "gemm_comp_kernel 128x128 P3"},
      {"gemm_skinny_kernel P1", "gemm_skinny_kernel P2", "gemm_skinny_kernel P3"}};
  if (M <= 0 || N <= 0 || products < 1 || products > 3) return "none";
  const TileKind kind = choose_tile(M, N, products == 2);
  if (kind == kTile128x256) return "gemm_comp_kernel 128x256 P2";
  if (kind == kSkinny && stream_fits(M, N, K, products >= 2)) {
    static const char* st[3] = {"gemm_stream_kernel M<=16 P1", "gemm_stream_kernel M<=16 P2",
                                "gemm_stream_kernel M<=16 P3"};
    return st[products - 1];
  }
  if (kind == kSkinny) {
    // [rows class][column blocks 1, 2, 4][products]
    static const char* sk[3][3][3] = {
        {{"gemm_skinny_kernel M<=16 NC1 P1", "gemm_skinny_kernel M<=16 NC1 P2", "gemm_skinny_kernel M<=16 NC1 P3"},
         {"gemm_skinny_kernel M<=16 NC2 P1", "gemm_skinny_kernel M<=16 NC2 P2", "gemm_skinny_kernel M<=16 NC2 P3"},
         {"gemm_skinny_kernel M<=16 NC4 P1", "gemm_skinny_kernel M<=16 NC4 P2", "gemm_skinny_kernel M<=16 NC4 P3"}},
        {{"gemm_skinny_kernel M<=32 NC1 P1", "gemm_skinny_kernel M<=32 NC1 P2", "gemm_skinny_kernel M<=32 NC1 P3"},
         {"gemm_skinny_kernel M<=32 NC2 P1", "gemm_skinny_kernel M<=32 NC2 P2", "gemm_skinny_kernel M<=32 NC2 P3"},
         {"gemm_skinny_kernel M<=32 NC4 P1", "gemm_skinny_kernel M<=32 NC4 P2", "gemm_skinny_kernel M<=32 NC4 P3"}},
        {{"gemm_skinny_kernel M<=64 NC1 P1", "gemm_skinny_kernel M<=64 NC1 P2", "gemm_skinny_kernel M<=64 NC1 P3"},
         {"gemm_skinny_kernel M<=64 NC2 P1", "gemm_skinny_kernel M<=64 NC2 P2", "gemm_skinny_kernel M<=64 NC2 P3"},
         {"gemm_skinny_kernel M<=64 NC4 P1", "gemm_skinny_kernel M<=64 NC4 P2", "gemm_skinny_kernel M<=64 NC4 P3"}}};
    const int nc = skinny_nc(M, N);
    return sk[M <= 16 ? 0 : (M <= 32 ? 1 : 2)][nc == 4 ? 2 : nc - 1][products - 1];
  }
  return names[kind][products - 1];
}

template <int BM, int BN>
hipError_t launch_tile_quant(int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al,
                             const int32_t* ea, int64_t lda, const uint16_t* bh, const uint16_t* bl,
                             const int32_t* eb, int64_t ldb, int16_t* q, int64_t ldq, float* s, int64_t ld_s,
                             hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (!grid_fits(tiles, kThreads)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)tiles), block(kThreads);
  float* const c = nullptr;
  if (al && bl)
    hipLaunchKernelGGL((gemm_comp_kernel<HEAL_F16, BM, BN, true, true, true>), grid, block, 0, stream, M, N, K,
                       ah, al, ea, lda, bh, bl, eb, ldb, c, (int64_t)0, q, ldq, s, ld_s);
  else if (al)
    hipLaunchKernelGGL((gemm_comp_kernel<HEAL_F16, BM, BN, true, false, true>), grid, block, 0, stream, M, N, K,
                       ah, al, ea, lda, bh, bl, eb, ldb, c, (int64_t)0, q, ldq, s, ld_s);
  else if (bl)
    hipLaunchKernelGGL((gemm_comp_kernel<HEAL_F16, BM, BN, false, true, true>), grid, block, 0, stream, M, N, K,
                       ah, al, ea, lda, bh, bl, eb, ldb, c, (int64_t)0, q, ldq, s, ld_s);
  else
    hipLaunchKernelGGL((gemm_comp_kernel<HEAL_F16, BM, BN, false, false, true>), grid, block, 0, stream, M, N,
                       K, ah, al, ea, lda, bh, bl, eb, ldb, c, (int64_t)0, q, ldq, s, ld_s);
  return hipGetLastError();
}

hipError_t launch_gemm_comp_quant(int64_t M, int64_t N, int64_t K, const uint16_t* a_hi, const uint16_t* a_lo,
                                  const int32_t* a_exp, int64_t lda, const uint16_t* b_hi, const uint16_t* b_lo,
                                  const int32_t* b_exp, int64_t ldb, int16_t* q, int64_t ldq, float* s,
                                  int64_t ld_s, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  // the tile kernels only: a skinny workgroup holds fewer columns than a head
  switch (choose_tile(M, N, a_lo && !b_lo)) {
    case kTile128x256:
      return launch_tile_128x256<HEAL_F16, true>(M, N, K, a_hi, a_lo, a_exp, lda, b_hi, b_exp, ldb, nullptr, 0, q,
                                                 ldq, s, ld_s, stream);
    case kTile256x256:
      return launch_tile_quant<256, 256>(M, N, K, a_hi, a_lo, a_exp, lda, b_hi, b_lo, b_exp, ldb, q, ldq, s, ld_s,
                                         stream);
    case kTile256x128:
      return launch_tile_quant<256, 128>(M, N, K, a_hi, a_lo, a_exp, lda, b_hi, b_lo, b_exp, ldb, q, ldq, s, ld_s,
                                         stream);
    default:
      return launch_tile_quant<128, 128>(M, N, K, a_hi, a_lo, a_exp, lda, b_hi, b_lo, b_exp, ldb, q, ldq, s, ld_s,
                                         stream);
  }
}

namespace {

// FP32 A split in the GEMM: the same kernel choice as launch_gemm_comp (with both A parts), so both paths
// run the same MFMAs in the same accumulation order on the same operand bits.  (Every tile kernel sums an
// element over the same 16-wide k steps, with the same products per step in the same order, so the block
// tile does not change the result: the three-product 256 x 256 case, whose registers the in-register
// split does not fit, runs on 256 x 128 tiles with identical output.)
// BLO: whether this (MT, NC) is instantiated with B's low part; the wide 64-row ones are not (their
// registers would spill), and the dispatcher sends three-product calls at M > 32 to NC = 1.
// LDS bytes of A's split hi and lo planes for the ALDS skinny kernel, or 0 when they exceed 64 KB (the kernel
// then splits A at each step): M (<= 16) rows of ceil(K / 8) + 1 chunks of 16 bytes, two planes.
size_t skinny_alds_bytes(int64_t M, int64_t K) {
  if (M < 1 || M > 16) return 0;
  const int64_t b = 2 * M * ((K + 7) / 8 + 1) * 16;
  return b <= 65536 ? (size_t)b : 0;
}

// at most 16 rows: exponents given (AEXP false) or derived; A split per step, or once into LDS (ALDS)
template <int NC, bool BLO, bool AEXP>
hipError_t launch_skinny_f32a_m16(int64_t M, int64_t N, int64_t K, const float* af, const int32_t* ea, int64_t lda,
                                  const uint16_t* bh, const uint16_t* bl, const int32_t* eb, int64_t ldb, float* c,
                                  int64_t ldc, dim3 grid, dim3 block, hipStream_t stream) {
  const uint16_t* const none = nullptr;
  const size_t lds = skinny_alds_bytes(M, K);
  if (lds)
    hipLaunchKernelGGL((gemm_skinny_kernel<HEAL_F16, 1, NC, true, BLO, true, false, AEXP, true>), grid, block,
                       (unsigned)lds, stream, M, N, K, none, none, ea, lda, bh, bl, eb, ldb, c, ldc, af, (int64_t)0);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<HEAL_F16, 1, NC, true, BLO, true, false, AEXP, false>), grid, block, 0,
                       stream, M, N, K, none, none, ea, lda, bh, bl, eb, ldb, c, ldc, af, (int64_t)0);
  return hipGetLastError();
}

template <int MT, int NC, bool BLO = true>
hipError_t launch_skinny_f32a_nc(int64_t M, int64_t N, int64_t K, const float* af, const int32_t* ea, int64_t lda,
                                 const uint16_t* bh, const uint16_t* bl, const int32_t* eb, int64_t ldb, float* c,
                                 int64_t ldc, hipStream_t stream) {
  if (!grid_fits((N + 16 * NC - 1) / (16 * NC), 64 * kSkWaves)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((N + 16 * NC - 1) / (16 * NC))), block(64 * kSkWaves);
  const uint16_t* const none = nullptr;
  if constexpr (!BLO) {
    if (bl) return hipErrorInvalidValue;
  }
  if constexpr (MT == 1) {
    if (bl) {
      if constexpr (BLO) {
        return ea ? launch_skinny_f32a_m16<NC, true, false>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, grid, block,
                                                            stream)
                  : launch_skinny_f32a_m16<NC, true, true>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, grid, block,
                                                           stream);
      }
    }
    return ea ? launch_skinny_f32a_m16<NC, false, false>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, grid, block,
                                                         stream)
              : launch_skinny_f32a_m16<NC, false, true>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, grid, block,
                                                        stream);
  } else {
    if (!ea) return hipErrorInvalidValue;  // derived exponents: at most 16 rows
    if constexpr (BLO) {
      if (bl) {
        hipLaunchKernelGGL((gemm_skinny_kernel<HEAL_F16, MT, NC, true, true, true>), grid, block, 0, stream, M, N,
                           K, none, none, ea, lda, bh, bl, eb, ldb, c, ldc, af);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((gemm_skinny_kernel<HEAL_F16, MT, NC, true, false, true>), grid, block, 0, stream, M, N, K,
                       none, none, ea, lda, bh, bl, eb, ldb, c, ldc, af);
    return hipGetLastError();
  }
}

hipError_t launch_skinny_f32a(int64_t M, int64_t N, int64_t K, const float* af, const int32_t* ea, int64_t lda,
                              const uint16_t* bh, const uint16_t* bl, const int32_t* eb, int64_t ldb, float* c,
                              int64_t ldc, hipStream_t stream) {
  if (stream_fits(M, N, K, true))
    return ea ? launch_stream<HEAL_F16, 1>(M, N, K, nullptr, nullptr, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream)
              : launch_stream<HEAL_F16, 2>(M, N, K, nullptr, nullptr, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  const int nc = skinny_nc(M, N);
  if (M <= 16) {
    if (nc >= 4) return launch_skinny_f32a_nc<1, 4>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    if (nc == 2) return launch_skinny_f32a_nc<1, 2>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    return launch_skinny_f32a_nc<1, 1>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  }
  if (M <= 32) {
    if (nc >= 4) return launch_skinny_f32a_nc<2, 4>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    if (nc == 2) return launch_skinny_f32a_nc<2, 2>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
    return launch_skinny_f32a_nc<2, 1>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  }
  // three products at 64 rows: NC = 1 (the wider ones spill; every NC gives the same sums)
  if (nc >= 4 && !bl) return launch_skinny_f32a_nc<4, 4, false>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  if (nc == 2 && !bl) return launch_skinny_f32a_nc<4, 2, false>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
  return launch_skinny_f32a_nc<4, 1>(M, N, K, af, ea, lda, bh, bl, eb, ldb, c, ldc, stream);
}

template <int BM, int BN, bool BLO>
hipError_t launch_tile_f32a(int64_t M, int64_t N, int64_t K, const float* af, const int32_t* ea, int64_t lda,
                            const uint16_t* bh, const uint16_t* bl, const int32_t* eb, int64_t ldb, float* c,
                            int64_t ldc, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (!grid_fits(tiles, kThreads)) return hipErrorInvalidConfiguration;
  const uint16_t* const none = nullptr;
  hipLaunchKernelGGL((gemm_comp_kernel<HEAL_F16, BM, BN, true, BLO, false, true>), dim3((unsigned)tiles),
                     dim3(kThreads), 0, stream, M, N, K, none, none, ea, lda, bh, bl, eb, ldb, c, ldc,
                     (int16_t*)nullptr, (int64_t)0, (float*)nullptr, (int64_t)0, af);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_comp_f32a(int64_t M, int64_t N, int64_t K, const float* a, int64_t lda, const int32_t* a_exp,
                                 const uint16_t* b_hi, const uint16_t* b_lo, const int32_t* b_exp, int64_t ldb,
                                 float* c, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (!a_exp && M > 16) return hipErrorInvalidValue;  // derived exponents: the skinny kernel, at most 16 rows
  const bool blo = b_lo != nullptr;
  switch (choose_tile(M, N, !blo)) {
    case kSkinny:
      return launch_skinny_f32a(M, N, K, a, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream);
    case kTile256x256:
      return blo ? launch_tile_f32a<256, 128, true>(M, N, K, a, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream)
                 : launch_tile_f32a<256, 256, false>(M, N, K, a, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream);
    case kTile128x256:  // chosen only when B has no low part
      return launch_tile_f32a<128, 256, false>(M, N, K, a, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream);
    case kTile256x128:
      return blo ? launch_tile_f32a<256, 128, true>(M, N, K, a, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream)
                 : launch_tile_f32a<256, 128, false>(M, N, K, a, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream);
    default:
      return blo ? launch_tile_f32a<128, 128, true>(M, N, K, a, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream)
                 : launch_tile_f32a<128, 128, false>(M, N, K, a, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream);
  }
}

hipError_t launch_gemm_comp(int64_t M, int64_t N, int64_t K, const uint16_t* a_hi, const uint16_t* a_lo,
                            const int32_t* a_exp, int64_t lda, const uint16_t* b_hi, const uint16_t* b_lo,
                            const int32_t* b_exp, int64_t ldb, int part, float* c, int64_t ldc,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (part == HEAL_F16)
    return launch_part<HEAL_F16>(M, N, K, a_hi, a_lo, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream);
  return launch_part<HEAL_BF16>(M, N, K, a_hi, a_lo, a_exp, lda, b_hi, b_lo, b_exp, ldb, c, ldc, stream);
}


// ============================================================================ split K through a workspace
// When heal_gemm_comp's own launch would leave CUs without work (at most 128 tiles of 128 x 128, or a skinny
// GEMM of 17..64 rows whose every workgroup re-reads all of A), K is cut into S slices: each workgroup
// multiplies one slice of one tile into an FP32 partial, and a second kernel adds the S partials of an
// output in slice order (0, 1, ..., S - 1) and applies the exponents once.  Every slice keeps its products
// in one FP32 accumulator, so the result has the same error bound as the unsplit GEMM and is the same bits on
// every run; it differs from heal_gemm_comp's bits only by the grouping of the FP32 additions.
namespace {

constexpr int64_t kSplitTileMinK = 1024;   // K per slice, at least, for the tile kernel
constexpr int64_t kSplitSkinnyMinK = 512;  // and for the skinny kernel
// rows and K from which a skinny GEMM of at most 16 rows is split
constexpr int64_t kSplitSkinnyMinRows = 8;
constexpr int64_t kSplitSkinnyFewRowsMinK = 8192;

constexpr int kMaxSlices = 16;             // K slices, at most

// Split K for 8..16 rows through gemm_stream_sk_kernel: slices of whole 128-column stages, as wide as A's parts
// allow in its LDS (1408 columns at 16 rows with both parts), the same width for every slice but the last, and
// about one workgroup per CU over the S x G grid.  Measured on MI355X (16 x 14336 -> 4096, FP32 A, bf16 weights
// rotated through HBM, graph-replayed, the reduction included): 35.6-36.3 us in 11 slices, against 38.2-38.4 us
// for the skinny kernel's 8 slices of four column blocks.  Splitting from K = 4096 instead of 8192 lost: 20.8
// against 16.7 us unsplit at 16 x 4096 -> 4096, and no gain at 16 x 4096 -> 14336.
struct StreamSkPlan {
  bool ok;
  int64_t S, kslice, G;
};
StreamSkPlan plan_stream_sk(int64_t M, int64_t N, int64_t K, bool a_lo) {
  StreamSkPlan q{false, 1, K, 0};
  if (M < 1 || M > 16 || N < 1 || K < 1) return q;
  const int64_t rs_max = kSkACap / ((a_lo ? 2 : 1) * M);
  int64_t wmax = 0;  // the widest slice whose planes fit
  for (int64_t w = kStK; stream_rs(w) <= rs_max; w += kStK) wmax = w;
  if (wmax < kStK) return q;
  int64_t S = (K + wmax - 1) / wmax;
  if (S < 2 || S > kMaxSlices) return q;
  const int64_t ks = ((K + S - 1) / S + kStK - 1) / kStK * kStK;  // equal slices, whole stages
  S = (K + ks - 1) / ks;
  const int64_t nblk = (N + 15) / 16;
  int64_t G = cu_count() / S;
  if (G < 1) G = 1;
  if (G > nblk) G = nblk;
  if ((nblk + G - 1) / G > 4 * kSkMaxJ) G = (nblk + 4 * kSkMaxJ - 1) / (4 * kSkMaxJ);
  q.ok = S >= 2;
  q.S = S;
  q.kslice = ks;
  q.G = G;
  return q;
}

struct SplitPlan {
  bool split;      // false: heal_gemm_comp's own launch
  bool skinny;     // skinny kernel (four column blocks) or 128 x 128 tiles
  int64_t S;       // slices
  int64_t kslice;  // K per slice (a multiple of 64; the last slice takes the rest)
  int64_t ldw;     // row stride of a partial (N rounded up to 4 floats)
  bool stream = false;  // 8..16 rows: gemm_stream_sk_kernel over a G x S grid
  int64_t G = 0;
};

SplitPlan plan_split(int64_t M, int64_t N, int64_t K, bool a_lo, bool b_lo) {
  SplitPlan p{false, false, 1, K, 0};
  if (M <= 0 || N <= 0 || K <= 0) return p;
  const TileKind kind = choose_tile(M, N, a_lo && !b_lo);
  int64_t wgs, target, min_k;
  if (kind == kSkinny) {
    // At most 16 rows, each workgroup of the unsplit launch re-reads all of A (M x K x 4 bytes of parts) for its
    // 16 NC columns of B: at 16 rows and one column block that is twice B's bytes.  The split launch takes four
    // column blocks per workgroup (A re-read a quarter as often) and restores the workgroup count with K slices,
    // at the price of the reduction's launch (a few microseconds): measured on the Llama-3-8B projections, that
    // pays from 8 rows and K = 8192 (down projection at 16 rows: 52 -> 38 us) and loses below.  Where A's
    // slice parts fit in LDS, the slices run on gemm_stream_sk_kernel instead (plan_stream_sk: 38 -> 36 us).
    // Above 16 rows, split only where every workgroup's re-read of A is over twice its share of B (16 NC
    // columns x K x 2 bytes): the unsplit launch's column blocks already serve the rest.
    if (M > 16 && M <= 16 * (int64_t)skinny_nc(M, N)) return p;
    if (M <= 16 && (M < kSplitSkinnyMinRows || K < kSplitSkinnyFewRowsMinK)) return p;
    if (M <= 16) {
      const StreamSkPlan q = plan_stream_sk(M, N, K, a_lo);
      if (q.ok) {
        p.split = true;
        p.S = q.S;
        p.kslice = q.kslice;
        p.ldw = (N + 3) / 4 * 4;
        p.stream = true;
        p.G = q.G;
        return p;
      }
    }
    wgs = (N + 63) / 64;
    target = 512;
    min_k = kSplitSkinnyMinK;
  } else if (kind == kTile128x128) {
    wgs = ((M + 127) / 128) * ((N + 127) / 128);
    target = 256;
    min_k = kSplitTileMinK;
  } else {
    return p;  // at least one full round of tiles already
  }
  int64_t S = target / wgs;  // at most one round: a partial second round costs more than the split gains
  if (S > K / min_k) S = K / min_k;
  if (S > kMaxSlices) S = kMaxSlices;
  if (S < 2) return p;
  const int64_t ks = ((K + S - 1) / S + 63) / 64 * 64;
  p.split = true;
  p.skinny = kind == kSkinny;
  p.kslice = ks;
  p.S = (K + ks - 1) / ks;
  p.ldw = (N + 3) / 4 * 4;
  return p;
}

// C[i, j] = 2^-(ea_i + eb_j) * (((w_0 + w_1) + w_2) + ... + w_{S-1})[i, j]; one thread per 4 columns
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int S, int64_t M, int64_t N,
                                                            int64_t ldw, const int32_t* __restrict__ ea,
                                                            const int32_t* __restrict__ eb, float* __restrict__ C,
                                                            int64_t ldc) {
  const int64_t nq = ldw >> 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * nq) return;
  const int64_t i = idx / nq, j0 = (idx - i * nq) * 4;
  const float* p = ws + i * ldw + j0;  // columns N .. ldw - 1 of a partial are never written and never stored
  const int64_t slice = M * ldw;
  // all S partials are requested before the first addition (one memory latency instead of S in a row); the
  // additions then run in slice order
  float4 v[kMaxSlices];
#pragma unroll
  for (int s = 0; s < kMaxSlices; ++s)
    if (s < S) v[s] = *reinterpret_cast<const float4*>(p + s * slice);
  float4 acc = v[0];
#pragma unroll
  for (int s = 1; s < kMaxSlices; ++s) {
    if (s < S) {
      acc.x += v[s].x;
      acc.y += v[s].y;
      acc.z += v[s].z;
      acc.w += v[s].w;
    }
  }
  const int e = ea ? ea[i] : 0;
  const float r[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t j = j0 + t;
    if (j < N) C[i * ldc + j] = __builtin_amdgcn_ldexpf(r[t], -(e + (eb ? eb[j] : 0)));
  }
}

template <int PART, bool ALO, bool BLO>
void launch_split_kernel(const SplitPlan& p, int64_t M, int64_t N, int64_t K, const uint16_t* ah,
                         const uint16_t* al, int64_t lda, const uint16_t* bh, const uint16_t* bl, int64_t ldb,
                         float* ws, hipStream_t stream) {
  const int32_t* const none = nullptr;
  if (p.stream) {
    constexpr int D = BLO ? kStDLo : kStD;
    hipLaunchKernelGGL((gemm_stream_sk_kernel<PART, D, ALO, BLO, 0>), dim3((unsigned)p.G, (unsigned)p.S), dim3(256),
                       0, stream, M, N, K, ah, al, (const float*)nullptr, none, lda, bh, bl, ldb, ws, p.ldw,
                       p.kslice);
  } else if (p.skinny) {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)p.S), block(64 * kSkWaves);
    if (M <= 16)
      hipLaunchKernelGGL((gemm_skinny_kernel<PART, 1, 4, ALO, BLO, false, true>), grid, block, 0, stream, M, N, K,
                         ah, al, none, lda, bh, bl, none, ldb, ws, p.ldw, (const float*)nullptr, p.kslice);
    else if (M <= 32)
      hipLaunchKernelGGL((gemm_skinny_kernel<PART, 2, 4, ALO, BLO, false, true>), grid, block, 0, stream, M, N, K,
                         ah, al, none, lda, bh, bl, none, ldb, ws, p.ldw, (const float*)nullptr, p.kslice);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<PART, 4, 4, ALO, BLO, false, true>), grid, block, 0, stream, M, N, K,
                         ah, al, none, lda, bh, bl, none, ldb, ws, p.ldw, (const float*)nullptr, p.kslice);
  } else {
    const dim3 grid((unsigned)(((M + 127) / 128) * ((N + 127) / 128)), (unsigned)p.S), block(kThreads);
    hipLaunchKernelGGL((gemm_comp_kernel<PART, 128, 128, ALO, BLO, false, false, true>), grid, block, 0, stream, M,
                       N, K, ah, al, none, lda, bh, bl, none, ldb, ws, p.ldw, (int16_t*)nullptr, (int64_t)0,
                       (float*)nullptr, (int64_t)0, (const float*)nullptr, p.kslice);
  }
}

// FP32 A (split in the kernel with the given row exponents): the skinny plan at 8..16 rows only
SplitPlan plan_split_f32a(int64_t M, int64_t N, int64_t K, bool b_lo) {
  SplitPlan p = plan_split(M, N, K, true, b_lo);
  if (!(p.skinny || p.stream) || M > 16) p = SplitPlan{false, false, 1, K, 0};
  return p;
}

template <bool BLO>
void launch_split_kernel_f32a(const SplitPlan& p, int64_t M, int64_t N, int64_t K, const float* af,
                              const int32_t* ea, int64_t lda, const uint16_t* bh, const uint16_t* bl, int64_t ldb,
                              float* ws, hipStream_t stream) {
  const uint16_t* const none = nullptr;
  if (p.stream) {
    constexpr int D = BLO ? kStDLo : kStD;
    hipLaunchKernelGGL((gemm_stream_sk_kernel<HEAL_F16, D, true, BLO, 1>), dim3((unsigned)p.G, (unsigned)p.S),
                       dim3(256), 0, stream, M, N, K, none, none, af, ea, lda, bh, bl, ldb, ws, p.ldw, p.kslice);
    return;
  }
  const dim3 grid((unsigned)((N + 63) / 64), (unsigned)p.S), block(64 * kSkWaves);
  hipLaunchKernelGGL((gemm_skinny_kernel<HEAL_F16, 1, 4, true, BLO, true, true>), grid, block, 0, stream, M, N, K,
                     none, none, ea, lda, bh, bl, (const int32_t*)nullptr, ldb, ws, p.ldw, af, p.kslice);
}

template <int PART>
void launch_split_part(const SplitPlan& p, int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al,
                       int64_t lda, const uint16_t* bh, const uint16_t* bl, int64_t ldb, float* ws,
                       hipStream_t stream) {
  if (al && bl)
    launch_split_kernel<PART, true, true>(p, M, N, K, ah, al, lda, bh, bl, ldb, ws, stream);
  else if (al)
    launch_split_kernel<PART, true, false>(p, M, N, K, ah, al, lda, bh, bl, ldb, ws, stream);
  else if (bl)
    launch_split_kernel<PART, false, true>(p, M, N, K, ah, al, lda, bh, bl, ldb, ws, stream);
  else
    launch_split_kernel<PART, false, false>(p, M, N, K, ah, al, lda, bh, bl, ldb, ws, stream);
}

}  // namespace

size_t gemm_comp_workspace(int64_t M, int64_t N, int64_t K, bool a_lo, bool b_lo) {
  const SplitPlan p = plan_split(M, N, K, a_lo, b_lo);
  return p.split ? (size_t)mul_sat(mul_sat(p.S, M), p.ldw * (int64_t)sizeof(float)) : 0;
}

int gemm_comp_slices(int64_t M, int64_t N, int64_t K, bool a_lo, bool b_lo) {
  return (int)plan_split(M, N, K, a_lo, b_lo).S;
}

size_t gemm_comp_f32a_workspace(int64_t M, int64_t N, int64_t K, bool b_lo) {
  const SplitPlan p = plan_split_f32a(M, N, K, b_lo);
  return p.split ? (size_t)mul_sat(mul_sat(p.S, M), p.ldw * (int64_t)sizeof(float)) : 0;
}

int gemm_comp_f32a_slices(int64_t M, int64_t N, int64_t K, bool b_lo) {
  return (int)plan_split_f32a(M, N, K, b_lo).S;
}

hipError_t launch_gemm_comp_f32a_splitk(int64_t M, int64_t N, int64_t K, const float* a, int64_t lda,
                                        const int32_t* a_exp, const uint16_t* b_hi, const uint16_t* b_lo,
                                        const int32_t* b_exp, int64_t ldb, float* c, int64_t ldc, void* workspace,
                                        hipStream_t stream) {
  const SplitPlan p = plan_split_f32a(M, N, K, b_lo != nullptr);
  if (!p.split || !a_exp)
    return launch_gemm_comp_f32a(M, N, K, a, lda, a_exp, b_hi, b_lo, b_exp, ldb, c, ldc, stream);
  const int64_t red_blocks = (M * (p.ldw / 4) + 255) / 256;
  if (!grid_fits(p.stream ? p.G : (N + 63) / 64, p.stream ? 256 : 64 * kSkWaves) || !grid_fits(red_blocks, 256))
    return hipErrorInvalidConfiguration;
  float* ws = reinterpret_cast<float*>(workspace);
  if (b_lo)
    launch_split_kernel_f32a<true>(p, M, N, K, a, a_exp, lda, b_hi, b_lo, ldb, ws, stream);
  else
    launch_split_kernel_f32a<false>(p, M, N, K, a, a_exp, lda, b_hi, b_lo, ldb, ws, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)red_blocks), dim3(256), 0, stream, (const float*)ws,
                     (int)p.S, M, N, p.ldw, a_exp, b_exp, c, ldc);
  return hipGetLastError();
}

hipError_t launch_gemm_comp_splitk(int64_t M, int64_t N, int64_t K, const uint16_t* a_hi, const uint16_t* a_lo,
                                   const int32_t* a_exp, int64_t lda, const uint16_t* b_hi, const uint16_t* b_lo,
                                   const int32_t* b_exp, int64_t ldb, int part, float* c, int64_t ldc, void* workspace,
                                   hipStream_t stream) {
  const SplitPlan p = plan_split(M, N, K, a_lo != nullptr, b_lo != nullptr);
  if (!p.split)
    return launch_gemm_comp(M, N, K, a_hi, a_lo, a_exp, lda, b_hi, b_lo, b_exp, ldb, part, c, ldc, stream);
  const int64_t gemm_blocks = p.stream ? p.G : p.skinny ? (N + 63) / 64 : ((M + 127) / 128) * ((N + 127) / 128);
  const int64_t red_blocks = (M * (p.ldw / 4) + 255) / 256;
  if (!grid_fits(gemm_blocks, p.stream ? 256 : p.skinny ? 64 * kSkWaves : kThreads) || !grid_fits(red_blocks, 256))
    return hipErrorInvalidConfiguration;
  float* ws = reinterpret_cast<float*>(workspace);
  if (part == HEAL_F16)
    launch_split_part<HEAL_F16>(p, M, N, K, a_hi, a_lo, lda, b_hi, b_lo, ldb, ws, stream);
  else
    launch_split_part<HEAL_BF16>(p, M, N, K, a_hi, a_lo, lda, b_hi, b_lo, ldb, ws, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)red_blocks), dim3(256), 0, stream, (const float*)ws,
                     (int)p.S, M, N, p.ldw, a_exp, b_exp, c, ldc);
  return hipGetLastError();
}

}  // namespace heal
