// attn.hip -- Dual-FP16 attention over INT16 Q/K/V on gfx950 matrix cores (HEAL, [TS 2A]).
//
// [TS 2A Solution/Mechanism/Benefit]: Q, K and V are stored as INT16; at run time each INT16 value is
// unpacked into two FP16 values that are exact, so QK^T and PV run on 16-bit matrix units while the
// stored footprint stays 16 bits.  [TS] = gist.science explainer "Demystifying Numerical Instability in
// LLM Inference: Achieving Reproducible Inference for Mission-Critical Tasks with HEAL", Technical Summary.
//
// Arithmetic (identical in both kernels):
//   * unpack (default, the byte split)  q = 256 * (q >> 8) + (q & 0xFF):  H = q >> 8 (-128..127) and
//     L = (q & 0xFF) / 256, both exact FP16 values, H + L = q / 256.  Two other exact readings of the pair
//     are selectable: the shift-10 split H = q >> 10, L = (q & 0x3FF) / 1024 (H + L = q / 1024), and the
//     float-float pair H = fp16_rn(q), L = q - H.  The power of two the halves carry (2^-8, 2^-10, 1) is
//     given back through the k-scales (squared) and the output exponent, exactly.
//   * S_int = q_i . k_j as two FP32 accumulators: Hq.Hk (byte split: integer partial sums below 2^21,
//     exact; shift-10: below 2^17, exact) and Hq.Lk + Lq.Hk + Lq.Lk (about 2^-7 of the first); S_int =
//     their FP32 sum.  The float-float pair drops Lq.Lk and Lv.P~l (3 + 3 products), and its Hq.Hk sum
//     rounds: about 2^-24 of sum |Hq Hk| per logit.
//   * t_ij = S_int * s_k,j * (s_q,i * softmax_scale * log2 e), carried as an FP32 pair (hi + FMA-captured
//     rounding error) so that t - max keeps its precision for logits of any size; online softmax in
//     base 2, FP32 running maximum and sum.  Prefill keeps u_ij = S_int * s_k,j as the pair and its maximum
//     in the same units, and multiplies only the difference by the query's factor: t - m = cq (u - m_u).
//   * P~ = p * (s_v,j * 2^E) with E = 14 - ilogb(max_j s_v,j) over the keys a workgroup reads (prefill: 8 less,
//     since its lazily moved maximum lets p reach 2^8), so P~ < 2^15 and its FP16 split P~ = P~h + P~l
//     (P~l = fp16(P~ - P~h), exact residual) keeps 22 bits;
//     O += P~h.H + P~h.L + P~l.H + P~l.L (4 products, one FP32 accumulator); O = acc * 2^(shift - E) / l
//     for the halves' scale 2^-shift.
//
// Prefill (q_len > 1): flash-style forward.  A workgroup of 8 wavefronts owns 256 queries of one
// (batch, head); each wavefront owns 32.  K/V tiles of 32 keys (PF_BKV) arrive in LDS as raw INT16 rows by
// direct-to-LDS transfers; the workgroup unpacks each tile once into FP16 hi / lo planes in LDS while the
// previous tile is multiplied (two raw stages and two plane stages); K fragments are 16-byte LDS reads and the
// V^T operand comes from the V planes through gfx950's transposing LDS read.
// Each wavefront computes S^T = K Q^T with v_mfma_f32_32x32x16_f16, so the 16 scores a lane holds all
// belong to ONE query: the softmax maximum/sum are lane-local plus one exchange with lane ^ 32.  The same
// registers, in MFMA order, are the P^T operand of O^T = V^T P^T, so P never leaves registers.
// Causal workgroups are dispatched longest first.
//
// Decode (q_len = 1): HBM-streaming, split over the keys.  A workgroup of 4 wavefronts owns one
// (batch, kv-head) and a chunk of 4 kpw keys; the G = n_q/n_kv query heads of the group are the 16 columns
// of v_mfma_f32_16x16x32_f16 (G <= 16).  Each wavefront streams its kpw keys in steps of 32 (kpw = 512, or
// less when a short cache or a small batch would leave most CUs idle: see decode_kpw): K straight
// into MFMA operand registers, V and the scales through two private LDS stages filled by direct-to-LDS
// transfers, so the next step's 16 KB are in flight while the current step is multiplied (66 KB of LDS
// per workgroup: two workgroups, eight wavefronts, per CU); the V^T operand comes straight from the
// [key][d] rows through gfx950's transposing LDS read.  The P~
// renormalisation exponent is kept as a running value (O rescaled by an exact power of two when a larger
// v-scale arrives), so no pre-pass over the scales is needed.  The four wavefronts' partial (max, sum, O)
// are merged in LDS in a fixed order and written to the workspace; a second kernel merges the chunks of
// each (batch, head) in a fixed order.  No atomics: results are bitwise reproducible.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "heal_internal.h"

namespace heal {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;

__device__ __forceinline__ uint32_t pack2(_Float16 a, _Float16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Dual-FP16 unpack of 8 INT16 values (one 16-byte chunk) into FP16 halves H + L, two values per 32-bit
// word.  Each reading's two exact parts are held scaled by 2^-kShift<SPLIT>, so that H + L = q 2^-kShift and
// the products of any two operands land in the same accumulators; a score then carries 2^-2 kShift and an O
// accumulator 2^-kShift, powers of two that the k-scales and the output exponent take back exactly.
//   HEAL_DUAL_BYTE     hi = q >> 8, lo = q & 0xFF, H = hi, L = lo / 256 (kShift 8).  With x = q ^ 0x8000 (the
//     high byte becomes hi + 128), a byte permute places each byte of x under the FP16 pattern 0x64__, the
//     value 1024 + byte (ulp 1 in [1024, 2048)): 1024 + lo and 1024 + hi + 128.  Then L = (1024 + lo) 2^-8 - 4
//     by one packed FMA (exact: the result needs 8 fraction bits) and H = (1152 + hi) - 1152.  No step rounds.
//   HEAL_DUAL_SHIFT10  hi = q >> 10, lo = q & 0x3FF, H = hi, L = lo / 1024 (kShift 10).
//     L: 0x6400 | lo is 1024 + lo, times 2^-10 minus 1.
//     H: with the 6-bit field f of q >> 10, 0x6400 | (f ^ 0x20) is 1024 + hi + 32; minus 1056 gives hi.
//   HEAL_DUAL_FLOAT    H = fp16_rn(q), L = q - H (an integer, |L| <= 16): the float-float pair, exact
//     (kShift 0).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <int SPLIT>
constexpr int kShift = SPLIT == HEAL_DUAL_BYTE ? 8 : (SPLIT == HEAL_DUAL_SHIFT10 ? 10 : 0);
template <int SPLIT>
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t& h, uint32_t& l) {
  if constexpr (SPLIT == HEAL_DUAL_BYTE) {
    const uint32_t x = w ^ 0x80008000u;
    // v_perm_b32: selector bytes 0..3 pick bytes of x, 4 picks a byte of 0x64646464
    const f16x2 lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, x, 0x04020400u));
    const f16x2 hb = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, x, 0x04030401u));
    const f16x2 c2m8 = {(_Float16)0.00390625f, (_Float16)0.00390625f};
    const f16x2 cm4 = {(_Float16)-4.0f, (_Float16)-4.0f};
    const f16x2 c1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
    l = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(lo, c2m8, cm4));
    h = __builtin_bit_cast(uint32_t, hb - c1152);
  } else if constexpr (SPLIT == HEAL_DUAL_SHIFT10) {
    const f16x2 lo = __builtin_bit_cast(f16x2, (w & 0x03FF03FFu) | 0x64006400u);
    const f16x2 hb = __builtin_bit_cast(f16x2, ((w >> 10) & 0x003F003Fu) ^ 0x64206420u);
    const f16x2 c2m10 = {(_Float16)0.0009765625f, (_Float16)0.0009765625f};
    const f16x2 cm1 = {(_Float16)-1.0f, (_Float16)-1.0f};
    const f16x2 c1056 = {(_Float16)1056.0f, (_Float16)1056.0f};
    l = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(lo, c2m10, cm1));
    h = __builtin_bit_cast(uint32_t, hb - c1056);
  } else {
    const float f0 = (float)(int16_t)(w & 0xFFFFu), f1 = (float)(int16_t)(w >> 16);
    const _Float16 h0 = (_Float16)f0, h1 = (_Float16)f1;  // round to nearest even
    const _Float16 l0 = (_Float16)(f0 - (float)h0), l1 = (_Float16)(f1 - (float)h1);  // exact residuals
    h = pack2(h0, h1);
    l = pack2(l0, l1);
  }
}
template <int SPLIT>
__device__ __forceinline__ void unpack8(const uint4& raw, uint4& H, uint4& L) {
  unpack_word<SPLIT>(raw.x, H.x, L.x);
  unpack_word<SPLIT>(raw.y, H.y, L.y);
  unpack_word<SPLIT>(raw.z, H.z, L.z);
  unpack_word<SPLIT>(raw.w, H.w, L.w);
}
// The float-float pair drops L.L (|L| <= 16 beside |H| up to 2^15: the product is below 2^-22 of H.H);
// the integer readings need all four products for an exact q.k.
template <int SPLIT>
constexpr bool kLoLo = SPLIT != HEAL_DUAL_FLOAT;

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
}

__device__ __forceinline__ int ilogb_pos(float x) { return __builtin_amdgcn_frexp_expf(x) - 1; }

// Logit t = (shh + srest) * s_k * cq as an unevaluated pair t_hi + t_lo.  A single FP32 rounding of t
// costs 2^-24 |t|, which for logits of magnitude 10^3 moves exp2(t - m) by ~1e-4; carrying the product's
// rounding error (FMA) keeps t - m accurate to ~2^-24 |t - m| instead.
// S_int = shh + srest is first rounded with its error kept: s_hi + s_lo == shh + srest exactly.  Fast2Sum
// suffices here although |srest| may exceed |shh|.  Byte split: shh sums products of two multiples of 256,
// so it is a multiple of 2^16, while |srest| < 2^31 makes ulp(srest) <= 2^8.  Shift-10 split: shh is a
// multiple of 2^20 and |srest| < 2^34, ulp(srest) <= 2^10.  An addend that is a multiple of the other's ulp
// makes the error term exact in either order.  t_hi is then the correctly rounded logit and
// |t_lo| <= ~2^-23 |t_hi| whatever cancellation happens.  Float-float split: shh (a sum of 22-bit products
// at different exponents) has already been rounded by its FP32 accumulator; Fast2Sum is exact whenever
// |shh| >= |srest|, the usual case since |srest| is about 2^-11 |shh|.
__device__ __forceinline__ void logit2(float shh, float srest, float sk, float cq, float& t_hi, float& t_lo) {
  const float s_hi = shh + srest;
  const float s_lo = srest - (s_hi - shh);
  const float c_hi = sk * cq;
  const float c_lo = __builtin_fmaf(sk, cq, -c_hi);
  t_hi = s_hi * c_hi;
  t_lo = __builtin_fmaf(s_hi, c_hi, -t_hi) + __builtin_fmaf(s_lo, c_hi, s_hi * c_lo);
}

// Prefill's form of the same pair: u = S_int * s_k as u_hi + u_lo (the query's factor cq is applied later, to
// the difference u - max, so t - m = cq ((u_hi - m_hi) + (u_lo - m_lo)) keeps ~2^-24 |t - m| for logits of
// any size with fewer operations per score than forming t itself).
__device__ __forceinline__ void score2(float shh, float srest, float sk, float& u_hi, float& u_lo) {
  const float s_hi = shh + srest;
  const float s_lo = srest - (s_hi - shh);
  u_hi = s_hi * sk;
  u_lo = __builtin_fmaf(s_lo, sk, __builtin_fmaf(s_hi, sk, -u_hi));
}

// 2^x by the hardware instruction (about 1 ulp; results below 2^-126 flush to 0).  Softmax weights are
// at most about 1, so a flushed weight is below the rounding error of the largest one.
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// (hi, lo) maximum: larger hi wins, equal hi -> larger lo.  The rule is symmetric, so lanes that exchange
// candidates agree on the result, and the arg-max key then gets p = exp2(0 + 0) = 1 exactly.
__device__ __forceinline__ void pair_max(float& mh, float& ml, float oh, float ol) {
  const bool take = (oh > mh) | ((oh == mh) & (ol > ml));
  mh = take ? oh : mh;
  ml = take ? ol : ml;
}

// split p~ into fp16 hi + lo (lo = fp16(p~ - hi), the residual is exact in fp32)
__device__ __forceinline__ void split_p(float p, _Float16& h, _Float16& l) {
  h = (_Float16)p;
  l = (_Float16)(p - (float)h);
}

// ================================================================================ direct-to-LDS helpers
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;
// CPOL: the transfer's cache policy bits (kNT: non-temporal, for cache rows that one launch reads once)
constexpr int kNT = 2;
template <int CPOL = 0>
__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_wave_base, 16, 0, CPOL);
}
template <int CPOL = 0>
__device__ __forceinline__ void dma4(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_wave_base, 4, 0, CPOL);
}

// s_waitcnt immediate: at most N vector-memory operations outstanding, all LDS operations done
template <int N>
constexpr int waitcnt_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4);
}
// K rows (FP16 halves) in LDS: [key][16 chunks of 8 d], chunk c of key j at j * 16 + (c ^ (j & 15)), so the
// 16 keys one 16-byte fragment read touches sit in 16 different bank groups
__device__ __forceinline__ int kv_pos(int key, int c) { return key * 16 + (c ^ (key & 15)); }
// V rows for the transposing reads: chunk c of key j at j * 16 + (c ^ vt_swz(j)).  A ds_read_b64_tr_b16 of a
// wavefront moves 512 bytes in two halves of 32 lanes; the swizzle spreads each half's 16 chunks over the 16
// distinct 16-byte bank groups of a 256-byte row, per read pattern:
//   VT_PREFILL: each half reads 4 consecutive keys x 4 consecutive chunks: XOR the chunk's top 2 bits with j % 4;
//   VT_DECODE:  each half reads 8 consecutive keys x 2 consecutive chunks: XOR chunk bits 1..3 with j % 8.
constexpr int VT_PREFILL = 0, VT_DECODE = 1;
template <int L>
__device__ __forceinline__ int vt_swz(int key) {
  return L == VT_PREFILL ? (key & 3) << 2 : (key & 7) << 1;
}
template <int L>
__device__ __forceinline__ int vt_pos(int key, int c) { return key * 16 + (c ^ vt_swz<L>(key)); }

// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element (i % 4) of the 8-byte rows read by
// lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.  So when lane r of a group reads V[k0 + r/4][d0 + 4 (r % 4) .. + 3]
// (4 keys x 16 d), lane i receives V[k0 .. k0 + 3][d0 + i]: four keys of one d, the V^T operand layout.
template <int L>
__device__ __forceinline__ v4i16 read_vt(const uint4* v_rows, int k0, int d0, int r) {
  const int key = k0 + (r >> 2), d = d0 + 4 * (r & 3);
  const char* src = reinterpret_cast<const char*>(v_rows) + vt_pos<L>(key, d >> 3) * 16 + (d & 7) * 2;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(src));
}
__device__ __forceinline__ uint4 join_v4i16(const v4i16& a, const v4i16& b) {
  const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
  return make_uint4(x.x, x.y, y.x, y.y);
}

// ============================================================================================ prefill
constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_BQ = 32 * PF_WAVES;  // queries per workgroup
constexpr int PF_BKV = 32;            // keys per tile
constexpr int PF_TAU = 8;             // slack of the lazy running maximum (log2 units)
static_assert(PF_BKV * 16 == PF_THREADS, "one 16-byte chunk of K and one of V per thread and tile");
// A tile as the direct-to-LDS transfers leave it: thread tid's chunk (key tid / 16, chunk tid % 16) of K and
// of V at slot tid, then the tile's 32 k-scales and 32 v-scales (brought by wavefront 0).  Every slot is
// written and read by the same thread, so only that thread's own transfer count guards it.
struct PfRaw {
  uint4 k[PF_THREADS];
  uint4 v[PF_THREADS];
  float sc[64];
};
// The tile's Dual-FP16 operands, unpacked once for all wavefronts: K halves in the kv_pos layout, V halves
// in the VT_PREFILL layout, the k-scales, then the v-scales times 2^E.
struct PfPlanes {
  uint4 kh[PF_BKV * 16];
  uint4 kl[PF_BKV * 16];
  uint4 vh[PF_BKV * 16];
  uint4 vl[PF_BKV * 16];
  float sc[64];
};

struct AttnParams {
  const int16_t* q;
  const int16_t* k;
  const int16_t* v;
  const float* qs;
  const float* ks;
  const float* vs;
  float* out;
  int64_t q_st[3], kv_st[3], qs_st[3], kvs_st[3], o_st[3];
  int64_t B, Lq, Lkv, Hq, Hkv;
  float scale_log2;  // softmax_scale * log2(e)
  int causal;
  // paged KV cache (decode): Lkv bounds the lengths lens[b]; key j of sequence b is slot
  // j & ((1 << page_shift) - 1) of page bt[b * bt_st + (j >> page_shift)], and kv_st[0] / kvs_st[0] are
  // the page strides
  const int32_t* bt;
  const int32_t* lens;
  int64_t bt_st, num_pages;
  int page_shift;
};

template <int SPLIT>
__global__ __launch_bounds__(PF_THREADS) void attn_prefill_kernel(AttnParams a) {
  __shared__ PfRaw r0;
  __shared__ PfRaw r1;
  __shared__ PfPlanes p0;
  __shared__ PfPlanes p1;
  __shared__ float red[PF_WAVES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bh = blockIdx.x;  // (batch, q-head)
  const int64_t b = bh / a.Hq, h = bh - b * a.Hq;
  const int64_t hk = h / (a.Hq / a.Hkv);
  const int ntq = (int)((a.Lq + PF_BQ - 1) / PF_BQ);
  const int64_t q0 = (int64_t)(ntq - 1 - (int)blockIdx.y) * PF_BQ;  // longest tiles first
  const int64_t off = a.Lkv - a.Lq;                                  // bottom-right causal offset

  int64_t kv_end = a.Lkv;
  if (a.causal) {
    const int64_t lim = q0 + PF_BQ + off;
    if (lim < kv_end) kv_end = lim;
  }
  if (kv_end < 0) kv_end = 0;
  const int ntk = (int)((kv_end + PF_BKV - 1) / PF_BKV);

  const int16_t* kbase = a.k + b * a.kv_st[0] + hk * a.kv_st[2];
  const int16_t* vbase = a.v + b * a.kv_st[0] + hk * a.kv_st[2];
  const float* ksb = a.ks + b * a.kvs_st[0] + hk * a.kvs_st[2];
  const float* vsb = a.vs + b * a.kvs_st[0] + hk * a.kvs_st[2];
  const int64_t kvs1 = a.kv_st[1], ss1 = a.kvs_st[1];

  // ---- one tile's transfers: wavefront 0 brings the scales first, then every thread its K and V chunk, so
  //      "at most 2 outstanding" after issuing tile t + 1 means this thread's part of tile t has landed.
  //      Keys past the end are clamped to the last key (read, never used). ----
  const int ckey = tid >> 4, cchunk = tid & 15;
  auto issue = [&](PfRaw& R, int t) {
    if (wave == 0) {
      int64_t js = (int64_t)t * PF_BKV + (lane & 31);
      if (js > a.Lkv - 1) js = a.Lkv - 1;
      dma4((lane < 32 ? ksb : vsb) + js * ss1, &R.sc[0]);
    }
    int64_t j = (int64_t)t * PF_BKV + ckey;
    if (j > a.Lkv - 1) j = a.Lkv - 1;
    dma16(kbase + j * kvs1 + 8 * cchunk, &R.k[64 * wave]);
    dma16(vbase + j * kvs1 + 8 * cchunk, &R.v[64 * wave]);
  };
  if (ntk > 0) {
    issue(r0, 0);
    issue(r1, 1);
  }

  // ---- E = 14 - PF_TAU - ilogb(max v-scale over the keys this workgroup reads) ----
  float vmax = 0.0f;
  for (int64_t j = tid; j < kv_end; j += PF_THREADS) vmax = fmaxf(vmax, vsb[j * ss1]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, m, 64));
  if (lane == 0) red[wave] = vmax;
  __syncthreads();
  vmax = red[0];
#pragma unroll
  for (int w = 1; w < PF_WAVES; ++w) vmax = fmaxf(vmax, red[w]);
  // p <= 2^PF_TAU under the lazy running maximum, so P~ = p s_v 2^E stays below 2^15
  const int E = vmax > 0.0f ? 14 - PF_TAU - ilogb_pos(vmax) : 0;

  // ---- unpack this thread's chunks of a landed tile into the Dual-FP16 planes ----
  auto unpack = [&](const PfRaw& R, PfPlanes& P) {
    uint4 hi, lo;
    unpack8<SPLIT>(R.k[tid], hi, lo);
    P.kh[kv_pos(ckey, cchunk)] = hi;
    P.kl[kv_pos(ckey, cchunk)] = lo;
    unpack8<SPLIT>(R.v[tid], hi, lo);
    P.vh[vt_pos<VT_PREFILL>(ckey, cchunk)] = hi;
    P.vl[vt_pos<VT_PREFILL>(ckey, cchunk)] = lo;
    if (wave == 0) {
      const float s = R.sc[lane];
      P.sc[lane] = __builtin_amdgcn_ldexpf(s, lane < 32 ? 2 * kShift<SPLIT> : E);
    }
  };

  // ---- this lane's query and its Dual-FP16 fragments (B operand of S^T = K Q^T), unpacked once ----
  const int qcol = lane & 31, half = lane >> 5;
  const int64_t qi = q0 + 32 * wave + qcol;
  const bool qvalid = qi < a.Lq;
  const int64_t qi_c = qvalid ? qi : a.Lq - 1;
  const int16_t* qrow = a.q + b * a.q_st[0] + qi_c * a.q_st[1] + h * a.q_st[2];
  uint4 QH[8], QL[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    unpack8<SPLIT>(*reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * half), QH[ks], QL[ks]);
  // the query's factor of every logit; at least the smallest normal float, so that a zero scale (a query of
  // zeros: every logit 0) never meets an infinity in cq * (u - m)
  const float cq = fmaxf(a.qs[b * a.qs_st[0] + qi_c * a.qs_st[1] + h * a.qs_st[2]] * a.scale_log2, 1.17549435e-38f);
  // queries of this wave: [q0 + 32 wave, q0 + 32 wave + 31]; key j visible to query i iff j <= i + off
  const int64_t wq_first = q0 + 32 * wave, wq_last = wq_first + 31;

  f32x16 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.0f;
  float m_run = -INFINITY, m_run_lo = 0.0f, l_run = 0.0f;
  const int vq = lane >> 4, vi = lane & 15;  // 16-lane group and position for the transposing reads

  // MASK: the tile holds keys this wavefront's queries cannot all see (past the end, or above the causal limit
  // of some query); without it every score of the tile is visible and the mask's vector work is skipped
  auto compute = [&](const PfPlanes& P, int t, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int64_t kb = (int64_t)t * PF_BKV;
    if (a.causal && kb > wq_last + off) return;  // every key masked for this wave (wave-uniform)
    // ---- S^T tile [32 keys x 32 queries] = K Q^T, two accumulators ----
    f32x16 shh, srest;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      shh[r] = 0.0f;
      srest[r] = 0.0f;
    }
    // K fragments one k step ahead: step ks + 1's reads are issued before step ks's MFMAs (a scheduling barrier
    // keeps the compiler from sinking them), so the LDS latency runs under the matrix work
    uint4 KH = P.kh[kv_pos(qcol, half)], KL = P.kl[kv_pos(qcol, half)];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 KHn = KH, KLn = KL;
      if (ks + 1 < 8) {
        KHn = P.kh[kv_pos(qcol, 2 * (ks + 1) + half)];
        KLn = P.kl[kv_pos(qcol, 2 * (ks + 1) + half)];
      }
      __builtin_amdgcn_sched_barrier(0);
      shh = mfma32(KH, QH[ks], shh);
      srest = mfma32(KH, QL[ks], srest);
      srest = mfma32(KL, QH[ks], srest);
      if constexpr (kLoLo<SPLIT>) srest = mfma32(KL, QL[ks], srest);
      KH = KHn;
      KL = KLn;
    }
    // ---- scores of this lane's query for its 16 keys: key = 8 (r/4) + 4 half + r%4.  Keys past the end
    //      or above this query's causal limit are hidden: tile key kk is visible iff kk < lim, so the lane's
    //      key 8 (r/4) + 4 half + r%4 is hidden iff 8 (r/4) + r%4 >= lim - 4 half.  A hidden key's lo stays
    //      finite, so its p = exp2(-inf + ...) is 0 all the same. ----
    int lim2 = PF_BKV;
    if constexpr (MASK) {
      int64_t lim = a.Lkv - kb;
      if (a.causal && qi + off + 1 - kb < lim) lim = qi + off + 1 - kb;
      lim2 = (int)(lim < 0 ? 0 : (lim > PF_BKV ? PF_BKV : lim)) - 4 * half;
    }
    // u = S_int * s_k per key (logit / cq), as a pair; hidden keys get u = -inf
    float tv[16], tl[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 k4 = *reinterpret_cast<const float4*>(&P.sc[8 * g + 4 * half]);
      const float skv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        score2(shh[r], srest[r], skv[i], tv[r], tl[r]);
        if constexpr (MASK) tv[r] = 8 * g + i >= lim2 ? -INFINITY : tv[r];
      }
    }
    // (hi, lo) maximum of the 16: the largest hi, then the lo of a key attaining it.  When keys tie in hi,
    // one with a larger lo than the chosen key gets p a few ulp above 1, which is harmless.
    float tmax = tv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, tv[r]);
    float tmax_lo = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) tmax_lo = tv[r] == tmax ? tl[r] : tmax_lo;
    pair_max(tmax, tmax_lo, __shfl_xor(tmax, 32, 64), __shfl_xor(tmax_lo, 32, 64));
    // ---- lazy running maximum: it moves to the tile maximum only where that exceeds it by more than
    //      PF_TAU, and then for the whole wavefront at once, so most tiles skip rescaling O.  Otherwise
    //      every p <= 2^PF_TAU, which the P~ scale 2^E leaves room for.  The first visible tile always
    //      moves it (m_run = -inf), so a key that is alone at the maximum still gets p = 1 exactly. ----
    // (in logit units: cq > 0 turns the u-space difference into t - m; NaN when both are -inf: no growth)
    const bool grow = ((tmax - m_run) + (tmax_lo - m_run_lo)) * cq > PF_TAU;
    if (__ballot(grow)) {  // wave-uniform
      const float alpha = grow ? exp2_raw(cq * ((m_run - tmax) + (m_run_lo - tmax_lo))) : 1.0f;  // 0 from -inf
      m_run = grow ? tmax : m_run;
      m_run_lo = grow ? tmax_lo : m_run_lo;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
    }
    const bool none = m_run == -INFINITY;  // no visible key yet: every p below is exp2(-inf) = 0
    const float m_use = none ? 0.0f : m_run, m_use_lo = none ? 0.0f : m_run_lo;
    float psum = 0.0f;
    uint32_t ph[8], pl[8];  // P~ fragments: k-step kk2 uses registers 4 kk2 .. 4 kk2 + 3
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 v4 = *reinterpret_cast<const float4*>(&P.sc[32 + 8 * g + 4 * half]);
      const float svv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int r = 4 * g + i;
        const float p0 = exp2_raw(cq * ((tv[r] - m_use) + (tl[r] - m_use_lo)));
        const float p1 = exp2_raw(cq * ((tv[r + 1] - m_use) + (tl[r + 1] - m_use_lo)));
        psum += p0 + p1;
        _Float16 h0, l0, h1, l1;
        split_p(p0 * svv[i], h0, l0);
        split_p(p1 * svv[i + 1], h1, l1);
        ph[r >> 1] = pack2(h0, h1);
        pl[r >> 1] = pack2(l0, l1);
      }
    }
    l_run += psum;
    // ---- O^T [128 d x 32 queries] += V^T P~^T over these 32 keys (2 k-steps of 16).  The V^T operand of
    //      lane (d = 32 dt + l % 32, k-group g = l / 32) holds keys 16 kk2 + 4 g + 0..3 and
    //      16 kk2 + 8 + 4 g + 0..3: the same keys, in the same order, as the P~ registers ----
    // the V^T fragments of (kk2, dt) step i = 4 kk2 + dt, read one step ahead of their MFMAs as K's above
    auto read_v = [&](int i, uint4& VH, uint4& VL) {
      const int k1 = 16 * (i >> 2) + 4 * (vq >> 1), d0 = 32 * (i & 3) + 16 * (vq & 1);
      VH = join_v4i16(read_vt<VT_PREFILL>(P.vh, k1, d0, vi), read_vt<VT_PREFILL>(P.vh, k1 + 8, d0, vi));
      VL = join_v4i16(read_vt<VT_PREFILL>(P.vl, k1, d0, vi), read_vt<VT_PREFILL>(P.vl, k1 + 8, d0, vi));
    };
    uint4 VH, VL;
    read_v(0, VH, VL);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk2 = i >> 2, dt = i & 3;
      const uint4 PH = make_uint4(ph[4 * kk2], ph[4 * kk2 + 1], ph[4 * kk2 + 2], ph[4 * kk2 + 3]);
      const uint4 PL = make_uint4(pl[4 * kk2], pl[4 * kk2 + 1], pl[4 * kk2 + 2], pl[4 * kk2 + 3]);
      uint4 VHn = VH, VLn = VL;
      if (i + 1 < 8) read_v(i + 1, VHn, VLn);
      __builtin_amdgcn_sched_barrier(0);
      O[dt] = mfma32(VH, PH, O[dt]);
      O[dt] = mfma32(VL, PH, O[dt]);
      O[dt] = mfma32(VH, PL, O[dt]);
      if constexpr (kLoLo<SPLIT>) O[dt] = mfma32(VL, PL, O[dt]);
      VH = VHn;
      VL = VLn;
    }
  };

  // ---- key loop.  In the step for tile t: tile t + 2's transfers are issued, tile t + 1 (landed) is
  //      unpacked into the other plane set, and tile t is multiplied; one barrier per tile.  The body is
  //      straight-line: transfers and unpacks past the last tile touch valid (clamped) keys and idle
  //      buffers only, and the transfers are drained before the epilogue. ----
  if (ntk > 0) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm<2>());
    unpack(r0, p0);
  }
  __syncthreads();
  // tile t is wholly visible to this wavefront (wave-uniform): all its keys exist and lie at or below the causal
  // limit of the wavefront's first query
  auto whole = [&](int t) {
    const int64_t kl = (int64_t)t * PF_BKV + PF_BKV - 1;
    return kl < a.Lkv && (!a.causal || kl <= wq_first + off);
  };
  using Unmasked = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  for (int t = 0; t < ntk; t += 2) {
    issue(r0, t + 2);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm<2>());
    unpack(r1, p1);
    if (whole(t))
      compute(p0, t, Unmasked{});
    else
      compute(p0, t, Masked{});
    __syncthreads();
    if (t + 1 >= ntk) break;
    issue(r1, t + 3);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm<2>());
    unpack(r0, p0);
    if (whole(t + 1))
      compute(p1, t + 1, Unmasked{});
    else
      compute(p1, t + 1, Masked{});
    __syncthreads();
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());

  // ---- epilogue: O = acc * 2^-E / l; lane holds query qcol, d = 32 dt + 8 (r/4) + 4 half + r%4 ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float* orow = a.out + b * a.o_st[0] + qi * a.o_st[1] + h * a.o_st[2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 o;
      o.x = __builtin_amdgcn_ldexpf(O[dt][4 * g + 0], kShift<SPLIT> - E) * inv;
      o.y = __builtin_amdgcn_ldexpf(O[dt][4 * g + 1], kShift<SPLIT> - E) * inv;
      o.z = __builtin_amdgcn_ldexpf(O[dt][4 * g + 2], kShift<SPLIT> - E) * inv;
      o.w = __builtin_amdgcn_ldexpf(O[dt][4 * g + 3], kShift<SPLIT> - E) * inv;
      *reinterpret_cast<float4*>(orow + 32 * dt + 8 * g + 4 * half) = o;
    }
}

// ============================================================================================= decode
constexpr int DC_WAVES = 4;
constexpr int DC_THREADS = 64 * DC_WAVES;
constexpr int DC_KPW = 512;                   // keys per wavefront, at most
constexpr int DC_SUB = 32;                    // keys per step
constexpr int DC_PART = 4 + D;                // floats per partial: m_hi, m_lo, l, (pad), O[128]
constexpr int DC_NDMA = 17;                   // direct-to-LDS transfers per lane per step

// One step's V in a wavefront-private LDS stage, filled by direct-to-LDS transfers: [32 keys][16 chunks of
// 8 d] INT16 in the VT_DECODE layout, then the 32 k-scales and 32 v-scales.  K needs no LDS: its MFMA operand
// layout (one key's 8 consecutive d per lane) is a plain 16-byte load into registers.
struct DcStage {
  uint4 v[DC_SUB * 16];
  float sc[2 * DC_SUB];
};

// Keys per wavefront: 512, halved (down to one 32-key step) while the grid would hold fewer than 512
// workgroups, the number two per CU makes resident.  With 512 keys a workgroup runs 16 dependent steps, so
// a grid of a few dozen workgroups (one sequence of a few hundred keys) is bound by that chain's latency,
// not by HBM; shorter runs spread the same keys over more workgroups at the price of more partials for the
// merge.  Every wavefront range stays kpw-aligned, a power of two from 32 to 512.
int decode_kpw(int64_t B, int64_t Hkv, int64_t Lkv) {
  int kpw = DC_KPW;
  while (kpw > DC_SUB && mul_sat(mul_sat(B, Hkv), (Lkv + 4 * kpw - 1) / (4 * kpw)) < 512) kpw >>= 1;
  return kpw;
}

size_t decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lkv) {
  const int64_t chunk = (int64_t)DC_WAVES * decode_kpw(B, Hkv, Lkv);
  const int64_t nsplit = (Lkv + chunk - 1) / chunk;
  // saturates rather than wraps: an impossible size is refused, never under-sized
  return (size_t)mul_sat(mul_sat(mul_sat(B, Hq), nsplit > 0 ? nsplit : 1), DC_PART * (int64_t)sizeof(float));
}

// PAGED: the keys of each sequence are in pages of a shared pool (AttnParams::bt / lens) and every sequence
// has its own length; otherwise one contiguous run of a.Lkv keys per (batch, kv head).
template <bool PAGED, int SPLIT>
__global__ __launch_bounds__(DC_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_decode_kernel(
    AttnParams a, float* __restrict__ ws, int nsplit, int kpw) {
  // two stages per wavefront, each stage its own object (the compiler can tell the stage being read
  // from the one being filled); after the key loop the same bytes hold the wavefront partials
  __shared__ DcStage st0[DC_WAVES];
  __shared__ DcStage st1[DC_WAVES];
  static_assert(sizeof(float) * DC_WAVES * 16 * DC_PART <= sizeof(DcStage) * DC_WAVES,
                "partials must fit in one stage array");
  float(*part)[16][DC_PART] = reinterpret_cast<float(*)[16][DC_PART]>(&st0[0]);

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x;
  const int64_t bk = blockIdx.y;  // (batch, kv-head)
  const int64_t b = bk / a.Hkv, hk = bk - b * a.Hkv;
  const int G = (int)(a.Hq / a.Hkv);
  // keys of this sequence (paged: its own length, clamped into [0, a.Lkv])
  int64_t L = a.Lkv;
  if constexpr (PAGED) {
    const int64_t len = a.lens[b];
    L = len < 0 ? 0 : (len > a.Lkv ? a.Lkv : len);
  }
  const int64_t c0 = (int64_t)split * DC_WAVES * kpw;
  int64_t c1 = c0 + DC_WAVES * kpw;
  if (c1 > L) c1 = L;
  const int64_t w0 = c0 + (int64_t)wave * kpw;
  int64_t w1 = w0 + kpw;
  if (w1 > c1) w1 = c1;

  // contiguous: the (batch, kv head) runs; paged: the kv head's offset inside a page
  const int64_t kvoff = (PAGED ? 0 : b * a.kv_st[0]) + hk * a.kv_st[2];
  const int64_t soff = (PAGED ? 0 : b * a.kvs_st[0]) + hk * a.kvs_st[2];

  // query column of this lane: head hk*G + qc for qc < G (other columns are zero padding)
  const int qc = lane & 15, grp = lane >> 4;
  const bool qvalid = qc < G;
  const int64_t hq = hk * G + (qvalid ? qc : 0);
  uint4 QH[4], QL[4];
  {
    const int16_t* qrow = a.q + b * a.q_st[0] + hq * a.q_st[2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 raw = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * grp);
      if (!qvalid) raw = make_uint4(0u, 0u, 0u, 0u);
      unpack8<SPLIT>(raw, QH[ks], QL[ks]);
    }
  }
  // the query's factor of every logit, times 2^(2 kShift) for the scale the unpacked halves carry
  const float cq = qvalid ? __builtin_amdgcn_ldexpf(a.qs[b * a.qs_st[0] + hq * a.qs_st[2]] * a.scale_log2,
                                                    2 * kShift<SPLIT>)
                          : 0.0f;

  // one step's loads: K straight into operand registers (key 16 mt + qc, d 32 ks + 8 grp .. + 7), V and the
  // scales direct-to-LDS (position p = 64 i + l holds key p / 16 in the VT_DECODE layout).  The V and scale
  // transfers are non-temporal (each launch reads the cache once; each V transfer covers whole 256-byte rows):
  // 397 against 411 us at 64 x 8192 x 8 heads, 362 against 390 us for head-major pages.  K's loads stay plain:
  // each reads 64 bytes of 16 rows, and non-temporal K loads ran slower (415 us).
  //  A step's keys past this wavefront's range are clamped to its last key (read, never used).  Paged: the
  //  page size is a power of two >= 32 and steps start at multiples of 32, so after that clamp every key of
  //  a step lies in the page of its first (clamped) key.  The wavefront's range (kpw <= 512 keys,
  //  kpw-aligned, kpw a power of two) spans at most 16 pages, whose ids lane l holds from the start (pid_lane); a step takes its page id from
  //  the lane of its page, so no table read waits in front of the step's loads.
  const int64_t kvs1 = a.kv_st[1], ss1 = a.kvs_st[1];
  const int64_t jmax = w1 - 1;
  int pid_lane = 0;
  int64_t p0 = 0;
  if constexpr (PAGED) {
    p0 = w0 >> a.page_shift;
    const int64_t pend = (w1 + ((int64_t)1 << a.page_shift) - 1) >> a.page_shift;  // pages of [w0, w1)
    if (w1 > w0 && p0 + lane < pend) pid_lane = a.bt[b * a.bt_st + p0 + lane];
  }
  auto issue = [&](DcStage& S, uint4 (&kr)[2][4], int64_t j0) {
    int64_t row0 = 0, srow0 = 0;  // element offsets of the step's page (paged) or run (contiguous)
    int64_t jmask = -1;           // key -> slot within that page
    if constexpr (PAGED) {
      const int64_t jc = j0 < jmax ? j0 : jmax;
      int64_t pg = __builtin_amdgcn_readlane(pid_lane, (int)((jc >> a.page_shift) - p0));
      pg = pg < 0 ? 0 : (pg > a.num_pages - 1 ? a.num_pages - 1 : pg);
      row0 = pg * a.kv_st[0];
      srow0 = pg * a.kvs_st[0];
      jmask = ((int64_t)1 << a.page_shift) - 1;
    }
    const int16_t* kb = a.k + kvoff + row0;
    const int16_t* vb = a.v + kvoff + row0;
    const float* ksp = a.ks + soff + srow0;
    const float* vsp = a.vs + soff + srow0;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      int64_t j = j0 + 16 * mt + qc;
      if (j > jmax) j = jmax;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kr[mt][ks] = *reinterpret_cast<const uint4*>(kb + (j & jmask) * kvs1 + 32 * ks + 8 * grp);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = 64 * i + lane, key = p >> 4, c = (p & 15) ^ vt_swz<VT_DECODE>(key);
      int64_t j = j0 + key;
      if (j > jmax) j = jmax;
      dma16<kNT>(vb + (j & jmask) * kvs1 + 8 * c, &S.v[64 * i]);
    }
    int64_t j = j0 + (lane & 31);
    if (j > jmax) j = jmax;
    dma4<kNT>((lane < 32 ? ksp : vsp) + (j & jmask) * ss1, &S.sc[0]);
  };

  f32x4 O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, m_run_lo = 0.0f, l_run = 0.0f;
  int E = 0;            // O is held in units of 2^-E (running P~ renormalisation)
  float sv_seen = 0.0f;  // largest v-scale seen so far

  auto compute = [&](const DcStage& S, const uint4 (&kraw)[2][4], int64_t j0) {
    // ---- every LDS read of the step first (one round of latency): V^T fragments through the
    //      transposing read, the scales of this lane's 8 keys ----
    // ds_read_b64_tr_b16: in each 16-lane group, lane i receives element (i % 4) of the 8-byte rows read
    // by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.  Lane r of group grp reads V[key 16 hh + 4 grp + r/4]
    // [d 16 dt + 4 (r % 4) .. + 3], so lane i gets V[keys 16 hh + 4 grp + 0..3][16 dt + i]: the V^T
    // operand rows in the score registers' key order.
    v4i16 vtr[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) vtr[dt][hh] = read_vt<VT_DECODE>(S.v, 16 * hh + 4 * grp, 16 * dt, qc);
    float4 skq[2], svq[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      skq[mt] = *reinterpret_cast<const float4*>(&S.sc[16 * mt + 4 * grp]);
      svq[mt] = *reinterpret_cast<const float4*>(&S.sc[DC_SUB + 16 * mt + 4 * grp]);
    }
    // ---- S^T [32 keys x 16 query columns] ----
    f32x4 shh[2], srest[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      shh[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      srest[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        uint4 KH, KL;
        unpack8<SPLIT>(kraw[mt][ks], KH, KL);
        shh[mt] = mfma16(KH, QH[ks], shh[mt]);
        srest[mt] = mfma16(KH, QL[ks], srest[mt]);
        srest[mt] = mfma16(KL, QH[ks], srest[mt]);
        if constexpr (kLoLo<SPLIT>) srest[mt] = mfma16(KL, QL[ks], srest[mt]);
      }
    }
    float skr[2][4] = {{skq[0].x, skq[0].y, skq[0].z, skq[0].w}, {skq[1].x, skq[1].y, skq[1].z, skq[1].w}};
    float svr[2][4] = {{svq[0].x, svq[0].y, svq[0].z, svq[0].w}, {svq[1].x, svq[1].y, svq[1].z, svq[1].w}};
    // ---- running exponent of the v-scales: P~ = p * s_v * 2^E < 2^15 ----
    float svm = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (j0 + 16 * mt + 4 * grp + i >= w1) svr[mt][i] = 0.0f;
        svm = fmaxf(svm, svr[mt][i]);
      }
    svm = fmaxf(svm, __shfl_xor(svm, 16, 64));
    svm = fmaxf(svm, __shfl_xor(svm, 32, 64));
    if (svm > sv_seen) {
      sv_seen = svm;
      const int En = 14 - ilogb_pos(svm);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[dt][i] = __builtin_amdgcn_ldexpf(O[dt][i], En - E);
      E = En;
    }
    // ---- scores, online softmax (FP32 pairs) ----
    float tv[2][4], tl[2][4];
    float tmax = -INFINITY, tmax_lo = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s, sl;
        logit2(shh[mt][i], srest[mt][i], skr[mt][i], cq, s, sl);
        if (j0 + 16 * mt + 4 * grp + i >= w1) {
          s = -INFINITY;
          sl = 0.0f;
        }
        tv[mt][i] = s;
        tl[mt][i] = sl;
        pair_max(tmax, tmax_lo, s, sl);
      }
    pair_max(tmax, tmax_lo, __shfl_xor(tmax, 16, 64), __shfl_xor(tmax_lo, 16, 64));
    pair_max(tmax, tmax_lo, __shfl_xor(tmax, 32, 64), __shfl_xor(tmax_lo, 32, 64));
    float m_new = m_run, m_new_lo = m_run_lo;
    pair_max(m_new, m_new_lo, tmax, tmax_lo);
    const bool none = m_new == -INFINITY;
    const float m_use = none ? 0.0f : m_new, m_use_lo = none ? 0.0f : m_new_lo;
    const float alpha = exp2_raw((m_run - m_use) + (m_run_lo - m_use_lo));
    m_run = m_new;
    m_run_lo = m_new_lo;
    float psum = 0.0f;
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float p0 = exp2_raw((tv[mt][i] - m_use) + (tl[mt][i] - m_use_lo));
        const float p1 = exp2_raw((tv[mt][i + 1] - m_use) + (tl[mt][i + 1] - m_use_lo));
        psum += p0 + p1;
        _Float16 h0, l0, h1, l1;
        split_p(p0 * __builtin_amdgcn_ldexpf(svr[mt][i], E), h0, l0);
        split_p(p1 * __builtin_amdgcn_ldexpf(svr[mt][i + 1], E), h1, l1);
        ph[2 * mt + (i >> 1)] = pack2(h0, h1);
        pl[2 * mt + (i >> 1)] = pack2(l0, l1);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) O[dt] *= alpha;
    // ---- O^T [128 d x 16 columns] += V^T P~^T ----
    const uint4 PH = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    const uint4 PL = make_uint4(pl[0], pl[1], pl[2], pl[3]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint4 VH, VL;
      unpack8<SPLIT>(join_v4i16(vtr[dt][0], vtr[dt][1]), VH, VL);
      O[dt] = mfma16(VH, PH, O[dt]);
      O[dt] = mfma16(VL, PH, O[dt]);
      O[dt] = mfma16(VH, PL, O[dt]);
      if constexpr (kLoLo<SPLIT>) O[dt] = mfma16(VL, PL, O[dt]);
    }
  };

  // ---- key loop: the next step's transfers are in flight while the current step is computed.  The
  //      body is straight-line: a transfer past the last step re-reads valid keys (clamped) into the
  //      idle stage and is drained after the loop. ----
  const int nsteps = w1 > w0 ? (int)((w1 - w0 + DC_SUB - 1) / DC_SUB) : 0;
  uint4 kr0[2][4], kr1[2][4];
  if (nsteps > 0) issue(st0[wave], kr0, w0);
  for (int s = 0; s < nsteps; s += 2) {
    const int64_t j0 = w0 + (int64_t)s * DC_SUB;
    issue(st1[wave], kr1, j0 + DC_SUB);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm<DC_NDMA>());
    __asm__ __volatile__("" ::: "memory");
    compute(st0[wave], kr0, j0);
    if (s + 1 >= nsteps) break;
    issue(st0[wave], kr0, j0 + 2 * DC_SUB);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm<DC_NDMA>());
    __asm__ __volatile__("" ::: "memory");
    compute(st1[wave], kr1, j0 + DC_SUB);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());

  // ---- wave partial: the sum over the 4 lane groups, O^T brought back from units of 2^-E ----
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  __syncthreads();  // every wavefront is done with its stages before they are reused
  {
    float* pw = part[wave][qc];
    if (grp == 0) {
      pw[0] = m_run;
      pw[1] = m_run_lo;
      pw[2] = l_tot;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[4 + 16 * dt + 4 * grp + i] = __builtin_amdgcn_ldexpf(O[dt][i], kShift<SPLIT> - E);
  }
  __syncthreads();
  // ---- merge the 4 wavefronts in order: thread -> (column, 8 d values) ----
  for (int idx = tid; idx < G * 16; idx += DC_THREADS) {
    const int col = idx >> 4, d0 = (idx & 15) * 8;
    float m = -INFINITY, ml = 0.0f;
#pragma unroll
    for (int w = 0; w < DC_WAVES; ++w) pair_max(m, ml, part[w][col][0], part[w][col][1]);
    const bool none = m == -INFINITY;
    const float mu = none ? 0.0f : m, mul = none ? 0.0f : ml;
    float l = 0.0f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < DC_WAVES; ++w) {
      const float f = exp2f((part[w][col][0] - mu) + (part[w][col][1] - mul));
      l += part[w][col][2] * f;
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] += part[w][col][4 + d0 + u] * f;
    }
    float* dst = ws + (((b * a.Hq + hk * G + col) * nsplit) + split) * DC_PART;
    if (d0 == 0) {
      dst[0] = m;
      dst[1] = ml;
      dst[2] = l;
      dst[3] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) dst[4 + d0 + u] = o[u];
  }
}

// merge the nsplit partials of each (batch, q-head) in split order
__global__ __launch_bounds__(128) void attn_decode_merge_kernel(AttnParams a, const float* __restrict__ ws,
                                                                int nsplit) {
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / a.Hq, h = bh - b * a.Hq;
  const int d = threadIdx.x;
  const float* src = ws + bh * nsplit * DC_PART;
  float m = -INFINITY, ml = 0.0f;
  for (int s = 0; s < nsplit; ++s) pair_max(m, ml, src[s * DC_PART], src[s * DC_PART + 1]);
  const bool none = m == -INFINITY;
  const float mu = none ? 0.0f : m, mul = none ? 0.0f : ml;
  float l = 0.0f, o = 0.0f;
  for (int s = 0; s < nsplit; ++s) {
    const float f = exp2f((src[s * DC_PART] - mu) + (src[s * DC_PART + 1] - mul));
    l += src[s * DC_PART + 2] * f;
    o += src[s * DC_PART + 4 + d] * f;
  }
  a.out[b * a.o_st[0] + h * a.o_st[2] + d] = l > 0.0f ? o / l : 0.0f;
}

AttnParams make_params(const heal_attn_args& x) {
  AttnParams p;
  p.q = x.q; p.k = x.k; p.v = x.v;
  p.qs = x.q_scale; p.ks = x.k_scale; p.vs = x.v_scale;
  p.out = x.out;
  for (int i = 0; i < 3; ++i) {
    p.q_st[i] = x.q_strides[i];
    p.kv_st[i] = x.kv_strides[i];
    p.qs_st[i] = x.qs_strides[i];
    p.kvs_st[i] = x.kvs_strides[i];
    p.o_st[i] = x.o_strides[i];
  }
  p.B = x.batch; p.Lq = x.q_len; p.Lkv = x.kv_len; p.Hq = x.n_q_heads; p.Hkv = x.n_kv_heads;
  const double sm = x.softmax_scale > 0.0f ? (double)x.softmax_scale : 1.0 / sqrt((double)x.head_dim);
  p.scale_log2 = (float)(sm * 1.4426950408889634);
  p.causal = x.causal != 0;
  p.bt = nullptr;
  p.lens = nullptr;
  p.bt_st = 0;
  p.num_pages = 0;
  p.page_shift = 0;
  return p;
}

AttnParams make_params_paged(const heal_paged_decode_args& x) {
  AttnParams p;
  p.q = x.q; p.k = x.k_pages; p.v = x.v_pages;
  p.qs = x.q_scale; p.ks = x.k_scale; p.vs = x.v_scale;
  p.out = x.out;
  // (batch, token, head) triples with a single query token; kv / kvs: (page, slot, head)
  p.q_st[0] = x.q_strides[0]; p.q_st[1] = 0; p.q_st[2] = x.q_strides[1];
  p.qs_st[0] = x.qs_strides[0]; p.qs_st[1] = 0; p.qs_st[2] = x.qs_strides[1];
  p.o_st[0] = x.o_strides[0]; p.o_st[1] = 0; p.o_st[2] = x.o_strides[1];
  for (int i = 0; i < 3; ++i) {
    p.kv_st[i] = x.kv_strides[i];
    p.kvs_st[i] = x.kvs_strides[i];
  }
  p.B = x.batch; p.Lq = 1; p.Lkv = x.max_kv_len; p.Hq = x.n_q_heads; p.Hkv = x.n_kv_heads;
  const double sm = x.softmax_scale > 0.0f ? (double)x.softmax_scale : 1.0 / sqrt((double)x.head_dim);
  p.scale_log2 = (float)(sm * 1.4426950408889634);
  p.causal = 0;
  p.bt = x.block_table;
  p.lens = x.seq_lens;
  p.bt_st = x.bt_stride;
  p.num_pages = x.num_pages;
  int sh = 0;
  while (((int64_t)1 << sh) < x.page_size) ++sh;
  p.page_shift = sh;
  return p;
}

bool use_decode(const heal_attn_args& x) {
  return x.q_len == 1 && x.kv_len > 0 && x.n_kv_heads > 0 && (x.n_q_heads / x.n_kv_heads) <= 16;
}

__global__ void zero_rows_kernel(AttnParams a) {
  // kv_len == 0: every query sees no key; the output is defined as 0
  const int64_t row = blockIdx.x;  // (b, i, h)
  const int64_t h = row % a.Hq, i = (row / a.Hq) % a.Lq, b = row / (a.Hq * a.Lq);
  a.out[b * a.o_st[0] + i * a.o_st[1] + h * a.o_st[2] + threadIdx.x] = 0.0f;
}

}  // namespace

size_t attn_workspace_bytes(const heal_attn_args& x) {
  if (!use_decode(x) || x.batch <= 0 || x.n_q_heads <= 0) return 0;
  return decode_workspace(x.batch, x.n_q_heads, x.n_kv_heads, x.kv_len);
}

hipError_t launch_attn(const heal_attn_args& x, hipStream_t stream) {
  const AttnParams p = make_params(x);
  if (x.kv_len == 0) {
    if (!grid_fits(mul_sat(mul_sat(x.batch, x.q_len), x.n_q_heads), D)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)(x.batch * x.q_len * x.n_q_heads)), dim3(D), 0, stream,
                       p);
    return hipGetLastError();
  }
  if (use_decode(x)) {
    const int kpw = decode_kpw(x.batch, x.n_kv_heads, x.kv_len);
    const int64_t nsplit64 = (x.kv_len + DC_WAVES * kpw - 1) / (DC_WAVES * kpw);
    if (!grid_fits(nsplit64, DC_THREADS) || !grid_fits(mul_sat(x.batch, x.n_kv_heads), 1) ||
        !grid_fits(mul_sat(x.batch, x.n_q_heads), D))
      return hipErrorInvalidConfiguration;
    const int nsplit = (int)nsplit64;
    float* ws = reinterpret_cast<float*>(x.workspace);
    const dim3 grid((unsigned)nsplit, (unsigned)(x.batch * x.n_kv_heads));
    if (x.dual_split == HEAL_DUAL_SHIFT10)
      hipLaunchKernelGGL((attn_decode_kernel<false, HEAL_DUAL_SHIFT10>), grid, dim3(DC_THREADS), 0, stream, p, ws,
                         nsplit, kpw);
    else if (x.dual_split == HEAL_DUAL_FLOAT)
      hipLaunchKernelGGL((attn_decode_kernel<false, HEAL_DUAL_FLOAT>), grid, dim3(DC_THREADS), 0, stream, p, ws,
                         nsplit, kpw);
    else
      hipLaunchKernelGGL((attn_decode_kernel<false, HEAL_DUAL_BYTE>), grid, dim3(DC_THREADS), 0, stream, p, ws,
                         nsplit, kpw);
    hipLaunchKernelGGL(attn_decode_merge_kernel, dim3((unsigned)(x.batch * x.n_q_heads)), dim3(D), 0, stream,
                       p, (const float*)ws, nsplit);
    return hipGetLastError();
  }
  if (!grid_fits(mul_sat(x.batch, x.n_q_heads), PF_THREADS) || !grid_fits((x.q_len + PF_BQ - 1) / PF_BQ, 1))
    return hipErrorInvalidConfiguration;
  const unsigned ntq = (unsigned)((x.q_len + PF_BQ - 1) / PF_BQ);
  const dim3 grid((unsigned)(x.batch * x.n_q_heads), ntq);
  if (x.dual_split == HEAL_DUAL_SHIFT10)
    hipLaunchKernelGGL(attn_prefill_kernel<HEAL_DUAL_SHIFT10>, grid, dim3(PF_THREADS), 0, stream, p);
  else if (x.dual_split == HEAL_DUAL_FLOAT)
    hipLaunchKernelGGL(attn_prefill_kernel<HEAL_DUAL_FLOAT>, grid, dim3(PF_THREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<HEAL_DUAL_BYTE>, grid, dim3(PF_THREADS), 0, stream, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------------ decode without a caller workspace
// The partials of heal_attn_dual_fp16_noalloc live in this array: one copy per GPU, allocated by the runtime
// with the code object and kept until the process ends.  In host code `scratch` names a host-side stand-in,
// never the device memory: its device address is looked up once per device (with that device current) and
// only that address is ever passed to a kernel.
static __device__ __align__(256) float scratch[HEAL_ATTN_NOALLOC_MAX_WORKSPACE / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// the device address of `scratch` on the device that runs `stream`
hipError_t scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_noalloc(const heal_attn_args& x, hipStream_t stream) {
  heal_attn_args y = x;
  y.workspace = nullptr;
  y.workspace_bytes = 0;
  if (attn_workspace_bytes(x) > 0) {
    void* p = nullptr;
    const hipError_t e = scratch_address(stream, &p);
    if (e != hipSuccess) return e;
    y.workspace = p;
    y.workspace_bytes = HEAL_ATTN_NOALLOC_MAX_WORKSPACE;
  }
  return launch_attn(y, stream);
}

size_t paged_workspace_bytes(const heal_paged_decode_args& x) {
  if (x.batch <= 0 || x.n_q_heads <= 0) return 0;
  return decode_workspace(x.batch, x.n_q_heads, x.n_kv_heads, x.max_kv_len);
}

hipError_t launch_attn_paged(const heal_paged_decode_args& x, hipStream_t stream) {
  const AttnParams p = make_params_paged(x);
  if (x.max_kv_len == 0) {
    if (!grid_fits(mul_sat(x.batch, x.n_q_heads), D)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)(x.batch * x.n_q_heads)), dim3(D), 0, stream, p);
    return hipGetLastError();
  }
  // the grid covers max_kv_len; splits past a sequence's own length write empty partials
  const int kpw = decode_kpw(x.batch, x.n_kv_heads, x.max_kv_len);
  const int64_t nsplit64 = (x.max_kv_len + DC_WAVES * kpw - 1) / (DC_WAVES * kpw);
  if (!grid_fits(nsplit64, DC_THREADS) || !grid_fits(mul_sat(x.batch, x.n_kv_heads), 1) ||
      !grid_fits(mul_sat(x.batch, x.n_q_heads), D))
    return hipErrorInvalidConfiguration;
  const int nsplit = (int)nsplit64;
  float* ws = reinterpret_cast<float*>(x.workspace);
  const dim3 grid((unsigned)nsplit, (unsigned)(x.batch * x.n_kv_heads));
  if (x.dual_split == HEAL_DUAL_SHIFT10)
    hipLaunchKernelGGL((attn_decode_kernel<true, HEAL_DUAL_SHIFT10>), grid, dim3(DC_THREADS), 0, stream, p, ws,
                       nsplit, kpw);
  else if (x.dual_split == HEAL_DUAL_FLOAT)
    hipLaunchKernelGGL((attn_decode_kernel<true, HEAL_DUAL_FLOAT>), grid, dim3(DC_THREADS), 0, stream, p, ws,
                       nsplit, kpw);
  else
    hipLaunchKernelGGL((attn_decode_kernel<true, HEAL_DUAL_BYTE>), grid, dim3(DC_THREADS), 0, stream, p, ws,
                       nsplit, kpw);
  hipLaunchKernelGGL(attn_decode_merge_kernel, dim3((unsigned)(x.batch * x.n_q_heads)), dim3(D), 0, stream, p,
                     (const float*)ws, nsplit);
  return hipGetLastError();
}

}  // namespace heal
