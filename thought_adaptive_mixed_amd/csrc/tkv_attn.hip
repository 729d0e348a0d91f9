// Split-K paged decode attention over the mixed-precision, hole-bearing cache,
// with the sparsity statistics (entropy, top-k mass) in the same pass.
//
// Method passages: ThinKV abstract (a kernel extending PagedAttention that
// reuses evicted tokens' slots without compaction) and the technical summary,
// "Methodologie": thought decomposition via attention sparsity, Continuous
// Thinking (block table with eviction masks).
//
// Work decomposition: one work-group of nw 64-lane waves per (batch entry, KV
// head, split); a split owns a byte-balanced range of the sequence's block
// lists [8-bit | 4-bit | 2-bit].  The live blocks (fully evicted ones are
// dropped) are taken PK at a time, steps dealt round-robin to the waves.  A
// wave holds two steps of records (codes and metadata of PK blocks) in
// registers: the loads of the next step are in flight while the current one
// is computed.  The codes are read through one buffer resource per block
// record (scalar base, constant lane offset); the query operands, the same
// for every step, are read from LDS.  Per 16-token block, lane l takes chunk l of the K codes and
// chunk l of the V codes (D*bits/32 bytes each), which puts the codes straight
// into MFMA operand layout (v_mfma_f32_16x16x32_f16; k = 8 (lane / 16) + e):
//   S^T[t][h] = sum_d K[t][d] Q[h][d]     A = K codes, two 8-dim halves of a
//                                         lane's 16 dims of a group per k slice
//   O^T[d][h] += sum_t V[t][d] P'[t][h]   A = V codes, a lane's 4 tokens of two
//                                         blocks per k slice
// Integer codes enter the MFMA as fp16 subnormals (8-bit code c as the bit
// pattern c, value c * 2^-24; 4- and 2-bit codes at the top of the subnormal
// mantissa, c * 2^-18 and c * 2^-16), so an operand is the masked (and
// shifted) code word itself; products are exact and the power of two is
// folded back in fp32, per class.  The fp16 scales and zero-points are
// applied per (token, group) in fp32:
//   logit = (sum_g sK * (q_g . c_g) + zK * sum(q_g)) / sqrt(D)
//   out   = sum_t (p sV) c  +  sum_t p zV          (per group of dims)
// with p sV fed as an fp16 hi + lo pair (two MFMAs), so the product reaches
// the fp32 accumulator with ~21 significant bits.  The query heads of the GQA
// group sit in the 16 MFMA columns; with G heads only the first G' =
// roundup(G, 4) columns of each 16-lane row are real, so the PK = 16 / G'
// blocks of a step are packed side by side (DPP row shifts with bank masks)
// and the softmax epilogue runs once for all of them on fully used lanes, then
// P' is unpacked block by block for the P.V products.
// Softmax runs online in the log2 domain; the running max is shared by the
// lanes holding a head's tokens and is raised whenever a step exceeds it, so
// every weight is at most 1 and p sV at most sV (below 2^15 for inputs below
// 2^15 in magnitude: an fp16 operand).  Each lane keeps partial Z, S' = sum p (s - m)
// and a sorted top-8 of its logits, filtered by the head-wide 8th-best bound.
// The waves of a work-group merge their records through LDS; with one split
// the work-group then adds the staged self token and the sink and writes the
// outputs and statistics, otherwise it writes a partial record that a small
// combine kernel merges across splits.
#include "tkv_internal.h"
#include <mutex>

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

#define PART_X 16          // extra floats per partial record: m2, Z, S2, n, top8[8], pad
#define TOPK 8
#define LOG2E 1.4426950408889634f
#define LN2 0.6931471805599453f

// v_exp_f32 directly: no denormal-range fixup (weights below 2^-126 are 0)
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// work-group barrier that orders LDS only: global reads in flight (the
// padding loads past a wave's last step, the self token) are not waited for
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// code -> fp16 operands.  An integer code c enters the MFMA as an fp16
// subnormal, the value c * 2^-kUnitExp: products with the fp16 queries or
// probabilities are exact in fp32 and every partial sum is the plain code
// product times that power of two, folded back exactly afterwards (into the
// logit factor on the K side, into the accumulator's unit on the V side).
// ---------------------------------------------------------------------------
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
constexpr float kCodeUnit = 0x1p-24f;     // value of the fp16 subnormal with bit pattern 1
constexpr float kCodeScale = 0x1p24f;
// The 4- and 2-bit codes are placed at the top of the 10-bit subnormal
// mantissa (bits 6..9 and 8..9), so that code 1 is 2^-18 and 2^-16: measured
// on gfx950, the f16 MFMA loses precision on subnormal inputs whose leading
// mantissa bits are zero (codes at bits 0..1 gave errors of 2.6e-4 of the
// largest product, at bits 8..9 6e-7; 8-bit codes at bits 0..7 1e-5).
template <int BITS>
constexpr int kUnitExp = BITS == 8 ? 24 : (BITS == 4 ? 18 : 16);   // integer code 1 is 2^-kUnitExp
// fields p and p + W/2 of word w (elements 2p, 2p+1 of the word), one per half
template <int BITS>
__device__ inline uint32_t code_pair(uint32_t w, int p) {
  if constexpr (BITS == 8) {
    // bytes [w.p, 0, w.p+2, 0] (selector 0x0c reads a zero byte)
    const uint32_t sel = (uint32_t)p | (0x0cu << 8) | ((uint32_t)(p + 2) << 16) | (0x0cu << 24);
    return __builtin_amdgcn_perm(0u, w, sel);
  } else {
    // field p of each half moved to bits 10-BITS .. 9 of that half
    constexpr uint32_t M = (((1u << BITS) - 1u) << (10 - BITS)) * 0x00010001u;
    const int sh = p * BITS - (10 - BITS);
    return (sh >= 0 ? (w >> sh) : (w << -sh)) & M;
  }
}
// Elements e0 .. e0+3 (e0 a multiple of 4) of a lane's chunk as an fp16
// quad.  Integer codes (FMT 0, and ternary codes in either format): the
// subnormals above.  Float codes (FMT 1): the FP8 E4M3 or FP4 E2M1 values
// themselves, converted pairwise to fp32 by the hardware and packed to fp16,
// both exact (E4M3 and E2M1 values are fp16 values); the codes of a word sit
// in element order.
template <int BITS, int FMT>
__device__ inline half4_t operand4(const uint32_t* words, int e0) {
  constexpr int W = 32 / BITS;
  const uint32_t w = words[e0 / W];
  if constexpr (FMT == 1 && BITS == 8) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);          // bytes 0, 1
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);           // bytes 2, 3
    const half2_t lo = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(a[0], a[1]));
    const half2_t hi = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(b[0], b[1]));
    return (half4_t){lo[0], lo[1], hi[0], hi[1]};
  } else if constexpr (FMT == 1 && BITS == 4) {
    const bool up = (e0 % W) != 0;                                    // elements 4..7 of the word: bytes 2, 3
    const auto a = up ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2)
                      : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const auto b = up ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3)
                      : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const half2_t lo = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(a[0], a[1]));
    const half2_t hi = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(b[0], b[1]));
    return (half4_t){lo[0], lo[1], hi[0], hi[1]};
  } else {
    const int p = (e0 % W) >> 1;
    const half2_t a = __builtin_bit_cast(half2_t, code_pair<BITS>(w, p));
    const half2_t b = __builtin_bit_cast(half2_t, code_pair<BITS>(w, p + 1));
    half4_t r = {a[0], a[1], b[0], b[1]};
    return r;
  }
}

__device__ inline half8_t cat8(half4_t a, half4_t b) {
  return (half8_t){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// v (k) or zeros (!k)
__device__ inline half4_t keep4(half4_t v, bool k) {
  const uint2 u = __builtin_bit_cast(uint2, v);
  return __builtin_bit_cast(half4_t, make_uint2(k ? u.x : 0u, k ? u.y : 0u));
}
// v_mfma_f32_16x16x32_f16: k = 8 * (lane / 16) + e in both operands
__device__ inline float4_t mfma32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// top-8 lists (descending)
// ---------------------------------------------------------------------------
__device__ inline void topk_insert(float (&L)[TOPK], float v) {
#pragma unroll
  for (int i = 0; i < TOPK; i++) {
    float hi = fmaxf(L[i], v), lo = fminf(L[i], v);
    L[i] = hi; v = lo;
  }
}
__device__ inline void cswap(float& a, float& b) { float hi = fmaxf(a, b), lo = fminf(a, b); a = hi; b = lo; }
// L <- top 8 of (L u O), both sorted descending (bitonic merge)
__device__ inline void topk_merge(float (&L)[TOPK], const float (&O)[TOPK]) {
#pragma unroll
  for (int i = 0; i < TOPK; i++) L[i] = fmaxf(L[i], O[TOPK - 1 - i]);
#pragma unroll
  for (int i = 0; i < 4; i++) cswap(L[i], L[i + 4]);
  cswap(L[0], L[2]); cswap(L[1], L[3]); cswap(L[4], L[6]); cswap(L[5], L[7]);
  cswap(L[0], L[1]); cswap(L[2], L[3]); cswap(L[4], L[5]); cswap(L[6], L[7]);
}
// ---------------------------------------------------------------------------
struct AttnParams {
  DevState S;
  const int32_t* seq_ids;
  const int32_t* q_pos;
  const uint16_t* q;
  const float* k_self;
  const float* v_self;
  const float* sinks;
  int window, splits, topk;
  int layer;                   // the layer attended: KV heads layer*Hkv.. of each block
  int stats_stride;            // floats between batch entries of stats
  float* part;                 // [batch][Hq][splits][D + PART_X]
  const int32_t* order;        // nullable: [1 + batch] batch size, then the entry of each grid row
  float* out;
  float* stats;
  int32_t* n_attended;
};

template <int D, int GS>
struct AttnState {
  static constexpr int NG = D / GS, NT = D / 16;
  float4_t acc[NT];
  float zacc[NG];
  float m2, Z, S2;
  float top[TOPK];
  float thr;                   // head-wide 8th-best of the top lists
  float vunit;                 // value of one V-side accumulator unit (the unit of the class last computed)
  int natt;
};

__device__ inline float h_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFF)); }
__device__ inline float h_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// max over the lanes holding one head's values in the packed layout (lanes
// h + GP*i of every row): DPP row rotations by 4 and 8 inside a 16-lane row,
// then the row-pair and wave-half swaps.
template <int GP>
__device__ inline float head_max(float v) {
  if constexpr (GP <= 4) v = fmaxf(v, dpp_f<0x124>(v));          // row_ror:4
  if constexpr (GP <= 8) v = fmaxf(v, dpp_f<0x128>(v));          // row_ror:8
  return pair_max<32>(pair_max<16>(v));
}
template <int K>
__device__ inline void pair_topk(float (&L)[TOPK]) {
  float O[TOPK];
  if constexpr (K <= 8) {
#pragma unroll
    for (int i = 0; i < TOPK; i++) O[i] = xchg<K>(L[i]);
  } else {
#pragma unroll
    for (int i = 0; i < TOPK; i++) swap_pair<K>(L[i], L[i], O[i]);
  }
  topk_merge(L, O);
}
template <int GP>
__device__ inline float head_sum(float v) {
  if constexpr (GP <= 4) v = pair_sum<4>(v);
  if constexpr (GP <= 8) v = pair_sum<8>(v);
  return pair_sum<32>(pair_sum<16>(v));
}
template <int GP>
__device__ inline void head_topk(float (&L)[TOPK]) {
  if constexpr (GP <= 4) pair_topk<4>(L);
  if constexpr (GP <= 8) pair_topk<8>(L);
  pair_topk<16>(L);
  pair_topk<32>(L);
}
// reductions over the first n lanes (the rest hold the neutral value),
// broadcast from lane 0
__device__ inline float first_lanes_sum(float v, int n) {
  if (n > 1) v = pair_sum<1>(v);
  if (n > 2) v = pair_sum<2>(v);
  if (n > 4) v = pair_sum<4>(v);
  if (n > 8) v = pair_sum<8>(v);
  if (n > 16) v = pair_sum<16>(v);
  if (n > 32) v = pair_sum<32>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ inline float first_lanes_max(float v, int n) {
  if (n > 1) v = pair_max<1>(v);
  if (n > 2) v = pair_max<2>(v);
  if (n > 4) v = pair_max<4>(v);
  if (n > 8) v = pair_max<8>(v);
  if (n > 16) v = pair_max<16>(v);
  if (n > 32) v = pair_max<32>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ inline void first_lanes_topk(float (&L)[TOPK], int n) {
  if (n > 1) pair_topk<1>(L);
  if (n > 2) pair_topk<2>(L);
  if (n > 4) pair_topk<4>(L);
  if (n > 8) pair_topk<8>(L);
  if (n > 16) pair_topk<16>(L);
  if (n > 32) pair_topk<32>(L);
}

// Blocks per step of class C when the layout packs PK blocks side by side:
// the 8-bit class at D = 128 takes at most two (four blocks of its codes
// would not fit the registers of two steps); its steps leave the columns of
// the missing block positions empty.  32-bit words of a lane's chunk: D*bits/128.
template <int D, int PK, int C>
constexpr int pk_class() { return (C == 0 && D == 128 && PK > 2) ? 2 : PK; }
template <int D, int C>
constexpr int chunk_words() { return D * (C == 0 ? 8 : (C == 1 ? 4 : 2)) / 128; }
template <int D, int PK>
constexpr int step_words() {
  constexpr int a = pk_class<D, PK, 0>() * chunk_words<D, 0>(), b = pk_class<D, PK, 1>() * chunk_words<D, 1>(),
                c = pk_class<D, PK, 2>() * chunk_words<D, 2>();
  return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

// One step's data in registers: the K and V code chunks of the step's blocks
// (lane l: chunk l of each; block j's words at j * chunk_words), the metadata
// of this lane's own block (quad lg) and, with a window, the positions of its
// four tokens.  Sized for the class whose step holds the most words.
template <int D, int GS, bool WINDOW, int PK>
struct Buf {
  static constexpr int NG = D / GS;
  static constexpr int KW = step_words<D, PK>();
  uint32_t kw[KW], vw[KW];
  uint32_t mk[4 * NG], mv[4 * NG];
  int pos[WINDOW ? 4 : 1];
};

template <int D, int GS, int BITS, int FMT, bool WINDOW, int PK, int PKC>
__device__ inline void compute_step(const Buf<D, GS, WINDOW, PK>& b, uint32_t mj, int lo_pos,
                                    int lane, bool head_ok, const half4_t (&qB)[D / 16],
                                    const half8_t* qk_lds, const float (&sumq)[D / GS],
                                    float alpha, AttnState<D, GS>& st) {
  constexpr int NG = D / GS;
  constexpr int KM = GS / 16;
  constexpr int NT = D / 16;
  constexpr int GP = 16 / PK;
  constexpr int CW = D * BITS / 128;
  const int lg = lane >> 4, jl = (lane & 15) / GP;
  // integer codes of this class are in units of 2^-kUnitExp; the zero-point
  // term's sum of q (in units of 2^-24) is brought to the same unit
  constexpr float kSumqScale = (FMT == 1 && BITS != 2) ? 1.0f : (float)(1u << (24 - kUnitExp<BITS>));
  // S^T = K Q^T per group, the PK blocks packed side by side.  PK = 1: a
  // lane's 16 elements of a group are two 8-element k slices.  PK > 1: a k
  // slice holds the same 4 elements of blocks 2p and 2p+1, and the query
  // operand qK[p] of a lane is zero outside its own block's half, so column
  // h receives block h / GP's logits directly.
  // The query operands are read from LDS at every step (kept in registers
  // they would hold 4 or 8 VGPRs per 16 dims through the whole loop); the
  // empty asm makes the lane offset opaque so the reads stay in the loop.
  int qoff = lane * 16;
  asm volatile("" : "+v"(qoff));
  const char* qrow = (const char*)qk_lds + qoff;
  float4_t spk[NG];
  if constexpr (PK == 1) {
#pragma unroll
    for (int gi = 0; gi < NG; gi++) {
      spk[gi] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mm = 0; mm < KM; mm += 2)
        spk[gi] = mfma32(cat8(operand4<BITS, FMT>(b.kw, gi * (GS / 4) + 4 * mm),
                              operand4<BITS, FMT>(b.kw, gi * (GS / 4) + 4 * mm + 4)),
                         *(const half8_t*)(qrow + ((gi * KM + mm) / 2) * 1024), spk[gi]);
    }
  } else {
#pragma unroll
    for (int gi = 0; gi < NG; gi++) spk[gi] = (float4_t){0.f, 0.f, 0.f, 0.f};
    // pair by pair (the scheduling barrier keeps a pair's query operands from
    // being read ahead of the previous pair's products: 4 VGPRs each)
    // The operands of pair 1 (blocks 2 and 3, PK = 4) are those of pair 0
    // moved by 8 lanes (two block positions of 4 columns): lane l reads lane
    // l ^ 8's entry of the one table.
#pragma unroll
    for (int p = 0; p < PKC / 2; p++) {
      const char* qp = qrow;
      if (p == 1) {
        int qoff1 = (lane ^ 8) * 16;
        asm volatile("" : "+v"(qoff1));
        qp = (const char*)qk_lds + qoff1;
      }
#pragma unroll
      for (int gi = 0; gi < NG; gi++)
#pragma unroll
        for (int mm = 0; mm < KM; mm++)
          spk[gi] = mfma32(cat8(operand4<BITS, FMT>(b.kw + 2 * p * CW, gi * (GS / 4) + 4 * mm),
                                operand4<BITS, FMT>(b.kw + (2 * p + 1) * CW, gi * (GS / 4) + 4 * mm)),
                           *(const half8_t*)(qp + (gi * KM + mm) * 1024), spk[gi]);
      if (p + 1 < PKC / 2) __builtin_amdgcn_sched_barrier(0);
    }
  }
  // this lane's block (mask mj) and token quad (lg)
  uint32_t valid = (mj >> (4 * lg)) & 0xFu;
  if constexpr (WINDOW) {
#pragma unroll
    for (int r = 0; r < 4; r++)
      if (b.pos[r] < lo_pos) valid &= ~(1u << r);
  }
  st.natt += __builtin_popcount(valid);
  const uint32_t vb = head_ok ? valid : 0u;
  // (made opaque so that the three classes' scaled copies are not all held
  // in registers across the loop)
  float sq_c[NG];
#pragma unroll
  for (int gi = 0; gi < NG; gi++) {
    float t = sumq[gi];
    if constexpr (kSumqScale != 1.0f) asm volatile("" : "+v"(t));
    sq_c[gi] = t * kSumqScale;
  }
  float s2[4];
  float lmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    float x = 0.f;
#pragma unroll
    for (int gi = 0; gi < NG; gi++) {
      const uint32_t m = b.mk[r * NG + gi];
      x = fmaf(h_lo(m), spk[gi][r], fmaf(h_hi(m), sq_c[gi], x));
    }
    s2[r] = ((vb >> r) & 1u) ? x * alpha : -INFINITY;
    lmax = fmaxf(lmax, s2[r]);
  }
  // the running max is exact (every weight p <= 1, so P' = p sV stays within
  // the fp16 range for every scale the input range allows).  A head's running
  // max is held by all its lanes, so a lane's own values decide whether any
  // head grows; the head-wide max is only formed then.
  if (__builtin_amdgcn_ballot_w64(lmax > st.m2)) {
    const float bm = head_max<GP>(lmax);
    if (bm > st.m2) {
      if (st.m2 == -INFINITY) {
        st.Z = 0.f; st.S2 = 0.f;
      } else {
        const float sc = fast_exp2(st.m2 - bm);
        st.S2 = sc * (st.S2 + (st.m2 - bm) * st.Z);
        st.Z *= sc;
#pragma unroll
        for (int n = 0; n < NT; n++) st.acc[n] *= sc;
#pragma unroll
        for (int gi = 0; gi < NG; gi++) st.zacc[gi] *= sc;
      }
      st.m2 = bm;
    }
  }
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const float t = s2[r] - st.m2;
    p[r] = fast_exp2(t);                   // 0 for masked tokens (t = -inf)
    st.Z += p[r];
    st.S2 = fmaf(p[r], fmaxf(t, -200.f), st.S2);
  }
  // top-8: only values above the head-wide 8th-best bound can enter (the
  // bound changes only when values enter, so it is formed only then)
  if (__builtin_amdgcn_ballot_w64(lmax > st.thr)) {
#pragma unroll
    for (int r = 0; r < 4; r++)
      if (s2[r] > st.thr) topk_insert(st.top, s2[r]);
    st.thr = head_max<GP>(st.top[TOPK - 1]);
  }
  // P' = p sV per group as fp16 hi + lo (packed layout), and the zero-point
  // term.  A masked token has p = 0 and finite metadata: pools are cleared
  // when the cache is created, so a slot never written (the tail of an open
  // block, the block repeated to pad a last step) holds zeros.  hi = f16(p sV)
  // and lo = f16(p sV - hi) are each one mixed-precision fma rounded to
  // nearest into a half of the operand word (the product p sV is exact inside
  // the fma, so hi + lo carries ~22 significant bits); rounding toward zero
  // made every term's error one-signed, and with sharp attention the many
  // small P' terms (whose lo part sits in the fp16 subnormal range) then added
  // up to ~2e-3 on large-valued channels.
  half4_t pbh[NG], pbl[NG];
#pragma unroll
  for (int gi = 0; gi < NG; gi++) {
    float z = st.zacc[gi];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const uint32_t m = b.mv[r * NG + gi];
      const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(m & 0xFFFF));
      const _Float16 hi = (_Float16)fmaf(p[r], (float)sv, 0.f);
      pbh[gi][r] = hi;
      pbl[gi][r] = (_Float16)fmaf(p[r], (float)sv, -(float)hi);
      z = fmaf(p[r], h_hi(m), z);
    }
    st.zacc[gi] = z;
  }
  // O^T += V^T P', P' unpacked to each block's own columns
  if constexpr (PK == 1) {
#pragma unroll
    for (int n = 0; n < NT; n++) {
      const half4_t a = operand4<BITS, FMT>(b.vw, 4 * n);
      st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pbh[(16 * n) / GS], st.acc[n], 0, 0, 0);
      st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pbl[(16 * n) / GS], st.acc[n], 0, 0, 0);
    }
  } else {
    // blocks 2p and 2p+1 form one 32-token k slice (16x16x32): a lane's 4
    // tokens of block 2p, then the same 4 of block 2p+1.  P' stays packed: a
    // lane keeps its own block's half of the slice and zeroes the other, so
    // accumulator column h collects head h % GP over the blocks at position
    // h / GP of every step; the positions are summed once at the end.
#pragma unroll
    for (int jp = 0; jp < PKC; jp += 2) {
      const bool k0 = jl == jp, k1 = jl == jp + 1;
      half8_t bh[NG], bl[NG];
#pragma unroll
      for (int gi = 0; gi < NG; gi++) {
        bh[gi] = cat8(keep4(pbh[gi], k0), keep4(pbh[gi], k1));
        bl[gi] = cat8(keep4(pbl[gi], k0), keep4(pbl[gi], k1));
      }
#pragma unroll
      for (int n = 0; n < NT; n++) {
        const half8_t a = cat8(operand4<BITS, FMT>(b.vw + jp * CW, 4 * n),
                               operand4<BITS, FMT>(b.vw + (jp + 1) * CW, 4 * n));
        st.acc[n] = mfma32(a, bh[(16 * n) / GS], st.acc[n]);
        st.acc[n] = mfma32(a, bl[(16 * n) / GS], st.acc[n]);
      }
      if (jp + 2 < PKC) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Load step sigma of class C into a register buffer: lane l takes chunk l
// of the K and V codes of each of the PK blocks, the metadata of its own
// block's token quad and, with a window, its tokens' positions.  A last,
// partial step repeats a live block (its mask is read as 0).  The codes are
// read through a buffer resource per block record (base address in scalar
// registers, the lane's offset a constant), so no per-lane address arithmetic
// is spent on them; a padding step past the wave's last one gives its records
// zero length, and its code loads then return zeros without touching memory.
// The metadata and positions of a padding step are read from the first line
// of the repeated block in every lane (one cached line).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kRawBufferWord3 = 0x00020000;     // gfx9 raw buffer: 32-bit elements, no swizzle
template <int D, int GS, bool WINDOW, int PK, int C>
__device__ inline void load_step(Buf<D, GS, WINDOW, PK>& b, const uint8_t* pool_kvh, int64_t stride,
                                 const int32_t* slot_c, const int2* lv, int n, int sigma, int lane, bool pad) {
  constexpr int BITS = C == 0 ? 8 : (C == 1 ? 4 : 2);
  constexpr int NG = D / GS, CB = D * BITS / 32, CW = CB / 4, R = 128 * CB + 128 * NG, GP = 16 / PK;
  constexpr int PKC = pk_class<D, PK, C>();
  const int lg = lane >> 4, jl = (lane & 15) / GP;
  int ids[PKC];
#pragma unroll
  for (int j = 0; j < PKC; j++) {
    const int e = sigma * PKC + j;
    ids[j] = __builtin_amdgcn_readfirstlane(lv[e < n ? e : n - 1].x);
  }
#pragma unroll
  for (int j = 0; j < PKC; j++) {
    const uint8_t* rec = pool_kvh + (int64_t)ids[j] * stride;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, pad ? 0 : R, kRawBufferWord3);
    if constexpr (CW % 4 == 0) {
      // 16-byte unit i of chunk l sits at byte (64 i + l) 16 of the region
#pragma unroll
      for (int i = 0; i < CW / 4; i++) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + 1024 * i, 0, 0);
        const u32x4_t y = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + 1024 * i + 64 * CB, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; e++) { b.kw[j * CW + 4 * i + e] = x[e]; b.vw[j * CW + 4 * i + e] = y[e]; }
      }
    } else if constexpr (CW == 2) {
      const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(rs, lane * 8, 0, 0);
      const u32x2_t y = __builtin_amdgcn_raw_buffer_load_b64(rs, lane * 8 + 64 * CB, 0, 0);
      b.kw[j * CW] = x[0]; b.kw[j * CW + 1] = x[1]; b.vw[j * CW] = y[0]; b.vw[j * CW + 1] = y[1];
    } else {
      b.kw[j * CW] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4, 0, 0);
      b.vw[j * CW] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4 + 64 * CB, 0, 0);
    }
  }
  int idj = ids[0];                                 // this lane's block (block 0's when it has none)
#pragma unroll
  for (int j = 1; j < PKC; j++) idj = (jl == j && !pad) ? ids[j] : idj;
  const int lq = pad ? 0 : lg;
  const uint8_t* rj = pool_kvh + (int64_t)idj * stride + 128 * CB;
  const uint4* mkp = (const uint4*)(rj + lq * 16 * NG);
  const uint4* mvp = (const uint4*)(rj + 64 * NG + lq * 16 * NG);
#pragma unroll
  for (int i = 0; i < NG; i++) {
    const uint4 x = mkp[i], y = mvp[i];
    b.mk[4 * i] = x.x; b.mk[4 * i + 1] = x.y; b.mk[4 * i + 2] = x.z; b.mk[4 * i + 3] = x.w;
    b.mv[4 * i] = y.x; b.mv[4 * i + 1] = y.y; b.mv[4 * i + 2] = y.z; b.mv[4 * i + 3] = y.w;
  }
  if constexpr (WINDOW) {
    const int4* pr = (const int4*)(slot_c + ((int64_t)idj * TKV_BS + 4 * lq) * 2);
    const int4 x = pr[0], y = pr[1];
    b.pos[0] = x.x; b.pos[1] = x.z; b.pos[2] = y.x; b.pos[3] = y.z;
  }
}

// The wave's steps across the three classes, in order: the live blocks of a
// class (compacted: id, mask), PK per step, steps dealt round-robin to the nw
// waves.  Two register buffers alternate: the next step's loads are in flight
// while the current step is computed, also across a class boundary.  Past the
// last step a wave issues the same load instructions (code loads of
// zero-length records, metadata from one cached line), so every path issues
// the same loads, the compiler's waits stay exact, and the padding is cheap.
template <int D, int GS, bool WINDOW, int PK, int FMT>
__device__ inline void run_steps(const AttnParams& P, const int2* live, int lmax, const int* nl, int kvh, int lo_pos,
                                 int lane, int w, int nw, bool head_ok, const half4_t (&qB)[D / 16],
                                 const half8_t* qk_lds, const float (&sumq)[D / GS],
                                 float alpha, AttnState<D, GS>& st) {
  typedef Buf<D, GS, WINDOW, PK> B;
  constexpr int GP = 16 / PK;
  const int jl = (lane & 15) / GP;
  // wave-uniform (read from LDS, so the compiler cannot tell): the step
  // index, the class branches and the block addresses stay scalar
  const int n0 = __builtin_amdgcn_readfirstlane(nl[0]), n1 = __builtin_amdgcn_readfirstlane(nl[1]),
            n2 = __builtin_amdgcn_readfirstlane(nl[2]);
  constexpr int P0 = pk_class<D, PK, 0>(), P1 = pk_class<D, PK, 1>(), P2 = pk_class<D, PK, 2>();
  const int c1 = (n0 + P0 - 1) / P0, c2 = c1 + (n1 + P1 - 1) / P1, T = c2 + (n2 + P2 - 1) / P2;
  const int2* l0 = live;
  const int2* l1 = live + lmax;
  const int2* l2 = live + 2 * lmax;
  // the per-class pools and slot tables in registers (indexing the argument
  // struct by a run-time class would copy it to scratch)
  const uint8_t* pool0 = P.S.pool[0];
  const uint8_t* pool1 = P.S.pool[1];
  const uint8_t* pool2 = P.S.pool[2];
  const int32_t* slt0 = P.S.slot[0];
  const int32_t* slt1 = P.S.slot[1];
  const int32_t* slt2 = P.S.slot[2];
  // a block stores every layer's KV heads: this layer's head kvh is head
  // layer*Hkv + kvh of Hst per block
  const int64_t Hst = P.S.Hst, hk = (int64_t)P.layer * P.S.Hkv + kvh;
  const int64_t R0 = P.S.bh_bytes[0], R1 = P.S.bh_bytes[1], R2 = P.S.bh_bytes[2];
  const uint8_t* pk0 = pool0 + hk * R0;
  const uint8_t* pk1 = pool1 + hk * R1;
  const uint8_t* pk2 = pool2 + hk * R2;
  auto load = [&](B& b, int g) {
    const bool pad = g >= T;
    g = pad ? T - 1 : g;
    if (g < c1) load_step<D, GS, WINDOW, PK, 0>(b, pk0, Hst * R0, slt0, l0, n0, g, lane, pad);
    else if (g < c2) load_step<D, GS, WINDOW, PK, 1>(b, pk1, Hst * R1, slt1, l1, n1, g - c1, lane, pad);
    else load_step<D, GS, WINDOW, PK, 2>(b, pk2, Hst * R2, slt2, l2, n2, g - c2, lane, pad);
  };
  auto mask_of = [&](const int2* lv, int n, int sigma, int pkc) -> uint32_t {
    const int e = sigma * pkc + jl;                 // this lane's block
    return (jl < pkc && e < n) ? (uint32_t)lv[e].y : 0u;
  };
  // alpha is the logit factor for plain values.  The operands of a class are
  // its codes in units of 2^-kUnitExp (integer codes) or the values themselves
  // (float codes), so each class has its own logit factor, and the V-side
  // accumulator has a unit too.  A wave's steps go through the classes in
  // order: at its first step of a class with another unit, the accumulator is
  // brought to that unit once (a power of two, exact), and st.vunit carries
  // the unit to the epilogue.
  constexpr float u0 = FMT ? 1.0f : (float)(1u << kUnitExp<8>);
  constexpr float u1 = FMT ? 1.0f : (float)(1u << kUnitExp<4>);
  constexpr float u2 = (float)(1u << kUnitExp<2>);
  auto to_unit = [&](float u) {
    if (st.vunit != u) {
      const float f = st.vunit / u;
#pragma unroll
      for (int n = 0; n < D / 16; n++) st.acc[n] *= f;
      st.vunit = u;
    }
  };
  int g = w;
  if (g >= T) return;
  // The two waves of a SIMD compete for issue and the arbiter favours the
  // older one; a wave lowers its priority as it advances through its steps,
  // so the one behind is favoured and the pair ends closer together.
  const int Tw = (T - w + nw - 1) / nw;          // this wave's steps
  int k = 0;
  auto set_priority = [&]() {
    const int lv = 3 - (4 * k) / Tw;
    if (lv >= 3) __builtin_amdgcn_s_setprio(3);
    else if (lv == 2) __builtin_amdgcn_s_setprio(2);
    else if (lv == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  };
  B nxt;
  load(nxt, g);
  __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
  // one loop per class (a wave's steps go through the classes in order), so
  // that each loop body holds one compute path: the three paths in one body
  // kept the union of their temporaries live and copied the accumulators at
  // the back edge (253 VGPRs; one path per loop: 194)
#pragma nounroll
  while (g < c1) {
    const B cur = nxt;
    load(nxt, g + nw);
    __builtin_amdgcn_sched_barrier(0);
    set_priority();
    compute_step<D, GS, 8, FMT, WINDOW, PK, P0>(cur, mask_of(l0, n0, g, P0), lo_pos, lane, head_ok, qB, qk_lds, sumq,
                                             alpha * u0, st);
    k++;
    g += nw;
  }
  if (g < c2) to_unit(u1);
#pragma nounroll
  while (g < c2) {
    const B cur = nxt;
    load(nxt, g + nw);
    __builtin_amdgcn_sched_barrier(0);
    set_priority();
    compute_step<D, GS, 4, FMT, WINDOW, PK, P1>(cur, mask_of(l1, n1, g - c1, P1), lo_pos, lane, head_ok, qB, qk_lds,
                                             sumq, alpha * u1, st);
    k++;
    g += nw;
  }
  if (g < T) to_unit(u2);
#pragma nounroll
  while (g < T) {
    const B cur = nxt;
    load(nxt, g + nw);
    __builtin_amdgcn_sched_barrier(0);
    set_priority();
    compute_step<D, GS, 2, 0, WINDOW, PK, P2>(cur, mask_of(l2, n2, g - c2, P2), lo_pos, lane, head_ok, qB, qk_lds, sumq,
                                           alpha * u2, st);
    k++;
    g += nw;
  }
  __builtin_amdgcn_s_setprio(0);
}

// ---------------------------------------------------------------------------
// Records: [D accumulator][m2, Z, S2, n][top8] with the zero-point term folded
// into the accumulator, all relative to the record's own max m2 (log2 units).
// merge_records folds nrec records (stride floats apart) into registers of
// one wave (the split combine): acc for dims lane and lane + 64, and the
// merged scalars.
// ---------------------------------------------------------------------------
struct Merged {
  float a0, a1, m, Z, S2;
  int n;
  float top[TOPK];
};

template <int D>
__device__ inline void merge_records(const float* recs, int stride, int nrec, int lane, Merged& M) {
  float mr = -INFINITY, zr = 0.f, sr = 0.f, nr = 0.f;
  if (lane < nrec) {
    const float* rec = recs + (int64_t)lane * stride;
    nr = rec[D + 3];
    if (nr > 0.f) { mr = rec[D]; zr = rec[D + 1]; sr = rec[D + 2]; }
  }
  const float m = first_lanes_max(mr, nrec);
  const float sc = nr > 0.f ? exp2f(mr - m) : 0.f;
  const float Z = first_lanes_sum(sc * zr, nrec);
  const float S2 = first_lanes_sum(nr > 0.f ? sc * (sr + (mr - m) * zr) : 0.f, nrec);
  const float nn = first_lanes_sum(nr, nrec);
#pragma unroll
  for (int i = 0; i < TOPK; i++) M.top[i] = (lane < nrec && nr > 0.f) ? recs[(int64_t)lane * stride + D + 4 + i] : -INFINITY;
  first_lanes_topk(M.top, nrec);
  float a0 = 0.f, a1 = 0.f;
  for (int r = 0; r < nrec; r++) {
    const float f = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc), r));
    if (f == 0.f) continue;
    const float* rec = recs + (int64_t)r * stride;
    a0 = fmaf(f, rec[lane], a0);
    if (D > 64) a1 = fmaf(f, rec[lane + 64], a1);
  }
  M.a0 = a0; M.a1 = a1; M.m = m; M.Z = Z; M.S2 = S2; M.n = (int)nn;
}

// The staged self token of one query head: its logit (log2 units) and its V
// row at dims lane and lane + 64.  Loaded in the prologue when the head's
// wave is known, so that its latency hides behind the block loads.
struct SelfTok {
  float s2, v0, v1;
};
template <int D>
__device__ inline SelfTok load_self(const AttnParams& P, int b, int hq, int lane) {
  const DevState& S = P.S;
  const int G = S.Hq / S.Hkv, kvh = hq / G;
  const uint16_t* qr = P.q + ((int64_t)b * S.Hq + hq) * D;
  const float* kr = P.k_self + ((int64_t)b * S.Hkv + kvh) * D;
  const float* vr = P.v_self + ((int64_t)b * S.Hkv + kvh) * D;
  float d = 0.f;
  for (int i = lane; i < D; i += 64) d = fmaf(__builtin_bit_cast(float, (uint32_t)qr[i] << 16), kr[i], d);
  d = pair_sum<32>(pair_sum<16>(pair_sum<8>(pair_sum<4>(pair_sum<2>(pair_sum<1>(d))))));
  SelfTok t;
  t.s2 = d * (LOG2E / sqrtf((float)D));
  t.v0 = vr[lane];
  t.v1 = D > 64 ? vr[lane + 64] : 0.f;
  return t;
}

// Add the staged self token and the sink; write the output and statistics.
// sink: the head's sink logit (read by the caller ahead of time; unused
// without sinks).
template <int D>
__device__ inline void finalize_head(const AttnParams& P, int b, int hq, int lane, Merged M, const SelfTok& self,
                                     float sink) {
  const DevState& S = P.S;
  int n = M.n;
  if (P.k_self) {
    const float self2 = self.s2;
    const float m = fmaxf(M.m, self2);
    const float sc = M.n > 0 ? exp2f(M.m - m) : 0.f;
    const float ps = exp2f(self2 - m);
    M.S2 = sc * (M.S2 + (M.n > 0 ? (M.m - m) * M.Z : 0.f)) + ps * (self2 - m);
    M.Z = sc * M.Z + ps;
    M.a0 = fmaf(ps, self.v0, sc * M.a0);
    if (D > 64) M.a1 = fmaf(ps, self.v1, sc * M.a1);
    M.m = m;
    topk_insert(M.top, self2);
    n += 1;
  }
  float* out = P.out + ((int64_t)b * S.Hq + hq) * D;
  float* st = P.stats ? P.stats + (int64_t)b * P.stats_stride + hq * 3 : nullptr;
  if (n == 0) {
    out[lane] = 0.f;
    if (D > 64) out[lane + 64] = 0.f;
    if (st && lane == 0) { st[0] = 0.f; st[1] = 0.f; st[2] = 0.f; }
  } else {
    float den = M.Z;
    if (P.sinks) den += exp2f(sink * LOG2E - M.m);
    const float inv = 1.0f / den;
    out[lane] = M.a0 * inv;
    if (D > 64) out[lane + 64] = M.a1 * inv;
    if (st && lane == 0) {
      const float H = logf(M.Z) - LN2 * M.S2 / M.Z;
      float mk = 0.f;
      const int kk = P.topk < n ? P.topk : n;
#pragma unroll
      for (int i = 0; i < TOPK; i++) mk += i < kk ? exp2f(M.top[i] - M.m) : 0.f;
      st[0] = H;
      st[1] = n >= 2 ? H / logf((float)n) : 0.f;
      st[2] = mk / M.Z;
    }
  }
  if (P.n_attended && hq == 0 && lane == 0) P.n_attended[b] = n;
}

// Merge the records of the NW waves of a work-group (LDS, [wave][head][RS]
// floats from base, rstride floats apart): the merged scalars of this lane's
// head, and the slices n = w, w + NW, ... of its accumulator.  Every record's
// reads are issued before the sums, which run in wave order; a record with
// no tokens (scale 0) adds zeros, so the sums equal those over the non-empty
// records alone.
template <int NW, int NT>
__device__ inline void merge_waves(const float* base, int rstride, int w, int lg, float& m, float& Z, float& S2,
                                   float& natt, float4_t (&a)[NT]) {
  float mr[NW], zr[NW], sr[NW], nr[NW];
#pragma unroll
  for (int r = 0; r < NW; r++) {
    const float4 x = *(const float4*)(base + r * rstride + NT * 16);
    mr[r] = x.x; zr[r] = x.y; sr[r] = x.z; nr[r] = x.w;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < NW; r++) mx = nr[r] > 0.f ? fmaxf(mx, mr[r]) : mx;
  float sc[NW];
  Z = 0.f; S2 = 0.f; natt = 0.f;
#pragma unroll
  for (int r = 0; r < NW; r++) {
    sc[r] = nr[r] > 0.f ? exp2f(mr[r] - mx) : 0.f;
    Z = fmaf(sc[r], zr[r], Z);
    S2 = nr[r] > 0.f ? fmaf(sc[r], sr[r] + (mr[r] - mx) * zr[r], S2) : S2;
    natt += nr[r];
  }
  m = mx;
#pragma unroll
  for (int n = 0; n < NT; n++) {
    if (n % NW != w) continue;
    float4_t x[NW];
#pragma unroll
    for (int r = 0; r < NW; r++) x[r] = *(const float4_t*)(base + r * rstride + 16 * n + 4 * lg);
    float4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < NW; r++) t += sc[r] * x[r];
    a[n] = t;
  }
}

template <int D, int GS, bool WINDOW, int PK, int FMT>
__global__ __launch_bounds__(512) void k_attn(AttnParams P) {
  constexpr int NG = D / GS;
  constexpr int KM = GS / 16;
  constexpr int NT = D / 16;
  constexpr int GP = 16 / PK;
  constexpr int RS = D + PART_X;                 // record stride (floats)
  // Dynamic LDS: the waves' records; the live block lists are a static array.
  // Dynamic LDS: the waves' records [nw][G][RS] floats, then the split's live
  // block lists [3][max_blocks] (id, mask) and their counts.
  extern __shared__ __align__(16) float lds[];
  const DevState& S = P.S;
  // grid row blockIdx.z is batch entry b, or, with a dispatch order made for
  // this batch size, the entry the order puts there (clamped into the batch)
  const int split = blockIdx.x, kvh = blockIdx.y, batch = gridDim.z;
  int b = blockIdx.z;
  if (P.order && P.order[0] == batch) b = min(max(P.order[1 + blockIdx.z], 0), batch - 1);
  const int s = P.seq_ids[b];
  // the wave index is uniform across its lanes: say so to the compiler
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nw = blockDim.x >> 6;
  const int lg = lane >> 4, h = lane & 15;
  const int G = S.Hq / S.Hkv;
  const bool col_ok = h < G;                     // MFMA column h is a real head
  const int hp = h % GP;                         // head of this lane in the packed layout
  const bool head_ok = hp < G;
  const bool seq_ok = s >= 0 && s < S.max_seqs;
  // Query rows, read now and converted after the block lists (so that their
  // latency overlaps the list reads).  Lane (h, lg) holds the query of the
  // head of its packed column, h mod GP (zero for a padding column).
  uint4 qraw[NG][GS / 32];
  {
    const uint16_t* qr = P.q + ((int64_t)b * S.Hq + (int64_t)kvh * G + (head_ok ? hp : 0)) * D;
#pragma unroll
    for (int gi = 0; gi < NG; gi++)
#pragma unroll
      for (int i = 0; i < GS / 32; i++) qraw[gi][i] = ((const uint4*)(qr + gi * GS + lg * (GS / 4)))[i];
  }
  // What the finalize needs besides the records is read now by wave 0 and
  // kept in LDS through the loop (s_fin): the sink logits of the group's
  // heads and, when the self token is finalized here (one split), its V row
  // (shared by the group's heads) and its logit for each head, computed from
  // its K row over this lane's query dims with the query conversion below.
  __shared__ __align__(16) float s_fin[2 * 64 + 2 * 16];   // V row [128], self logits [16], sinks [16]
  const bool self_here = P.splits == 1 && P.k_self != nullptr && w == 0;
  const float sinks_g = (w == 0 && P.sinks && lane < G) ? P.sinks[kvh * G + lane] : 0.f;
  float4 kself[NG][GS / 16];
  float selfv0 = 0.f, selfv1 = 0.f;
  if (self_here) {
    const float* kr = P.k_self + ((int64_t)b * S.Hkv + kvh) * D;
    const float* vr = P.v_self + ((int64_t)b * S.Hkv + kvh) * D;
#pragma unroll
    for (int gi = 0; gi < NG; gi++)
#pragma unroll
      for (int i = 0; i < GS / 16; i++) kself[gi][i] = ((const float4*)(kr + gi * GS + lg * (GS / 4)))[i];
    selfv0 = vr[lane];
    selfv1 = D > 64 ? vr[lane + 64] : 0.f;
  }
  const float alpha = LOG2E / sqrtf((float)D);
  AttnState<D, GS> st;
#pragma unroll
  for (int n = 0; n < NT; n++) st.acc[n] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int gi = 0; gi < NG; gi++) st.zacc[gi] = 0.f;
  st.m2 = -INFINITY; st.Z = 0.f; st.S2 = 0.f; st.natt = 0;
#pragma unroll
  for (int i = 0; i < TOPK; i++) st.top[i] = -INFINITY;
  st.thr = -INFINITY;
  st.vunit = FMT ? 1.0f : kCodeScale;        // the unit of the first class (8-bit codes)
  // The split's live blocks of each class, into LDS, in list order: wave w
  // takes the classes c = w, w + nw, ... (all three with one wave), reads
  // their block-table entries 64 at a time and their block records, and
  // keeps, by ballot, the blocks with a valid token (and, with a window, a
  // position inside it).  The first 64 entries of each of a wave's classes
  // are read together with the sequence record, before the split's range is
  // known, and the block records of those first entries are read together
  // for all of the wave's classes, so the chain of dependent reads before
  // the first codes is three deep (sequence id; sequence record and table;
  // block records) whatever the number of waves.
  const int lo_pos = WINDOW ? P.q_pos[b] - P.window + 1 : 0;
  const int lmax = S.max_blocks;
  int2* live = (int2*)(lds + (int64_t)nw * G * RS);       // [3][lmax]
  int* nlive = (int*)(live + 3 * lmax);
  if (seq_ok) {
    const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
    const int32_t* bt = S.btab + (int64_t)s * 3 * lmax;
    int spec[3];
#pragma unroll
    for (int k = 0; k < 3; k++) {
      const int c = w + k * nw;
      spec[k] = c < 3 && lane < lmax ? bt[c * lmax + lane] : 0;
    }
    const int nb0 = q[Q_NBLK + 0], nb1 = q[Q_NBLK + 1], nb2 = q[Q_NBLK + 2];
    // byte-balanced split of [8-bit | 4-bit | 2-bit] block lists (< 2^31 bytes per sequence)
    const int w0 = (int)S.bh_bytes[0], w1 = (int)S.bh_bytes[1], w2 = (int)S.bh_bytes[2];
    const int P1 = nb0 * w0, P2 = P1 + nb1 * w1, W = P2 + nb2 * w2;
    const int lo = (int)((int64_t)W * split / P.splits), hi = (int)((int64_t)W * (split + 1) / P.splits);
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
    int j0s[3], j1s[3], ids[3], ms[3];
#pragma unroll
    for (int k = 0; k < 3; k++) {
      const int c = w + k * nw;
      j0s[k] = j1s[k] = 0;
      if (c < 3) {
        const int off = c == 0 ? 0 : (c == 1 ? P1 : P2);
        const int wb = c == 0 ? w0 : (c == 1 ? w1 : w2);
        const int nbc = c == 0 ? nb0 : (c == 1 ? nb1 : nb2);
        const int a = lo - off, z = hi - off;
        j0s[k] = a <= 0 ? 0 : min(nbc, (a + wb - 1) / wb);
        j1s[k] = z <= 0 ? 0 : min(nbc, (z + wb - 1) / wb);
      }
      const int jj = j0s[k] + lane;
      ids[k] = jj < j1s[k] ? (j0s[k] == 0 ? spec[k] : bt[c * lmax + jj]) : 0;
    }
#pragma unroll
    for (int k = 0; k < 3; k++) {
      const int c = w + k * nw;
      ms[k] = 0;
      if (c < 3 && j0s[k] + lane < j1s[k]) {
        const int2 rec = *(const int2*)(pick3(S.blk, c) + (int64_t)ids[k] * TKV_BLK_W);
        ms[k] = rec.x;
        if (WINDOW && rec.y < lo_pos) ms[k] = 0;
      }
    }
#pragma unroll
    for (int k = 0; k < 3; k++) {
      const int c = w + k * nw;
      if (c >= 3) break;
      const int32_t* blk = pick3(S.blk, c);
      const uint64_t bal0 = __builtin_amdgcn_ballot_w64(ms[k] != 0);
      if (ms[k] != 0) live[c * lmax + __popcll(bal0 & lt)] = make_int2(ids[k], ms[k]);
      int cnt = __popcll(bal0);
      for (int j = j0s[k] + 64; j < j1s[k]; j += 64) {
        const int jj = j + lane;
        int id = 0, m = 0;
        if (jj < j1s[k]) {
          id = bt[c * lmax + jj];
          const int2 rec = *(const int2*)(blk + (int64_t)id * TKV_BLK_W);
          m = rec.x;
          if (WINDOW && rec.y < lo_pos) m = 0;
        }
        const uint64_t bal = __builtin_amdgcn_ballot_w64(m != 0);
        if (m != 0) live[c * lmax + cnt + __popcll(bal & lt)] = make_int2(id, m);
        cnt += __popcll(bal);
      }
      if (lane == 0) nlive[c] = cnt;
    }
  } else {
    for (int c = w; c < 3; c += nw)
      if (lane == 0) nlive[c] = 0;
  }
  // query B operand: qB[gi*KM + mm][e] of lane (h, lg) holds dim
  // gi*GS + lg*(GS/4) + 4mm + e of column h's head; and sum(q) per group (over
  // the four lane groups of the column), in code units
  half4_t qB[NG * KM];
  float sumq[NG];
  float selfdot = 0.f;                                   // q . k_self over this lane's dims
#pragma unroll
  for (int gi = 0; gi < NG; gi++) {
    uint32_t wq[GS / 8];
#pragma unroll
    for (int i = 0; i < GS / 32; i++) {
      wq[4 * i] = qraw[gi][i].x; wq[4 * i + 1] = qraw[gi][i].y; wq[4 * i + 2] = qraw[gi][i].z; wq[4 * i + 3] = qraw[gi][i].w;
    }
    float sq = 0.f;
#pragma unroll
    for (int mm = 0; mm < KM; mm++) {
      half4_t v;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int j = 4 * mm + e;
        const uint32_t bits = (j & 1) ? (wq[j >> 1] & 0xFFFF0000u) : (wq[j >> 1] << 16);
        const float x = head_ok ? __builtin_bit_cast(float, bits) : 0.f;
        v[e] = (_Float16)x;
        sq += (float)v[e];
        if (self_here) {
          const float4 k4 = kself[gi][j >> 2];
          selfdot = fmaf(x, (j & 3) == 0 ? k4.x : (j & 3) == 1 ? k4.y : (j & 3) == 2 ? k4.z : k4.w, selfdot);
        }
      }
      qB[gi * KM + mm] = v;
    }
    sumq[gi] = pair_sum<32>(pair_sum<16>(sq)) * kCodeUnit;
  }
  // lane (h, lg) now holds the self logit (log2 units) of its column's head
  if (w == 0) {
    const float self2 = pair_sum<32>(pair_sum<16>(selfdot)) * alpha;
    s_fin[lane] = selfv0;
    s_fin[64 + lane] = selfv1;
    if (lane < 16) { s_fin[128 + lane] = self2; s_fin[144 + lane] = sinks_g; }
  }
  // K-side query operands in LDS, identical in every wave (wave 0 stores
  // them), [k slice][lane].  One block per step: 16 dims per k slice.  Packed
  // blocks: the lane's query in the half of the k slice that holds its own
  // block (position 0 or 1; zeros at positions 2 and 3), [16 dims][lane].
  __shared__ half8_t s_qk[NT * 64];
  if (w == 0) {
    if constexpr (PK == 1) {
#pragma unroll
      for (int i = 0; i < NT; i += 2) s_qk[(i / 2) * 64 + lane] = cat8(qB[i], qB[i + 1]);
    } else {
      const int jq = (lane & 15) / GP;
#pragma unroll
      for (int i = 0; i < NT; i++) s_qk[i * 64 + lane] = cat8(keep4(qB[i], jq == 0), keep4(qB[i], jq == 1));
    }
  }
  __syncthreads();
  run_steps<D, GS, WINDOW, PK, FMT>(P, live, lmax, nlive, kvh, lo_pos, lane, w, nw, head_ok, qB, s_qk, sumq,
                                    alpha, st);
  // accumulator columns h and h + GP*i hold one head (block positions): sum
  // them into every column of the row (rotations inside the 16-lane row)
  if constexpr (PK > 1) {
#pragma unroll
    for (int n = 0; n < NT; n++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        float v = st.acc[n][r];
        if constexpr (GP <= 4) v += dpp_f<0x124>(v);              // row_ror:4
        v += dpp_f<0x128>(v);                                     // row_ror:8
        st.acc[n][r] = v;
      }
  }
  // this wave's state per head: sums over the lanes holding the head.  From
  // here on lane 16 lg + h (h < G) holds head h: dims 16 n + 4 lg .. + 3 of
  // every 16-dim slice n and the head's scalars, and the epilogue runs for all
  // heads at once on those lanes.
  st.Z = head_sum<GP>(st.Z);
  st.S2 = head_sum<GP>(st.S2);
#pragma unroll
  for (int gi = 0; gi < NG; gi++) st.zacc[gi] = head_sum<GP>(st.zacc[gi]);
  st.natt = (int)head_sum<GP>((float)st.natt);
  head_topk<GP>(st.top);
  const int he = col_ok ? h : 0;                  // the head these lanes finish (lanes h >= G repeat head 0)
  float4_t a[NT];
#pragma unroll
  for (int n = 0; n < NT; n++) a[n] = st.acc[n] * st.vunit + st.zacc[(16 * n) / GS];
  float m = st.m2, Z = st.Z, S2 = st.S2, natt = (float)st.natt;
  if (nw > 1) {
    // Merge the waves' records (through LDS): every wave forms the merged
    // scalars of its lanes' heads, finishes the slices n = w, w + nw, ... and
    // wave 0 also the top-8 list.
    if (col_ok) {
      float* rec = lds + ((int64_t)w * G + h) * RS;
#pragma unroll
      for (int n = 0; n < NT; n++) *(float4_t*)(rec + 16 * n + 4 * lg) = a[n];
      if (lg == 0) {
        *(float4*)(rec + D) = make_float4(m, Z, S2, natt);
#pragma unroll
        for (int i = 0; i < TOPK; i += 4) *(float4*)(rec + D + 4 + i) = make_float4(st.top[i], st.top[i + 1], st.top[i + 2], st.top[i + 3]);
      }
    }
    lds_barrier();
    const float* base = lds + (int64_t)he * RS;
    const int rstride = G * RS;
    if (nw == 2) merge_waves<2, NT>(base, rstride, w, lg, m, Z, S2, natt, a);
    else if (nw == 4) merge_waves<4, NT>(base, rstride, w, lg, m, Z, S2, natt, a);
    else merge_waves<8, NT>(base, rstride, w, lg, m, Z, S2, natt, a);
    if (w == 0) {
      // lane group lg merges the lists of records lg, lg + 4; then across groups
#pragma unroll
      for (int i = 0; i < TOPK; i++) st.top[i] = lg < nw ? base[lg * rstride + D + 4 + i] : -INFINITY;
      if (lg + 4 < nw) {
        float O[TOPK];
#pragma unroll
        for (int i = 0; i < TOPK; i++) O[i] = base[(lg + 4) * rstride + D + 4 + i];
        topk_merge(st.top, O);
      }
      pair_topk<16>(st.top);
      pair_topk<32>(st.top);
    }
  }
  // slices of this wave: n = w, w + nw, ... (every slice with one wave)
  auto mine = [&](int n) { return nw == 1 || n % nw == w; };
  const int hq = kvh * G + he;
  if (P.splits == 1) {
    // add the staged self token and the sink; write the outputs and statistics
    if (P.k_self) {
      const float self2 = s_fin[128 + he];
      const float mm = fmaxf(m, self2);
      const float sc = natt > 0.f ? exp2f(m - mm) : 0.f;
      const float ps = exp2f(self2 - mm);
      S2 = sc * (S2 + (natt > 0.f ? (m - mm) * Z : 0.f)) + ps * (self2 - mm);
      Z = fmaf(sc, Z, ps);
#pragma unroll
      for (int n = 0; n < NT; n++)
        if (mine(n)) {
          const float4 v = *(const float4*)(s_fin + 16 * n + 4 * lg);
          a[n] = (float4_t){fmaf(ps, v.x, sc * a[n][0]), fmaf(ps, v.y, sc * a[n][1]), fmaf(ps, v.z, sc * a[n][2]),
                            fmaf(ps, v.w, sc * a[n][3])};
        }
      m = mm;
      if (w == 0) topk_insert(st.top, self2);
      natt += 1.f;
    }
    const int nn = (int)natt;
    float inv = 0.f;
    if (nn > 0) {
      float den = Z;
      if (P.sinks) den += exp2f(s_fin[144 + he] * LOG2E - m);
      inv = 1.0f / den;
    }
    if (col_ok) {
      float* out = P.out + ((int64_t)b * S.Hq + hq) * D;
#pragma unroll
      for (int n = 0; n < NT; n++)
        if (mine(n)) *(float4_t*)(out + 16 * n + 4 * lg) = a[n] * inv;
      if (w == 0 && lg == 0 && P.stats) {
        float* sp = P.stats + (int64_t)b * P.stats_stride + hq * 3;
        if (nn == 0) {
          sp[0] = 0.f; sp[1] = 0.f; sp[2] = 0.f;
        } else {
          const float H = logf(Z) - LN2 * S2 / Z;
          float mk = 0.f;
          const int kk = P.topk < nn ? P.topk : nn;
#pragma unroll
          for (int i = 0; i < TOPK; i++) mk += i < kk ? exp2f(st.top[i] - m) : 0.f;
          sp[0] = H;
          sp[1] = nn >= 2 ? H / logf((float)nn) : 0.f;
          sp[2] = mk / Z;
        }
      }
      if (w == 0 && lane == 0 && kvh == 0 && P.n_attended) P.n_attended[b] = nn;
    }
  } else if (col_ok) {
    // this split's partial record; the combine kernel merges the splits
    float* rec = P.part + (((int64_t)b * S.Hq + hq) * P.splits + split) * RS;
#pragma unroll
    for (int n = 0; n < NT; n++)
      if (mine(n)) *(float4_t*)(rec + 16 * n + 4 * lg) = a[n];
    if (w == 0 && lg == 0) {
      *(float4*)(rec + D) = make_float4(m, Z, S2, natt);
#pragma unroll
      for (int i = 0; i < TOPK; i += 4) *(float4*)(rec + D + 4 + i) = make_float4(st.top[i], st.top[i + 1], st.top[i + 2], st.top[i + 3]);
    }
  }
  if (split == 0 && kvh == 0 && threadIdx.x == 0 && !seq_ok) record_error(S.hdr, TKV_EINVAL, s < 0 ? TKV_INF : s);
}

// Merge the splits of each (batch entry, query head): one wave per head.
template <int D>
__global__ __launch_bounds__(256) void k_combine(AttnParams P) {
  const DevState& S = P.S;
  const int lane = threadIdx.x & 63;
  const int hq = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6), b = blockIdx.y;
  if (hq >= S.Hq) return;
  const float* recs = P.part + ((int64_t)b * S.Hq + hq) * P.splits * (D + PART_X);
  const SelfTok self = P.k_self ? load_self<D>(P, b, hq, lane) : SelfTok{0.f, 0.f, 0.f};
  const float sink = P.sinks ? P.sinks[hq] : 0.f;
  Merged M;
  merge_records<D>(recs, D + PART_X, P.splits, lane, M);
  finalize_head<D>(P, b, hq, lane, M, self, sink);
}

// ---------------------------------------------------------------------------
// Launch shape: one work-group of nw waves per (batch entry, KV head, split);
// about two resident waves per SIMD (1024 SIMDs), the waves of a work-group
// sharing the sequence's blocks; extra splits only when the batch is small.
// LDS per work-group: nw step slots of PK records, the block lists.
// ---------------------------------------------------------------------------
static const int kTargetWaves = 2048;
static const int kMaxLds = 160 * 1024;

// blocks packed side by side per step: 16 / roundup(G, 4), and none with
// more than two groups per head.  At D = 128 the 8-bit class takes two blocks
// per step whatever the packing (pk_class); with a window, where each lane
// also holds its tokens' positions, the packing stays at two there: four
// spill.  (A spill reload in the loop waits for every load in flight, the
// next step's included.)
static int pack_of(const tkv_cache* c, int G, bool window) {
  if (c->S.D / c->S.g > 2) return 1;
  if (G <= 4 && (c->S.D == 64 || !window)) return 4;
  return G <= 8 ? 2 : 1;
}

// dynamic LDS: the waves' records, the live block lists and their counts
static int lds_bytes(const tkv_cache* c, int nw) {
  const int D = c->S.D, G = c->S.Hq / c->S.Hkv;
  return nw * G * (D + PART_X) * (int)sizeof(float) + 3 * c->S.max_blocks * 8 + 16;
}
static const int kStaticLds = 8192 + 640 + 384;                     // query operands, finalize inputs (and slack)

void attn_plan(const tkv_cache* c, int batch, int num_splits, bool ordered, int* nw_out, int* splits_out) {
  const int units = batch * c->S.Hkv > 0 ? batch * c->S.Hkv : 1;
  int nw = 1;
  while (nw < 8 && units * nw * 2 <= kTargetWaves && lds_bytes(c, nw * 2) + kStaticLds <= kMaxLds) nw *= 2;
  // A grid dispatched longest first runs in two rounds of two-wave
  // work-groups: the first round holds the longest sequences, each with two
  // waves, and the short ones follow as slots free up.  (Only where the
  // units fill the machine by themselves, so the split count is 1 either way.)
  if (ordered && units >= kTargetWaves && lds_bytes(c, 2) + kStaticLds <= kMaxLds) nw = 2;
  int splits = num_splits;
  if (splits <= 0) {
    splits = (kTargetWaves + units * nw - 1) / (units * nw);
    // at most as many splits as give each wave about four steps when the
    // block lists are full (more would leave waves idle and add a combine)
    const int pk = pack_of(c, c->S.Hq / c->S.Hkv, false);
    const int cap = (3 * c->S.max_blocks) / (4 * nw * pk) > 1 ? (3 * c->S.max_blocks) / (4 * nw * pk) : 1;
    if (splits > cap) splits = cap;
    if (splits > 64) splits = 64;
    if (splits < 1) splits = 1;
  }
  *nw_out = nw;
  *splits_out = splits;
}

// Dispatch order of the batch entries, longest first.  The dispatcher deals
// consecutive work-groups round-robin over the XCDs and their compute units,
// so a compute unit receives work-groups far apart in the grid; in batch
// order (lengths at random) some compute units then get several long
// sequences and finish last, while in length order every compute unit gets
// one work-group of each length range.  Entries are counted into 256 length
// buckets (a counting sort on the sequence's code bytes per KV head; the
// order inside a bucket is the order of arrival).  The attention's results do
// not depend on this order.  One work-group, one thread per batch entry.
__global__ __launch_bounds__(1024) void k_attn_order(DevState S, const int32_t* seq_ids, int batch, int32_t* order) {
  __shared__ int s_hist[256];
  __shared__ unsigned s_max;
  const int b = threadIdx.x;
  if (b < 256) s_hist[b] = 0;
  if (b == 0) s_max = 1;
  int s = -1;
  unsigned w = 0;
  if (b < batch) {
    s = seq_ids[b];
    if (s >= 0 && s < S.max_seqs) {
      const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
      w = (unsigned)q[Q_NBLK + 0] * (unsigned)S.bh_bytes[0] + (unsigned)q[Q_NBLK + 1] * (unsigned)S.bh_bytes[1] +
          (unsigned)q[Q_NBLK + 2] * (unsigned)S.bh_bytes[2];
    }
  }
  __syncthreads();
  if (b < batch) atomicMax(&s_max, w);
  __syncthreads();
  // bucket 0 holds the longest entries
  const int d = 255 - (int)(((unsigned long long)w * 255u) / s_max);
  int at = 0;
  if (b < batch) at = atomicAdd(&s_hist[d], 1);
  __syncthreads();
  // exclusive prefix of the bucket counts (one wave, four buckets per lane)
  if (b < 64) {
    int v[4], t = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) { v[i] = s_hist[4 * b + i]; t += v[i]; }
    int incl = t;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int y = __shfl_up(incl, sh, 64);
      if (b >= sh) incl += y;
    }
    int run = incl - t;
#pragma unroll
    for (int i = 0; i < 4; i++) { const int x = v[i]; s_hist[4 * b + i] = run; run += x; }
  }
  __syncthreads();
  if (b < batch) order[1 + s_hist[d] + at] = b;
  if (b == 0) order[0] = batch;
}

int launch_attn_order(tkv_cache* c, int batch, const int32_t* seq_ids, int32_t* order, hipStream_t st) {
  TKV_TIMED(c, st, "k_attn_order", k_attn_order<<<1, 1024, 0, st>>>(c->S, seq_ids, batch, order));
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

size_t attn_workspace_bytes(const tkv_cache* c, int batch, int splits) {
  if (splits <= 1) return 0;
  return (size_t)batch * c->S.Hq * splits * (c->S.D + PART_X) * sizeof(float);
}

template <int D, int GS, bool W, int PK, int FMT>
static bool launch_one(const AttnParams& P, dim3 grid, int nw, int lds, hipStream_t st) {
  // dynamic LDS above 64 KiB must be allowed once per kernel and device
  constexpr int kDevs = 64;
  static bool attr_set[kDevs] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return false;
  if (!attr_set[dev]) {
    if (hipFuncSetAttribute((const void*)k_attn<D, GS, W, PK, FMT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kMaxLds - kStaticLds) != hipSuccess)
      return false;
    attr_set[dev] = true;
  }
  k_attn<D, GS, W, PK, FMT><<<grid, 64 * nw, lds, st>>>(P);
  return true;
}

template <int D, int GS, int FMT>
static bool launch_attn_t(const AttnParams& P, int batch, int Hkv, int Hq, int nw, int lds, bool window, int pk,
                          hipStream_t st) {
  dim3 grid(P.splits, Hkv, batch);
  constexpr int PK2 = D / GS <= 2 ? 2 : 1;              // (pack_of packs blocks only with at most two groups)
  constexpr int PK4 = D / GS <= 2 ? 4 : 1;
  constexpr int PK4W = (D == 64 && D / GS <= 2) ? 4 : PK2;  // (with a window, four only at D = 64)
  bool ok;
  if (window) {
    if (pk == 4) ok = launch_one<D, GS, true, PK4W, FMT>(P, grid, nw, lds, st);
    else if (pk == 2) ok = launch_one<D, GS, true, PK2, FMT>(P, grid, nw, lds, st);
    else ok = launch_one<D, GS, true, 1, FMT>(P, grid, nw, lds, st);
  } else {
    if (pk == 4) ok = launch_one<D, GS, false, PK4, FMT>(P, grid, nw, lds, st);
    else if (pk == 2) ok = launch_one<D, GS, false, PK2, FMT>(P, grid, nw, lds, st);
    else ok = launch_one<D, GS, false, 1, FMT>(P, grid, nw, lds, st);
  }
  return ok;
}

int launch_attention(tkv_cache* c, const tkv_attn_args* a, int nw, int splits, hipStream_t st, void* workspace) {
  if (a->batch == 0) return TKV_OK;
  AttnParams P;
  P.S = c->S; P.seq_ids = a->seq_ids; P.q_pos = a->q_pos; P.q = a->q;
  P.k_self = a->k_self; P.v_self = a->v_self; P.sinks = a->sinks;
  P.window = a->window; P.splits = splits; P.topk = a->topk;
  P.layer = a->layer; P.stats_stride = a->stats_stride ? a->stats_stride : c->S.Hq * 3;
  P.part = (float*)(workspace ? workspace : a->workspace); P.out = a->out; P.stats = a->stats; P.n_attended = a->n_attended;
  P.order = a->order;
  const int D = c->S.D, g = c->S.g, lds = lds_bytes(c, nw);
  const bool win = a->window > 0;
  const int pk = pack_of(c, c->S.Hq / c->S.Hkv, win);
  const int B = a->batch, Hkv = c->S.Hkv, Hq = c->S.Hq;
  bool ok = false;
  {
    KernelScope ks(c, st, "k_attn");
    if (c->S.fmt == 0) {
      if (D == 128 && g == 64) ok = launch_attn_t<128, 64, 0>(P, B, Hkv, Hq, nw, lds, win, pk, st);
      else if (D == 128 && g == 32) ok = launch_attn_t<128, 32, 0>(P, B, Hkv, Hq, nw, lds, win, pk, st);
      else if (D == 64 && g == 64) ok = launch_attn_t<64, 64, 0>(P, B, Hkv, Hq, nw, lds, win, pk, st);
      else ok = launch_attn_t<64, 32, 0>(P, B, Hkv, Hq, nw, lds, win, pk, st);
    } else {
      if (D == 128 && g == 64) ok = launch_attn_t<128, 64, 1>(P, B, Hkv, Hq, nw, lds, win, pk, st);
      else if (D == 128 && g == 32) ok = launch_attn_t<128, 32, 1>(P, B, Hkv, Hq, nw, lds, win, pk, st);
      else if (D == 64 && g == 64) ok = launch_attn_t<64, 64, 1>(P, B, Hkv, Hq, nw, lds, win, pk, st);
      else ok = launch_attn_t<64, 32, 1>(P, B, Hkv, Hq, nw, lds, win, pk, st);
    }
  }
  if (ok && P.splits > 1)
    TKV_TIMED(c, st, "k_combine", {
      if (D == 128) k_combine<128><<<dim3((Hq + 3) / 4, B), 256, 0, st>>>(P);
      else k_combine<64><<<dim3((Hq + 3) / 4, B), 256, 0, st>>>(P);
    });
  if (!ok) return TKV_EHIP;
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// Allocation-free variant of the attention call: the split-K partial records
// live in a file-scope device array instead of the caller's workspace.  Each
// device holds its own copy of the array at its own address, which is looked
// up once per device (with that device current) when a cache is created; the
// host uses that address, never the array's name.  Every call on a device
// shares the array, so calls that overlap on one device race; nothing in it
// needs to start at zero (each call writes every partial record it reads).
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[TKV_STATIC_WORKSPACE_BYTES];

#define TKV_MAX_DEVICES 64
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[TKV_MAX_DEVICES];

int static_workspace_setup(int device) {
  if (device < 0 || device >= TKV_MAX_DEVICES) return TKV_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return TKV_OK;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TKV_EHIP;
  g_scratch_ptr[device] = p;
  return TKV_OK;
}

void* static_workspace(int device) {
  if (device < 0 || device >= TKV_MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}
