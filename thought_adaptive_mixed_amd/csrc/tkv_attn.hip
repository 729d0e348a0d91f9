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
// lists [8-bit | 4-bit | 2-bit] and its live blocks are dealt round-robin to
// the waves.  Block ids and valid masks are read 64 at a time into lanes;
// fully evicted blocks are skipped; the next block's codes and metadata are
// loaded while the current one is computed.  Per
// 16-token block, lane l loads chunk l of the K codes and chunk l of the V
// codes (D*bits/32 contiguous bytes each), which puts the codes straight into
// MFMA operand layout:
//   S^T[t][h] = sum_d K[t][d] Q[h][d]     v_mfma_f32_16x16x16_f16, A = K codes
//   O^T[d][h] += sum_t V[t][d] P'[t][h]   v_mfma_f32_16x16x16_f16, A = V codes
// Codes enter the MFMA as exact fp16 integers ((0x6400 | code) - 1024); the
// fp16 scales and zero-points are applied per (token, group) in fp32:
//   logit = (sum_g sK * (q_g . c_g) + zK * sum(q_g)) / sqrt(D)
//   out   = sum_t (p sV) c  +  sum_t p zV          (per group of dims)
// with p sV fed as an fp16 hi + lo pair (two MFMAs), so the product reaches
// the fp32 accumulator with ~21 significant bits.  The query heads of the GQA
// group sit in the 16 MFMA columns (heads >= G are padding and masked).
// Softmax runs online in the log2 domain; the running max is shared by the 4
// lanes holding a head's tokens and is raised only when a block exceeds it
// by more than 2^8 (lazy rescale).  Each lane keeps partial Z, S' = sum
// p (s - m) and a sorted top-8 of its logits, filtered by the head-wide 8th-
// best bound.  The waves of a work-group merge their records through LDS;
// with one split the work-group then adds the staged self token and the sink
// and writes the outputs and statistics, otherwise it writes a partial record
// that a small combine kernel merges across splits.
#include "tkv_internal.h"

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

#define PART_X 16          // extra floats per partial record: m2, Z, S2, n, top8[8], pad
#define TOPK 8
#define SLACK 8.0f         // lazy-rescale slack, log2 units
#define LOG2E 1.4426950408889634f
#define LN2 0.6931471805599453f

// v_exp_f32 directly: no denormal-range fixup (weights below 2^-126 are 0)
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float xorf(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ inline uint32_t rdlane(uint32_t v, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)v, l); }

// ---------------------------------------------------------------------------
// code -> exact fp16 operands
// ---------------------------------------------------------------------------
__device__ inline half2_t exact_codes(uint32_t u) {
  half2_t h = __builtin_bit_cast(half2_t, u);
  const half2_t off = {(_Float16)1024.0f, (_Float16)1024.0f};
  return h - off;
}
// fields p and p + W/2 of word w (elements 2p, 2p+1 of the word) as two fp16 1024 + code
template <int BITS>
__device__ inline uint32_t code_pair(uint32_t w, int p) {
  if constexpr (BITS == 8) {
    // bytes [w.p, 0x64, w.p+2, 0x64]: v_perm_b32 with {0x64646464, w}
    const uint32_t sel = (uint32_t)p | (4u << 8) | ((uint32_t)(p + 2) << 16) | (4u << 24);
    return __builtin_amdgcn_perm(0x64646464u, w, sel);
  } else {
    constexpr uint32_t M = ((1u << BITS) - 1u) * 0x00010001u;
    return ((w >> (p * BITS)) & M) | 0x64006400u;
  }
}
template <int BITS>
__device__ inline half4_t operand4(const uint32_t* words, int e0) {
  constexpr int W = 32 / BITS;
  const uint32_t w = words[e0 / W];
  const int p = (e0 % W) >> 1;
  half2_t a = exact_codes(code_pair<BITS>(w, p));
  half2_t b = exact_codes(code_pair<BITS>(w, p + 1));
  half4_t r = {a[0], a[1], b[0], b[1]};
  return r;
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
__device__ inline void topk_merge_xor(float (&L)[TOPK], int m) {
  float O[TOPK];
#pragma unroll
  for (int i = 0; i < TOPK; i++) O[i] = xorf(L[i], m);
  topk_merge(L, O);
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
  float* part;                 // [batch][Hq][splits][D + PART_X]
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
  int natt;
};

template <int D, int GS, int BITS, bool WINDOW>
struct Blk {
  static constexpr int NG = D / GS;
  static constexpr int CW = D * BITS / 128;     // 32-bit words per lane chunk
  uint32_t kw[CW], vw[CW];
  uint32_t mk[4 * NG], mv[4 * NG];
  int pos[WINDOW ? 4 : 1];
};

template <int D, int GS, int BITS, bool WINDOW>
__device__ inline void load_block(Blk<D, GS, BITS, WINDOW>& b, const uint8_t* base, const int32_t* slotrec,
                                  int lane) {
  constexpr int NG = D / GS;
  constexpr int CB = D * BITS / 32;
  constexpr int CW = CB / 4;
  const int lg = lane >> 4;
  const uint32_t* kp = (const uint32_t*)(base + lane * CB);
  const uint32_t* vp = (const uint32_t*)(base + 64 * CB + lane * CB);
  if constexpr (CW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < CW / 4; i++) {
      uint4 a = ((const uint4*)kp)[i], c = ((const uint4*)vp)[i];
      b.kw[4 * i] = a.x; b.kw[4 * i + 1] = a.y; b.kw[4 * i + 2] = a.z; b.kw[4 * i + 3] = a.w;
      b.vw[4 * i] = c.x; b.vw[4 * i + 1] = c.y; b.vw[4 * i + 2] = c.z; b.vw[4 * i + 3] = c.w;
    }
  } else if constexpr (CW == 2) {
    uint2 a = *(const uint2*)kp, c = *(const uint2*)vp;
    b.kw[0] = a.x; b.kw[1] = a.y; b.vw[0] = c.x; b.vw[1] = c.y;
  } else {
    b.kw[0] = kp[0]; b.vw[0] = vp[0];
  }
  const uint4* mkp = (const uint4*)(base + 2 * 64 * CB + lg * 16 * NG);
  const uint4* mvp = (const uint4*)(base + 2 * 64 * CB + 16 * NG * 4 + lg * 16 * NG);
#pragma unroll
  for (int i = 0; i < NG; i++) {
    uint4 a = mkp[i], c = mvp[i];
    b.mk[4 * i] = a.x; b.mk[4 * i + 1] = a.y; b.mk[4 * i + 2] = a.z; b.mk[4 * i + 3] = a.w;
    b.mv[4 * i] = c.x; b.mv[4 * i + 1] = c.y; b.mv[4 * i + 2] = c.z; b.mv[4 * i + 3] = c.w;
  }
  if constexpr (WINDOW) {
    const int4* pr = (const int4*)(slotrec + 4 * lg * 2);
    int4 a = pr[0], c = pr[1];
    b.pos[0] = a.x; b.pos[1] = a.z; b.pos[2] = c.x; b.pos[3] = c.z;
  }
}

__device__ inline float h_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFF)); }
__device__ inline float h_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

template <int D, int GS, int BITS, bool WINDOW>
__device__ inline void compute_block(const Blk<D, GS, BITS, WINDOW>& b, uint32_t mask, int lo_pos, int lane, bool head_ok,
                                     const half4_t (&qB)[D / 16], const float (&sumq)[D / GS], float alpha,
                                     AttnState<D, GS>& st) {
  constexpr int NG = D / GS;
  constexpr int KM = GS / 16;
  constexpr int NT = D / 16;
  const int lg = lane >> 4;
  uint32_t valid = (mask >> (4 * lg)) & 0xFu;
  if constexpr (WINDOW) {
#pragma unroll
    for (int r = 0; r < 4; r++)
      if (b.pos[r] < lo_pos) valid &= ~(1u << r);
  }
  st.natt += __builtin_popcount(valid);
  const uint32_t vb = head_ok ? valid : 0u;
  // S^T = K Q^T, one accumulator per group
  float4_t sacc[NG];
#pragma unroll
  for (int gi = 0; gi < NG; gi++) {
    sacc[gi] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mm = 0; mm < KM; mm++) {
      half4_t a = operand4<BITS>(b.kw, gi * (GS / 4) + 4 * mm);
      sacc[gi] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, qB[gi * KM + mm], sacc[gi], 0, 0, 0);
    }
  }
  float s2[4];
  float lmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    float x = 0.f;
#pragma unroll
    for (int gi = 0; gi < NG; gi++) {
      const uint32_t m = b.mk[r * NG + gi];
      x = fmaf(h_lo(m), sacc[gi][r], fmaf(h_hi(m), sumq[gi], x));
    }
    s2[r] = ((vb >> r) & 1u) ? x * alpha : -INFINITY;
    lmax = fmaxf(lmax, s2[r]);
  }
  float bm = fmaxf(lmax, xorf(lmax, 16));
  bm = fmaxf(bm, xorf(bm, 32));
  // lazy rescale: raise the running max only when a block exceeds it by SLACK
  const bool grow = bm > st.m2 + SLACK;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    if (grow) {
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
  // top-8: only values above the head-wide 8th-best bound can enter
  float thr = fmaxf(st.top[TOPK - 1], xorf(st.top[TOPK - 1], 16));
  thr = fmaxf(thr, xorf(thr, 32));
  if (__builtin_amdgcn_ballot_w64(lmax > thr)) {
#pragma unroll
    for (int r = 0; r < 4; r++)
      if (s2[r] > thr) topk_insert(st.top, s2[r]);
  }
  // P' = p sV per group as fp16 hi + lo, and the zero-point term
  half4_t pbh[NG], pbl[NG];
#pragma unroll
  for (int gi = 0; gi < NG; gi++) {
    float pv[4];
    float z = st.zacc[gi];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const uint32_t m = b.mv[r * NG + gi];
      pv[r] = p[r] * h_lo(m);
      z = fmaf(p[r], h_hi(m), z);
    }
    st.zacc[gi] = z;
    half2_t h01 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pv[0], pv[1]));
    half2_t h23 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pv[2], pv[3]));
    half2_t l01 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pv[0] - (float)h01[0], pv[1] - (float)h01[1]));
    half2_t l23 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pv[2] - (float)h23[0], pv[3] - (float)h23[1]));
    pbh[gi] = (half4_t){h01[0], h01[1], h23[0], h23[1]};
    pbl[gi] = (half4_t){l01[0], l01[1], l23[0], l23[1]};
  }
  // O^T += V^T P'
#pragma unroll
  for (int n = 0; n < NT; n++) {
    half4_t a = operand4<BITS>(b.vw, 4 * n);
    st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pbh[(16 * n) / GS], st.acc[n], 0, 0, 0);
    st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pbl[(16 * n) / GS], st.acc[n], 0, 0, 0);
  }
}

// The live blocks of one class, as listed in LDS (block id, mask; mask 0 =
// skip), dealt round-robin to the nw waves.  Three block buffers rotate: while
// one block is computed, the next two are in flight.  The loads are always
// issued (past the end they repeat the last block), so no wait drains them.
__device__ inline int next_live(const int2* lst, int n, int e, int nw) {
  while (e < n && lst[e].y == 0) e += nw;
  return e;
}

template <int D, int GS, int BITS, bool WINDOW>
__device__ inline void run_class(const AttnParams& P, int c, const int2* lst, int n, int kvh, int lo_pos, int lane,
                                 int w, int nw, bool head_ok, const half4_t (&qB)[D / 16],
                                 const float (&sumq)[D / GS], float alpha, AttnState<D, GS>& st) {
  typedef Blk<D, GS, BITS, WINDOW> B;
  const DevState& S = P.S;
  const int64_t stride = (int64_t)S.Hkv * pick3(S.bh_bytes, c);
  const uint8_t* pool = pick3(S.pool, c) + (int64_t)kvh * pick3(S.bh_bytes, c);
  const int32_t* slot = pick3(S.slot, c);
  int e0 = next_live(lst, n, w, nw);
  if (e0 >= n) return;
  int e1 = next_live(lst, n, e0 + nw, nw);
  int e2 = e1 < n ? next_live(lst, n, e1 + nw, nw) : n;
  int last = e0;
  auto issue = [&](B& buf, int e) {
    const int ee = e < n ? e : last;
    last = ee;
    const int id = __builtin_amdgcn_readfirstlane(lst[ee].x);
    load_block(buf, pool + (int64_t)id * stride, slot + (int64_t)id * TKV_BS * 2, lane);
  };
  auto mask_of = [&](int e) { return (uint32_t)__builtin_amdgcn_readfirstlane(lst[e].y); };
  B A, Bb, C;
  issue(A, e0);
  issue(Bb, e1);
  while (true) {
    // A holds e0, Bb holds e1 (in flight), C gets e2
    issue(C, e2);
    compute_block<D, GS, BITS, WINDOW>(A, mask_of(e0), lo_pos, lane, head_ok, qB, sumq, alpha, st);
    if (e1 >= n) break;
    int e3 = e2 < n ? next_live(lst, n, e2 + nw, nw) : n;
    issue(A, e3);
    compute_block<D, GS, BITS, WINDOW>(Bb, mask_of(e1), lo_pos, lane, head_ok, qB, sumq, alpha, st);
    if (e2 >= n) break;
    int e4 = e3 < n ? next_live(lst, n, e3 + nw, nw) : n;
    issue(Bb, e4);
    compute_block<D, GS, BITS, WINDOW>(C, mask_of(e2), lo_pos, lane, head_ok, qB, sumq, alpha, st);
    if (e3 >= n) break;
    e0 = e3; e1 = e4;
    e2 = e4 < n ? next_live(lst, n, e4 + nw, nw) : n;
  }
}

// ---------------------------------------------------------------------------
// Records: [D accumulator][m2, Z, S2, n][top8] with the zero-point term folded
// into the accumulator, all relative to the record's own max m2 (log2 units).
// merge_records folds nrec records (stride floats apart) into registers of
// one wave: acc for dims lane and lane + 64, and the merged scalars.
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
  float m = mr;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, xorf(m, o));
  const float sc = nr > 0.f ? exp2f(mr - m) : 0.f;
  float Z = sc * zr, S2 = nr > 0.f ? sc * (sr + (mr - m) * zr) : 0.f, nn = nr;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { Z += xorf(Z, o); S2 += xorf(S2, o); nn += xorf(nn, o); }
#pragma unroll
  for (int i = 0; i < TOPK; i++) M.top[i] = (lane < nrec && nr > 0.f) ? recs[(int64_t)lane * stride + D + 4 + i] : -INFINITY;
  for (int o = 1; o < nrec; o <<= 1) topk_merge_xor(M.top, o);
  float a0 = 0.f, a1 = 0.f;
  for (int r = 0; r < nrec; r++) {
    const float f = __shfl(sc, r, 64);
    if (f == 0.f) continue;
    const float* rec = recs + (int64_t)r * stride;
    a0 = fmaf(f, rec[lane], a0);
    if (D > 64) a1 = fmaf(f, rec[lane + 64], a1);
  }
  M.a0 = a0; M.a1 = a1; M.m = m; M.Z = Z; M.S2 = S2; M.n = (int)nn;
}

// Add the staged self token and the sink; write the output and statistics.
template <int D>
__device__ inline void finalize_head(const AttnParams& P, int b, int hq, int lane, Merged M) {
  const DevState& S = P.S;
  const int G = S.Hq / S.Hkv, kvh = hq / G;
  const float alpha = LOG2E / sqrtf((float)D);
  int n = M.n;
  if (P.k_self) {
    const uint16_t* qr = P.q + ((int64_t)b * S.Hq + hq) * D;
    const float* kr = P.k_self + ((int64_t)b * S.Hkv + kvh) * D;
    float d = 0.f;
    for (int i = lane; i < D; i += 64) d = fmaf(__builtin_bit_cast(float, (uint32_t)qr[i] << 16), kr[i], d);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) d += xorf(d, o);
    const float self2 = d * alpha;
    const float m = fmaxf(M.m, self2);
    const float sc = M.n > 0 ? exp2f(M.m - m) : 0.f;
    const float ps = exp2f(self2 - m);
    M.S2 = sc * (M.S2 + (M.n > 0 ? (M.m - m) * M.Z : 0.f)) + ps * (self2 - m);
    M.Z = sc * M.Z + ps;
    const float* vr = P.v_self + ((int64_t)b * S.Hkv + kvh) * D;
    M.a0 = fmaf(ps, vr[lane], sc * M.a0);
    if (D > 64) M.a1 = fmaf(ps, vr[lane + 64], sc * M.a1);
    M.m = m;
    topk_insert(M.top, self2);
    n += 1;
  }
  float* out = P.out + ((int64_t)b * S.Hq + hq) * D;
  float* st = P.stats ? P.stats + ((int64_t)b * S.Hq + hq) * 3 : nullptr;
  if (n == 0) {
    out[lane] = 0.f;
    if (D > 64) out[lane + 64] = 0.f;
    if (st && lane == 0) { st[0] = 0.f; st[1] = 0.f; st[2] = 0.f; }
  } else {
    float den = M.Z;
    if (P.sinks) den += exp2f(P.sinks[hq] * LOG2E - M.m);
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

template <int D, int GS, bool WINDOW>
__global__ __launch_bounds__(512) void k_attn(AttnParams P) {
  constexpr int NG = D / GS;
  constexpr int KM = GS / 16;
  constexpr int NT = D / 16;
  constexpr int RS = D + PART_X;                 // record stride (floats)
  extern __shared__ float lds[];                 // [nw][G][RS] records, then [3][max_blocks] (id, mask)
  const DevState& S = P.S;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int lg = lane >> 4, h = lane & 15;
  const int G = S.Hq / S.Hkv;
  const bool head_ok = h < G;
  const int s = P.seq_ids[b];
  const bool seq_ok = s >= 0 && s < S.max_seqs;
  // query B operand: column h, k = 4lg + e <-> dim gi*GS + lg*(GS/4) + 4mm + e
  half4_t qB[NG * KM];
  float sumq[NG];
  {
    const uint16_t* qr = P.q + ((int64_t)b * S.Hq + (int64_t)kvh * G + (head_ok ? h : 0)) * D;
#pragma unroll
    for (int gi = 0; gi < NG; gi++) {
      const uint4* src = (const uint4*)(qr + gi * GS + lg * (GS / 4));
      uint32_t wq[GS / 8];
#pragma unroll
      for (int i = 0; i < GS / 32; i++) {
        uint4 v = src[i];
        wq[4 * i] = v.x; wq[4 * i + 1] = v.y; wq[4 * i + 2] = v.z; wq[4 * i + 3] = v.w;
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
        }
        qB[gi * KM + mm] = v;
      }
      sq += xorf(sq, 16);
      sq += xorf(sq, 32);
      sumq[gi] = sq;
    }
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
  // the split's block ids and masks, all three classes, into LDS
  int2* lst = (int2*)(lds + nw * G * RS);            // [3][lmax]
  const int lmax = S.max_blocks;
  int ncls[3] = {0, 0, 0};
  const int lo_pos = WINDOW ? P.q_pos[b] - P.window + 1 : 0;
  if (seq_ok) {
    const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
    const int nb0 = q[Q_NBLK + 0], nb1 = q[Q_NBLK + 1], nb2 = q[Q_NBLK + 2];
    // byte-balanced split of [8-bit | 4-bit | 2-bit] block lists (< 2^31 bytes per sequence)
    const int w0 = (int)S.bh_bytes[0], w1 = (int)S.bh_bytes[1], w2 = (int)S.bh_bytes[2];
    const int P1 = nb0 * w0, P2 = P1 + nb1 * w1, W = P2 + nb2 * w2;
    const int lo = (int)((int64_t)W * split / P.splits), hi = (int)((int64_t)W * (split + 1) / P.splits);
    const int32_t* bt = S.btab + (int64_t)s * 3 * S.max_blocks;
    int j0s[3], j1s[3];
    const int off[3] = {0, P1, P2}, wb[3] = {w0, w1, w2}, nb[3] = {nb0, nb1, nb2};
#pragma unroll
    for (int c = 0; c < 3; c++) {
      const int a = lo - off[c], z = hi - off[c];
      j0s[c] = a <= 0 ? 0 : min(nb[c], (a + wb[c] - 1) / wb[c]);
      j1s[c] = z <= 0 ? 0 : min(nb[c], (z + wb[c] - 1) / wb[c]);
      ncls[c] = j1s[c] > j0s[c] ? j1s[c] - j0s[c] : 0;
    }
    const int tot = ncls[0] + ncls[1] + ncls[2];
    for (int e = threadIdx.x; e < tot; e += blockDim.x) {
      const int c = e < ncls[0] ? 0 : (e < ncls[0] + ncls[1] ? 1 : 2);
      const int i = e - (c == 0 ? 0 : (c == 1 ? ncls[0] : ncls[0] + ncls[1]));
      const int id = bt[c * S.max_blocks + j0s[c] + i];
      const int2 rec = *(const int2*)(pick3(S.blk, c) + (int64_t)id * TKV_BLK_W);
      int m = rec.x;
      if (WINDOW && rec.y < lo_pos) m = 0;
      lst[c * lmax + i] = make_int2(id, m);
    }
  }
  __syncthreads();
  if (ncls[0]) run_class<D, GS, 8, WINDOW>(P, 0, lst, ncls[0], kvh, lo_pos, lane, w, nw, head_ok, qB, sumq, alpha, st);
  if (ncls[1])
    run_class<D, GS, 4, WINDOW>(P, 1, lst + lmax, ncls[1], kvh, lo_pos, lane, w, nw, head_ok, qB, sumq, alpha, st);
  if (ncls[2])
    run_class<D, GS, 2, WINDOW>(P, 2, lst + 2 * lmax, ncls[2], kvh, lo_pos, lane, w, nw, head_ok, qB, sumq, alpha,
                                st);
  // this wave's record per head, over its 4 lane groups
  st.Z += xorf(st.Z, 16); st.Z += xorf(st.Z, 32);
  st.S2 += xorf(st.S2, 16); st.S2 += xorf(st.S2, 32);
#pragma unroll
  for (int gi = 0; gi < NG; gi++) { st.zacc[gi] += xorf(st.zacc[gi], 16); st.zacc[gi] += xorf(st.zacc[gi], 32); }
  {
    float n = (float)st.natt;
    n += xorf(n, 16); n += xorf(n, 32);
    st.natt = (int)n;
  }
  topk_merge_xor(st.top, 16);
  topk_merge_xor(st.top, 32);
  if (head_ok) {
    float* rec = lds + ((int64_t)w * G + h) * RS;
#pragma unroll
    for (int n = 0; n < NT; n++) {
      const float z = st.zacc[(16 * n) / GS];
#pragma unroll
      for (int r = 0; r < 4; r++) rec[16 * n + 4 * lg + r] = st.acc[n][r] + z;
    }
    if (lg == 0) {
      rec[D] = st.m2; rec[D + 1] = st.Z; rec[D + 2] = st.S2; rec[D + 3] = (float)st.natt;
#pragma unroll
      for (int i = 0; i < TOPK; i++) rec[D + 4 + i] = st.top[i];
    }
  }
  __syncthreads();
  // merge the waves' records; finalize here when the sequence is one split
  for (int hh = w; hh < G; hh += nw) {
    Merged M;
    merge_records<D>(lds + (int64_t)hh * RS, G * RS, nw, lane, M);
    const int hq = kvh * G + hh;
    if (P.splits == 1) {
      finalize_head<D>(P, b, hq, lane, M);
    } else {
      float* rec = P.part + (((int64_t)b * S.Hq + hq) * P.splits + split) * RS;
      rec[lane] = M.a0;
      if (D > 64) rec[lane + 64] = M.a1;
      if (lane < 4) rec[D + lane] = lane == 0 ? M.m : lane == 1 ? M.Z : lane == 2 ? M.S2 : (float)M.n;
      if (lane < TOPK) {
        float v = M.top[0];
#pragma unroll
        for (int i = 1; i < TOPK; i++) v = lane == i ? M.top[i] : v;
        rec[D + 4 + lane] = v;
      }
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
  Merged M;
  merge_records<D>(recs, D + PART_X, P.splits, lane, M);
  finalize_head<D>(P, b, hq, lane, M);
}

// ---------------------------------------------------------------------------
// Launch shape: one work-group of nw waves per (batch entry, KV head, split);
// about two resident waves per SIMD (1024 SIMDs), the waves of a work-group
// sharing the sequence's blocks; extra splits only when the batch is small.
// ---------------------------------------------------------------------------
static const int kTargetWaves = 2048;

static int lds_bytes(const tkv_cache* c, int nw) {
  return nw * (c->S.Hq / c->S.Hkv) * (c->S.D + PART_X) * (int)sizeof(float) + 3 * c->S.max_blocks * 8;
}

void attn_plan(const tkv_cache* c, int batch, int num_splits, int* nw_out, int* splits_out) {
  const int units = batch * c->S.Hkv > 0 ? batch * c->S.Hkv : 1;
  int nw = 1;
  while (nw < 8 && units * nw * 2 <= kTargetWaves && lds_bytes(c, nw * 2) <= 65536) nw *= 2;
  int splits = num_splits;
  if (splits <= 0) {
    splits = (kTargetWaves + units * nw - 1) / (units * nw);
    const int cap = (3 * c->S.max_blocks) / (4 * nw) > 1 ? (3 * c->S.max_blocks) / (4 * nw) : 1;
    if (splits > cap) splits = cap;
    if (splits > 64) splits = 64;
    if (splits < 1) splits = 1;
  }
  *nw_out = nw;
  *splits_out = splits;
}

size_t attn_workspace_bytes(const tkv_cache* c, int batch, int splits) {
  if (splits <= 1) return 0;
  return (size_t)batch * c->S.Hq * splits * (c->S.D + PART_X) * sizeof(float);
}

template <int D, int GS>
static void launch_attn_t(const AttnParams& P, int batch, int Hkv, int Hq, int nw, int lds, bool window,
                          hipStream_t st) {
  dim3 grid(P.splits, Hkv, batch);
  if (window) k_attn<D, GS, true><<<grid, 64 * nw, lds, st>>>(P);
  else k_attn<D, GS, false><<<grid, 64 * nw, lds, st>>>(P);
  if (P.splits > 1) k_combine<D><<<dim3((Hq + 3) / 4, batch), 256, 0, st>>>(P);
}

int launch_attention(tkv_cache* c, const tkv_attn_args* a, int nw, int splits, hipStream_t st) {
  if (a->batch == 0) return TKV_OK;
  AttnParams P;
  P.S = c->S; P.seq_ids = a->seq_ids; P.q_pos = a->q_pos; P.q = a->q;
  P.k_self = a->k_self; P.v_self = a->v_self; P.sinks = a->sinks;
  P.window = a->window; P.splits = splits; P.topk = a->topk;
  P.part = (float*)a->workspace; P.out = a->out; P.stats = a->stats; P.n_attended = a->n_attended;
  const int D = c->S.D, g = c->S.g, lds = lds_bytes(c, nw);
  const bool win = a->window > 0;
  if (D == 128 && g == 64) launch_attn_t<128, 64>(P, a->batch, c->S.Hkv, c->S.Hq, nw, lds, win, st);
  else if (D == 128 && g == 32) launch_attn_t<128, 32>(P, a->batch, c->S.Hkv, c->S.Hq, nw, lds, win, st);
  else if (D == 64 && g == 64) launch_attn_t<64, 64>(P, a->batch, c->S.Hkv, c->S.Hq, nw, lds, win, st);
  else launch_attn_t<64, 32>(P, a->batch, c->S.Hkv, c->S.Hq, nw, lds, win, st);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}
