// Split-K paged decode attention over the mixed-precision, hole-bearing cache,
// with the sparsity statistics (entropy, top-k mass) in the same pass.
//
// Method passages: ThinKV abstract (a kernel extending PagedAttention that
// reuses evicted tokens' slots without compaction) and the technical summary,
// "Methodologie": thought decomposition via attention sparsity, Continuous
// Thinking (block table with eviction masks).
//
// Work decomposition: one 64-lane wave per (batch entry, KV head, split);
// a split owns a byte-balanced range of the sequence's block lists
// [8-bit | 4-bit | 2-bit].  Per 16-token block, lane l loads chunk l of the K
// codes and chunk l of the V codes (D*bits/32 bytes each, contiguous across
// the wave), so the codes land directly in MFMA operand layout:
//   S^T[t][h] = sum_d K[t][d] Q[h][d]     v_mfma_f32_16x16x16_f16, A = K codes
//   O^T[d][h] += sum_t V[t][d] P'[t][h]   v_mfma_f32_16x16x16_f16, A = V codes
// Codes enter the MFMA as exact fp16 integers (0x6400|code minus 1024); the
// fp16 scales and zero-points are applied per (token, group) in fp32:
//   logit = (sum_g sK * (q_g . c_g) + zK * sum(q_g)) / sqrt(D)
//   out   = sum_t (p sV) c  +  sum_t p zV          (per group of dims)
// with p sV fed as an fp16 hi + lo pair (two MFMAs) so the absolute error of
// large outputs stays at fp32 level.
// Query heads of the GQA group sit in the 16 MFMA columns (heads >= G are
// zero padding).  Softmax runs online in the log2 domain per head with the
// running max shared by the 4 lanes holding a head's tokens; each lane keeps
// partial Z, S' = sum p (s - m) and a sorted top-8 list of its logits.
#include "tkv_internal.h"

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

#define PART_X 16          // extra floats per partial record: m2, Z, S2, n, top8[8], pad
#define TOPK 8
#define LOG2E 1.4426950408889634f
#define LN2 0.6931471805599453f

__device__ inline float wave_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// two fp16 codes (1024 + code) from fields p and p + W/2 of a 32-bit word
template <int BITS>
__device__ inline uint32_t code_pair(uint32_t w, int p) {
  constexpr uint32_t M = ((1u << BITS) - 1u) * 0x00010001u;
  return ((w >> (p * BITS)) & M) | 0x64006400u;
}
__device__ inline half2_t exact_codes(uint32_t u) {
  half2_t h = __builtin_bit_cast(half2_t, u);
  const half2_t off = {(_Float16)1024.0f, (_Float16)1024.0f};
  return h - off;
}
// A operand (4 consecutive chunk elements e0..e0+3) from the chunk words
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

__device__ inline void topk_insert(float (&L)[TOPK], float v) {
  if (v > L[TOPK - 1]) {
#pragma unroll
    for (int i = 0; i < TOPK; i++) {
      float hi = fmaxf(L[i], v), lo = fminf(L[i], v);
      L[i] = hi; v = lo;
    }
  }
}
// merge with the list held by lane ^ m (both sorted descending)
__device__ inline void topk_merge_xor(float (&L)[TOPK], int m) {
  float O[TOPK];
#pragma unroll
  for (int i = 0; i < TOPK; i++) O[i] = wave_xor(L[i], m);
#pragma unroll
  for (int i = 0; i < TOPK; i++) topk_insert(L, O[i]);
}

template <int D, int G_>
struct AttnGeom {
  static constexpr int NT = D / 16;         // dim tiles of the P.V product
};

struct AttnParams {
  DevState S;
  const int32_t* seq_ids;
  const int32_t* q_pos;
  const uint16_t* q;
  int window;
  int splits;
  float* part;                 // [batch][Hq][splits][D + PART_X]
};

// One block of class BITS: loads, q.K^T, online softmax, P.V.
template <int D, int GS, int BITS, bool WINDOW>
__device__ inline void attn_block(const AttnParams& P, int c, int blk, int kvh, int lo_pos, int lane,
                                  const half4_t (&qB)[D / 16], const float (&sumq)[D / GS], float alpha,
                                  float4_t (&acc)[D / 16], float (&zacc)[D / GS], float& m2, float& Z, float& S2,
                                  float (&top)[TOPK], int& natt) {
  constexpr int NG = D / GS;
  constexpr int KM = GS / 16;               // MFMAs per group for S^T
  constexpr int NT = D / 16;
  constexpr int CB = D * BITS / 32;         // bytes per lane chunk
  constexpr int CW = CB / 4;                // words per lane chunk
  const DevState& S = P.S;
  const int lg = lane >> 4;
  const int32_t* brec = S.blk[c] + (int64_t)blk * TKV_BLK_W;
  const uint32_t mask = (uint32_t)brec[0];
  if (mask == 0) return;
  uint32_t vbits = (mask >> (4 * lg)) & 0xFu;   // validity of this lane's 4 tokens
  if (WINDOW) {
    if (brec[1] < lo_pos) return;
    const int4* pr = (const int4*)(S.slot[c] + ((int64_t)blk * TKV_BS + 4 * lg) * 2);
    int4 a = pr[0], b = pr[1];
    if (a.x < lo_pos) vbits &= ~1u;
    if (a.z < lo_pos) vbits &= ~2u;
    if (b.x < lo_pos) vbits &= ~4u;
    if (b.z < lo_pos) vbits &= ~8u;
    if (__ballot(vbits != 0) == 0) return;
  }
  const uint8_t* base = S.pool[c] + ((int64_t)blk * S.Hkv + kvh) * S.bh_bytes[c];
  uint32_t kw[CW], vw[CW];
  {
    const uint32_t* kp = (const uint32_t*)(base + lane * CB);
    const uint32_t* vp = (const uint32_t*)(base + 64 * CB + lane * CB);
    if constexpr (CW % 4 == 0) {
#pragma unroll
      for (int i = 0; i < CW / 4; i++) {
        uint4 a = ((const uint4*)kp)[i], b = ((const uint4*)vp)[i];
        kw[4 * i] = a.x; kw[4 * i + 1] = a.y; kw[4 * i + 2] = a.z; kw[4 * i + 3] = a.w;
        vw[4 * i] = b.x; vw[4 * i + 1] = b.y; vw[4 * i + 2] = b.z; vw[4 * i + 3] = b.w;
      }
    } else if constexpr (CW == 2) {
      uint2 a = *(const uint2*)kp, b = *(const uint2*)vp;
      kw[0] = a.x; kw[1] = a.y; vw[0] = b.x; vw[1] = b.y;
    } else {
      kw[0] = kp[0]; vw[0] = vp[0];
    }
  }
  // meta of tokens 4lg .. 4lg+3: (scale, zero) fp16 per group
  float sK[4][NG], zK[4][NG], sV[4][NG], zV[4][NG];
  {
    const uint32_t* mk = (const uint32_t*)(base + 2 * 64 * CB) + 4 * lg * NG;
    const uint32_t* mv = (const uint32_t*)(base + 2 * 64 * CB + 16 * NG * 4) + 4 * lg * NG;
#pragma unroll
    for (int r = 0; r < 4; r++)
#pragma unroll
      for (int gi = 0; gi < NG; gi++) {
        uint32_t a = mk[r * NG + gi], b = mv[r * NG + gi];
        sK[r][gi] = f16_bits_to_f32((uint16_t)(a & 0xFFFF)); zK[r][gi] = f16_bits_to_f32((uint16_t)(a >> 16));
        sV[r][gi] = f16_bits_to_f32((uint16_t)(b & 0xFFFF)); zV[r][gi] = f16_bits_to_f32((uint16_t)(b >> 16));
      }
  }
  // S^T = K Q^T, one accumulator per group
  float4_t sacc[NG];
#pragma unroll
  for (int gi = 0; gi < NG; gi++) {
    sacc[gi] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mm = 0; mm < KM; mm++) {
      half4_t a = operand4<BITS>(kw, gi * (GS / 4) + 4 * mm);
      sacc[gi] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, qB[gi * KM + mm], sacc[gi], 0, 0, 0);
    }
  }
  float s2[4];
  float bm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    float x = 0.f;
#pragma unroll
    for (int gi = 0; gi < NG; gi++) x = fmaf(sK[r][gi], sacc[gi][r], fmaf(zK[r][gi], sumq[gi], x));
    x *= alpha;
    s2[r] = ((vbits >> r) & 1u) ? x : -INFINITY;
    bm = fmaxf(bm, s2[r]);
  }
  bm = fmaxf(bm, wave_xor(bm, 16));
  bm = fmaxf(bm, wave_xor(bm, 32));
  const float mn = fmaxf(m2, bm);
  if (mn > m2) {
    if (m2 == -INFINITY) {
      Z = 0.f; S2 = 0.f;
    } else {
      const float sc = exp2f(m2 - mn);
      S2 = sc * (S2 + (m2 - mn) * Z);
      Z *= sc;
#pragma unroll
      for (int n = 0; n < NT; n++) acc[n] *= sc;
#pragma unroll
      for (int gi = 0; gi < NG; gi++) zacc[gi] *= sc;
    }
    m2 = mn;
  }
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const bool v = (vbits >> r) & 1u;
    p[r] = v ? exp2f(s2[r] - m2) : 0.f;
    Z += p[r];
    S2 = v ? fmaf(p[r], s2[r] - m2, S2) : S2;
    natt += v ? 1 : 0;
  }
#pragma unroll
  for (int r = 0; r < 4; r++) topk_insert(top, s2[r]);
  // P' = p * sV per group, split into fp16 hi + lo so that the product
  // reaches the fp32 accumulator with ~22 significant bits, and the
  // zero-point term
  half4_t pbh[NG], pbl[NG];
#pragma unroll
  for (int gi = 0; gi < NG; gi++) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const float pv = p[r] * sV[r][gi];
      const _Float16 hi = (_Float16)pv;
      pbh[gi][r] = hi;
      pbl[gi][r] = (_Float16)(pv - (float)hi);
    }
    float z = zacc[gi];
#pragma unroll
    for (int r = 0; r < 4; r++) z = fmaf(p[r], zV[r][gi], z);
    zacc[gi] = z;
  }
  // O^T += V^T P'
#pragma unroll
  for (int n = 0; n < NT; n++) {
    half4_t a = operand4<BITS>(vw, 4 * n);
    acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pbh[(16 * n) / GS], acc[n], 0, 0, 0);
    acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pbl[(16 * n) / GS], acc[n], 0, 0, 0);
  }
}

template <int D, int GS, bool WINDOW>
__global__ __launch_bounds__(64) void k_attn(AttnParams P) {
  constexpr int NG = D / GS;
  constexpr int KM = GS / 16;
  constexpr int NT = D / 16;
  const DevState& S = P.S;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, lg = lane >> 4, h = lane & 15;
  const int G = S.Hq / S.Hkv;
  const int s = P.seq_ids[b];
  const bool seq_ok = s >= 0 && s < S.max_seqs;
  // query B operand: column h, k = 4lg + e -> dim gi*GS + lg*(GS/4) + 4mm + e
  half4_t qB[NG * KM];
  float sumq[NG];
  {
    const uint16_t* qr = P.q + ((int64_t)b * S.Hq + (int64_t)kvh * G + (h < G ? h : 0)) * D;
#pragma unroll
    for (int gi = 0; gi < NG; gi++) sumq[gi] = 0.f;
#pragma unroll
    for (int gi = 0; gi < NG; gi++)
#pragma unroll
      for (int mm = 0; mm < KM; mm++) {
        half4_t v;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          int d = gi * GS + lg * (GS / 4) + 4 * mm + e;
          float x = h < G ? __builtin_bit_cast(float, (uint32_t)qr[d] << 16) : 0.f;
          v[e] = (_Float16)x;
        }
        qB[gi * KM + mm] = v;
      }
    // sum of q over each group (all 64 dims of the group, this head)
#pragma unroll
    for (int gi = 0; gi < NG; gi++) {
      float sq = 0.f;
      for (int j = 0; j < GS / 4; j++) {
        int d = gi * GS + lg * (GS / 4) + j;
        sq += h < G ? (float)(_Float16)__builtin_bit_cast(float, (uint32_t)qr[d] << 16) : 0.f;
      }
      sq += wave_xor(sq, 16);
      sq += wave_xor(sq, 32);
      sumq[gi] = sq;
    }
  }
  const float alpha = LOG2E / sqrtf((float)D);
  float4_t acc[NT];
#pragma unroll
  for (int n = 0; n < NT; n++) acc[n] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float zacc[NG];
#pragma unroll
  for (int gi = 0; gi < NG; gi++) zacc[gi] = 0.f;
  float m2 = -INFINITY, Z = 0.f, S2 = 0.f;
  float top[TOPK];
#pragma unroll
  for (int i = 0; i < TOPK; i++) top[i] = -INFINITY;
  int natt = 0;
  if (seq_ok) {
    const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
    const int nb0 = q[Q_NBLK + 0], nb1 = q[Q_NBLK + 1], nb2 = q[Q_NBLK + 2];
    // byte-balanced split of [8-bit | 4-bit | 2-bit] block lists
    const long long w0 = S.bh_bytes[0], w1 = S.bh_bytes[1], w2 = S.bh_bytes[2];
    const long long P1 = nb0 * w0, P2 = P1 + nb1 * w1, W = P2 + nb2 * w2;
    const long long lo = W * split / P.splits, hi = W * (split + 1) / P.splits;
    const int lo_pos = WINDOW ? P.q_pos[b] - P.window + 1 : 0;
    const int32_t* bt = S.btab + (int64_t)s * 3 * S.max_blocks;
    auto range = [&](long long off, long long w, int nb, int& j0, int& j1) {
      long long a = lo - off, z = hi - off;
      j0 = a <= 0 ? 0 : (int)((a + w - 1) / w);
      j1 = z <= 0 ? 0 : (int)((z + w - 1) / w);
      if (j0 > nb) j0 = nb;
      if (j1 > nb) j1 = nb;
    };
    int j0, j1;
    range(0, w0, nb0, j0, j1);
    for (int j = j0; j < j1; j++)
      attn_block<D, GS, 8, WINDOW>(P, 0, bt[j], kvh, lo_pos, lane, qB, sumq, alpha, acc, zacc, m2, Z, S2, top, natt);
    range(P1, w1, nb1, j0, j1);
    for (int j = j0; j < j1; j++)
      attn_block<D, GS, 4, WINDOW>(P, 1, bt[S.max_blocks + j], kvh, lo_pos, lane, qB, sumq, alpha, acc, zacc, m2, Z,
                                   S2, top, natt);
    range(P2, w2, nb2, j0, j1);
    for (int j = j0; j < j1; j++)
      attn_block<D, GS, 2, WINDOW>(P, 2, bt[2 * S.max_blocks + j], kvh, lo_pos, lane, qB, sumq, alpha, acc, zacc, m2,
                                   Z, S2, top, natt);
  }
  // reduce the lane partials of each head over the 4 lane groups
  Z += wave_xor(Z, 16); Z += wave_xor(Z, 32);
  S2 += wave_xor(S2, 16); S2 += wave_xor(S2, 32);
#pragma unroll
  for (int gi = 0; gi < NG; gi++) { zacc[gi] += wave_xor(zacc[gi], 16); zacc[gi] += wave_xor(zacc[gi], 32); }
  {
    float n = (float)natt;
    n += wave_xor(n, 16); n += wave_xor(n, 32);
    natt = (int)n;
  }
  topk_merge_xor(top, 16);
  topk_merge_xor(top, 32);
  if (h < G) {
    const int hq = kvh * G + h;
    float* rec = P.part + (((int64_t)b * S.Hq + hq) * P.splits + split) * (D + PART_X);
#pragma unroll
    for (int n = 0; n < NT; n++) {
      const float z = zacc[(16 * n) / GS];
      float4 o = make_float4(acc[n][0] + z, acc[n][1] + z, acc[n][2] + z, acc[n][3] + z);
      *(float4*)(rec + 16 * n + 4 * lg) = o;
    }
    if (lg == 0) {
      rec[D + 0] = m2; rec[D + 1] = Z; rec[D + 2] = S2; rec[D + 3] = (float)natt;
#pragma unroll
      for (int i = 0; i < TOPK; i++) rec[D + 4 + i] = top[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Combine the splits of one (batch entry, query head); add the self token
// and the sink; write out and the statistics.
// ---------------------------------------------------------------------------
struct CombineParams {
  int batch, Hq, Hkv, D, splits, topk, max_seqs;
  const int32_t* seq_ids;
  const uint16_t* q;
  const float* k_self;
  const float* v_self;
  const float* sinks;
  const float* part;
  float* out;
  float* stats;
  int32_t* n_attended;
  int32_t* hdr;
};

__global__ __launch_bounds__(64) void k_combine(CombineParams C) {
  const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int D = C.D, G = C.Hq / C.Hkv, kvh = hq / G;
  const float* rec0 = C.part + ((int64_t)b * C.Hq + hq) * C.splits * (D + PART_X);
  const float alpha = LOG2E / sqrtf((float)D);
  // self token logit (log2 units)
  float self2 = -INFINITY;
  if (C.k_self) {
    const uint16_t* qr = C.q + ((int64_t)b * C.Hq + hq) * D;
    const float* kr = C.k_self + ((int64_t)b * C.Hkv + kvh) * D;
    float d = 0.f;
    for (int i = lane; i < D; i += 64) d = fmaf(__builtin_bit_cast(float, (uint32_t)qr[i] << 16), kr[i], d);
    for (int o = 32; o > 0; o >>= 1) d += wave_xor(d, o);
    self2 = d * alpha;
  }
  float m = self2;
  int n = C.k_self ? 1 : 0;
  for (int r = 0; r < C.splits; r++) {
    const float* rec = rec0 + (int64_t)r * (D + PART_X);
    if (rec[D + 3] > 0.f) m = fmaxf(m, rec[D]);
    n += (int)rec[D + 3];
  }
  float Z = 0.f, S2 = 0.f;
  float o0 = 0.f, o1 = 0.f;   // dims lane and lane + 64
  float top[TOPK];
#pragma unroll
  for (int i = 0; i < TOPK; i++) top[i] = -INFINITY;
  for (int r = 0; r < C.splits; r++) {
    const float* rec = rec0 + (int64_t)r * (D + PART_X);
    if (!(rec[D + 3] > 0.f)) continue;
    const float mr = rec[D], zr = rec[D + 1], sr = rec[D + 2];
    const float sc = exp2f(mr - m);
    Z = fmaf(sc, zr, Z);
    S2 = fmaf(sc, sr + (mr - m) * zr, S2);
    if (lane < D) o0 = fmaf(sc, rec[lane], o0);
    if (lane + 64 < D) o1 = fmaf(sc, rec[lane + 64], o1);
    for (int i = 0; i < TOPK; i++) topk_insert(top, rec[D + 4 + i]);
  }
  if (C.k_self) {
    const float ps = exp2f(self2 - m);
    Z += ps;
    S2 = fmaf(ps, self2 - m, S2);
    const float* vr = C.v_self + ((int64_t)b * C.Hkv + kvh) * D;
    if (lane < D) o0 = fmaf(ps, vr[lane], o0);
    if (lane + 64 < D) o1 = fmaf(ps, vr[lane + 64], o1);
    topk_insert(top, self2);
  }
  float* out = C.out + ((int64_t)b * C.Hq + hq) * D;
  if (n == 0) {
    if (lane < D) out[lane] = 0.f;
    if (lane + 64 < D) out[lane + 64] = 0.f;
    if (C.stats && lane == 0) {
      float* st = C.stats + ((int64_t)b * C.Hq + hq) * 3;
      st[0] = 0.f; st[1] = 0.f; st[2] = 0.f;
    }
  } else {
    float den = Z;
    if (C.sinks) den += exp2f(C.sinks[hq] * LOG2E - m);
    const float inv = 1.0f / den;
    if (lane < D) out[lane] = o0 * inv;
    if (lane + 64 < D) out[lane + 64] = o1 * inv;
    if (C.stats && lane == 0) {
      const float H = logf(Z) - LN2 * S2 / Z;
      float mk = 0.f;
      const int kk = C.topk < n ? C.topk : n;
      for (int i = 0; i < kk; i++) mk += exp2f(top[i] - m);
      float* st = C.stats + ((int64_t)b * C.Hq + hq) * 3;
      st[0] = H;
      st[1] = n >= 2 ? H / logf((float)n) : 0.f;
      st[2] = mk / Z;
    }
  }
  if (C.n_attended && hq == 0 && lane == 0) C.n_attended[b] = n;
  if (hq == 0 && lane == 0) {
    const int s = C.seq_ids[b];
    if (s < 0 || s >= C.max_seqs) record_error(C.hdr, TKV_EINVAL, s < 0 ? TKV_INF : s);
  }
}

// ---------------------------------------------------------------------------
int attn_choose_splits(const tkv_cache* c, int batch) {
  const int units = batch * c->S.Hkv;
  int s = (4096 + units - 1) / (units > 0 ? units : 1);
  const int maxb = 3 * c->S.max_blocks;
  int cap = maxb / 4 > 1 ? maxb / 4 : 1;
  if (s > cap) s = cap;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return s;
}

size_t attn_workspace_bytes(const tkv_cache* c, int batch, int splits) {
  return (size_t)batch * c->S.Hq * splits * (c->S.D + PART_X) * sizeof(float);
}

template <int D, int GS>
static void launch_attn_t(const AttnParams& P, int batch, int Hkv, bool window, hipStream_t st) {
  dim3 grid(P.splits, Hkv, batch);
  if (window) k_attn<D, GS, true><<<grid, 64, 0, st>>>(P);
  else k_attn<D, GS, false><<<grid, 64, 0, st>>>(P);
}

int launch_attention(tkv_cache* c, const tkv_attn_args* a, int splits, hipStream_t st) {
  if (a->batch == 0) return TKV_OK;
  AttnParams P;
  P.S = c->S; P.seq_ids = a->seq_ids; P.q_pos = a->q_pos; P.q = a->q; P.window = a->window; P.splits = splits;
  P.part = (float*)a->workspace;
  const int D = c->S.D, g = c->S.g;
  const bool win = a->window > 0;
  if (D == 128 && g == 64) launch_attn_t<128, 64>(P, a->batch, c->S.Hkv, win, st);
  else if (D == 128 && g == 32) launch_attn_t<128, 32>(P, a->batch, c->S.Hkv, win, st);
  else if (D == 64 && g == 64) launch_attn_t<64, 64>(P, a->batch, c->S.Hkv, win, st);
  else launch_attn_t<64, 32>(P, a->batch, c->S.Hkv, win, st);
  CombineParams C;
  C.batch = a->batch; C.Hq = c->S.Hq; C.Hkv = c->S.Hkv; C.D = D; C.splits = splits; C.topk = a->topk;
  C.max_seqs = c->S.max_seqs; C.seq_ids = a->seq_ids; C.q = a->q; C.k_self = a->k_self; C.v_self = a->v_self;
  C.sinks = a->sinks; C.part = P.part; C.out = a->out; C.stats = a->stats; C.n_attended = a->n_attended;
  C.hdr = c->S.hdr;
  k_combine<<<dim3(c->S.Hq, a->batch), 64, 0, st>>>(C);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}
