/*
 * ThinKV decode hot path -- CPU ORACLE.  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the graft smoke entry and the bench's cpu_baseline leg may
 * load this library.  The product path never calls it.  It shares no source,
 * header, table or helper with the HIP library; every layout constant below is
 * re-derived here from the state-format description.
 *
 * Plain, sequential and slow on purpose:
 *   - quantizer in IEEE fp32 (no contraction; build with -ffp-contract=off),
 *     with its own round-to-nearest-even fp32 -> fp16 conversion;
 *   - allocator / segment / eviction state machine applied item by item in
 *     list order;
 *   - attention gathered, dequantized and soft-maxed in fp64.
 *
 * What the method computes (pages: "ThinKV: Thought-Adaptive KV Cache
 * Compression for Efficient Reasoning Models", the arXiv abstract page and
 * the technical summary pages, section "Methodologie"/"Methodology"):
 *   - thought types R/E/T are read off attention sparsity (bullets on thought
 *     decomposition; T most sparse, then R, E least);
 *   - tokens are group-quantized at a precision set by thought type, R > E > T
 *     (TBQ bullet), here asymmetric integer 8/4/2-bit with fp16 scale and
 *     zero-point per group;
 *   - less critical thought segments are evicted at segment granularity
 *     (TBE bullet);
 *   - evicted slots are reused in place by new tokens of the same precision
 *     class through a block table holding thought type, start index and
 *     eviction mask, so the cache is never compacted (Continuous Thinking
 *     bullet).
 * Readings taken where the pages are silent are listed beside each function.
 *
 * Parity pins: see tests/test_oracle_*.py.  Thought semantics of the labels
 * (whether R/E/T mean anything for a real model) are parity unpinned: that
 * needs trained weights and data.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define ORA_OK      0
#define ORA_EINVAL (-1)
#define ORA_ENOMEM (-2)
#define ORA_ENOSEG (-3)

#define BS 16            /* tokens per block (PagedAttention block size) */
#define SEQ_W 16         /* int32 words per sequence record              */
#define HDR_W 16         /* int32 words in the header                    */
#define SEG_W 8          /* int32 words per segment record               */
#define BLK_W 4          /* int32 words per block record                 */
#define SLOT_W 2         /* int32 words per slot record                  */

/* class index c = 0,1,2 holds 8-, 4-, 2-bit codes */
static const int CLASS_BITS[3] = {8, 4, 2};

typedef struct {
  int32_t num_kv_heads, num_q_heads, head_dim, group_size;
  int32_t bits[3];               /* bits for thought type R, E, T */
  int32_t pool_blocks[3];
  int32_t max_seqs, max_blocks_per_seq, max_segments_per_seq;
  int32_t num_layers;            /* layers sharing block tables and eviction; 0 counts as 1 */
  int32_t code_format;           /* 0: integer codes; 1: FP8 E4M3 / FP4 E2M1 / ternary by class */
} ora_layout;

typedef struct {
  uint8_t *pool[3];
  int32_t *blk[3];
  int32_t *slot[3];
  int32_t *freestk[3];
  int32_t *hdr;
  int32_t *seq;
  int32_t *btab;
  int32_t *sstk;
  int32_t *segt;
} ora_state;

/* ---------------------------------------------------------------------- */
/* fp16 <-> fp32, written from the IEEE-754 binary16 definition.           */
/* ---------------------------------------------------------------------- */

/* Round-to-nearest-even conversion of an fp32 value to binary16 bits.
   Subnormal results are kept; overflow goes to infinity; NaN stays NaN. */
uint16_t ora_f32_to_f16(float f) {
  uint32_t x; memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  int32_t  e    = (int32_t)((x >> 23) & 0xff);
  uint32_t m    = x & 0x7fffffu;
  if (e == 0xff) return (uint16_t)(sign | 0x7c00u | (m ? 0x200u : 0u));
  /* value = 1.m * 2^(e-127) for normal inputs; fp32 subnormals are far
     below half of the smallest fp16 subnormal and round to zero. */
  if (e == 0) return (uint16_t)sign;
  int32_t he = e - 127 + 15;                 /* biased fp16 exponent */
  uint32_t mant = m | 0x800000u;             /* 24-bit significand   */
  if (he >= 31) return (uint16_t)(sign | 0x7c00u);
  int shift;                                 /* bits dropped from the 24-bit significand */
  uint32_t base_exp;
  if (he >= 1) { shift = 13; base_exp = (uint32_t)he; }
  else {                                     /* subnormal result: 2^-24 units */
    shift = 14 - he;                         /* he=0 -> 14, he=-10 -> 24 */
    if (shift > 25) return (uint16_t)sign;   /* below half the smallest subnormal */
    base_exp = 0;
  }
  uint32_t kept = mant >> shift;
  uint32_t rem  = mant & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (kept & 1u))) kept += 1u;
  uint32_t bits;
  if (base_exp == 0) bits = kept;                       /* may carry into the normal range: still correct */
  else bits = (base_exp << 10) + (kept - 0x400u);       /* drop the implicit bit; carry bumps the exponent */
  if (bits >= 0x7c00u) bits = 0x7c00u;
  return (uint16_t)(sign | bits);
}

double ora_f16_to_f64(uint16_t h) {
  int e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m | 0x400), e - 25);
  return (h & 0x8000) ? -v : v;
}

static float f16_to_f32(uint16_t h) { return (float)ora_f16_to_f64(h); }

static double bf16_to_f64(uint16_t b) {
  uint32_t x = (uint32_t)b << 16; float f; memcpy(&f, &x, 4); return (double)f;
}

/* ---------------------------------------------------------------------- */
/* State-format geometry                                                   */
/* ---------------------------------------------------------------------- */

static int64_t chunk_bytes(const ora_layout *L, int c) { return (int64_t)L->head_dim * CLASS_BITS[c] / 32; }
static int64_t codes_bytes(const ora_layout *L, int c) { return 64 * chunk_bytes(L, c); }
static int64_t meta_bytes(const ora_layout *L) { return (int64_t)BS * (L->head_dim / L->group_size) * 4; }
/* KV heads stored per block: every layer's (the layers share block tables,
   segments and eviction, so a token's rows of all layers sit in one slot). */
int ora_stored_heads(const ora_layout *L) { return L->num_kv_heads * (L->num_layers > 1 ? L->num_layers : 1); }
int64_t ora_block_head_bytes(const ora_layout *L, int c) { return 2 * codes_bytes(L, c) + 2 * meta_bytes(L); }

static uint8_t *block_head(const ora_layout *L, ora_state *S, int c, int blk, int head) {
  return S->pool[c] + ((int64_t)blk * ora_stored_heads(L) + head) * ora_block_head_bytes(L, c);
}

/* Bit offset of element e within a chunk of `bits`-wide codes.  Codes are
   grouped in little-endian 32-bit words of W = 32/bits codes; the low 16
   bits of a word hold the word's even-indexed codes and the high 16 bits its
   odd-indexed codes, each half least-significant field first. */
static int64_t elem_bit(int64_t e, int bits) {
  int64_t W = 32 / bits, w = e / W, f = e % W;
  int64_t p = (f >> 1) + (f & 1) * (W / 2);
  return w * 32 + p * bits;
}
/* Float codes (code_format 1, 8- and 4-bit classes) sit in their words in
   element order, least significant field first; ternary codes, which are
   integers on a three-level grid, keep the integer order. */
static int64_t elem_bit_of(const ora_layout *L, int64_t e, int bits) {
  return (L->code_format && bits > 2) ? e * bits : elem_bit(e, bits);
}

/* A code region holds 64 chunks.  A chunk of CB bytes is cut into units of
   U = min(CB, 16) bytes; unit u of chunk k occupies bytes [(64u + k) U,
   (64u + k + 1) U) of the region (for CB <= 16: chunk k at byte k*CB).
   Bit `bit` of chunk k -> bit offset within the region. */
static int64_t chunk_bit(const ora_layout *L, int c, int64_t k, int64_t bit) {
  int64_t CB = chunk_bytes(L, c), U = CB < 16 ? CB : 16;
  int64_t byte = bit / 8, u = byte / U;
  return ((64 * u + k) * U + byte % U) * 8 + bit % 8;
}

/* K code of token t (0..15), dim d: chunk 16*lg + t, element gi*(g/4) + e',
   where gi = d / g, lg = (d % g) / (g/4), e' = d % (g/4). */
static int64_t k_code_bit(const ora_layout *L, int c, int t, int d) {
  int g = L->group_size, q4 = g / 4;
  int gi = d / g, w = d % g, lg = w / q4, ep = w % q4;
  int64_t chunk = 16 * lg + t;
  return chunk_bit(L, c, chunk, elem_bit_of(L, (int64_t)gi * q4 + ep, CLASS_BITS[c]));
}

/* V code of token t = 4q + r, dim d = 16n + i: chunk 16*q + i, element 4n + r. */
static int64_t v_code_bit(const ora_layout *L, int c, int t, int d) {
  int q = t / 4, r = t % 4, n = d / 16, i = d % 16;
  int64_t chunk = 16 * q + i;
  return codes_bytes(L, c) * 8 + chunk_bit(L, c, chunk, elem_bit_of(L, (int64_t)n * 4 + r, CLASS_BITS[c]));
}

/* byte offset of the (scale, zero) fp16 pair of token t, group gi, tensor kv (0=K, 1=V) */
static int64_t meta_off(const ora_layout *L, int c, int kv, int t, int gi) {
  int NG = L->head_dim / L->group_size;
  return 2 * codes_bytes(L, c) + kv * meta_bytes(L) + ((int64_t)t * NG + gi) * 4;
}

static unsigned get_code(const uint8_t *base, int64_t bit, int bits) {
  unsigned v = 0;
  for (int b = 0; b < bits; b++) v |= (unsigned)((base[(bit + b) >> 3] >> ((bit + b) & 7)) & 1u) << b;
  return v;
}
static void put_code(uint8_t *base, int64_t bit, int bits, unsigned code) {
  for (int b = 0; b < bits; b++) {
    int64_t at = bit + b;
    uint8_t mask = (uint8_t)(1u << (at & 7));
    if ((code >> b) & 1u) base[at >> 3] |= mask; else base[at >> 3] &= (uint8_t)~mask;
  }
}
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }

/* record accessors */
static int32_t *SEQ(const ora_layout *L, ora_state *S, int s) { (void)L; return S->seq + (int64_t)s * SEQ_W; }
static int32_t *BTAB(const ora_layout *L, ora_state *S, int s, int c) { return S->btab + ((int64_t)s * 3 + c) * L->max_blocks_per_seq; }
static int32_t *SSTK(const ora_layout *L, ora_state *S, int s, int c) { return S->sstk + ((int64_t)s * 3 + c) * L->max_blocks_per_seq * BS; }
static int32_t *SEGR(const ora_layout *L, ora_state *S, int s, int k) { return S->segt + ((int64_t)s * L->max_segments_per_seq + k) * SEG_W; }
/* SEQ words */
enum { Q_NBLK = 0, Q_NSLOT = 3, Q_NSEG = 6, Q_LEN = 7, Q_NRET = 8, Q_NAPP = 9 };
/* SEG words */
enum { G_TYPE = 0, G_BITS, G_FIRST, G_LAST, G_NTOT, G_NRET };
/* HDR words */
enum { H_FREE = 0, H_EFLAGS = 3, H_EMINSEQ = 4, H_ECOUNT = 5 };

static int class_of_bits(int bits) { return bits == 8 ? 0 : bits == 4 ? 1 : bits == 2 ? 2 : -1; }

static void record_error(ora_state *S, int code, int seq) {
  S->hdr[H_EFLAGS] |= 1 << (-code);
  if (seq < S->hdr[H_EMINSEQ]) S->hdr[H_EMINSEQ] = seq;
  S->hdr[H_ECOUNT] += 1;
}

/* ---------------------------------------------------------------------- */
/* Initial state                                                           */
/* ---------------------------------------------------------------------- */

/* order[c] (nullable) lists the blocks of pool c in the order they will be
   popped; NULL means 0, 1, 2, ...  The stack array holds that order reversed
   (top of stack = last element). */
void ora_init(const ora_layout *L, ora_state *S, const int32_t *const order[3]) {
  for (int c = 0; c < 3; c++) {
    int P = L->pool_blocks[c];
    memset(S->pool[c], 0, (size_t)(P * ora_block_head_bytes(L, c)));
    for (int b = 0; b < P; b++) {
      S->blk[c][b * BLK_W + 0] = 0; S->blk[c][b * BLK_W + 1] = -1;
      S->blk[c][b * BLK_W + 2] = -1; S->blk[c][b * BLK_W + 3] = 0;
      for (int t = 0; t < BS; t++) { S->slot[c][(b * BS + t) * SLOT_W] = -1; S->slot[c][(b * BS + t) * SLOT_W + 1] = -1; }
      S->freestk[c][b] = order && order[c] ? order[c][P - 1 - b] : P - 1 - b;
    }
  }
  memset(S->hdr, 0, HDR_W * 4);
  for (int c = 0; c < 3; c++) S->hdr[H_FREE + c] = L->pool_blocks[c];
  S->hdr[H_EMINSEQ] = 0x7fffffff;
  memset(S->seq, 0, (size_t)L->max_seqs * SEQ_W * 4);
  for (int64_t i = 0; i < (int64_t)L->max_seqs * 3 * L->max_blocks_per_seq; i++) S->btab[i] = -1;
  for (int64_t i = 0; i < (int64_t)L->max_seqs * 3 * L->max_blocks_per_seq * BS; i++) S->sstk[i] = -1;
  memset(S->segt, 0, (size_t)L->max_seqs * L->max_segments_per_seq * SEG_W * 4);
}

/* ---------------------------------------------------------------------- */
/* Quantizer (TBQ bullet: group quantization by thought category).         */
/* Reading: asymmetric integer codes, groups of g consecutive dims of one  */
/* token, one KV head, one tensor; scale = fp16((max-min)/(2^c-1)),        */
/* zero = fp16(min), -0 canonicalized to +0; codes = clamp(rint-even(      */
/* (x - zero)/scale), 0, 2^c-1); a zero scale gives all-zero codes.        */
/* ---------------------------------------------------------------------- */
void ora_quantize_group(const float *x, int n, int bits, unsigned *codes, uint16_t *s16, uint16_t *z16) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < n; i++) { if (x[i] < mn) mn = x[i]; if (x[i] > mx) mx = x[i]; }
  float levels = (float)((1 << bits) - 1);
  float range = mx - mn;
  float s32 = range / levels;
  uint16_t sh = ora_f32_to_f16(s32), zh = ora_f32_to_f16(mn);
  if (sh == 0x8000u) sh = 0;
  if (zh == 0x8000u) zh = 0;
  float sf = f16_to_f32(sh), zf = f16_to_f32(zh);
  for (int i = 0; i < n; i++) {
    if (sf == 0.0f) { codes[i] = 0; continue; }
    float diff = x[i] - zf;
    float qv = diff / sf;
    float r = nearbyintf(qv);               /* default rounding mode: to nearest, ties to even */
    if (r < 0.0f) r = 0.0f;
    if (r > levels) r = levels;
    codes[i] = (unsigned)r;
  }
  *s16 = sh; *z16 = zh;
}

/* ---------------------------------------------------------------------- */
/* Float and ternary codes (code_format 1; TBQ bullet: 8-bit FP8 for       */
/* Reasoning tokens, a 4-bit float for Execution, 2-bit ternary for        */
/* Transition).  Symmetric, one fp16 scale per group, zero-point 0.        */
/*   FP8 E4M3 (class 0): s = fp16(amax / 448); code = E4M3 of x / s,       */
/*     round to nearest even, saturated at +-448.                          */
/*   FP4 E2M1 (class 1): s = fp16(amax / 6); code = E2M1 of x / s, round   */
/*     to nearest, ties to the even mantissa, saturated at +-6.            */
/*   Ternary (class 2), the rule of Ternary Weight Networks (Li, Zhang,    */
/*     Liu 2016): threshold 0.7 * mean |x|; t = sign(x) where |x| exceeds  */
/*     it, else 0; s = fp16(mean |x| over the nonzero t).  Sums are        */
/*     pairwise over index halves.  Stored as the integer code t + 1 with  */
/*     zero-point -s, so x^ = s * code + zero as for integer codes.        */
/* A zero scale gives all-zero codes and zero-point; zero and -0 float     */
/* codes are +0.                                                           */
/* ---------------------------------------------------------------------- */
static double e4m3_value(unsigned c) {
  int e = (c >> 3) & 15, m = c & 7;
  double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  return (c & 0x80) ? -v : v;
}
static double e2m1_value(unsigned c) {
  int e = (c >> 1) & 3, m = c & 1;
  double v = e ? ldexp(1.0 + m / 2.0, e - 1) : m * 0.5;
  return (c & 8) ? -v : v;
}

static unsigned e4m3_code(float y) {
  double a = fabs((double)y);
  unsigned mag;
  if (a >= 448.0) mag = 0x7E;
  else if (a < ldexp(1.0, -6)) mag = (unsigned)nearbyint(a * 512.0);          /* subnormal steps of 2^-9 */
  else {
    int E; frexp(a, &E); E -= 1;                                              /* 2^E <= a < 2^(E+1) */
    double q = (ldexp(a, -E) - 1.0) * 8.0;
    int m = (int)nearbyint(q);
    if (m == 8) { m = 0; E += 1; }
    mag = (unsigned)(((E + 7) << 3) | m);
  }
  return mag == 0 ? 0 : mag | (y < 0.0f ? 0x80u : 0u);
}
static unsigned e2m1_code(float y) {
  double a = fabs((double)y);
  unsigned mag;
  if (a >= 6.0) mag = 7;
  else if (a < 1.0) mag = (unsigned)nearbyint(a * 2.0);                       /* 0, 0.5, 1 */
  else {
    int E; frexp(a, &E); E -= 1;
    double q = (ldexp(a, -E) - 1.0) * 2.0;
    int m = (int)nearbyint(q);
    if (m == 2) { m = 0; E += 1; }
    mag = (unsigned)(((E + 1) << 1) | m);
  }
  return mag == 0 ? 0 : mag | (y < 0.0f ? 8u : 0u);
}
static float pairwise_sum(const float *x, int n) {
  return n == 1 ? x[0] : pairwise_sum(x, n / 2) + pairwise_sum(x + n / 2, n / 2);
}

void ora_quantize_group_fmt(int c, const float *x, int n, unsigned *codes, uint16_t *s16, uint16_t *z16) {
  float a[256];
  float amax = 0.0f;
  for (int i = 0; i < n; i++) { a[i] = fabsf(x[i]); if (a[i] > amax) amax = a[i]; }
  uint16_t sh;
  if (c == 2) {
    float thr = 0.7f * (pairwise_sum(a, n) / (float)n);
    float kept[256]; int cnt = 0;
    for (int i = 0; i < n; i++) { int on = x[i] > thr || x[i] < -thr; kept[i] = on ? a[i] : 0.0f; cnt += on; }
    sh = cnt ? ora_f32_to_f16(pairwise_sum(kept, n) / (float)cnt) : 0;
    for (int i = 0; i < n; i++)
      codes[i] = sh == 0 ? 0 : (x[i] > thr ? 2u : (x[i] < -thr ? 0u : 1u));
  } else {
    sh = ora_f32_to_f16(amax / (c == 0 ? 448.0f : 6.0f));
    float sf = f16_to_f32(sh);
    for (int i = 0; i < n; i++)
      codes[i] = sh == 0 ? 0 : (c == 0 ? e4m3_code(x[i] / sf) : e2m1_code(x[i] / sf));
  }
  if (sh == 0x8000u) sh = 0;
  *s16 = sh;
  *z16 = (c == 2 && sh) ? (uint16_t)(sh ^ 0x8000u) : 0;
}
/* value of a stored code, before the group's scale and zero-point */
static double code_value(const ora_layout *L, int c, unsigned code) {
  if (!L->code_format || c == 2) return (double)code;
  return c == 0 ? e4m3_value(code) : e2m1_value(code);
}
double ora_code_value(int code_format, int c, unsigned code) {
  ora_layout L; memset(&L, 0, sizeof L); L.code_format = code_format;
  return code_value(&L, c, code);
}

/* Quantize one token's K and V rows of one KV head into block-head memory. */
static void store_token(const ora_layout *L, ora_state *S, int c, int blk, int t, int head,
                        const float *krow, const float *vrow) {
  int D = L->head_dim, g = L->group_size, NG = D / g, bits = CLASS_BITS[c];
  uint8_t *bh = block_head(L, S, c, blk, head);
  unsigned codes[256]; uint16_t sh, zh;
  for (int kv = 0; kv < 2; kv++) {
    const float *row = kv ? vrow : krow;
    for (int gi = 0; gi < NG; gi++) {
      if (L->code_format) ora_quantize_group_fmt(c, row + gi * g, g, codes, &sh, &zh);
      else ora_quantize_group(row + gi * g, g, bits, codes, &sh, &zh);
      for (int j = 0; j < g; j++) {
        int d = gi * g + j;
        int64_t bit = kv ? v_code_bit(L, c, t, d) : k_code_bit(L, c, t, d);
        put_code(bh, bit, bits, codes[j]);
      }
      uint8_t *m = bh + meta_off(L, c, kv, t, gi);
      put_u16(m, sh); put_u16(m + 2, zh);
    }
  }
}

/* Dequantize one token's row (fp32, as the downgrade path re-reads it). */
static void load_token_f32(const ora_layout *L, ora_state *S, int c, int blk, int t, int head, int kv, float *row) {
  int D = L->head_dim, g = L->group_size, bits = CLASS_BITS[c];
  uint8_t *bh = block_head(L, S, c, blk, head);
  for (int d = 0; d < D; d++) {
    int gi = d / g;
    uint8_t *m = bh + meta_off(L, c, kv, t, gi);
    float sf = f16_to_f32(get_u16(m)), zf = f16_to_f32(get_u16(m + 2));
    unsigned code = get_code(bh, kv ? v_code_bit(L, c, t, d) : k_code_bit(L, c, t, d), bits);
    float prod = sf * (float)code_value(L, c, code);   /* exact: 11-bit by <=8-bit significands */
    row[d] = prod + zf;
  }
}

/* The fp32 rows (K then V) of the token in slot `slot` of class c, head h
   (test access to stored tokens). */
void ora_token_rows(const ora_layout *L, ora_state *S, int c, int slot, int head, float *k, float *v) {
  load_token_f32(L, S, c, slot / BS, slot % BS, head, 0, k);
  load_token_f32(L, S, c, slot / BS, slot % BS, head, 1, v);
}

/* Dequantize one code exactly in fp64. */
static double deq64(const ora_layout *L, ora_state *S, int c, int blk, int t, int head, int kv, int d) {
  uint8_t *bh = block_head(L, S, c, blk, head);
  uint8_t *m = bh + meta_off(L, c, kv, t, d / L->group_size);
  unsigned code = get_code(bh, kv ? v_code_bit(L, c, t, d) : k_code_bit(L, c, t, d), CLASS_BITS[c]);
  return ora_f16_to_f64(get_u16(m)) * code_value(L, c, code) + ora_f16_to_f64(get_u16(m + 2));
}

/* ---------------------------------------------------------------------- */
/* Slot allocation (Continuous Thinking bullet: evicted slots are reused   */
/* in place).  Reading: per (sequence, class) a LIFO free-slot stack; when */
/* it is empty one block is popped from the class's global LIFO block      */
/* stack, appended to the sequence's block list, and its 16 slots pushed   */
/* so that slot 0 is popped first.  Blocks go back to the global stack     */
/* only on sequence reset.                                                 */
/* ---------------------------------------------------------------------- */
static int pop_slot(const ora_layout *L, ora_state *S, int s, int c) {
  int32_t *q = SEQ(L, S, s);
  if (q[Q_NSLOT + c] == 0) {
    int blk = S->freestk[c][--S->hdr[H_FREE + c]];
    BTAB(L, S, s, c)[q[Q_NBLK + c]++] = blk;
    S->blk[c][blk * BLK_W + 2] = s;
    int32_t *st = SSTK(L, S, s, c);
    for (int t = BS - 1; t >= 0; t--) st[q[Q_NSLOT + c]++] = blk * BS + t;
  }
  return SSTK(L, S, s, c)[--q[Q_NSLOT + c]];
}
static void push_slot(const ora_layout *L, ora_state *S, int s, int c, int slot) {
  int32_t *q = SEQ(L, S, s);
  SSTK(L, S, s, c)[q[Q_NSLOT + c]++] = slot;
}

static void occupy(const ora_layout *L, ora_state *S, int c, int slot, int pos, int segid) {
  (void)L;
  int blk = slot / BS, t = slot % BS;
  S->blk[c][blk * BLK_W + 0] |= 1 << t;
  if (pos > S->blk[c][blk * BLK_W + 1]) S->blk[c][blk * BLK_W + 1] = pos;
  S->slot[c][slot * SLOT_W + 0] = pos;
  S->slot[c][slot * SLOT_W + 1] = segid;
}
static void vacate(const ora_layout *L, ora_state *S, int c, int slot) {
  (void)L;
  S->blk[c][(slot / BS) * BLK_W + 0] &= ~(1 << (slot % BS));
}

/* ---------------------------------------------------------------------- */
/* kv_append_quant: tokens applied one by one in list order.               */
/* k, v: fp32 [n][L][Hkv][D].  slot_out (nullable): (class << 28) | slot, or */
/* -1 for a token that was not stored.                                     */
/* Segments (TBE bullet: eviction acts on runs of one thought type): a maximal run of */
/* consecutively appended tokens of one sequence with the same type (and   */
/* the same precision class, should the open segment have been downgraded).*/
/* Failure rules (per call): a token whose sequence already failed in this */
/* call is skipped; bad arguments give EINVAL, a full segment table or     */
/* block list ENOMEM, and the first pool exhaustion of a class makes every */
/* later block-needing token of that class fail with ENOMEM.  A failing    */
/* token leaves the state untouched and marks its sequence failed.         */
/* ---------------------------------------------------------------------- */
void ora_append(const ora_layout *L, ora_state *S, int n, const int32_t *seq_ids, const int32_t *pos,
                const uint8_t *thought, const float *k, const float *v, int32_t *slot_out) {
  int H = ora_stored_heads(L), D = L->head_dim;
  char *failed = calloc((size_t)L->max_seqs, 1);
  int dry[3] = {0, 0, 0};
  for (int i = 0; i < n; i++) {
    if (slot_out) slot_out[i] = -1;
    int s = seq_ids[i];
    if (s < 0 || s >= L->max_seqs) { record_error(S, ORA_EINVAL, s < 0 ? 0x7fffffff : s); continue; }
    if (failed[s]) continue;
    int32_t *q = SEQ(L, S, s);
    int y = thought[i];
    if (y > 2 || pos[i] < q[Q_LEN]) { record_error(S, ORA_EINVAL, s); failed[s] = 1; continue; }
    int c = class_of_bits(L->bits[y]);
    int nseg = q[Q_NSEG];
    /* a new segment opens when the type changes, or when the open segment
       was moved to another precision class (downgraded) meanwhile */
    int new_seg = (nseg == 0) || (SEGR(L, S, s, nseg - 1)[G_TYPE] != y) ||
                  (SEGR(L, S, s, nseg - 1)[G_BITS] != CLASS_BITS[c]);
    if (new_seg && nseg == L->max_segments_per_seq) { record_error(S, ORA_ENOMEM, s); failed[s] = 1; continue; }
    if (q[Q_NSLOT + c] == 0) {
      if (q[Q_NBLK + c] == L->max_blocks_per_seq) { record_error(S, ORA_ENOMEM, s); failed[s] = 1; continue; }
      if (dry[c] || S->hdr[H_FREE + c] == 0) { dry[c] = 1; record_error(S, ORA_ENOMEM, s); failed[s] = 1; continue; }
    }
    int slot = pop_slot(L, S, s, c);
    if (new_seg) {
      int32_t *g = SEGR(L, S, s, nseg);
      g[G_TYPE] = y; g[G_BITS] = CLASS_BITS[c]; g[G_FIRST] = pos[i]; g[G_LAST] = pos[i];
      g[G_NTOT] = 0; g[G_NRET] = 0; g[6] = 0; g[7] = 0;
      q[Q_NSEG] = nseg + 1;
    }
    int segid = q[Q_NSEG] - 1;
    int32_t *g = SEGR(L, S, s, segid);
    g[G_LAST] = pos[i]; g[G_NTOT] += 1; g[G_NRET] += 1;
    for (int h = 0; h < H; h++)
      store_token(L, S, c, slot / BS, slot % BS, h, k + ((int64_t)i * H + h) * D, v + ((int64_t)i * H + h) * D);
    occupy(L, S, c, slot, pos[i], segid);
    q[Q_LEN] = pos[i] + 1; q[Q_NRET] += 1; q[Q_NAPP] += 1;
    if (slot_out) slot_out[i] = (c << 28) | slot;
  }
  free(failed);
}

/* Collect the valid slots of segment k of sequence s, sorted by position. */
static int segment_slots(const ora_layout *L, ora_state *S, int s, int k, int c, int32_t *slots) {
  int32_t *q = SEQ(L, S, s);
  int n = 0;
  for (int j = 0; j < q[Q_NBLK + c]; j++) {
    int blk = BTAB(L, S, s, c)[j];
    int mask = S->blk[c][blk * BLK_W];
    for (int t = 0; t < BS; t++)
      if (((mask >> t) & 1) && S->slot[c][(blk * BS + t) * SLOT_W + 1] == k) slots[n++] = blk * BS + t;
  }
  /* insertion sort by position (positions of one sequence are unique) */
  for (int a = 1; a < n; a++) {
    int32_t x = slots[a]; int px = S->slot[c][x * SLOT_W]; int b = a - 1;
    while (b >= 0 && S->slot[c][slots[b] * SLOT_W] > px) { slots[b + 1] = slots[b]; b--; }
    slots[b + 1] = x;
  }
  return n;
}

/* ---------------------------------------------------------------------- */
/* kv_evict_segment (TBE bullet: segment-granular, progressive eviction).  */
/* Op (s, k, keep_n, new_bits): keep the keep_n newest retained tokens of  */
/* segment k (0 = none), evict the rest (valid bit cleared, slot pushed on */
/* the sequence's stack in ascending position order).  new_bits below the  */
/* segment's bits re-quantizes the kept tokens from their dequantized fp32 */
/* values into slots of the lower class (popped in ascending position      */
/* order), then frees the old slots (pushed in ascending position order).  */
/* A segment may appear in one op per call.                                */
/* ---------------------------------------------------------------------- */
void ora_evict(const ora_layout *L, ora_state *S, int n_ops, const int32_t *seq_ids, const int32_t *seg_ids,
               const int32_t *keep_n, const uint8_t *new_bits) {
  int H = ora_stored_heads(L), D = L->head_dim;
  char *failed = calloc((size_t)L->max_seqs, 1);
  int dry[3] = {0, 0, 0};
  int32_t *slots = malloc(sizeof(int32_t) * (size_t)L->max_blocks_per_seq * BS);
  float *krow = malloc(sizeof(float) * (size_t)D), *vrow = malloc(sizeof(float) * (size_t)D);
  for (int i = 0; i < n_ops; i++) {
    int s = seq_ids[i];
    if (s < 0 || s >= L->max_seqs) { record_error(S, ORA_EINVAL, s < 0 ? 0x7fffffff : s); continue; }
    if (failed[s]) continue;
    int32_t *q = SEQ(L, S, s);
    int k = seg_ids[i];
    if (k < 0 || k >= q[Q_NSEG]) { record_error(S, ORA_ENOSEG, s); failed[s] = 1; continue; }
    int dup = 0;
    for (int j = 0; j < i; j++) if (seq_ids[j] == s && seg_ids[j] == k) dup = 1;
    int nb = new_bits[i];
    int32_t *g = SEGR(L, S, s, k);
    if (dup || keep_n[i] < 0 || !(nb == 0 || nb == 2 || nb == 4 || nb == 8) || (nb != 0 && nb > g[G_BITS])) {
      record_error(S, ORA_EINVAL, s); failed[s] = 1; continue;
    }
    if (g[G_NRET] == 0) { record_error(S, ORA_ENOSEG, s); failed[s] = 1; continue; }
    int c = class_of_bits(g[G_BITS]);
    int r = g[G_NRET];
    int keep = keep_n[i] < r ? keep_n[i] : r;
    int down = (nb != 0 && nb < g[G_BITS] && keep > 0);
    int c2 = down ? class_of_bits(nb) : c;
    if (down) {
      int have = q[Q_NSLOT + c2];
      int need = keep > have ? (keep - have + BS - 1) / BS : 0;
      if (q[Q_NBLK + c2] + need > L->max_blocks_per_seq) { record_error(S, ORA_ENOMEM, s); failed[s] = 1; continue; }
      if (need > 0 && (dry[c2] || need > S->hdr[H_FREE + c2])) { dry[c2] = 1; record_error(S, ORA_ENOMEM, s); failed[s] = 1; continue; }
    }
    int n = segment_slots(L, S, s, k, c, slots);
    int ev = n - keep;
    for (int j = 0; j < ev; j++) { vacate(L, S, c, slots[j]); push_slot(L, S, s, c, slots[j]); }
    if (down) {
      for (int j = ev; j < n; j++) {
        int old = slots[j];
        int p = S->slot[c][old * SLOT_W];
        int ns = pop_slot(L, S, s, c2);
        for (int h = 0; h < H; h++) {
          load_token_f32(L, S, c, old / BS, old % BS, h, 0, krow);
          load_token_f32(L, S, c, old / BS, old % BS, h, 1, vrow);
          store_token(L, S, c2, ns / BS, ns % BS, h, krow, vrow);
        }
        occupy(L, S, c2, ns, p, k);
      }
      for (int j = ev; j < n; j++) { vacate(L, S, c, slots[j]); push_slot(L, S, s, c, slots[j]); }
      g[G_BITS] = nb;
    }
    g[G_NRET] = keep;
    q[Q_NRET] -= ev;
  }
  free(krow); free(vrow); free(slots); free(failed);
}

/* ---------------------------------------------------------------------- */
/* Budget ladder.  Budget in tokens: B = floor(len * num / den), len = the */
/* sequence's logical length (last appended position + 1).  While the     */
/* retained count exceeds B, evict whole T segments oldest first, never    */
/* the open (last) segment nor the newest retained T segment (the safety   */
/* net of Transition thoughts, lay summary "Astuce B").  If still over,     */
/* downgrade the single oldest non-open E segment still above 2 bits to    */
/* 2 bits.  Ops go out in list order of the sequences; at most max_ops.    */
/* ---------------------------------------------------------------------- */
int ora_plan_budget(const ora_layout *L, ora_state *S, int n, const int32_t *seq_ids, int num, int den, int max_ops,
                    int32_t *op_seq, int32_t *op_seg, int32_t *op_keep, uint8_t *op_bits) {
  int m = 0;
  for (int i = 0; i < n; i++) {
    int s = seq_ids[i];
    if (s < 0 || s >= L->max_seqs) continue;
    int32_t *q = SEQ(L, S, s);
    int nseg = q[Q_NSEG];
    long long B = (long long)q[Q_LEN] * num / den;
    long long nr = q[Q_NRET];
    if (nr <= B) continue;
    int newest_t = -1;
    for (int k = 0; k < nseg; k++) { int32_t *g = SEGR(L, S, s, k); if (g[G_TYPE] == 2 && g[G_NRET] > 0) newest_t = k; }
    for (int k = 0; k < nseg - 1 && nr > B; k++) {
      int32_t *g = SEGR(L, S, s, k);
      if (g[G_TYPE] != 2 || g[G_NRET] == 0 || k == newest_t) continue;
      if (m < max_ops) { op_seq[m] = s; op_seg[m] = k; op_keep[m] = 0; op_bits[m] = 0; m++; }
      nr -= g[G_NRET];
    }
    if (nr > B) {
      for (int k = 0; k < nseg - 1; k++) {
        int32_t *g = SEGR(L, S, s, k);
        if (g[G_TYPE] == 1 && g[G_BITS] > 2 && g[G_NRET] > 0) {
          if (m < max_ops) { op_seq[m] = s; op_seg[m] = k; op_keep[m] = g[G_NRET]; op_bits[m] = 2; m++; }
          break;
        }
      }
    }
  }
  return m;
}

/* ---------------------------------------------------------------------- */
/* Annealing schedule of TBE (Methodology, TBE bullet: once a Transition  */
/* thought is detected, tokens of the earlier, less critical Reasoning or  */
/* Execution segments are evicted progressively on an annealing schedule   */
/* of the retention, e.g. 64, then 32, then 16, at segment granularity;    */
/* lay summary "Astuce B": a small safety net of Transition thoughts is    */
/* always kept).  Reading: a T event is the opening of a T segment; an R   */
/* or E segment followed by e >= 1 T segments has retention cap            */
/* r0 / 2^(e-1) (integer halving, 0 once halved to nothing), and keeps its */
/* cap newest retained tokens; T segments are never planned.  The cap      */
/* depends only on the segment table, so planning twice gives no new ops.  */
/* Ops (s, k, keep_n = cap, bits 0) in list order of the sequences and     */
/* segment order; at most max_ops are written and counted.                 */
/* ---------------------------------------------------------------------- */
int ora_plan_anneal(const ora_layout *L, ora_state *S, int n, const int32_t *seq_ids, int r0, int max_ops,
                    int32_t *op_seq, int32_t *op_seg, int32_t *op_keep, uint8_t *op_bits) {
  int m = 0;
  for (int i = 0; i < n; i++) {
    int s = seq_ids[i];
    if (s < 0 || s >= L->max_seqs) continue;
    int32_t *q = SEQ(L, S, s);
    int nseg = q[Q_NSEG];
    for (int k = 0; k < nseg; k++) {
      int32_t *g = SEGR(L, S, s, k);
      if (g[G_TYPE] == 2 || g[G_NRET] == 0) continue;
      int events = 0;                       /* T segments opened after segment k */
      for (int j = k + 1; j < nseg; j++)
        if (SEGR(L, S, s, j)[G_TYPE] == 2) events++;
      if (events == 0) continue;
      int cap = r0;
      for (int e = 1; e < events && cap > 0; e++) cap /= 2;
      if (g[G_NRET] > cap && m < max_ops) {
        op_seq[m] = s; op_seg[m] = k; op_keep[m] = cap; op_bits[m] = 0; m++;
      }
    }
  }
  return m;
}

/* ---------------------------------------------------------------------- */
/* Gather compaction: the baseline that in-place reuse avoids (abstract:   */
/* the kernel reuses evicted tokens' slots, so no compaction is needed;    */
/* Continuous Thinking bullet).  Reading: for each listed sequence (an id  */
/* listed again is compacted once, at its first listing) and each class    */
/* holding blocks, its m retained tokens are copied bit for bit, in       */
/* position order, into ceil(m/16) blocks popped from the class's global   */
/* stack (token i into slot i % 16 of the (i/16)-th popped block); those   */
/* blocks become the class's block list and the free-slot stack becomes    */
/* the empty tail of the last one (lowest slot on top).  All pops of the   */
/* call come first, in list order; then the old blocks of every compacted  */
/* sequence go back to their global stacks (sequences in list order,       */
/* classes in order, blocks in list order, records cleared), so no copy    */
/* reads a block written in the same call.  A sequence that does not find  */
/* all its blocks fails with ENOMEM and is left untouched; after the first */
/* such failure of a class, every later sequence needing blocks of that    */
/* class fails too.  Ids outside [0, max_seqs): EINVAL.                    */
/* ---------------------------------------------------------------------- */
static int32_t token_pos(ora_state *S, int c, int slot) { return S->slot[c][slot * SLOT_W]; }

static void copy_token(const ora_layout *L, ora_state *S, int c, int src, int dst) {
  int D = L->head_dim, NG = D / L->group_size, bits = CLASS_BITS[c];
  for (int h = 0; h < ora_stored_heads(L); h++) {
    uint8_t *sb = block_head(L, S, c, src / BS, h), *db = block_head(L, S, c, dst / BS, h);
    int ts = src % BS, td = dst % BS;
    for (int d = 0; d < D; d++) {
      put_code(db, k_code_bit(L, c, td, d), bits, get_code(sb, k_code_bit(L, c, ts, d), bits));
      put_code(db, v_code_bit(L, c, td, d), bits, get_code(sb, v_code_bit(L, c, ts, d), bits));
    }
    for (int kv = 0; kv < 2; kv++)
      for (int gi = 0; gi < NG; gi++) memcpy(db + meta_off(L, c, kv, td, gi), sb + meta_off(L, c, kv, ts, gi), 4);
  }
}

void ora_compact(const ora_layout *L, ora_state *S, int n, const int32_t *seq_ids) {
  int MB = L->max_blocks_per_seq;
  char *seen = calloc((size_t)L->max_seqs, 1);
  int32_t *plan_s = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int32_t *newb = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1) * 3 * MB);
  int32_t *slots = malloc(sizeof(int32_t) * (size_t)MB * BS);
  int dry[3] = {0, 0, 0}, np = 0;
  /* pops, in list order */
  for (int i = 0; i < n; i++) {
    int s = seq_ids[i];
    if (s < 0 || s >= L->max_seqs) { record_error(S, ORA_EINVAL, s < 0 ? 0x7fffffff : s); continue; }
    if (seen[s]) continue;
    seen[s] = 1;
    int32_t *q = SEQ(L, S, s);
    int need[3], ok = 1;
    for (int c = 0; c < 3; c++) {
      int m = 0;
      for (int j = 0; j < q[Q_NBLK + c]; j++) {
        int mask = S->blk[c][BTAB(L, S, s, c)[j] * BLK_W];
        for (int t = 0; t < BS; t++) m += (mask >> t) & 1;
      }
      need[c] = (m + BS - 1) / BS;
    }
    for (int c = 0; c < 3; c++)
      if (need[c] > 0 && (dry[c] || need[c] > S->hdr[H_FREE + c])) { dry[c] = 1; ok = 0; }
    if (!ok) { record_error(S, ORA_ENOMEM, s); continue; }
    int32_t *nb = newb + (int64_t)np * 3 * MB;
    for (int c = 0; c < 3; c++)
      for (int j = 0; j < need[c]; j++) nb[c * MB + j] = S->freestk[c][--S->hdr[H_FREE + c]];
    plan_s[np++] = s;
  }
  /* copies: each class's retained tokens in position order into the popped blocks */
  int32_t *oldb = malloc(sizeof(int32_t) * (size_t)(np > 0 ? np : 1) * 3 * MB);
  int32_t *oldn = malloc(sizeof(int32_t) * (size_t)(np > 0 ? np : 1) * 3);
  for (int p = 0; p < np; p++) {
    int s = plan_s[p];
    int32_t *q = SEQ(L, S, s), *nb = newb + (int64_t)p * 3 * MB;
    for (int c = 0; c < 3; c++) {
      int32_t *bt = BTAB(L, S, s, c);
      int nold = q[Q_NBLK + c];
      oldn[p * 3 + c] = nold;
      memcpy(oldb + ((int64_t)p * 3 + c) * MB, bt, sizeof(int32_t) * (size_t)nold);
      if (nold == 0) continue;
      int m = 0;
      for (int j = 0; j < nold; j++) {
        int blk = bt[j], mask = S->blk[c][blk * BLK_W];
        for (int t = 0; t < BS; t++) if ((mask >> t) & 1) slots[m++] = blk * BS + t;
      }
      for (int a = 1; a < m; a++) {            /* insertion sort by position */
        int32_t x = slots[a]; int b = a - 1;
        while (b >= 0 && token_pos(S, c, slots[b]) > token_pos(S, c, x)) { slots[b + 1] = slots[b]; b--; }
        slots[b + 1] = x;
      }
      int need = (m + BS - 1) / BS;
      for (int i = 0; i < m; i++) {
        int dst = nb[c * MB + i / BS] * BS + i % BS;
        copy_token(L, S, c, slots[i], dst);
        occupy(L, S, c, dst, token_pos(S, c, slots[i]), S->slot[c][slots[i] * SLOT_W + 1]);
      }
      for (int j = 0; j < need; j++) { bt[j] = nb[c * MB + j]; S->blk[c][bt[j] * BLK_W + 2] = s; }
      q[Q_NBLK + c] = need;
      q[Q_NSLOT + c] = 0;
      if (m % BS) {
        int32_t *st = SSTK(L, S, s, c);
        for (int t = BS - 1; t >= m % BS; t--) st[q[Q_NSLOT + c]++] = bt[need - 1] * BS + t;
      }
    }
  }
  /* pushes: the old blocks back, records cleared */
  for (int p = 0; p < np; p++)
    for (int c = 0; c < 3; c++)
      for (int j = 0; j < oldn[p * 3 + c]; j++) {
        int blk = oldb[((int64_t)p * 3 + c) * MB + j];
        S->blk[c][blk * BLK_W + 0] = 0; S->blk[c][blk * BLK_W + 1] = -1; S->blk[c][blk * BLK_W + 2] = -1;
        S->freestk[c][S->hdr[H_FREE + c]++] = blk;
      }
  free(oldb); free(oldn); free(slots); free(newb); free(plan_s); free(seen);
}

/* Return the sequences' blocks to the global stacks (list order, classes
   in order, blocks in block-list order) and clear their records. */
void ora_seq_reset(const ora_layout *L, ora_state *S, int n, const int32_t *seq_ids) {
  for (int i = 0; i < n; i++) {
    int s = seq_ids[i];
    if (s < 0 || s >= L->max_seqs) { record_error(S, ORA_EINVAL, s < 0 ? 0x7fffffff : s); continue; }
    int32_t *q = SEQ(L, S, s);
    for (int c = 0; c < 3; c++) {
      for (int j = 0; j < q[Q_NBLK + c]; j++) {
        int blk = BTAB(L, S, s, c)[j];
        S->blk[c][blk * BLK_W + 0] = 0; S->blk[c][blk * BLK_W + 1] = -1; S->blk[c][blk * BLK_W + 2] = -1;
        S->freestk[c][S->hdr[H_FREE + c]++] = blk;
      }
    }
    memset(q, 0, SEQ_W * 4);
  }
}

/* ---------------------------------------------------------------------- */
/* Attention in fp64 over the current state.                               */
/* One layer per call: the rows of layer `layer` (stored head layer*Hkv+j).*/
/* For batch entry b (sequence seq_ids[b], query position t = q_pos[b])    */
/* and query head h (KV head h / (Hq/Hkv)): the attended set A holds every */
/* valid slot of the sequence in all three classes with pos >= t - W + 1   */
/* when window W > 0, plus the unquantized self token (k_self, v_self)     */
/* when given.  logits l = q.k / sqrt(D), q upcast exactly from bf16.      */
/* out = sum e^(l-m) v / (sum e^(l-m) + [sink] e^(sigma_h - m)).          */
/* Stats over tokens only (sink excluded): p~ = softmax(l); H = -sum p~   */
/* ln p~; H/ln|A| (0 if |A| < 2); sum of the min(topk,|A|) largest p~.     */
/* An empty A gives out = 0 and stats 0.                                   */
/* ---------------------------------------------------------------------- */
void ora_attention(const ora_layout *L, ora_state *S, int batch, const int32_t *seq_ids, const int32_t *q_pos,
                   const uint16_t *qbf, const float *k_self, const float *v_self, const float *sinks,
                   int window, int topk, int layer, double *out, double *stats, int32_t *n_attended) {
  int Hq = L->num_q_heads, Hkv = L->num_kv_heads, D = L->head_dim, G = Hq / Hkv;
  #pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < batch * Hkv; bh++) {
    int b = bh / Hkv, j = bh % Hkv, s = seq_ids[b], t = q_pos[b];
    int32_t *q = SEQ(L, S, s);
    int cap = 1;
    for (int c = 0; c < 3; c++) cap += q[Q_NBLK + c] * BS;
    double *K = malloc(sizeof(double) * (size_t)cap * D), *V = malloc(sizeof(double) * (size_t)cap * D);
    double *lg = malloc(sizeof(double) * (size_t)cap), *p = malloc(sizeof(double) * (size_t)cap);
    int n = 0;
    for (int c = 0; c < 3; c++)
      for (int jb = 0; jb < q[Q_NBLK + c]; jb++) {
        int blk = BTAB(L, S, s, c)[jb];
        int mask = S->blk[c][blk * BLK_W];
        for (int tt = 0; tt < BS; tt++) {
          if (!((mask >> tt) & 1)) continue;
          int ps = S->slot[c][(blk * BS + tt) * SLOT_W];
          if (window > 0 && ps < t - window + 1) continue;
          for (int d = 0; d < D; d++) {
            K[(int64_t)n * D + d] = deq64(L, S, c, blk, tt, layer * Hkv + j, 0, d);
            V[(int64_t)n * D + d] = deq64(L, S, c, blk, tt, layer * Hkv + j, 1, d);
          }
          n++;
        }
      }
    if (k_self) {
      for (int d = 0; d < D; d++) {
        K[(int64_t)n * D + d] = k_self[((int64_t)b * Hkv + j) * D + d];
        V[(int64_t)n * D + d] = v_self[((int64_t)b * Hkv + j) * D + d];
      }
      n++;
    }
    if (j == 0 && n_attended) n_attended[b] = n;
    for (int hh = 0; hh < G; hh++) {
      int h = j * G + hh;
      double *o = out + ((int64_t)b * Hq + h) * D;
      double *st = stats ? stats + ((int64_t)b * Hq + h) * 3 : NULL;
      const uint16_t *qr = qbf + ((int64_t)b * Hq + h) * D;
      for (int d = 0; d < D; d++) o[d] = 0.0;
      if (st) st[0] = st[1] = st[2] = 0.0;
      if (n == 0) continue;
      double m = -INFINITY;
      for (int i = 0; i < n; i++) {
        double acc = 0.0;
        for (int d = 0; d < D; d++) acc += bf16_to_f64(qr[d]) * K[(int64_t)i * D + d];
        lg[i] = acc / sqrt((double)D);
        if (lg[i] > m) m = lg[i];
      }
      double mm = m;
      if (sinks && (double)sinks[h] > mm) mm = (double)sinks[h];
      double z = 0.0, zt = 0.0;
      for (int i = 0; i < n; i++) { p[i] = exp(lg[i] - mm); z += p[i]; }
      double den = z + (sinks ? exp((double)sinks[h] - mm) : 0.0);
      for (int i = 0; i < n; i++) {
        double w = p[i] / den;
        for (int d = 0; d < D; d++) o[d] += w * V[(int64_t)i * D + d];
      }
      if (!st) continue;
      /* stats over the tokens' own softmax */
      for (int i = 0; i < n; i++) { p[i] = exp(lg[i] - m); }
      zt = 0.0; for (int i = 0; i < n; i++) zt += p[i];
      double H = 0.0;
      for (int i = 0; i < n; i++) { double pi = p[i] / zt; if (pi > 0.0) H -= pi * log(pi); }
      st[0] = H;
      st[1] = n >= 2 ? H / log((double)n) : 0.0;
      int kk = topk < n ? topk : n;
      /* partial selection sort of the kk largest */
      double mass = 0.0;
      for (int a = 0; a < kk; a++) {
        int best = a;
        for (int i = a + 1; i < n; i++) if (p[i] > p[best]) best = i;
        double tmp = p[a]; p[a] = p[best]; p[best] = tmp;
        mass += p[a] / zt;
      }
      st[2] = mass;
    }
    free(K); free(V); free(lg); free(p);
  }
}

/* ---------------------------------------------------------------------- */
/* thought_classify (thought decomposition bullets: T most sparse, then R, */
/* E least).  Reading: sparsity = concentration of the decode query's      */
/* attention; score = fp32 mean over query heads (in head order) of the    */
/* normalized entropy (kind 0) or of 1 - top-k mass (kind 1).  T if score  */
/* <= tau_T, E if score >= tau_E, else R.  Labels: R=0, E=1, T=2.          */
/* ---------------------------------------------------------------------- */
void ora_classify(int batch, int Hq, const float *stats, float tau_T, float tau_E, int kind, uint8_t *labels) {
  for (int b = 0; b < batch; b++) {
    float sum = 0.0f;
    for (int h = 0; h < Hq; h++) {
      const float *st = stats + ((int64_t)b * Hq + h) * 3;
      float v = kind == 0 ? st[1] : 1.0f - st[2];
      sum = sum + v;
    }
    float score = sum / (float)Hq;
    labels[b] = score <= tau_T ? 2 : (score >= tau_E ? 1 : 0);
  }
}

/* Vector form of the conversion, for the exhaustive pin against an
   independent binary16 implementation. */
void ora_f32_to_f16_vec(const float *x, uint16_t *h, int64_t n) {
  for (int64_t i = 0; i < n; i++) h[i] = ora_f32_to_f16(x[i]);
}

/* Bit offset (from the start of a block-head record) of the code of tensor
   kv (0=K, 1=V), token t, dim d in class c; exported for the packing pins. */
int64_t ora_code_bit(const ora_layout *L, int c, int kv, int t, int d) {
  return kv ? v_code_bit(L, c, t, d) : k_code_bit(L, c, t, d);
}
