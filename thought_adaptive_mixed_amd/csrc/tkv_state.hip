// State kernels of libthinkv: allocation + quantize-and-pack append, segment
// eviction and downgrade, the budget ladder, sequence reset, classification.
//
// Method passages (ThinKV technical summary, "Methodologie"): TBQ bullet
// (tokens group-quantized by thought category), TBE bullet (segment-granular
// progressive eviction), Continuous Thinking bullet (evicted slots reused in
// place through a block table with type, start index and eviction mask);
// lay summary "Astuce B" (a small safety net of Transition thoughts is kept).
//
// Determinism: items are applied in list order.  Per-sequence work runs on
// one thread (allocation walks) or one work-group (eviction) per sequence;
// pops from the shared global block stacks are ordered by an exclusive scan
// over the list, so block ids do not depend on scheduling.
#include "tkv_internal.h"

#define WG 1024

// ---------------------------------------------------------------------------
// Work-group exclusive scan of three counters per thread (list order follows
// thread order).  Returns the totals in tot[3].
// ---------------------------------------------------------------------------
__device__ void wg_scan3(int v[3], int excl[3], int tot[3], int* s_tmp /* [3][WG/64] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  int incl[3];
  for (int c = 0; c < 3; c++) {
    int x = v[c];
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    incl[c] = x;
    if (lane == 63) s_tmp[c * 16 + wave] = x;
  }
  __syncthreads();
  for (int c = 0; c < 3; c++) {
    int base = 0, all = 0;
    for (int w = 0; w < nwave; w++) {
      int t = s_tmp[c * 16 + w];
      if (w < wave) base += t;
      all += t;
    }
    excl[c] = base + incl[c] - v[c];
    tot[c] = all;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// init
// ---------------------------------------------------------------------------
__global__ void k_init_blocks(DevState S, int c) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= S.pool_blocks[c]) return;
  int32_t* r = S.blk[c] + (int64_t)b * TKV_BLK_W;
  r[0] = 0; r[1] = -1; r[2] = -1; r[3] = 0;
  for (int t = 0; t < TKV_BS; t++) {
    S.slot[c][((int64_t)b * TKV_BS + t) * 2] = -1;
    S.slot[c][((int64_t)b * TKV_BS + t) * 2 + 1] = -1;
  }
}
__global__ void k_fill(int32_t* p, int64_t n, int32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}
__global__ void k_init_hdr(DevState S) {
  if (threadIdx.x == 0) {
    for (int i = 0; i < 16; i++) S.hdr[i] = 0;
    for (int c = 0; c < 3; c++) S.hdr[H_FREE + c] = S.pool_blocks[c];
    S.hdr[H_EMINSEQ] = TKV_INF;
  }
}

static int fill(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return TKV_OK;
  int blocks = (int)((n + 255) / 256); if (blocks > 4096) blocks = 4096;
  k_fill<<<blocks, 256, 0, st>>>(p, n, v);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

int launch_init(tkv_cache* c, hipStream_t st) {
  DevState& S = c->S;
  for (int k = 0; k < 3; k++) {
    if (hipMemsetAsync(S.pool[k], 0, c->size[TKV_BUF_POOL0 + k], st) != hipSuccess) return TKV_EHIP;
    k_init_blocks<<<(S.pool_blocks[k] + 255) / 256, 256, 0, st>>>(S, k);
  }
  k_init_hdr<<<1, 64, 0, st>>>(S);
  if (hipMemsetAsync(S.seq, 0, c->size[TKV_BUF_SEQ], st) != hipSuccess) return TKV_EHIP;
  if (hipMemsetAsync(S.segt, 0, c->size[TKV_BUF_SEGT], st) != hipSuccess) return TKV_EHIP;
  int r = fill(S.btab, (int64_t)(c->size[TKV_BUF_BTAB] / 4), -1, st);
  if (r) return r;
  r = fill(S.sstk, (int64_t)(c->size[TKV_BUF_SSTK] / 4), -1, st);
  if (r) return r;
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// Append, part 1: allocation.  One work-group; thread s walks the token list
// for sequence s.  A first walk simulates the sequence's stacks to flag the
// tokens that need a fresh block; an exclusive scan over the list gives each
// flagged token its index among the class's global pops.  The earliest token
// whose index exceeds what the pool holds marks the class dry from there on
// and the walk is redone (at most once per class).  A final walk commits.
// ---------------------------------------------------------------------------
// Per-class counters as scalars (selected by class) so that walks never index
// private arrays dynamically (which would place them in scratch memory).
struct C3 {
  int a, b, c;
  __device__ int get(int k) const { return k == 0 ? a : (k == 1 ? b : c); }
  __device__ void add(int k, int d) { a += k == 0 ? d : 0; b += k == 1 ? d : 0; c += k == 2 ? d : 0; }
};
struct SeqRec {
  C3 nblk, nslot;
  int nseg, len, nret, napp, open_type, open_bits;
};

__device__ inline SeqRec load_seq(const DevState& S, int s) {
  const int4* q4 = (const int4*)(S.seq + (int64_t)s * TKV_SEQ_W);
  const int4 a = q4[0], b = q4[1], c = q4[2];
  SeqRec r;
  r.nblk = C3{a.x, a.y, a.z};
  r.nslot = C3{a.w, b.x, b.y};
  r.nseg = b.z; r.len = b.w;
  r.nret = c.x; r.napp = c.y;
  r.open_type = -1; r.open_bits = -1;
  if (r.nseg > 0) {
    const int2 g = *(const int2*)(S.segt + ((int64_t)s * S.max_segs + r.nseg - 1) * TKV_SEG_W);
    r.open_type = g.x; r.open_bits = g.y;
  }
  return r;
}

// s_flags: bits 0-1 thought type (3 = invalid), bit 2 = token needs a fresh block
#define F_TYPE 3u
#define F_NEED 4u

__device__ void append_walk(const DevState& S, int s, SeqRec w, int n, const uint16_t* s_seq, uint8_t* s_flags,
                            const int* s_pos, const int* dry_from, const int* avail, const uint16_t* s_idx,
                            int32_t* info, int32_t* slot_out, bool commit) {
  int failed = 0, fail_code = 0;
  int32_t* bt = S.btab + (int64_t)s * 3 * S.max_blocks;
  int32_t* st = S.sstk + (int64_t)s * 3 * S.max_blocks * TKV_BS;
  // Each walker advances a cursor to its next token with cheap LDS compares;
  // the body below then runs for all walkers of the wave together (not once
  // per lane, as a plain scan of the list would make it).
  int i = -1;
  while (true) {
    i++;
    while (i < n && s_seq[i] != s) i++;
    if (__builtin_amdgcn_ballot_w64(i < n) == 0) break;
    if (i >= n) continue;
    const uint32_t fl = s_flags[i];
    if (!commit) s_flags[i] = (uint8_t)(fl & F_TYPE);
    if (failed) continue;
    const int y = (int)(fl & F_TYPE);
    const int p = s_pos[i];
    if (y > 2 || p < w.len) { failed = 1; fail_code = TKV_EINVAL; continue; }
    const int c = S.type_class[y];
    const int cb = class_bits(c);
    const int new_seg = (w.nseg == 0) || (w.open_type != y) || (w.open_bits != cb);
    if (new_seg && w.nseg == S.max_segs) { failed = 1; fail_code = TKV_ENOMEM; continue; }
    const int need = w.nslot.get(c) == 0;
    if (need && (w.nblk.get(c) == S.max_blocks || i >= dry_from[c])) { failed = 1; fail_code = TKV_ENOMEM; continue; }
    if (!commit) {
      if (need) { s_flags[i] = (uint8_t)((fl & F_TYPE) | F_NEED); w.nblk.add(c, 1); w.nslot.add(c, TKV_BS); }
      w.nslot.add(c, -1);
      if (new_seg) { w.nseg++; w.open_type = y; w.open_bits = cb; }
      w.len = p + 1;
      continue;
    }
    // commit
    const int ix = s_idx[i];
    if (need && ix >= avail[c]) {   // cannot happen after the dry passes; keeps indexing in bounds
      failed = 1; fail_code = TKV_ENOMEM; continue;
    }
    int32_t* btc = bt + c * S.max_blocks;
    int32_t* stc = st + (int64_t)c * S.max_blocks * TKV_BS;
    int slot;
    if (need) {
      // a fresh block: push its 16 slots (slot 0 on top) and pop slot 0
      const int blk = S.freestk[c][avail[c] - 1 - ix];
      const int nb = w.nblk.get(c), ns = w.nslot.get(c);
      btc[nb] = blk;
      S.blk[c][(int64_t)blk * TKV_BLK_W + 2] = s;
      for (int t = TKV_BS - 1; t >= 1; t--) stc[ns + TKV_BS - 1 - t] = blk * TKV_BS + t;
      w.nblk.add(c, 1);
      w.nslot.add(c, TKV_BS - 1);
      slot = blk * TKV_BS;
    } else {
      w.nslot.add(c, -1);
      slot = stc[w.nslot.get(c)];
    }
    if (new_seg) {
      int32_t* g = S.segt + ((int64_t)s * S.max_segs + w.nseg) * TKV_SEG_W;
      *(int4*)g = make_int4(y, cb, p, p);
      *(int4*)(g + 4) = make_int4(1, 1, 0, 0);
      w.nseg++; w.open_type = y; w.open_bits = cb;
    } else {
      int32_t* g = S.segt + ((int64_t)s * S.max_segs + w.nseg - 1) * TKV_SEG_W;
      g[G_LAST] = p; g[G_NTOT] += 1; g[G_NRET] += 1;
    }
    const int blk = slot / TKV_BS, t = slot % TKV_BS;
    int32_t* br = S.blk[c] + (int64_t)blk * TKV_BLK_W;
    atomicOr(&br[0], 1 << t);
    atomicMax(&br[1], p);
    *(int2*)(S.slot[c] + (int64_t)slot * 2) = make_int2(p, w.nseg - 1);
    w.len = p + 1; w.nret++; w.napp++;
    const int code = (c << 28) | slot;
    info[i] = code;
    if (slot_out) slot_out[i] = code;
  }
  if (commit) {
    int4* q4 = (int4*)(S.seq + (int64_t)s * TKV_SEQ_W);
    q4[0] = make_int4(w.nblk.a, w.nblk.b, w.nblk.c, w.nslot.a);
    q4[1] = make_int4(w.nslot.b, w.nslot.c, w.nseg, w.len);
    S.seq[(int64_t)s * TKV_SEQ_W + Q_NRET] = w.nret;
    S.seq[(int64_t)s * TKV_SEQ_W + Q_NAPP] = w.napp;
    if (failed) record_error(S.hdr, fail_code, s);
  }
}

__global__ __launch_bounds__(WG) void k_append_alloc(DevState S, int n, const int32_t* seq_ids, const int32_t* pos,
                                                     const uint8_t* thought, int32_t* slot_out) {
  __shared__ uint16_t s_seq[TKV_MAX_TOK];
  __shared__ uint8_t s_flags[TKV_MAX_TOK];
  __shared__ int s_pos[TKV_MAX_TOK];
  __shared__ uint16_t s_idx[TKV_MAX_TOK];
  __shared__ int s_tmp[48];
  __shared__ int dry_from[3], avail[3], viol[3], total[3];
  const int tid = threadIdx.x;
  int32_t* info = scr_info(S.scratch);
  const bool walker = tid < S.max_seqs;
  SeqRec rec;
  if (walker) rec = load_seq(S, tid);
  for (int i = tid; i < n; i += WG) {
    const int s = seq_ids[i];
    info[i] = -1;
    if (slot_out) slot_out[i] = -1;
    if (s < 0 || s >= S.max_seqs) {
      s_seq[i] = 0xFFFF;
      record_error(S.hdr, TKV_EINVAL, s < 0 ? TKV_INF : s);
    } else {
      s_seq[i] = (uint16_t)s;
    }
    const uint32_t y = thought[i];
    s_flags[i] = (uint8_t)(y > 2 ? 3u : y);
    s_pos[i] = pos[i];
  }
  if (tid < 3) { dry_from[tid] = TKV_INF; avail[tid] = S.hdr[H_FREE + tid]; }
  __syncthreads();
  const int per = (n + WG - 1) / WG;
  const int lo = tid * per, hi = min(n, lo + per);
  for (int iter = 0; iter < 4; iter++) {
    if (walker) append_walk(S, tid, rec, n, s_seq, s_flags, s_pos, dry_from, avail, s_idx, info, slot_out, false);
    __syncthreads();
    int v[3] = {0, 0, 0}, ex[3], tot[3];
    for (int i = lo; i < hi; i++)
      if (s_flags[i] & F_NEED) v[S.type_class[s_flags[i] & F_TYPE]]++;
    wg_scan3(v, ex, tot, s_tmp);
    if (tid < 3) viol[tid] = TKV_INF;
    __syncthreads();
    for (int i = lo; i < hi; i++) {
      if (!(s_flags[i] & F_NEED)) continue;
      const int c = S.type_class[s_flags[i] & F_TYPE];
      const int ix = ex[c]++;
      s_idx[i] = (uint16_t)ix;
      if (ix >= avail[c]) atomicMin(&viol[c], i);
    }
    if (tid < 3) total[tid] = tot[tid];
    __syncthreads();
    int first = TKV_INF, fc = -1;
    for (int c = 0; c < 3; c++) if (viol[c] < first) { first = viol[c]; fc = c; }
    __syncthreads();
    if (first == TKV_INF) break;
    if (tid == 0) dry_from[fc] = first;
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();
  if (walker) append_walk(S, tid, rec, n, s_seq, s_flags, s_pos, dry_from, avail, s_idx, info, slot_out, true);
  __syncthreads();
  if (tid < 3) S.hdr[H_FREE + tid] = avail[tid] - total[tid];
}

// ---------------------------------------------------------------------------
// Append, part 2: quantize and pack.  One wave per (token, KV head, tensor)
// row: lane l holds elements E*l .. E*l+E-1 (E = D/64); a group's min and max
// are butterfly reductions over its g/E lanes; every lane of the group then
// derives the same fp16 scale and zero-point and quantizes its own elements.
// The codes go through a per-wave LDS row so that each lane can assemble
// whole 32-bit words: a token's K codes fill whole words of its own chunks
// (plain stores); its V codes share words with 3 other tokens, so 4- and
// 2-bit V fields are merged with atomic AND/OR (8-bit ones are byte stores).
// ---------------------------------------------------------------------------
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int E>
__device__ void quant_row_wave(const DevState& S, int c, int blk, int t, int h, int kv, int lane, const float (&x)[E],
                               uint8_t* codes /* per-wave LDS, D bytes */) {
#pragma clang fp contract(off)
  const int D = S.D, g = S.g, bits = class_bits(c);
  const int lpg = g / E;                       // lanes per group
  const int gi = (lane * E) / g;
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < E; e++) { mn = x[e] < mn ? x[e] : mn; mx = x[e] > mx ? x[e] : mx; }
  for (int o = 1; o < lpg; o <<= 1) {
    const float a = __shfl_xor(mn, o, 64), b = __shfl_xor(mx, o, 64);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  // (the sign of a zero extremum cannot change the scale, the zero-point or any code)
  const float levels = (float)((1 << bits) - 1);
  const float range = mx - mn;
  const float s32 = range / levels;
  const uint16_t sh = f16_bits_rne(s32), zh = f16_bits_rne(mn);
  const float sf = f16_bits_to_f32(sh), zf = f16_bits_to_f32(zh);
#pragma unroll
  for (int e = 0; e < E; e++) codes[lane * E + e] = (uint8_t)quant_code(x[e], sf, zf, bits);
  uint8_t* base = S.pool[c] + ((int64_t)blk * S.Hkv + h) * S.bh_bytes[c];
  if ((lane * E) % g == 0) *(uint32_t*)(base + meta_byte(D, g, bits, kv, t, gi)) = (uint32_t)sh | ((uint32_t)zh << 16);
  wave_lds_sync();
  const int W = 32 / bits;
  const int CB = D * bits / 32;                // bytes per chunk
  const int wpc = CB / 4;                      // words per chunk
  if (kv == 0) {
    // word l: chunk 16*lg + t, word w; element e = w*W + f holds dim (e/(g/4))*g + lg*(g/4) + e%(g/4)
    const int q4 = g / 4;
    for (int l = lane; l < 4 * wpc; l += 64) {
      const int lg = l / wpc, w = l % wpc;
      uint32_t word = 0;
      for (int f = 0; f < W; f++) {
        const int e = w * W + f;
        const int d = (e / q4) * g + lg * q4 + (e % q4);
        word |= (uint32_t)codes[d] << (((f >> 1) + (f & 1) * (W >> 1)) * bits);
      }
      *(uint32_t*)(base + (16 * lg + t) * CB + w * 4) = word;
    }
  } else {
    // chunk 16*q + i, element 4n + r: token t = 4q + r, dim d = 16n + i
    const int q = t >> 2, r = t & 3;
    uint8_t* vbase = base + 64 * CB;
    for (int l = lane; l < 16 * wpc; l += 64) {
      const int i = l / wpc, w = l % wpc;
      uint8_t* ch = vbase + (16 * q + i) * CB;
      if (bits == 8) {
        // word w holds dim n = w for tokens r = 0..3: our byte is field r
        const int f = r, p = (f >> 1) + (f & 1) * 2;
        ch[w * 4 + p] = codes[16 * w + i];
      } else {
        uint32_t mask = 0, val = 0;
        for (int f = 0; f < W; f++) {
          const int e = w * W + f;
          if ((e & 3) != r) continue;
          const int p = (f >> 1) + (f & 1) * (W >> 1);
          mask |= ((1u << bits) - 1u) << (p * bits);
          val |= (uint32_t)codes[16 * (e >> 2) + i] << (p * bits);
        }
        uint32_t* wp = (uint32_t*)ch + w;
        atomicAnd(wp, ~mask);
        atomicOr(wp, val);
      }
    }
  }
  wave_lds_sync();     // the LDS row may be reused by this wave's next row
}

template <int E>
__global__ __launch_bounds__(256) void k_append_store(DevState S, int n, const float* k, const float* v) {
  __shared__ uint8_t s_codes[4][128];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= (int64_t)n * S.Hkv * 2) return;
  const int kv = (int)(row & 1);
  const int h = (int)((row >> 1) % S.Hkv);
  const int i = (int)((row >> 1) / S.Hkv);
  const int info = scr_info(S.scratch)[i];
  if (info < 0) return;
  const int c = info >> 28, slot = info & 0x0FFFFFFF;
  const float* src = (kv ? v : k) + ((int64_t)i * S.Hkv + h) * S.D + lane * E;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; e++) x[e] = src[e];
  quant_row_wave<E>(S, c, slot / TKV_BS, slot % TKV_BS, h, kv, lane, x, s_codes[wv]);
}

int launch_append(tkv_cache* c, int n, const int32_t* seq_ids, const int32_t* pos, const uint8_t* thought,
                  const float* k, const float* v, int32_t* slot_out, hipStream_t st) {
  if (n == 0) return TKV_OK;
  k_append_alloc<<<1, WG, 0, st>>>(c->S, n, seq_ids, pos, thought, slot_out);
  const int64_t rows = (int64_t)n * c->S.Hkv * 2;
  const int blocks = (int)((rows + 3) / 4);
  if (c->S.D == 128) k_append_store<2><<<blocks, 256, 0, st>>>(c->S, n, k, v);
  else k_append_store<1><<<blocks, 256, 0, st>>>(c->S, n, k, v);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// Evict, part 1: validation and reservation of fresh lower-class blocks for
// downgrades, in list order (same walk / scan / dry scheme as append).
// status[j]: 1 = apply, 0 = skipped or failed.  need[j] = fresh blocks,
// idx[j] = index of its first global pop.
// ---------------------------------------------------------------------------
__device__ void evict_walk(const DevState& S, int s, const SeqRec& rec, int n, const uint16_t* s_seq,
                           const int32_t* seg_ids, const int32_t* keep_n, const uint8_t* new_bits,
                           const int2* s_seg, uint8_t* s_cls, int32_t* need, int32_t* status, const int* dry_from,
                           bool final_pass) {
  C3 nslot = rec.nslot, nblk = rec.nblk;
  const int nseg = rec.nseg;
  int failed = 0, code = 0;
  int j = -1;
  while (true) {
    j++;
    while (j < n && s_seq[j] != s) j++;
    if (__builtin_amdgcn_ballot_w64(j < n) == 0) break;
    if (j >= n) continue;
    need[j] = 0; status[j] = 0; s_cls[j] = 0;
    if (failed) continue;
    const int k = seg_ids[j];
    if (k < 0 || k >= nseg) { failed = 1; code = TKV_ENOSEG; continue; }
    int dup = 0;
    for (int j2 = 0; j2 < j; j2++) if (s_seq[j2] == s && seg_ids[j2] == k) { dup = 1; break; }
    const int nb = new_bits[j], gb = s_seg[j].x;
    if (dup || keep_n[j] < 0 || !(nb == 0 || nb == 2 || nb == 4 || nb == 8) || (nb != 0 && nb > gb)) {
      failed = 1; code = TKV_EINVAL; continue;
    }
    const int r = s_seg[j].y;
    if (r == 0) { failed = 1; code = TKV_ENOSEG; continue; }
    const int c = class_of_bits(gb);
    const int keep = keep_n[j] < r ? keep_n[j] : r;
    const int down = (nb != 0 && nb < gb && keep > 0);
    const int c2 = down ? class_of_bits(nb) : c;
    int nd = 0;
    if (down) {
      const int have = nslot.get(c2);
      nd = keep > have ? (keep - have + TKV_BS - 1) / TKV_BS : 0;
      if (nblk.get(c2) + nd > S.max_blocks) { failed = 1; code = TKV_ENOMEM; continue; }
      if (nd > 0 && j >= dry_from[c2]) { failed = 1; code = TKV_ENOMEM; continue; }
    }
    const int ev = r - keep;
    nslot.add(c, ev);
    if (down) {
      nblk.add(c2, nd);
      nslot.add(c2, TKV_BS * nd - keep);
      nslot.add(c, keep);
    }
    need[j] = nd; status[j] = 1; s_cls[j] = (uint8_t)c2;
  }
  if (final_pass && failed) record_error(S.hdr, code, s);
}

#define EV_STAGE 2048     // ops whose fields are staged in LDS
__global__ __launch_bounds__(WG) void k_evict_plan(DevState S, int n_cap, const int32_t* n_dev, const int32_t* seq_ids,
                                                   const int32_t* g_seg, const int32_t* g_keep,
                                                   const uint8_t* g_bits) {
  __shared__ uint16_t s_seq[TKV_MAX_TOK];
  __shared__ uint8_t s_cls[TKV_MAX_TOK];
  __shared__ int32_t s_seg[EV_STAGE], s_keep[EV_STAGE];
  __shared__ uint8_t s_bits[EV_STAGE];
  __shared__ int2 s_segrec[TKV_MAX_TOK];   // (bits, retained) of each op's segment, read up front
  __shared__ int s_tmp[48];
  __shared__ int dry_from[3], avail[3], viol[3], total[3];
  const int tid = threadIdx.x;
  int n = n_cap;
  if (n_dev) { int m = *n_dev; n = m < n_cap ? (m < 0 ? 0 : m) : n_cap; }
  int32_t* idx = scr_idx(S.scratch);
  int32_t* status = scr_status(S.scratch);
  int32_t* need = scr_need(S.scratch);
  int32_t* misc = scr_misc(S.scratch);
  // op fields: staged in LDS when they fit, read in place otherwise
  const bool staged = n <= EV_STAGE;
  const int32_t* seg_ids = staged ? s_seg : g_seg;
  const int32_t* keep_n = staged ? s_keep : g_keep;
  const uint8_t* new_bits = staged ? s_bits : g_bits;
  const bool walker = tid < S.max_seqs;
  SeqRec rec;
  if (walker) rec = load_seq(S, tid);
  for (int j = tid; j < n; j += WG) {
    int s = seq_ids[j];
    const int k = g_seg[j];
    if (staged) { s_seg[j] = k; s_keep[j] = g_keep[j]; s_bits[j] = g_bits[j]; }
    status[j] = 0; need[j] = 0; idx[j] = 0;
    s_segrec[j] = make_int2(0, 0);
    if (s < 0 || s >= S.max_seqs) { s_seq[j] = 0xFFFF; record_error(S.hdr, TKV_EINVAL, s < 0 ? TKV_INF : s); }
    else {
      s_seq[j] = (uint16_t)s;
      if (k >= 0 && k < S.max_segs) {
        const int2 gr = *(const int2*)(S.segt + ((int64_t)s * S.max_segs + k) * TKV_SEG_W + G_BITS);
        const int nr = S.segt[((int64_t)s * S.max_segs + k) * TKV_SEG_W + G_NRET];
        s_segrec[j] = make_int2(gr.x, nr);
      }
    }
  }
  if (tid < 3) { dry_from[tid] = TKV_INF; avail[tid] = S.hdr[H_FREE + tid]; }
  if (tid == 0) misc[3] = n;
  __syncthreads();
  const int per = (n + WG - 1) / WG;
  const int lo = tid * per, hi = min(n, lo + per);
  for (int iter = 0; iter < 4; iter++) {
    if (walker)
      evict_walk(S, tid, rec, n, s_seq, seg_ids, keep_n, new_bits, s_segrec, s_cls, need, status, dry_from, false);
    __threadfence_block();
    __syncthreads();
    int v[3] = {0, 0, 0}, ex[3], tot[3];
    for (int j = lo; j < hi; j++) if (need[j] > 0) v[s_cls[j]] += need[j];
    wg_scan3(v, ex, tot, s_tmp);
    if (tid < 3) viol[tid] = TKV_INF;
    __syncthreads();
    for (int j = lo; j < hi; j++) {
      if (need[j] <= 0) continue;
      int c = s_cls[j];
      idx[j] = ex[c];
      ex[c] += need[j];
      if (idx[j] + need[j] > avail[c]) atomicMin(&viol[c], j);
    }
    if (tid < 3) total[tid] = tot[tid];
    __syncthreads();
    int first = TKV_INF, fc = -1;
    for (int c = 0; c < 3; c++) if (viol[c] < first) { first = viol[c]; fc = c; }
    __syncthreads();
    if (first == TKV_INF) break;
    if (tid == 0) dry_from[fc] = first;
    __syncthreads();
  }
  // final walk records the errors (state of the last iteration is the truth)
  if (tid < S.max_seqs)
    evict_walk(S, tid, rec, n, s_seq, seg_ids, keep_n, new_bits, s_segrec, s_cls, need, status, dry_from, true);
  __syncthreads();
  if (tid < 3) { misc[tid] = avail[tid]; S.hdr[H_FREE + tid] = avail[tid] - total[tid]; }
}

// Evict, part 2: one work-group per sequence applies its ops in list order.
#define EV_THREADS 256
#define EV_MAXSLOT (TKV_MAX_BLOCKS * TKV_BS)   // every slot of one class of one sequence

__device__ float deq_code(const DevState& S, int c, int blk, int t, int h, int kv, int d) {
#pragma clang fp contract(off)
  const int bits = class_bits(c);
  const uint8_t* base = S.pool[c] + ((int64_t)blk * S.Hkv + h) * S.bh_bytes[c];
  int bit = kv ? v_code_bit(S.D, bits, t, d) : k_code_bit(S.D, S.g, bits, t, d);
  uint32_t word = *(const uint32_t*)(base + ((bit >> 5) << 2));
  unsigned code = (word >> (bit & 31)) & ((1u << bits) - 1u);
  uint32_t m = *(const uint32_t*)(base + meta_byte(S.D, S.g, bits, kv, t, d / S.g));
  float sf = f16_bits_to_f32((uint16_t)(m & 0xFFFF)), zf = f16_bits_to_f32((uint16_t)(m >> 16));
  float prod = sf * (float)code;
  return prod + zf;
}

// Sort m (position, slot) pairs by position (unique) in LDS: bitonic network
// over the next power of two, padded with +inf positions.
__device__ void lds_sort_pairs(int32_t* pos, int32_t* slot, int m, int tid, int nthreads) {
  int n2 = 1;
  while (n2 < m) n2 <<= 1;
  for (int i = m + tid; i < n2; i += nthreads) { pos[i] = TKV_INF; slot[i] = -1; }
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += nthreads) {
        const int l = i ^ j;
        if (l > i) {
          const bool up = (i & k) == 0;
          const int pi = pos[i], pl = pos[l];
          if ((pi > pl) == up) {
            pos[i] = pl; pos[l] = pi;
            const int t = slot[i]; slot[i] = slot[l]; slot[l] = t;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Re-quantize one moved row (K or V of one KV head of one token) from the
// fp32 values its old codes decode to, into its new slot.  One wave.
__device__ void requant_row(const DevState& S, int src, int dst, int h, int kv, int lane, uint8_t* codes) {
  const int c = src >> 28, old = src & 0x0FFFFFFF, c2 = dst >> 28, ns = dst & 0x0FFFFFFF;
  const int ob = old / TKV_BS, ot = old % TKV_BS;
  if (S.D == 128) {
    float x[2];
    for (int e = 0; e < 2; e++) x[e] = deq_code(S, c, ob, ot, h, kv, lane * 2 + e);
    quant_row_wave<2>(S, c2, ns / TKV_BS, ns % TKV_BS, h, kv, lane, x, codes);
  } else {
    float x[1];
    x[0] = deq_code(S, c, ob, ot, h, kv, lane);
    quant_row_wave<1>(S, c2, ns / TKV_BS, ns % TKV_BS, h, kv, lane, x, codes);
  }
}

// Deferred downgrade moves of all sequences, one wave per row: a flat grid
// strides over sum(moves) * Hkv * 2 rows.
#define RQ_THREADS 256
__global__ __launch_bounds__(RQ_THREADS) void k_requant(DevState S) {
  __shared__ int s_off[TKV_MAX_SEQS + 1];
  __shared__ int s_tmp[48];
  __shared__ uint8_t s_codes[RQ_THREADS / 64][128];
  const int tid = threadIdx.x;
  const int32_t* mcnt = scr_mcnt(S.scratch);
  const int32_t* moves = scr_moves(S.scratch, S.max_seqs);
  const int per_seq = S.max_blocks * TKV_BS * 2;
  // exclusive prefix of the per-sequence move counts (rows = moves * Hkv * 2)
  const int per = (S.max_seqs + RQ_THREADS - 1) / RQ_THREADS;
  const int lo = tid * per, hi = min(S.max_seqs, lo + per);
  int v[3] = {0, 0, 0}, ex[3], tot[3];
  for (int i = lo; i < hi; i++) v[0] += mcnt[i];
  wg_scan3(v, ex, tot, s_tmp);
  int run = ex[0];
  for (int i = lo; i < hi; i++) { s_off[i] = run; run += mcnt[i]; }
  if (tid == 0) s_off[S.max_seqs] = tot[0];
  __syncthreads();
  const int total_rows = tot[0] * S.Hkv * 2;
  const int wv = tid >> 6, lane = tid & 63;
  const int nwaves = gridDim.x * (RQ_THREADS / 64);
  for (int row = blockIdx.x * (RQ_THREADS / 64) + wv; row < total_rows; row += nwaves) {
    const int kv = row & 1, h = (row >> 1) % S.Hkv, mv = (row >> 1) / S.Hkv;
    // sequence owning move mv: last s with s_off[s] <= mv
    int a = 0, b = S.max_seqs;
    while (b - a > 1) { const int mid = (a + b) >> 1; if (s_off[mid] <= mv) a = mid; else b = mid; }
    const int j = mv - s_off[a];
    const int32_t* m2 = moves + (int64_t)a * per_seq + 2 * j;
    requant_row(S, m2[0], m2[1], h, kv, lane, s_codes[wv]);
  }
}

__global__ __launch_bounds__(EV_THREADS) void k_evict_apply(DevState S, const int32_t* seq_ids, const int32_t* seg_ids,
                                                            const int32_t* keep_n, const uint8_t* new_bits) {
  __shared__ int32_t s_pos[EV_MAXSLOT];
  __shared__ int32_t s_slot[EV_MAXSLOT];
  __shared__ uint8_t s_codes[EV_THREADS / 64][128];
  __shared__ int s_cnt;
  const int s = blockIdx.x, tid = threadIdx.x;
  const int32_t* status = scr_status(S.scratch);
  const int32_t* idx = scr_idx(S.scratch);
  const int32_t* need = scr_need(S.scratch);
  const int32_t* misc = scr_misc(S.scratch);
  const int n = misc[3];
  int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
  int32_t* bt = S.btab + (int64_t)s * 3 * S.max_blocks;
  int32_t* st = S.sstk + (int64_t)s * 3 * S.max_blocks * TKV_BS;
  int32_t* moves = scr_moves(S.scratch, S.max_seqs) + (int64_t)s * S.max_blocks * TKV_BS * 2;
  // With one downgrade for this sequence in the call, its re-quantization is
  // deferred to a wide kernel (the old slots cannot be overwritten within the
  // call); with several, a later one could reuse slots an earlier one still
  // reads from, so they are re-quantized here, in op order.
  int ndown = 0;
  for (int j = 0; j < n; j++)
    if (seq_ids[j] == s && status[j] == 1 && need[j] >= 0) {
      const int32_t* g = S.segt + ((int64_t)s * S.max_segs + seg_ids[j]) * TKV_SEG_W;
      const int gb = g[G_BITS], nb = new_bits[j];
      if (nb != 0 && nb < gb && keep_n[j] > 0) ndown++;
    }
  const bool defer = ndown <= 1;
  int nmoves = 0;
  for (int j = 0; j < n; j++) {
    if (seq_ids[j] != s || status[j] != 1) continue;
    const int k = seg_ids[j];
    int32_t* g = S.segt + ((int64_t)s * S.max_segs + k) * TKV_SEG_W;
    const int gb = g[G_BITS], c = class_of_bits(gb), r = g[G_NRET];
    int keep = keep_n[j] < r ? keep_n[j] : r;
    const int nb = new_bits[j];
    const int down = (nb != 0 && nb < gb && keep > 0);
    const int c2 = down ? class_of_bits(nb) : c;
    // gather the segment's valid slots
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    const int nbk = q[Q_NBLK + c];
    for (int x = tid; x < nbk * TKV_BS; x += EV_THREADS) {
      int blk = bt[c * S.max_blocks + x / TKV_BS], t = x % TKV_BS;
      int mask = S.blk[c][(int64_t)blk * TKV_BLK_W];
      if (((mask >> t) & 1) && S.slot[c][((int64_t)blk * TKV_BS + t) * 2 + 1] == k) {
        int at = atomicAdd(&s_cnt, 1);
        if (at >= EV_MAXSLOT) continue;
        s_pos[at] = S.slot[c][((int64_t)blk * TKV_BS + t) * 2];
        s_slot[at] = blk * TKV_BS + t;
      }
    }
    __syncthreads();
    const int m = s_cnt < EV_MAXSLOT ? s_cnt : EV_MAXSLOT;
    lds_sort_pairs(s_pos, s_slot, m, tid, EV_THREADS);
    const int32_t* s_sorted = s_slot;
    if (keep > m) keep = m;                 // m == r on a consistent state
    const int ev = m - keep;
    const int ns_c = q[Q_NSLOT + c];
    for (int a = tid; a < ev; a += EV_THREADS) {
      int sl = s_sorted[a];
      atomicAnd(&S.blk[c][(int64_t)(sl / TKV_BS) * TKV_BLK_W], ~(1 << (sl % TKV_BS)));
      st[(int64_t)c * S.max_blocks * TKV_BS + ns_c + a] = sl;
    }
    if (down) {
      const int S0 = q[Q_NSLOT + c2];
      const int nbk2 = q[Q_NBLK + c2];
      const int nd = need[j], base = idx[j], av = misc[c2];
      int32_t* st2 = st + (int64_t)c2 * S.max_blocks * TKV_BS;
      for (int b = tid; b < nd; b += EV_THREADS) {
        int blk = S.freestk[c2][av - 1 - (base + b)];
        bt[c2 * S.max_blocks + nbk2 + b] = blk;
        S.blk[c2][(int64_t)blk * TKV_BLK_W + 2] = s;
      }
      __threadfence_block();
      __syncthreads();
      // re-quantize each kept token (K and V rows of every head) into its new slot
      if (defer) {
        for (int p = tid; p < keep; p += EV_THREADS) {
          int ns;
          if (p < S0) ns = st2[S0 - 1 - p];
          else { int pp = p - S0; ns = bt[c2 * S.max_blocks + nbk2 + pp / TKV_BS] * TKV_BS + pp % TKV_BS; }
          moves[2 * (nmoves + p)] = (c << 28) | s_sorted[ev + p];
          moves[2 * (nmoves + p) + 1] = (c2 << 28) | ns;
        }
        nmoves += keep;
      } else {
        const int wv = tid >> 6, lane = tid & 63;
        for (int row = wv; row < keep * S.Hkv * 2; row += EV_THREADS / 64) {
          const int kv = row & 1, h = (row >> 1) % S.Hkv, p = (row >> 1) / S.Hkv;
          int ns;
          if (p < S0) ns = st2[S0 - 1 - p];
          else { int pp = p - S0; ns = bt[c2 * S.max_blocks + nbk2 + pp / TKV_BS] * TKV_BS + pp % TKV_BS; }
          requant_row(S, (c << 28) | s_sorted[ev + p], (c2 << 28) | ns, h, kv, lane, s_codes[wv]);
        }
      }
      __threadfence_block();
      __syncthreads();
      for (int p = tid; p < keep; p += EV_THREADS) {
        int old = s_sorted[ev + p];
        int ns;
        if (p < S0) ns = st2[S0 - 1 - p];
        else { int pp = p - S0; ns = bt[c2 * S.max_blocks + nbk2 + pp / TKV_BS] * TKV_BS + pp % TKV_BS; }
        int pos = S.slot[c][(int64_t)old * 2];
        atomicOr(&S.blk[c2][(int64_t)(ns / TKV_BS) * TKV_BLK_W], 1 << (ns % TKV_BS));
        atomicMax(&S.blk[c2][(int64_t)(ns / TKV_BS) * TKV_BLK_W + 1], pos);
        S.slot[c2][(int64_t)ns * 2] = pos;
        S.slot[c2][(int64_t)ns * 2 + 1] = k;
        atomicAnd(&S.blk[c][(int64_t)(old / TKV_BS) * TKV_BLK_W], ~(1 << (old % TKV_BS)));
        st[(int64_t)c * S.max_blocks * TKV_BS + ns_c + ev + p] = old;
      }
      __threadfence_block();
      __syncthreads();
      if (tid == 0) {
        int depth;
        if (keep <= S0) depth = S0 - keep;
        else {
          int used_last = (keep - S0) - TKV_BS * (nd - 1);
          int last = bt[c2 * S.max_blocks + nbk2 + nd - 1];
          depth = TKV_BS - used_last;
          for (int i2 = 0; i2 < depth; i2++) st2[i2] = last * TKV_BS + (TKV_BS - 1 - i2);
        }
        q[Q_NSLOT + c2] = depth;
        q[Q_NBLK + c2] = nbk2 + nd;
        q[Q_NSLOT + c] = ns_c + ev + keep;
        g[G_BITS] = nb;
      }
    } else if (tid == 0) {
      q[Q_NSLOT + c] = ns_c + ev;
    }
    if (tid == 0) {
      g[G_NRET] = keep;
      q[Q_NRET] -= ev;
    }
    __threadfence_block();
    __syncthreads();
  }
  if (tid == 0) scr_mcnt(S.scratch)[s] = nmoves;
}

int launch_evict(tkv_cache* c, int n_ops, const int32_t* n_ops_dev, const int32_t* seq_ids, const int32_t* seg_ids,
                 const int32_t* keep_n, const uint8_t* new_bits, hipStream_t st) {
  if (n_ops == 0) return TKV_OK;
  k_evict_plan<<<1, WG, 0, st>>>(c->S, n_ops, n_ops_dev, seq_ids, seg_ids, keep_n, new_bits);
  k_evict_apply<<<c->S.max_seqs, EV_THREADS, 0, st>>>(c->S, seq_ids, seg_ids, keep_n, new_bits);
  k_requant<<<512, RQ_THREADS, 0, st>>>(c->S);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// Budget ladder: one thread per listed sequence counts and then writes its
// ops at its exclusive-scan offset (list order).
// ---------------------------------------------------------------------------
__device__ int ladder(const DevState& S, int s, int num, int den, int base, int max_ops, int32_t* os, int32_t* og,
                      int32_t* ok, uint8_t* ob, bool write) {
  if (s < 0 || s >= S.max_seqs) return 0;
  const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
  const int nseg = q[Q_NSEG];
  long long B = (long long)q[Q_LEN] * num / den;
  long long nr = q[Q_NRET];
  if (nr <= B) return 0;
  const int32_t* segs = S.segt + (int64_t)s * S.max_segs * TKV_SEG_W;
  int newest_t = -1;
  for (int k = 0; k < nseg; k++)
    if (segs[k * TKV_SEG_W + G_TYPE] == TKV_T && segs[k * TKV_SEG_W + G_NRET] > 0) newest_t = k;
  int m = 0;
  for (int k = 0; k < nseg - 1 && nr > B; k++) {
    const int32_t* g = segs + k * TKV_SEG_W;
    if (g[G_TYPE] != TKV_T || g[G_NRET] == 0 || k == newest_t) continue;
    if (write && base + m < max_ops) { os[base + m] = s; og[base + m] = k; ok[base + m] = 0; ob[base + m] = 0; }
    m++;
    nr -= g[G_NRET];
  }
  if (nr > B) {
    for (int k = 0; k < nseg - 1; k++) {
      const int32_t* g = segs + k * TKV_SEG_W;
      if (g[G_TYPE] == TKV_E && g[G_BITS] > 2 && g[G_NRET] > 0) {
        if (write && base + m < max_ops) { os[base + m] = s; og[base + m] = k; ok[base + m] = g[G_NRET]; ob[base + m] = 2; }
        m++;
        break;
      }
    }
  }
  return m;
}

__global__ __launch_bounds__(WG) void k_plan(DevState S, int n, const int32_t* seq_ids, int num, int den, int max_ops,
                                             int32_t* n_ops, int32_t* os, int32_t* og, int32_t* ok, uint8_t* ob) {
  __shared__ int s_tmp[48];
  const int tid = threadIdx.x;
  const int per = (n + WG - 1) / WG;
  const int lo = tid * per, hi = min(n, lo + per);
  int v[3] = {0, 0, 0}, ex[3], tot[3];
  for (int i = lo; i < hi; i++) v[0] += ladder(S, seq_ids[i], num, den, 0, 0, os, og, ok, ob, false);
  wg_scan3(v, ex, tot, s_tmp);
  int base = ex[0];
  for (int i = lo; i < hi; i++) base += ladder(S, seq_ids[i], num, den, base, max_ops, os, og, ok, ob, true);
  if (tid == 0) *n_ops = tot[0] < max_ops ? tot[0] : max_ops;
}

int launch_plan(tkv_cache* c, int n, const int32_t* seq_ids, int num, int den, int max_ops, int32_t* n_ops_dev,
                int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits, hipStream_t st) {
  k_plan<<<1, WG, 0, st>>>(c->S, n, seq_ids, num, den, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// Sequence reset: blocks back to the global stacks in list order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(WG) void k_seq_reset(DevState S, int n, const int32_t* seq_ids) {
  __shared__ int s_tmp[48];
  __shared__ int base_cnt[3];
  const int tid = threadIdx.x;
  const int per = (n + WG - 1) / WG;
  const int lo = tid * per, hi = min(n, lo + per);
  if (tid < 3) base_cnt[tid] = S.hdr[H_FREE + tid];
  int v[3] = {0, 0, 0}, ex[3], tot[3];
  for (int i = lo; i < hi; i++) {
    int s = seq_ids[i];
    if (s < 0 || s >= S.max_seqs) continue;
    int dup = 0;
    for (int j = 0; j < i; j++) if (seq_ids[j] == s) { dup = 1; break; }
    if (dup) continue;
    for (int c = 0; c < 3; c++) v[c] += S.seq[(int64_t)s * TKV_SEQ_W + Q_NBLK + c];
  }
  __syncthreads();
  wg_scan3(v, ex, tot, s_tmp);
  for (int i = lo; i < hi; i++) {
    int s = seq_ids[i];
    if (s < 0 || s >= S.max_seqs) { record_error(S.hdr, TKV_EINVAL, s < 0 ? TKV_INF : s); continue; }
    int dup = 0;
    for (int j = 0; j < i; j++) if (seq_ids[j] == s) { dup = 1; break; }
    if (dup) continue;
    int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
    for (int c = 0; c < 3; c++) {
      for (int j = 0; j < q[Q_NBLK + c]; j++) {
        int blk = S.btab[((int64_t)s * 3 + c) * S.max_blocks + j];
        int32_t* br = S.blk[c] + (int64_t)blk * TKV_BLK_W;
        br[0] = 0; br[1] = -1; br[2] = -1;
        S.freestk[c][base_cnt[c] + ex[c]++] = blk;
      }
    }
    for (int w = 0; w < TKV_SEQ_W; w++) q[w] = 0;
  }
  __syncthreads();
  if (tid < 3) S.hdr[H_FREE + tid] = base_cnt[tid] + tot[tid];
}

int launch_seq_reset(tkv_cache* c, int n, const int32_t* seq_ids, hipStream_t st) {
  if (n == 0) return TKV_OK;
  k_seq_reset<<<1, WG, 0, st>>>(c->S, n, seq_ids);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// thought_classify: fp32 mean over heads in head order, then thresholds.
// ---------------------------------------------------------------------------
__global__ void k_classify(int batch, int Hq, const float* stats, float tT, float tE, int kind, uint8_t* labels) {
#pragma clang fp contract(off)
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  float sum = 0.0f;
  for (int h = 0; h < Hq; h++) {
    const float* st = stats + ((int64_t)b * Hq + h) * 3;
    float v = kind == 0 ? st[1] : 1.0f - st[2];
    sum = sum + v;
  }
  float score = sum / (float)Hq;
  labels[b] = score <= tT ? (uint8_t)TKV_T : (score >= tE ? (uint8_t)TKV_E : (uint8_t)TKV_R);
}

int launch_classify(int batch, int Hq, const float* stats, float tau_T, float tau_E, int kind, uint8_t* labels,
                    hipStream_t st) {
  if (batch == 0) return TKV_OK;
  k_classify<<<(batch + 255) / 256, 256, 0, st>>>(batch, Hq, stats, tau_T, tau_E, kind, labels);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}
