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
// Scans.  A wave's inclusive prefix sum in six DPP steps: shifts by 1, 2, 4
// and 8 lanes inside each row of 16, then row 15 / lane 31 broadcasts.
// ---------------------------------------------------------------------------
__device__ inline int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}
__device__ inline int wave_total(int incl) { return __builtin_amdgcn_readlane(incl, 63); }

// Work-group exclusive scan of three counters per thread (list order follows
// thread order; any multiple of 64 threads up to 1024).  Returns the totals.
__device__ void wg_scan3(int v[3], int excl[3], int tot[3], int* s_tmp /* [3][16] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  int incl[3];
#pragma unroll
  for (int c = 0; c < 3; c++) {
    incl[c] = wave_incl_scan(v[c]);
    if (lane == 63) s_tmp[c * 16 + wave] = incl[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 3; c++) {
    int base = 0, all = 0;
    for (int w = 0; w < nwave; w++) {
      const int t = s_tmp[c * 16 + w];
      if (w < wave) base += t;
      all += t;
    }
    excl[c] = base + incl[c] - v[c];
    tot[c] = all;
  }
  __syncthreads();
}

// Threads of the single-work-group state kernels: one walker per sequence.
static inline int walker_threads(int max_seqs) {
  const int t = (max_seqs + 63) / 64 * 64;
  return t < 64 ? 64 : (t > WG ? WG : t);
}

// ---------------------------------------------------------------------------
// init
// ---------------------------------------------------------------------------
__global__ void k_init_blocks(DevState S, int c) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= pick3(S.pool_blocks, c)) return;
  int32_t* r = pick3(S.blk, c) + (int64_t)b * TKV_BLK_W;
  r[0] = 0; r[1] = -1; r[2] = -1; r[3] = 0;
  for (int t = 0; t < TKV_BS; t++) {
    pick3(S.slot, c)[((int64_t)b * TKV_BS + t) * 2] = -1;
    pick3(S.slot, c)[((int64_t)b * TKV_BS + t) * 2 + 1] = -1;
  }
}
__global__ void k_fill(int32_t* p, int64_t n, int32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}
__global__ void k_init_hdr(DevState S) {
  if (threadIdx.x == 0) {
    for (int i = 0; i < 16; i++) S.hdr[i] = 0;
    for (int c = 0; c < 3; c++) S.hdr[H_FREE + c] = pick3(S.pool_blocks, c);
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
// Stable grouping of list items by sequence, in LDS: afterwards
// s_list[s_off[s] .. s_off[s] + s_cnt[s]) holds, in list order, the items whose
// key is s (keys >= max_seqs are left out); returns how many items were
// grouped.  s_cnt must be zero on entry.
// Whole work-group; max_seqs <= blockDim.x.
// ---------------------------------------------------------------------------
__device__ int group_by_seq(int n, int max_seqs, const uint16_t* s_key, int* s_cnt, int* s_off, uint16_t* s_list,
                            int* s_tmp) {
  const int tid = threadIdx.x, NT = blockDim.x;
  for (int i = tid; i < n; i += NT) {
    const int k = s_key[i];
    if (k < max_seqs) atomicAdd(&s_cnt[k], 1);
  }
  __syncthreads();
  int v[3] = {tid < max_seqs ? s_cnt[tid] : 0, 0, 0}, ex[3], tot[3];
  wg_scan3(v, ex, tot, s_tmp);
  if (tid < max_seqs) s_off[tid] = ex[0];
  __syncthreads();
  const uint32_t* kw = (const uint32_t*)s_key;
  for (int i = tid; i < n; i += NT) {
    const uint32_t k = s_key[i];
    if ((int)k >= max_seqs) continue;
    int rank = 0;
    if (s_cnt[k] > 1) {                      // rank among the earlier items of the same sequence
      int j = 0;
      for (; j + 1 < i; j += 2) {
        const uint32_t w = kw[j >> 1];
        rank += ((w & 0xFFFFu) == k) + ((w >> 16) == k);
      }
      if (j < i) rank += s_key[j] == k;
    }
    s_list[s_off[k] + rank] = (uint16_t)i;
  }
  __syncthreads();
  return tot[0];
}

// ---------------------------------------------------------------------------
// Append, part 1: allocation.  One work-group.  Items are grouped by sequence
// in LDS; thread s then walks sequence s's items in list order.  A first walk
// simulates the sequence's stacks to flag the tokens that need a fresh block;
// an exclusive scan over the list gives each flagged token its index among
// the class's global pops.  The earliest token whose index exceeds what the
// pool holds marks the class dry from there on and the walk is redone (at
// most once per class).  A final walk commits.  The sequence record, its open
// segment and the top of each slot stack are read before the grouping, so
// their latency overlaps it; a segment's record is written once per call.
// ---------------------------------------------------------------------------
// Per-class counters as scalars (selected by class) so that walks never index
// private arrays dynamically (which would place them in scratch memory).
struct C3 {
  int a, b, c;
  __device__ int get(int k) const { return k == 0 ? a : (k == 1 ? b : c); }
  __device__ void add(int k, int d) { a += k == 0 ? d : 0; b += k == 1 ? d : 0; c += k == 2 ? d : 0; }
  __device__ void set(int k, int v) { a = k == 0 ? v : a; b = k == 1 ? v : b; c = k == 2 ? v : c; }
};
struct SeqRec {
  C3 nblk, nslot;
  int nseg, len, nret, napp;
  int open_type, open_bits, open_first, open_last, open_ntot, open_nret;   // segment nseg-1
};

__device__ inline SeqRec load_seq_rec(const DevState& S, int s) {
  const int4* q4 = (const int4*)(S.seq + (int64_t)s * TKV_SEQ_W);
  const int4 a = q4[0], b = q4[1], c = q4[2];
  SeqRec r;
  r.nblk = C3{a.x, a.y, a.z};
  r.nslot = C3{a.w, b.x, b.y};
  r.nseg = b.z; r.len = b.w;
  r.nret = c.x; r.napp = c.y;
  r.open_type = -1; r.open_bits = -1; r.open_first = 0; r.open_last = 0; r.open_ntot = 0; r.open_nret = 0;
  return r;
}
__device__ inline void load_open_seg(const DevState& S, int s, SeqRec& r) {
  if (r.nseg > 0) {
    const int32_t* g = S.segt + ((int64_t)s * S.max_segs + r.nseg - 1) * TKV_SEG_W;
    const int4 a = *(const int4*)g;
    const int2 b = *(const int2*)(g + 4);
    r.open_type = a.x; r.open_bits = a.y; r.open_first = a.z; r.open_last = a.w;
    r.open_ntot = b.x; r.open_nret = b.y;
  }
}

// s_flags: bits 0-1 thought type (3 = invalid), bit 2 = token needs a fresh block
#define F_TYPE 3u
#define F_NEED 4u

__device__ void append_walk(const DevState& S, int s, SeqRec w, const C3& top, int cnt, const uint16_t* lst,
                            uint8_t* s_flags, const int* s_pos, const int* dry_from, const int* avail,
                            const uint16_t* s_idx, int32_t* info, int32_t* slot_out, bool commit) {
  int failed = 0, fail_code = 0;
  int32_t* bt = S.btab + (int64_t)s * 3 * S.max_blocks;
  const int32_t* st = S.sstk + (int64_t)s * 3 * S.max_blocks * TKV_BS;
  int popped = 0;              // bit c: class c's stack top (read up front) has been taken
  C3 fresh{-1, -1, -1};        // block whose slots refilled class c's empty stack in this call
  // the segment being extended: its index, whether this call opened it, and its fields
  int cur = -1, cur_new = 0, cur_type = 0, cur_bits = 0, cur_first = 0, cur_last = 0, cur_ntot = 0, cur_nret = 0;
  for (int r = 0; r < cnt; r++) {
    const int i = lst[r];
    const uint32_t fl = s_flags[i];
    if (!commit) s_flags[i] = (uint8_t)(fl & F_TYPE);
    if (failed) continue;
    const int y = (int)(fl & F_TYPE);
    const int p = s_pos[i];
    if (y > 2 || p < w.len) { failed = 1; fail_code = TKV_EINVAL; continue; }
    const int c = pick3(S.type_class, y);
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
    int32_t* stc = S.sstk + (int64_t)s * 3 * S.max_blocks * TKV_BS + (int64_t)c * S.max_blocks * TKV_BS;
    int slot;
    if (need) {
      // a fresh block: push its 16 slots (slot 0 on top) and pop slot 0
      const int blk = pick3(S.freestk, c)[avail[c] - 1 - ix];
      const int nb = w.nblk.get(c), ns = w.nslot.get(c);
      btc[nb] = blk;
      pick3(S.blk, c)[(int64_t)blk * TKV_BLK_W + 2] = s;
      for (int t = TKV_BS - 1; t >= 1; t--) stc[ns + TKV_BS - 1 - t] = blk * TKV_BS + t;
      w.nblk.add(c, 1);
      w.nslot.add(c, TKV_BS - 1);
      fresh.set(c, blk);
      slot = blk * TKV_BS;
    } else {
      w.nslot.add(c, -1);
      const int at = w.nslot.get(c);
      const int fb = fresh.get(c);
      if (fb >= 0) slot = fb * TKV_BS + (TKV_BS - 1 - at);       // stack positions 0..14 hold slots 15..1
      else if (!((popped >> c) & 1)) slot = top.get(c);
      else slot = st[(int64_t)c * S.max_blocks * TKV_BS + at];
      popped |= 1 << c;
    }
    if (new_seg) {
      if (cur >= 0) {   // close the previous segment of this call
        int32_t* g = S.segt + ((int64_t)s * S.max_segs + cur) * TKV_SEG_W;
        *(int4*)g = make_int4(cur_type, cur_bits, cur_first, cur_last);
        *(int2*)(g + 4) = make_int2(cur_ntot, cur_nret);
      }
      cur = w.nseg; cur_new = 1; cur_type = y; cur_bits = cb; cur_first = p; cur_ntot = 0; cur_nret = 0;
      w.nseg++; w.open_type = y; w.open_bits = cb;
    } else if (cur < 0) {   // extending the segment that was open before the call
      cur = w.nseg - 1; cur_new = 0; cur_type = w.open_type; cur_bits = w.open_bits; cur_first = w.open_first;
      cur_ntot = w.open_ntot; cur_nret = w.open_nret;
    }
    cur_last = p; cur_ntot++; cur_nret++;
    const int blk = slot / TKV_BS, t = slot % TKV_BS;
    int32_t* br = pick3(S.blk, c) + (int64_t)blk * TKV_BLK_W;
    atomicOr(&br[0], 1 << t);
    atomicMax(&br[1], p);
    *(int2*)(pick3(S.slot, c) + (int64_t)slot * 2) = make_int2(p, w.nseg - 1);
    w.len = p + 1; w.nret++; w.napp++;
    const int code = (c << 28) | slot;
    info[i] = code;
    if (slot_out) slot_out[i] = code;
  }
  if (commit) {
    if (cur >= 0) {
      int32_t* g = S.segt + ((int64_t)s * S.max_segs + cur) * TKV_SEG_W;
      if (cur_new) *(int4*)g = make_int4(cur_type, cur_bits, cur_first, cur_last);
      else g[G_LAST] = cur_last;
      *(int2*)(g + 4) = make_int2(cur_ntot, cur_nret);
    }
    int4* q4 = (int4*)(S.seq + (int64_t)s * TKV_SEQ_W);
    q4[0] = make_int4(w.nblk.a, w.nblk.b, w.nblk.c, w.nslot.a);
    q4[1] = make_int4(w.nslot.b, w.nslot.c, w.nseg, w.len);
    *(int2*)(S.seq + (int64_t)s * TKV_SEQ_W + Q_NRET) = make_int2(w.nret, w.napp);
    if (failed) record_error(S.hdr, fail_code, s);
  }
}

#define CL_STAGE 8448    // floats of statistics staged per chunk of rows (256 rows of 32 heads + padding)
__global__ __launch_bounds__(WG) void k_append_alloc(DevState S, int n, const int32_t* seq_ids, const int32_t* pos,
                                                     const uint8_t* thought, int32_t* slot_out, ClassifyIn cl) {
  __shared__ __align__(16) uint16_t s_seq[TKV_MAX_TOK];
  __shared__ uint16_t s_list[TKV_MAX_TOK];
  __shared__ uint16_t s_idx[TKV_MAX_TOK];
  __shared__ uint8_t s_flags[TKV_MAX_TOK];
  __shared__ int s_pos[TKV_MAX_TOK];
  __shared__ int s_cnt[TKV_MAX_SEQS], s_off[TKV_MAX_SEQS];
  __shared__ int s_tmp[48];
  __shared__ int dry_from[3], avail[3], viol[3], total[3];
  __shared__ float s_stat[CL_STAGE];
  const int tid = threadIdx.x, NT = blockDim.x;
  int32_t* info = scr_info(S.scratch);
  const bool walker = tid < S.max_seqs;
  SeqRec rec;
  if (walker) rec = load_seq_rec(S, tid);
  if (walker) s_cnt[tid] = 0;
  if (tid < 3) { dry_from[tid] = TKV_INF; avail[tid] = S.hdr[H_FREE + tid]; }
  // the tokens' thought types: given, or classified here from their entries'
  // statistics.  The classification's column of the rows (H/ln n or M_k of
  // every head) is staged in LDS a chunk of rows at a time, read coalesced by
  // the whole work-group (a row's heads are adjacent in memory; one thread
  // per row would touch a cache line per head); then thread i adds row i's
  // values in head order.  Rows are padded by one float so the row-per-thread
  // reads hit distinct banks.
  if (cl.stats) {
#pragma clang fp contract(off)
    const int H = cl.heads, RW = H + 1, off = cl.kind == 0 ? 1 : 2;
    const int per = CL_STAGE / RW;
    for (int r0 = 0; r0 < n; r0 += per) {
      const int nr = min(per, n - r0), ne = nr * H;
      const float* base = cl.stats + (int64_t)r0 * H * 3 + off;
#pragma unroll 8
      for (int e = tid; e < ne; e += NT) {
        const int r = e / H, h = e - r * H;
        s_stat[r * RW + h] = base[(int64_t)e * 3];
      }
      __syncthreads();
      for (int i = r0 + tid; i < r0 + nr; i += NT) {
        const float* row = s_stat + (i - r0) * RW;
        float sum = 0.0f;
#pragma unroll 8
        for (int h = 0; h < H; h++) sum = sum + (cl.kind == 0 ? row[h] : 1.0f - row[h]);
        const uint32_t y = thought_label(sum / (float)H, cl.tT, cl.tE);
        s_flags[i] = (uint8_t)y;
        if (cl.labels) cl.labels[i] = (uint8_t)y;
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < n; i += NT) {
    const int s = seq_ids[i];
    const uint32_t y = cl.stats ? s_flags[i] : thought[i];
    const int p = pos[i];
    info[i] = -1;
    if (slot_out) slot_out[i] = -1;
    if (s < 0 || s >= S.max_seqs) {
      s_seq[i] = 0xFFFF;
      record_error(S.hdr, TKV_EINVAL, s < 0 ? TKV_INF : s);
    } else {
      s_seq[i] = (uint16_t)s;
    }
    s_flags[i] = (uint8_t)(y > 2 ? 3u : y);
    s_pos[i] = p;
  }
  __syncthreads();
  // second round of reads (their latency overlaps the grouping below)
  C3 top{-1, -1, -1};
  if (walker) {
    load_open_seg(S, tid, rec);
    const int32_t* st = S.sstk + (int64_t)tid * 3 * S.max_blocks * TKV_BS;
    const int64_t cs = (int64_t)S.max_blocks * TKV_BS;
    if (rec.nslot.a > 0) top.a = st[rec.nslot.a - 1];
    if (rec.nslot.b > 0) top.b = st[cs + rec.nslot.b - 1];
    if (rec.nslot.c > 0) top.c = st[2 * cs + rec.nslot.c - 1];
  }
  group_by_seq(n, S.max_seqs, s_seq, s_cnt, s_off, s_list, s_tmp);
  const int my_cnt = walker ? s_cnt[tid] : 0;
  const uint16_t* my_list = s_list + (walker ? s_off[tid] : 0);
  const int per = (n + NT - 1) / NT;
  const int lo = tid * per, hi = min(n, lo + per);
  for (int iter = 0; iter < 4; iter++) {
    if (walker)
      append_walk(S, tid, rec, top, my_cnt, my_list, s_flags, s_pos, dry_from, avail, s_idx, info, slot_out, false);
    __syncthreads();
    int v[3] = {0, 0, 0}, ex[3], tot[3];
    for (int i = lo; i < hi; i++)
      if (s_flags[i] & F_NEED) v[pick3(S.type_class, s_flags[i] & F_TYPE)]++;
    wg_scan3(v, ex, tot, s_tmp);
    if (tid < 3) viol[tid] = TKV_INF;
    __syncthreads();
    for (int i = lo; i < hi; i++) {
      if (!(s_flags[i] & F_NEED)) continue;
      const int c = pick3(S.type_class, s_flags[i] & F_TYPE);
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
  if (walker)
    append_walk(S, tid, rec, top, my_cnt, my_list, s_flags, s_pos, dry_from, avail, s_idx, info, slot_out, true);
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

template <int K>
__device__ inline void minmax_level(float& mn, float& mx) {
  if constexpr (K <= 8) {
    const float a = xchg<K>(mn), b = xchg<K>(mx);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  } else {
    float m0, m1, x0, x1;
    swap_pair<K>(mn, m0, m1);
    swap_pair<K>(mx, x0, x1);
    mn = m1 < m0 ? m1 : m0;
    mx = x1 > x0 ? x1 : x0;
  }
}

// The body takes the geometry (D, g, bits) as arguments: called with
// constants, the index arithmetic of the code layout folds to shifts and masks.
template <int E>
__device__ __forceinline__ void quant_row_body(const DevState& S, const int D, const int g, const int bits, int c, int blk,
                                               int t, int h, int kv, int lane, const float (&x)[E],
                                               uint8_t* codes /* per-wave LDS, D bytes */) {
#pragma clang fp contract(off)
  const int lpg = g / E;                       // lanes per group
  const int gi = (lane * E) / g;
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < E; e++) { mn = x[e] < mn ? x[e] : mn; mx = x[e] > mx ? x[e] : mx; }
  // butterfly over the group's lpg lanes (exact; a zero extremum may keep
  // either sign, which no result depends on)
  if (lpg > 1) minmax_level<1>(mn, mx);
  if (lpg > 2) minmax_level<2>(mn, mx);
  if (lpg > 4) minmax_level<4>(mn, mx);
  if (lpg > 8) minmax_level<8>(mn, mx);
  if (lpg > 16) minmax_level<16>(mn, mx);
  if (lpg > 32) minmax_level<32>(mn, mx);
  // (the sign of a zero extremum cannot change the scale, the zero-point or any code)
  uint16_t sh, zh = 0;
  if (S.fmt == 0) {
    const float levels = (float)((1 << bits) - 1);
    const float range = mx - mn;
    const float s32 = range / levels;
    sh = f16_bits_rne(s32);
    zh = f16_bits_rne(mn);
    const float sf = f16_bits_to_f32(sh), zf = f16_bits_to_f32(zh);
#pragma unroll
    for (int e = 0; e < E; e++) codes[lane * E + e] = (uint8_t)quant_code(x[e], sf, zf, bits);
  } else if (c < 2) {
    // FP8 / FP4: scale fp16(amax / largest finite value); codes of x / scale
    const float amax = mx > -mn ? mx : -mn;
    sh = f16_bits_rne(amax / (c == 0 ? 448.0f : 6.0f));
    const float sf = f16_bits_to_f32(sh);
#pragma unroll
    for (int e = 0; e < E; e++)
      codes[lane * E + e] = (uint8_t)(sh == 0 ? 0u : (c == 0 ? e4m3_encode(x[e] / sf) : e2m1_encode(x[e] / sf)));
  } else {
    // ternary, stored as the integer code t + 1 with zero-point -scale: sums
    // pairwise over index halves, i.e. the lane's own elements first, then
    // butterfly levels 1, 2, 4, ... over the group's lanes
    float sa = __builtin_fabsf(x[0]);
#pragma unroll
    for (int e = 1; e < E; e++) sa = sa + __builtin_fabsf(x[e]);
    if (lpg > 1) sa = pair_sum<1>(sa);
    if (lpg > 2) sa = pair_sum<2>(sa);
    if (lpg > 4) sa = pair_sum<4>(sa);
    if (lpg > 8) sa = pair_sum<8>(sa);
    if (lpg > 16) sa = pair_sum<16>(sa);
    if (lpg > 32) sa = pair_sum<32>(sa);
    const float thr = 0.7f * (sa / (float)g);
    float sk = 0.0f, nk = 0.0f;
    unsigned t[E];
#pragma unroll
    for (int e = 0; e < E; e++) {
      t[e] = x[e] > thr ? 2u : (x[e] < -thr ? 0u : 1u);
      const float k = t[e] != 1u ? __builtin_fabsf(x[e]) : 0.0f;
      sk = e ? sk + k : k;
      nk += t[e] != 1u ? 1.0f : 0.0f;
    }
    if (lpg > 1) { sk = pair_sum<1>(sk); nk = pair_sum<1>(nk); }
    if (lpg > 2) { sk = pair_sum<2>(sk); nk = pair_sum<2>(nk); }
    if (lpg > 4) { sk = pair_sum<4>(sk); nk = pair_sum<4>(nk); }
    if (lpg > 8) { sk = pair_sum<8>(sk); nk = pair_sum<8>(nk); }
    if (lpg > 16) { sk = pair_sum<16>(sk); nk = pair_sum<16>(nk); }
    if (lpg > 32) { sk = pair_sum<32>(sk); nk = pair_sum<32>(nk); }
    sh = nk > 0.0f ? f16_bits_rne(sk / nk) : (uint16_t)0;
    zh = sh ? (uint16_t)(sh ^ 0x8000u) : (uint16_t)0;
#pragma unroll
    for (int e = 0; e < E; e++) codes[lane * E + e] = (uint8_t)(sh == 0 ? 0u : t[e]);
  }
  uint8_t* base = pick3(S.pool, c) + ((int64_t)blk * S.Hst + h) * pick3(S.bh_bytes, c);
  if ((lane * E) % g == 0) *(uint32_t*)(base + meta_byte(D, g, bits, kv, t, gi)) = (uint32_t)sh | ((uint32_t)zh << 16);
  wave_lds_sync();
  const int W = 32 / bits;
  const int CB = D * bits / 32;                // bytes per chunk
  const int wpc = CB / 4;                      // words per chunk
  const int nat = natural_order(S.fmt, c);
  if (kv == 0) {
    // word l: chunk 16*lg + t, word w; element e = w*W + f holds dim (e/(g/4))*g + lg*(g/4) + e%(g/4)
    const int q4 = g / 4;
    for (int l = lane; l < 4 * wpc; l += 64) {
      const int lg = l / wpc, w = l % wpc;
      uint32_t word = 0;
      for (int f = 0; f < W; f++) {
        const int e = w * W + f;
        const int d = (e / q4) * g + lg * q4 + (e % q4);
        word |= (uint32_t)codes[d] << (field_pos(f, W, nat) * bits);
      }
      *(uint32_t*)(base + chunk_byte(CB, 16 * lg + t, w * 4)) = word;
    }
  } else {
    // chunk 16*q + i, element 4n + r: token t = 4q + r, dim d = 16n + i
    const int q = t >> 2, r = t & 3;
    uint8_t* vbase = base + 64 * CB;
    for (int l = lane; l < 16 * wpc; l += 64) {
      const int i = l / wpc, w = l % wpc;
      uint8_t* wb = vbase + chunk_byte(CB, 16 * q + i, w * 4);     // word w of chunk 16q + i
      if (bits == 8) {
        // word w holds dim n = w for tokens r = 0..3: our byte is field r
        const int p = field_pos(r, 4, nat);
        wb[p] = codes[16 * w + i];
      } else {
        uint32_t mask = 0, val = 0;
        for (int f = 0; f < W; f++) {
          const int e = w * W + f;
          if ((e & 3) != r) continue;
          const int p = field_pos(f, W, nat);
          mask |= ((1u << bits) - 1u) << (p * bits);
          val |= (uint32_t)codes[16 * (e >> 2) + i] << (p * bits);
        }
        uint32_t* wp = (uint32_t*)wb;
        atomicAnd(wp, ~mask);
        atomicOr(wp, val);
      }
    }
  }
  wave_lds_sync();     // the LDS row may be reused by this wave's next row
}

// geometry read from the state
template <int E>
__device__ __forceinline__ void quant_row_wave(const DevState& S, int c, int blk, int t, int h, int kv, int lane,
                                               const float (&x)[E], uint8_t* codes) {
  quant_row_body<E>(S, S.D, S.g, class_bits(c), c, blk, t, h, kv, lane, x, codes);
}
// geometry fixed at compile time (D = 64 E, group G), class c chosen at run time
template <int E, int G>
__device__ __forceinline__ void quant_row_fixed(const DevState& S, int c, int blk, int t, int h, int kv, int lane,
                                                const float (&x)[E], uint8_t* codes) {
  if (c == 0) quant_row_body<E>(S, 64 * E, G, 8, c, blk, t, h, kv, lane, x, codes);
  else if (c == 1) quant_row_body<E>(S, 64 * E, G, 4, c, blk, t, h, kv, lane, x, codes);
  else quant_row_body<E>(S, 64 * E, G, 2, c, blk, t, h, kv, lane, x, codes);
}

template <int E, int G>
__global__ __launch_bounds__(256) void k_append_store(DevState S, int n, const float* k, const float* v) {
  __shared__ uint8_t s_codes[4][128];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= (int64_t)n * S.Hst * 2) return;
  const int kv = (int)(row & 1);
  const int h = (int)((row >> 1) % S.Hst);
  const int i = (int)((row >> 1) / S.Hst);
  // the row's values do not depend on the slot: read them first
  const float* src = (kv ? v : k) + ((int64_t)i * S.Hst + h) * S.D + lane * E;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; e++) x[e] = src[e];
  const int info = scr_info(S.scratch)[i];
  if (info < 0) return;
  const int c = info >> 28, slot = info & 0x0FFFFFFF;
  quant_row_fixed<E, G>(S, c, slot / TKV_BS, slot % TKV_BS, h, kv, lane, x, s_codes[wv]);
}

int launch_append(tkv_cache* c, int n, const int32_t* seq_ids, const int32_t* pos, const uint8_t* thought,
                  const float* k, const float* v, int32_t* slot_out, hipStream_t st, const ClassifyIn* cl) {
  if (n == 0) return TKV_OK;
  if (cl && cl->stats && cl->heads + 1 > CL_STAGE) return TKV_EINVAL;   // a row must fit the LDS stage
  const ClassifyIn none = {nullptr, 0, 0, 0.f, 0.f, nullptr};
  TKV_TIMED(c, st, "k_append_alloc",
            k_append_alloc<<<1, walker_threads(c->S.max_seqs), 0, st>>>(c->S, n, seq_ids, pos, thought, slot_out,
                                                                        cl ? *cl : none));
  const int64_t rows = (int64_t)n * c->S.Hst * 2;
  const int blocks = (int)((rows + 3) / 4);
  TKV_TIMED(c, st, "k_append_store", {
    if (c->S.D == 128) {
      if (c->S.g == 64) k_append_store<2, 64><<<blocks, 256, 0, st>>>(c->S, n, k, v);
      else k_append_store<2, 32><<<blocks, 256, 0, st>>>(c->S, n, k, v);
    } else {
      if (c->S.g == 64) k_append_store<1, 64><<<blocks, 256, 0, st>>>(c->S, n, k, v);
      else k_append_store<1, 32><<<blocks, 256, 0, st>>>(c->S, n, k, v);
    }
  });
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// Evict, part 1: validation and reservation of fresh lower-class blocks for
// downgrades, in list order (same grouping / walk / scan / dry scheme as
// append).  Results in scratch: status[j] (1 = apply), need[j] (fresh blocks),
// idx[j] (index of its first global pop); the ops of each sequence in list
// order (list, offset, count) and its number of downgrades.
// ---------------------------------------------------------------------------
#define ST_APPLY 4u       // s_st: bits 0-1 target class, bit 2 = apply
#define ST_DUP 8u         // s_st bit 3: an earlier op of the sequence names the same segment

__device__ void evict_walk(const DevState& S, int s, const SeqRec& rec, int cnt, const uint16_t* lst,
                           const int32_t* seg_ids, const int32_t* keep_n, const uint8_t* new_bits,
                           const uint16_t* s_segrec, uint8_t* s_st, int32_t* s_ni, const int* dry_from,
                           int* ndown_out, bool final_pass) {
  C3 nslot = rec.nslot, nblk = rec.nblk;
  const int nseg = rec.nseg;
  int failed = 0, code = 0, ndown = 0;
  for (int r = 0; r < cnt; r++) {
    const int j = lst[r];
    // the final pass repeats the last simulated walk: it only records errors
    // and leaves the per-op results (and the pop indices packed with them) alone
    if (!final_pass) { s_ni[j] = 0; s_st[j] &= ST_DUP; }
    if (failed) continue;
    const int k = seg_ids[j];
    if (k < 0 || k >= nseg) { failed = 1; code = TKV_ENOSEG; continue; }
    const int dup = (s_st[j] & ST_DUP) != 0;
    const int nb = new_bits[j];
    const int sr = s_segrec[j];
    const int c = sr >> 14, gb = class_bits(c);
    if (dup || keep_n[j] < 0 || !(nb == 0 || nb == 2 || nb == 4 || nb == 8) || (nb != 0 && nb > gb)) {
      failed = 1; code = TKV_EINVAL; continue;
    }
    const int rr = sr & 0x3FFF;
    if (rr == 0) { failed = 1; code = TKV_ENOSEG; continue; }
    const int keep = keep_n[j] < rr ? keep_n[j] : rr;
    const int down = (nb != 0 && nb < gb && keep > 0);
    const int c2 = down ? class_of_bits(nb) : c;
    int nd = 0;
    if (down) {
      const int have = nslot.get(c2);
      nd = keep > have ? (keep - have + TKV_BS - 1) / TKV_BS : 0;
      if (nblk.get(c2) + nd > S.max_blocks) { failed = 1; code = TKV_ENOMEM; continue; }
      if (nd > 0 && j >= dry_from[c2]) { failed = 1; code = TKV_ENOMEM; continue; }
    }
    const int ev = rr - keep;
    nslot.add(c, ev);
    if (down) {
      nblk.add(c2, nd);
      nslot.add(c2, TKV_BS * nd - keep);
      nslot.add(c, keep);
    }
    if (!final_pass) { s_ni[j] = nd; s_st[j] = (uint8_t)((s_st[j] & ST_DUP) | c2 | ST_APPLY); }
    ndown += down;
  }
  if (final_pass) {
    if (failed) record_error(S.hdr, code, s);
    *ndown_out = ndown;
  }
}

#define EV_STAGE 1024     // ops whose fields are staged in LDS
__device__ __forceinline__ void evict_plan_body(const DevState& S, int n_cap, const int32_t* n_dev,
                                                const int32_t* seq_ids, const int32_t* g_seg,
                                                const int32_t* g_keep, const uint8_t* g_bits) {
  __shared__ __align__(16) uint16_t s_seq[TKV_MAX_TOK];
  __shared__ uint16_t s_list[TKV_MAX_TOK];
  __shared__ int32_t s_ni[TKV_MAX_TOK];       // fresh blocks an op needs | index of its first pop << 9
  __shared__ uint16_t s_segrec[TKV_MAX_TOK];   // retained tokens | class << 14 of each op's segment
  __shared__ uint8_t s_st[TKV_MAX_TOK];
  __shared__ int s_cnt[TKV_MAX_SEQS], s_off[TKV_MAX_SEQS];
  __shared__ int32_t s_seg[EV_STAGE], s_keep[EV_STAGE];
  __shared__ uint8_t s_bits[EV_STAGE];
  __shared__ int s_tmp[48];
  __shared__ int dry_from[3], avail[3], viol[3], total[3];
  const int tid = threadIdx.x, NT = blockDim.x;
  int n = n_cap;
  if (n_dev) { int m = *n_dev; n = m < n_cap ? (m < 0 ? 0 : m) : n_cap; }
  int32_t* misc = scr_misc(S.scratch);
  // op fields: staged in LDS when they fit, read in place otherwise
  const bool staged = n <= EV_STAGE;
  const int32_t* seg_ids = staged ? s_seg : g_seg;
  const int32_t* keep_n = staged ? s_keep : g_keep;
  const uint8_t* new_bits = staged ? s_bits : g_bits;
  const bool walker = tid < S.max_seqs;
  if (n == 0) {                 // nothing listed: every sequence's op count is zero
    if (walker) scr_grp(S.scratch)[S.max_seqs + tid] = 0;
    if (tid == 0) misc[3] = 0;
    return;
  }
  SeqRec rec;
  if (walker) { rec = load_seq_rec(S, tid); s_cnt[tid] = 0; }
  for (int j = tid; j < n; j += NT) {
    const int s = seq_ids[j];
    const int k = g_seg[j];
    if (staged) { s_seg[j] = k; s_keep[j] = g_keep[j]; s_bits[j] = g_bits[j]; }
    s_segrec[j] = 0; s_ni[j] = 0; s_st[j] = 0;
    if (s < 0 || s >= S.max_seqs) { s_seq[j] = 0xFFFF; record_error(S.hdr, TKV_EINVAL, s < 0 ? TKV_INF : s); }
    else {
      s_seq[j] = (uint16_t)s;
      if (k >= 0 && k < S.max_segs) {
        const int32_t* g = S.segt + ((int64_t)s * S.max_segs + k) * TKV_SEG_W;
        const int gb = g[G_BITS], nr = g[G_NRET];
        s_segrec[j] = (uint16_t)((nr & 0x3FFF) | ((class_of_bits(gb) & 3) << 14));
      }
    }
  }
  if (tid < 3) { dry_from[tid] = TKV_INF; avail[tid] = S.hdr[H_FREE + tid]; }
  if (tid == 0) misc[3] = n;
  __syncthreads();
  const int n_valid = group_by_seq(n, S.max_seqs, s_seq, s_cnt, s_off, s_list, s_tmp);
  // repeated segments, flagged once for the walks below (an op per thread,
  // against the earlier ops of its sequence)
  for (int p = tid; p < n_valid; p += NT) {
    const int j = s_list[p], k = seg_ids[j];
    for (int p2 = s_off[s_seq[j]]; p2 < p; p2++)
      if (seg_ids[s_list[p2]] == k) { s_st[j] = ST_DUP; break; }
  }
  __syncthreads();
  const int my_cnt = walker ? s_cnt[tid] : 0;
  const uint16_t* my_list = s_list + (walker ? s_off[tid] : 0);
  int ndown = 0;
  const int per = (n + NT - 1) / NT;
  const int lo = tid * per, hi = min(n, lo + per);
  for (int iter = 0; iter < 4; iter++) {
    if (walker)
      evict_walk(S, tid, rec, my_cnt, my_list, seg_ids, keep_n, new_bits, s_segrec, s_st, s_ni, dry_from, &ndown,
                 false);
    __syncthreads();
    int v[3] = {0, 0, 0}, ex[3], tot[3];
    for (int j = lo; j < hi; j++) v[s_st[j] & 3] += s_ni[j] & 511;
    wg_scan3(v, ex, tot, s_tmp);
    if (tid < 3) viol[tid] = TKV_INF;
    __syncthreads();
    for (int j = lo; j < hi; j++) {
      const int nd = s_ni[j] & 511;
      if (nd == 0) continue;
      const int c = s_st[j] & 3;
      s_ni[j] = nd | (ex[c] << 9);
      if (ex[c] + nd > avail[c]) atomicMin(&viol[c], j);
      ex[c] += nd;
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
  if (walker)
    evict_walk(S, tid, rec, my_cnt, my_list, seg_ids, keep_n, new_bits, s_segrec, s_st, s_ni, dry_from, &ndown,
               true);
  __syncthreads();
  // one record per listed op, grouped by sequence in list order: what the
  // apply kernel needs, so that it reads nothing else about the op
  int32_t* recs = scr_oprec(S.scratch);
  for (int r = tid; r < n_valid; r += NT) {
    const int j = s_list[r];
    const int st = s_st[j], sr = s_segrec[j];
    const int c = sr >> 14, rr = sr & 0x3FFF, k = seg_ids[j], nb = new_bits[j];
    const int kn = keep_n[j], keep = kn < rr ? kn : rr;
    int first = 0, span = 0;
    if (st & ST_APPLY) {
      const int2 fl = *(const int2*)(S.segt + ((int64_t)s_seq[j] * S.max_segs + k) * TKV_SEG_W + G_FIRST);
      first = fl.x; span = fl.y - fl.x + 1;
    }
    int4* o = (int4*)(recs + 8 * r);
    o[0] = make_int4((st & ST_APPLY ? 1 : 0) | (c << 4) | ((st & 3) << 8), k, keep, nb);
    o[1] = make_int4(s_ni[j] & 511, s_ni[j] >> 9, first, span);
  }
  if (walker) {
    int32_t* grp = scr_grp(S.scratch);
    grp[tid] = s_off[tid];
    grp[S.max_seqs + tid] = my_cnt;
    grp[2 * S.max_seqs + tid] = ndown;
  }
  if (tid < 3) { misc[tid] = avail[tid]; S.hdr[H_FREE + tid] = avail[tid] - total[tid]; }
}
__global__ __launch_bounds__(WG) void k_evict_plan(DevState S, int n_cap, const int32_t* n_dev, const int32_t* seq_ids,
                                                   const int32_t* g_seg, const int32_t* g_keep,
                                                   const uint8_t* g_bits) {
  evict_plan_body(S, n_cap, n_dev, seq_ids, g_seg, g_keep, g_bits);
}

// Evict, part 2: one work-group per sequence applies its own ops in list order.
#define EV_THREADS 256
#define EV_MAXSLOT (TKV_MAX_BLOCKS * TKV_BS)   // every slot of one class of one sequence
#define EV_BMW 1024                            // position bitmap words: segments spanning <= 32768 positions

__device__ __forceinline__ float deq_code_body(const DevState& S, const int D, const int g, const int bits, int c, int blk,
                                              int t, int h, int kv, int d) {
#pragma clang fp contract(off)
  const uint8_t* base = pick3(S.pool, c) + ((int64_t)blk * S.Hst + h) * pick3(S.bh_bytes, c);
  const int nat = natural_order(S.fmt, c);
  int bit = kv ? v_code_bit(D, bits, nat, t, d) : k_code_bit(D, g, bits, nat, t, d);
  uint32_t word = *(const uint32_t*)(base + ((bit >> 5) << 2));
  unsigned code = (word >> (bit & 31)) & ((1u << bits) - 1u);
  uint32_t m = *(const uint32_t*)(base + meta_byte(D, g, bits, kv, t, d / g));
  float sf = f16_bits_to_f32((uint16_t)(m & 0xFFFF)), zf = f16_bits_to_f32((uint16_t)(m >> 16));
  float prod = sf * (nat ? fmt_value(c, code) : (float)code);     // exact product
  return prod + zf;
}

__device__ __forceinline__ float deq_code(const DevState& S, int c, int blk, int t, int h, int kv, int d) {
  return deq_code_body(S, S.D, S.g, class_bits(c), c, blk, t, h, kv, d);
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
// the same with the geometry fixed at compile time (D = 64 E, group G)
template <int E, int G>
__device__ __forceinline__ void requant_row_fixed(const DevState& S, int src, int dst, int h, int kv, int lane,
                                                  uint8_t* codes) {
  const int c = src >> 28, old = src & 0x0FFFFFFF, c2 = dst >> 28, ns = dst & 0x0FFFFFFF;
  const int ob = old / TKV_BS, ot = old % TKV_BS;
  const int bits = c == 0 ? 8 : (c == 1 ? 4 : 2);
  float x[E];
#pragma unroll
  for (int e = 0; e < E; e++) {
    const int d = lane * E + e;
    x[e] = bits == 8 ? deq_code_body(S, 64 * E, G, 8, c, ob, ot, h, kv, d)
         : (bits == 4 ? deq_code_body(S, 64 * E, G, 4, c, ob, ot, h, kv, d) : deq_code_body(S, 64 * E, G, 2, c, ob, ot, h, kv, d));
  }
  quant_row_fixed<E, G>(S, c2, ns / TKV_BS, ns % TKV_BS, h, kv, lane, x, codes);
}

// Deferred downgrade moves of all sequences, one wave per row: a flat grid
// strides over sum(moves) * Hkv * 2 rows.  A row is a short chain of
// dependent global reads (codes and scale of its old slot), a wave reduction
// and stores: the grid fills the machine at the kernel's occupancy (seven
// waves per SIMD on 256 compute units at D = 128) so that the chains overlap.
#define RQ_THREADS 256
#define RQ_GRID 1792
template <int E, int G>
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
  const int total_rows = tot[0] * S.Hst * 2;
  const int wv = tid >> 6, lane = tid & 63;
  const int nwaves = gridDim.x * (RQ_THREADS / 64);
  for (int row = blockIdx.x * (RQ_THREADS / 64) + wv; row < total_rows; row += nwaves) {
    const int kv = row & 1, h = (row >> 1) % S.Hst, mv = (row >> 1) / S.Hst;
    // sequence owning move mv: last s with s_off[s] <= mv
    int a = 0, b = S.max_seqs;
    while (b - a > 1) { const int mid = (a + b) >> 1; if (s_off[mid] <= mv) a = mid; else b = mid; }
    const int j = mv - s_off[a];
    const int32_t* m2 = moves + (int64_t)a * per_seq + 2 * j;
    requant_row_fixed<E, G>(S, m2[0], m2[1], h, kv, lane, s_codes[wv]);
  }
}
static void launch_requant(const tkv_cache* c, hipStream_t st) {
  TKV_TIMED(c, st, "k_requant", {
    if (c->S.D == 128) {
      if (c->S.g == 64) k_requant<2, 64><<<RQ_GRID, RQ_THREADS, 0, st>>>(c->S);
      else k_requant<2, 32><<<RQ_GRID, RQ_THREADS, 0, st>>>(c->S);
    } else {
      if (c->S.g == 64) k_requant<1, 64><<<RQ_GRID, RQ_THREADS, 0, st>>>(c->S);
      else k_requant<1, 32><<<RQ_GRID, RQ_THREADS, 0, st>>>(c->S);
    }
  });
}

// Evict, part 2, the ops of one sequence without downgrades, each class in
// one scan.  Ops of one class touch only that class's slots and stack, and a
// sequence's segments hold disjoint position ranges, so: map each op's
// segment to the op, gather the valid slots of those segments with one scan of
// the class's blocks into a bitmap over the union of the ops' position ranges,
// rank every slot by position (bitmap prefix counts), and evict the oldest
// m - keep of each op; an op's evicted slots go on the stack after those of
// the earlier ops of its class (list order), in ascending position order.
// The result is the one of applying the ops one after another.
#define EVB_MAXOPS 256          // ops of one sequence handled by the class-wise path
__device__ void evict_classwise(const DevState& S, int s, int cnt, const int32_t* recs, int32_t* q, const int32_t* bt,
                                int32_t* st, int32_t* s_pos, int32_t* s_slot, int32_t* s_segop, uint32_t* s_bm,
                                int32_t* s_bpre, int* s_tmp, int* s_cnt) {
  __shared__ int s_m[EVB_MAXOPS], s_ev[EVB_MAXOPS], s_base[EVB_MAXOPS], s_rk0[EVB_MAXOPS];
  __shared__ int s_evtot;
  const int tid = threadIdx.x;
  if (tid == 0) s_evtot = 0;
  for (int c = 0; c < 3; c++) {
    // the class's ops: union of their position ranges (the same in every thread)
    int lo = TKV_INF, hi = -1, nop = 0;
    for (int r = 0; r < cnt; r++) {
      const int4 o0 = *(const int4*)(recs + 8 * r), o1 = *(const int4*)(recs + 8 * r + 4);
      if (!(o0.x & 1) || ((o0.x >> 4) & 3) != c) continue;
      lo = min(lo, o1.z);
      hi = max(hi, o1.z + o1.w - 1);
      nop++;
    }
    if (nop == 0) continue;
    const int span = hi - lo + 1, nbw = (span + 31) >> 5;
    for (int k = tid; k < S.max_segs; k += EV_THREADS) s_segop[k] = -1;
    for (int w = tid; w < nbw; w += EV_THREADS) s_bm[w] = 0;
    for (int r = tid; r < cnt; r += EV_THREADS) s_m[r] = 0;
    if (tid == 0) *s_cnt = 0;
    __syncthreads();
    for (int r = tid; r < cnt; r += EV_THREADS) {
      const int4 o0 = *(const int4*)(recs + 8 * r);
      if ((o0.x & 1) && ((o0.x >> 4) & 3) == c) s_segop[o0.y] = r;
    }
    __syncthreads();
    // gather: (position offset | op << 15, slot) of every valid slot of a target segment
    const int nbk = q[Q_NBLK + c];
    for (int x = tid; x < nbk * TKV_BS; x += EV_THREADS) {
      const int blk = bt[c * S.max_blocks + x / TKV_BS], t = x % TKV_BS;
      const int mask = pick3(S.blk, c)[(int64_t)blk * TKV_BLK_W];
      const int2 sr = *(const int2*)(pick3(S.slot, c) + ((int64_t)blk * TKV_BS + t) * 2);
      if (!((mask >> t) & 1) || sr.y < 0 || sr.y >= S.max_segs) continue;
      const int r = s_segop[sr.y];
      if (r < 0) continue;
      const int4 o1 = *(const int4*)(recs + 8 * r + 4);
      if ((unsigned)(sr.x - o1.z) >= (unsigned)o1.w) continue;       // not on a consistent state
      const int at = atomicAdd(s_cnt, 1);
      if (at >= EV_MAXSLOT) continue;
      const int off = sr.x - lo;
      s_pos[at] = off | (r << 15);
      s_slot[at] = blk * TKV_BS + t;
      atomicOr(&s_bm[off >> 5], 1u << (off & 31));
      atomicAdd(&s_m[r], 1);
    }
    __syncthreads();
    const int m = *s_cnt < EV_MAXSLOT ? *s_cnt : EV_MAXSLOT;
    // exclusive prefix of the bitmap words' popcounts
    {
      int pc[EV_BMW / EV_THREADS], v[3] = {0, 0, 0}, ex[3], tot[3];
#pragma unroll
      for (int u = 0; u < EV_BMW / EV_THREADS; u++) {
        const int w = tid * (EV_BMW / EV_THREADS) + u;
        pc[u] = w < nbw ? __popc(s_bm[w]) : 0;
        v[0] += pc[u];
      }
      wg_scan3(v, ex, tot, s_tmp);
      int run = ex[0];
#pragma unroll
      for (int u = 0; u < EV_BMW / EV_THREADS; u++) {
        s_bpre[tid * (EV_BMW / EV_THREADS) + u] = run;
        run += pc[u];
      }
    }
    __syncthreads();
    // per op in list order: kept and evicted counts, stack offset, rank of its first position
    if (tid == 0) {
      int run = q[Q_NSLOT + c], evc = 0;
      for (int r = 0; r < cnt; r++) {
        const int4 o0 = *(const int4*)(recs + 8 * r), o1 = *(const int4*)(recs + 8 * r + 4);
        if (!(o0.x & 1) || ((o0.x >> 4) & 3) != c) continue;
        const int mr = s_m[r];
        const int keep = o0.z < mr ? o0.z : mr;
        const int off = o1.z - lo;
        s_ev[r] = mr - keep;
        s_base[r] = run;
        s_rk0[r] = s_bpre[off >> 5] + __popc(s_bm[off >> 5] & ((1u << (off & 31)) - 1u));
        run += mr - keep;
        evc += mr - keep;
        S.segt[((int64_t)s * S.max_segs + o0.y) * TKV_SEG_W + G_NRET] = keep;
      }
      q[Q_NSLOT + c] = run;
      s_evtot += evc;
    }
    __syncthreads();
    int32_t* stc = st + (int64_t)c * S.max_blocks * TKV_BS;
    for (int a = tid; a < m; a += EV_THREADS) {
      const int off = s_pos[a] & 0x7FFF, r = s_pos[a] >> 15;
      const int rk = s_bpre[off >> 5] + __popc(s_bm[off >> 5] & ((1u << (off & 31)) - 1u)) - s_rk0[r];
      if (rk >= s_ev[r]) continue;
      const int sl = s_slot[a];
      atomicAnd(&pick3(S.blk, c)[(int64_t)(sl / TKV_BS) * TKV_BLK_W], ~(1 << (sl % TKV_BS)));
      stc[s_base[r] + rk] = sl;
    }
    __threadfence_block();
    __syncthreads();
  }
  if (tid == 0) q[Q_NRET] -= s_evtot;
}

__global__ __launch_bounds__(EV_THREADS) void k_evict_apply(DevState S) {
  __shared__ int32_t s_pos[EV_MAXSLOT];
  __shared__ int32_t s_slot[EV_MAXSLOT];
  __shared__ int32_t s_rank[EV_MAXSLOT];
  __shared__ uint32_t s_bm[EV_BMW];
  __shared__ int32_t s_bpre[EV_BMW];
  __shared__ uint8_t s_codes[EV_THREADS / 64][128];
  __shared__ int s_tmp[48];
  __shared__ int s_cnt;
  const int s = blockIdx.x, tid = threadIdx.x;
  const int32_t* grp = scr_grp(S.scratch);
  const int cnt = grp[S.max_seqs + s];
  if (cnt == 0) {
    if (tid == 0) scr_mcnt(S.scratch)[s] = 0;
    return;
  }
  const int32_t* recs = scr_oprec(S.scratch) + 8 * grp[s];
  const int ndown = grp[2 * S.max_seqs + s];
  const int32_t* misc = scr_misc(S.scratch);
  int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
  int32_t* bt = S.btab + (int64_t)s * 3 * S.max_blocks;
  int32_t* st = S.sstk + (int64_t)s * 3 * S.max_blocks * TKV_BS;
  int32_t* moves = scr_moves(S.scratch, S.max_seqs) + (int64_t)s * S.max_blocks * TKV_BS * 2;
  // With one downgrade for this sequence in the call, its re-quantization is
  // deferred to a wide kernel (the old slots cannot be overwritten within the
  // call); with several, a later one could reuse slots an earlier one still
  // reads from, so they are re-quantized here, in op order.
  const bool defer = ndown <= 1;
  int nmoves = 0;
  // Several ops and no downgrade: each class in one scan (below); otherwise
  // (or when a bound of that path is exceeded) the ops one after another.
  if (ndown == 0 && cnt > 1 && cnt <= EVB_MAXOPS && S.max_segs <= EV_MAXSLOT) {
    __shared__ int s_ok;
    if (tid == 0) {
      int ok = 1;
      for (int c = 0; c < 3 && ok; c++) {
        int lo = TKV_INF, hi = -1;
        for (int r = 0; r < cnt; r++) {
          const int4 o0 = *(const int4*)(recs + 8 * r), o1 = *(const int4*)(recs + 8 * r + 4);
          if (!(o0.x & 1) || ((o0.x >> 4) & 3) != c) continue;
          lo = min(lo, o1.z);
          hi = max(hi, o1.z + o1.w - 1);
        }
        if (hi >= lo && hi - lo + 1 > EV_BMW * 32) ok = 0;
      }
      s_ok = ok;
    }
    __syncthreads();
    if (s_ok) {
      evict_classwise(S, s, cnt, recs, q, bt, st, s_pos, s_slot, s_rank, s_bm, s_bpre, s_tmp, &s_cnt);
      if (tid == 0) scr_mcnt(S.scratch)[s] = 0;
      return;
    }
  }
  for (int r0 = 0; r0 < cnt; r0++) {
    const int4 o0 = *(const int4*)(recs + 8 * r0), o1 = *(const int4*)(recs + 8 * r0 + 4);
    if (!(o0.x & 1)) continue;
    const int c = (o0.x >> 4) & 3, c2 = (o0.x >> 8) & 3;
    const int k = o0.y, nb = o0.w, gb = class_bits(c);
    int keep = o0.z;
    const int down = (nb != 0 && nb < gb && keep > 0);
    const int nd = o1.x, base = o1.y, first = o1.z, span = o1.w;
    int32_t* g = S.segt + ((int64_t)s * S.max_segs + k) * TKV_SEG_W;
    // gather the segment's valid slots; rank them by position with a bitmap of
    // the segment's position span (a sort when the span is too wide)
    const bool use_bm = span > 0 && span <= EV_BMW * 32;
    const int nbw = use_bm ? (span + 31) >> 5 : 0;
    for (int w = tid; w < nbw; w += EV_THREADS) s_bm[w] = 0;
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    const int nbk = q[Q_NBLK + c];
    for (int x = tid; x < nbk * TKV_BS; x += EV_THREADS) {
      const int blk = bt[c * S.max_blocks + x / TKV_BS], t = x % TKV_BS;
      // both reads depend only on the block id: issued together
      const int mask = pick3(S.blk, c)[(int64_t)blk * TKV_BLK_W];
      const int2 sr = *(const int2*)(pick3(S.slot, c) + ((int64_t)blk * TKV_BS + t) * 2);
      if (!((mask >> t) & 1) || sr.y != k) continue;
      const int at = atomicAdd(&s_cnt, 1);
      if (at >= EV_MAXSLOT) continue;
      s_pos[at] = sr.x;
      s_slot[at] = blk * TKV_BS + t;
      const unsigned off = (unsigned)(sr.x - first);
      if (use_bm && off < (unsigned)span) atomicOr(&s_bm[off >> 5], 1u << (off & 31));
    }
    __syncthreads();
    const int m = s_cnt < EV_MAXSLOT ? s_cnt : EV_MAXSLOT;
    const int32_t* sorted;
    if (use_bm) {
      // exclusive prefix of the bitmap words' popcounts (EV_BMW / EV_THREADS words per thread)
      int pc[EV_BMW / EV_THREADS], v[3] = {0, 0, 0}, ex[3], tot[3];
#pragma unroll
      for (int u = 0; u < EV_BMW / EV_THREADS; u++) {
        const int w = tid * (EV_BMW / EV_THREADS) + u;
        pc[u] = w < nbw ? __popc(s_bm[w]) : 0;
        v[0] += pc[u];
      }
      wg_scan3(v, ex, tot, s_tmp);
      int run = ex[0];
#pragma unroll
      for (int u = 0; u < EV_BMW / EV_THREADS; u++) {
        s_bpre[tid * (EV_BMW / EV_THREADS) + u] = run;
        run += pc[u];
      }
      __syncthreads();
      for (int a = tid; a < m; a += EV_THREADS) {
        const unsigned off = (unsigned)(s_pos[a] - first);
        if (off >= (unsigned)span) continue;          // not on a consistent state
        const int rk = s_bpre[off >> 5] + __popc(s_bm[off >> 5] & ((1u << (off & 31)) - 1u));
        if (rk < m) s_rank[rk] = s_slot[a];
      }
      __syncthreads();
      sorted = s_rank;
    } else {
      lds_sort_pairs(s_pos, s_slot, m, tid, EV_THREADS);
      sorted = s_slot;
    }
    if (keep > m) keep = m;                 // m == r on a consistent state
    const int ev = m - keep;
    const int ns_c = q[Q_NSLOT + c];
    for (int a = tid; a < ev; a += EV_THREADS) {
      int sl = sorted[a];
      atomicAnd(&pick3(S.blk, c)[(int64_t)(sl / TKV_BS) * TKV_BLK_W], ~(1 << (sl % TKV_BS)));
      st[(int64_t)c * S.max_blocks * TKV_BS + ns_c + a] = sl;
    }
    if (down) {
      const int S0 = q[Q_NSLOT + c2];
      const int nbk2 = q[Q_NBLK + c2];
      const int av = misc[c2];
      int32_t* st2 = st + (int64_t)c2 * S.max_blocks * TKV_BS;
      for (int b = tid; b < nd; b += EV_THREADS) {
        int blk = pick3(S.freestk, c2)[av - 1 - (base + b)];
        bt[c2 * S.max_blocks + nbk2 + b] = blk;
        pick3(S.blk, c2)[(int64_t)blk * TKV_BLK_W + 2] = s;
      }
      __threadfence_block();
      __syncthreads();
      // re-quantize each kept token (K and V rows of every head) into its new slot
      if (defer) {
        for (int p = tid; p < keep; p += EV_THREADS) {
          int ns;
          if (p < S0) ns = st2[S0 - 1 - p];
          else { int pp = p - S0; ns = bt[c2 * S.max_blocks + nbk2 + pp / TKV_BS] * TKV_BS + pp % TKV_BS; }
          moves[2 * (nmoves + p)] = (c << 28) | sorted[ev + p];
          moves[2 * (nmoves + p) + 1] = (c2 << 28) | ns;
        }
        nmoves += keep;
      } else {
        const int wv = tid >> 6, lane = tid & 63;
        for (int row = wv; row < keep * S.Hst * 2; row += EV_THREADS / 64) {
          const int kv = row & 1, h = (row >> 1) % S.Hst, p = (row >> 1) / S.Hst;
          int ns;
          if (p < S0) ns = st2[S0 - 1 - p];
          else { int pp = p - S0; ns = bt[c2 * S.max_blocks + nbk2 + pp / TKV_BS] * TKV_BS + pp % TKV_BS; }
          requant_row(S, (c << 28) | sorted[ev + p], (c2 << 28) | ns, h, kv, lane, s_codes[wv]);
        }
      }
      __threadfence_block();
      __syncthreads();
      for (int p = tid; p < keep; p += EV_THREADS) {
        int old = sorted[ev + p];
        int ns;
        if (p < S0) ns = st2[S0 - 1 - p];
        else { int pp = p - S0; ns = bt[c2 * S.max_blocks + nbk2 + pp / TKV_BS] * TKV_BS + pp % TKV_BS; }
        int pos = pick3(S.slot, c)[(int64_t)old * 2];
        atomicOr(&pick3(S.blk, c2)[(int64_t)(ns / TKV_BS) * TKV_BLK_W], 1 << (ns % TKV_BS));
        atomicMax(&pick3(S.blk, c2)[(int64_t)(ns / TKV_BS) * TKV_BLK_W + 1], pos);
        pick3(S.slot, c2)[(int64_t)ns * 2] = pos;
        pick3(S.slot, c2)[(int64_t)ns * 2 + 1] = k;
        atomicAnd(&pick3(S.blk, c)[(int64_t)(old / TKV_BS) * TKV_BLK_W], ~(1 << (old % TKV_BS)));
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
  TKV_TIMED(c, st, "k_evict_plan",
            k_evict_plan<<<1, walker_threads(c->S.max_seqs), 0, st>>>(c->S, n_ops, n_ops_dev, seq_ids, seg_ids, keep_n,
                                                                      new_bits));
  TKV_TIMED(c, st, "k_evict_apply", k_evict_apply<<<c->S.max_seqs, EV_THREADS, 0, st>>>(c->S));
  launch_requant(c, st);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// Budget ladder.  Every listed sequence's record is read in parallel to find
// those over budget; one wave then walks each of these, reading 64 segment
// records at a time: the newest retained T segment is the highest set bit of
// a ballot over the table read from its end; eviction candidates are T
// segments (oldest first) and a candidate is taken while the retained count
// before it still exceeds the budget, i.e. for a prefix of the candidates,
// found with a prefix sum of their retained counts; the downgrade is the
// lowest set bit of a ballot.  A first walk counts each sequence's ops, a scan
// over the list places them, a second walk writes them.
// ---------------------------------------------------------------------------
__device__ inline bool over_budget(const DevState& S, int s, int num, int den) {
  if (s < 0 || s >= S.max_seqs) return false;
  const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
  const int len = q[Q_LEN], nr = q[Q_NRET];
  return (long long)nr > (long long)len * num / den;
}

// write: place the ops at base.. in the output lists; otherwise only count
// them, keeping the first PL_STAGE_K (segment, keep, bits) in `stage` if given.
#define PL_STAGE_K 8
__device__ int ladder_wave(const DevState& S, int s, int num, int den, int base, int max_ops, int32_t* os,
                           int32_t* og, int32_t* ok, uint8_t* ob, bool write, int lane, int2* stage) {
  if (s < 0 || s >= S.max_seqs) return 0;
  const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
  const int nseg = __builtin_amdgcn_readfirstlane(q[Q_NSEG]);
  const int len = __builtin_amdgcn_readfirstlane(q[Q_LEN]);
  const int nr0 = __builtin_amdgcn_readfirstlane(q[Q_NRET]);
  const long long B = (long long)len * num / den;
  long long nr = nr0;
  if (nr <= B) return 0;
  const int32_t* segs = S.segt + (int64_t)s * S.max_segs * TKV_SEG_W;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  // newest retained T segment
  int newest_t = -1;
  for (int b0 = ((nseg - 1) >> 6) << 6; b0 >= 0; b0 -= 64) {
    const int k = b0 + lane;
    bool hit = false;
    if (k < nseg) {
      const int32_t* g = segs + (int64_t)k * TKV_SEG_W;
      hit = g[G_TYPE] == TKV_T && g[G_NRET] > 0;
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
    if (m) { newest_t = b0 + 63 - __builtin_clzll(m); break; }
  }
  // whole T segments, oldest first, never the open one nor the newest retained T
  int m = 0;
  for (int b0 = 0; b0 < nseg - 1 && nr > B; b0 += 64) {
    const int k = b0 + lane;
    int amt = 0;
    if (k < nseg - 1 && k != newest_t) {
      const int32_t* g = segs + (int64_t)k * TKV_SEG_W;
      if (g[G_TYPE] == TKV_T) amt = g[G_NRET];
    }
    const int incl = wave_incl_scan(amt);
    const bool take = amt > 0 && nr - (incl - amt) > B;
    const uint64_t tm = __builtin_amdgcn_ballot_w64(take);
    if (take) {
      const int rel = m + __popcll(tm & lt);
      if (write) {
        if (base + rel < max_ops) { os[base + rel] = s; og[base + rel] = k; ok[base + rel] = 0; ob[base + rel] = 0; }
      } else if (stage && rel < PL_STAGE_K) {
        stage[rel] = make_int2(k, 0);
      }
    }
    m += __popcll(tm);
    nr -= wave_total(wave_incl_scan(take ? amt : 0));
  }
  // then one downgrade: the oldest non-open E segment above 2 bits
  if (nr > B) {
    for (int b0 = 0; b0 < nseg - 1; b0 += 64) {
      const int k = b0 + lane;
      int r = 0;
      if (k < nseg - 1) {
        const int32_t* g = segs + (int64_t)k * TKV_SEG_W;
        if (g[G_TYPE] == TKV_E && g[G_BITS] > 2) r = g[G_NRET];
      }
      const uint64_t hm = __builtin_amdgcn_ballot_w64(r > 0);
      if (hm) {
        if (lane == __builtin_ctzll(hm)) {
          if (write) {
            if (base + m < max_ops) { os[base + m] = s; og[base + m] = k; ok[base + m] = r; ob[base + m] = 2; }
          } else if (stage && m < PL_STAGE_K) {
            stage[m] = make_int2(k, r | (2 << 24));
          }
        }
        m++;
        break;
      }
    }
  }
  return m;
}

#define PL_STAGE_R 256     // over-budget sequences whose first ops are staged in LDS
__device__ __forceinline__ void plan_body(const DevState& S, int n, const int32_t* seq_ids, int num, int den,
                                          int max_ops, int32_t* n_ops, int32_t* os, int32_t* og, int32_t* ok,
                                          uint8_t* ob) {
  __shared__ uint16_t s_over[TKV_MAX_TOK];   // items over budget, in list order
  __shared__ int s_cnt[TKV_MAX_TOK];         // their op counts
  __shared__ int s_base[TKV_MAX_TOK];        // their first op's index
  __shared__ int2 s_stage[PL_STAGE_R][PL_STAGE_K];
  __shared__ int s_tmp[48];
  const int tid = threadIdx.x, NT = blockDim.x, wv = tid >> 6, lane = tid & 63, NW = NT >> 6;
  // 1. the listed sequences over budget
  for (int i = tid; i < n; i += NT) s_cnt[i] = over_budget(S, seq_ids[i], num, den);
  __syncthreads();
  const int per = (n + NT - 1) / NT;
  const int lo = tid * per, hi = min(n, lo + per);
  int v[3] = {0, 0, 0}, ex[3], tot[3];
  for (int i = lo; i < hi; i++) v[0] += s_cnt[i];
  wg_scan3(v, ex, tot, s_tmp);
  for (int i = lo, r = ex[0]; i < hi; i++) if (s_cnt[i]) s_over[r++] = (uint16_t)i;
  const int nover = tot[0];
  __syncthreads();
  if (nover == 0) {
    if (tid == 0) *n_ops = 0;
    return;
  }
  // 2. count each one's ops (staging the first few), place them in list order, write them
  for (int r = wv; r < nover; r += NW) {
    const int s = __builtin_amdgcn_readfirstlane(seq_ids[s_over[r]]);
    const int m = ladder_wave(S, s, num, den, 0, 0, os, og, ok, ob, false, lane,
                              r < PL_STAGE_R ? s_stage[r] : nullptr);
    if (lane == 0) s_cnt[r] = m;
  }
  __syncthreads();
  const int per2 = (nover + NT - 1) / NT;
  const int lo2 = tid * per2, hi2 = min(nover, lo2 + per2);
  int v2[3] = {0, 0, 0}, ex2[3], tot2[3];
  for (int r = lo2; r < hi2; r++) v2[0] += s_cnt[r];
  wg_scan3(v2, ex2, tot2, s_tmp);
  for (int r = lo2, run = ex2[0]; r < hi2; r++) { s_base[r] = run; run += s_cnt[r]; }
  __syncthreads();
  for (int r = wv; r < nover; r += NW) {
    const int m = s_cnt[r], b0 = s_base[r];
    if (m == 0) continue;
    const int s = __builtin_amdgcn_readfirstlane(seq_ids[s_over[r]]);
    if (r < PL_STAGE_R && m <= PL_STAGE_K) {
      if (lane < m && b0 + lane < max_ops) {
        const int2 e = s_stage[r][lane];
        os[b0 + lane] = s; og[b0 + lane] = e.x; ok[b0 + lane] = e.y & 0xFFFFFF; ob[b0 + lane] = (uint8_t)(e.y >> 24);
      }
    } else {
      ladder_wave(S, s, num, den, b0, max_ops, os, og, ok, ob, true, lane, nullptr);
    }
  }
  if (tid == 0) *n_ops = tot2[0] < max_ops ? tot2[0] : max_ops;
}
__global__ __launch_bounds__(WG) void k_plan(DevState S, int n, const int32_t* seq_ids, int num, int den, int max_ops,
                                             int32_t* n_ops, int32_t* os, int32_t* og, int32_t* ok, uint8_t* ob) {
  plan_body(S, n, seq_ids, num, den, max_ops, n_ops, os, og, ok, ob);
}

// a wave per listed sequence, up to max_threads / 64 waves
static int launch_plan_t(tkv_cache* c, int n, const int32_t* seq_ids, int num, int den, int max_ops,
                         int32_t* n_ops_dev, int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits,
                         int max_threads, hipStream_t st) {
  const int nt = n < 1 ? 64 : (n >= max_threads / 64 ? max_threads : 64 * n);
  TKV_TIMED(c, st, "k_plan",
            k_plan<<<1, nt, 0, st>>>(c->S, n, seq_ids, num, den, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits));
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}
int launch_plan(tkv_cache* c, int n, const int32_t* seq_ids, int num, int den, int max_ops, int32_t* n_ops_dev,
                int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits, hipStream_t st) {
  return launch_plan_t(c, n, seq_ids, num, den, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits, WG, st);
}

// The ladder, then the eviction's kernels (kv_evict_segment with the ladder's
// device-side op count).  In a decode loop this call runs beside the next
// batch's attention, which holds every compute unit's registers but for a
// slot of about 112 VGPRs per SIMD lane and ~96 KB of LDS per compute unit:
// a ladder work-group of at most 8 waves (32 VGPRs, 57 KB of LDS) and the
// eviction's planning work-group (256 threads at B256, 47 VGPRs, 62 KB) fit
// there and start at once, where one work-group doing both (1024 threads,
// 120 KB of LDS; measured 5 us faster alone) waited for a compute unit the
// attention had left entirely.
#define PL_EVICT_THREADS 512
int launch_plan_evict(tkv_cache* c, int n, const int32_t* seq_ids, int num, int den, int max_ops, int32_t* n_ops_dev,
                      int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits, hipStream_t st) {
  const int r = launch_plan_t(c, n, seq_ids, num, den, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits,
                              PL_EVICT_THREADS, st);
  if (r != TKV_OK || max_ops == 0) return r;
  return launch_evict(c, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits, st);
}

// ---------------------------------------------------------------------------
// Annealing schedule of TBE (Methodologie, TBE bullet: on a Transition thought
// the earlier Reasoning/Execution segments are evicted progressively, the
// retention shrinking on a schedule such as 64, 32, 16; the lay summary keeps
// a small safety net of Transition thoughts).  An R or E segment with e >= 1
// T segments opened after it is capped at r0 halved e-1 times and keeps its
// cap newest retained tokens; T segments are never planned.  One wave per
// listed sequence walks its segment table 64 records at a time: a ballot over
// the T records gives the total, a running prefix of it gives each record's
// count of later T segments, and a ballot over the over-cap records places
// the ops in segment order.  A first walk counts each sequence's ops, a scan
// over the list places them, a second walk writes them.
// ---------------------------------------------------------------------------
__device__ int anneal_wave(const DevState& S, int s, int r0, int base, int max_ops, int32_t* os, int32_t* og,
                           int32_t* ok, uint8_t* ob, bool write, int lane) {
  if (s < 0 || s >= S.max_seqs) return 0;
  const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
  const int nseg = __builtin_amdgcn_readfirstlane(q[Q_NSEG]);
  const int32_t* segs = S.segt + (int64_t)s * S.max_segs * TKV_SEG_W;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int total_t = 0;
  for (int b0 = 0; b0 < nseg; b0 += 64) {
    const int k = b0 + lane;
    const bool t = k < nseg && segs[(int64_t)k * TKV_SEG_W + G_TYPE] == TKV_T;
    total_t += __popcll(__builtin_amdgcn_ballot_w64(t));
  }
  if (total_t == 0) return 0;
  int m = 0, seen_t = 0;                          // T segments in earlier chunks
  for (int b0 = 0; b0 < nseg; b0 += 64) {
    const int k = b0 + lane;
    int type = TKV_T, nret = 0;
    if (k < nseg) {
      const int32_t* g = segs + (int64_t)k * TKV_SEG_W;
      type = g[G_TYPE];
      nret = g[G_NRET];
    }
    const uint64_t tb = __builtin_amdgcn_ballot_w64(k < nseg && type == TKV_T);
    const int later = total_t - seen_t - __popcll(tb & (lt | (1ull << lane)));  // T segments after k
    const int sh = later - 1 < 31 ? later - 1 : 31;
    const int cap = later >= 1 ? (r0 >> sh) : 0;
    const bool take = k < nseg && type != TKV_T && later >= 1 && nret > cap;
    const uint64_t tm = __builtin_amdgcn_ballot_w64(take);
    if (take && write) {
      const int at = base + m + __popcll(tm & lt);
      if (at < max_ops) { os[at] = s; og[at] = k; ok[at] = cap; ob[at] = 0; }
    }
    m += __popcll(tm);
    seen_t += __popcll(tb);
  }
  return m;
}

__device__ __forceinline__ void anneal_body(const DevState& S, int n, const int32_t* seq_ids, int r0, int max_ops,
                                            int32_t* n_ops, int32_t* os, int32_t* og, int32_t* ok, uint8_t* ob) {
  __shared__ int s_cnt[TKV_MAX_TOK];         // ops of each listed sequence
  __shared__ int s_base[TKV_MAX_TOK];        // their first op's index
  __shared__ int s_tmp[48];
  const int tid = threadIdx.x, NT = blockDim.x, wv = tid >> 6, lane = tid & 63, NW = NT >> 6;
  for (int i = wv; i < n; i += NW) {
    const int s = __builtin_amdgcn_readfirstlane(seq_ids[i]);
    const int m = anneal_wave(S, s, r0, 0, 0, os, og, ok, ob, false, lane);
    if (lane == 0) s_cnt[i] = m;
  }
  __syncthreads();
  const int per = (n + NT - 1) / NT;
  const int lo = tid * per, hi = min(n, lo + per);
  int v[3] = {0, 0, 0}, ex[3], tot[3];
  for (int i = lo; i < hi; i++) v[0] += s_cnt[i];
  wg_scan3(v, ex, tot, s_tmp);
  for (int i = lo, run = ex[0]; i < hi; i++) { s_base[i] = run; run += s_cnt[i]; }
  __syncthreads();
  for (int i = wv; i < n; i += NW) {
    if (s_cnt[i] == 0 || s_base[i] >= max_ops) continue;
    const int s = __builtin_amdgcn_readfirstlane(seq_ids[i]);
    anneal_wave(S, s, r0, s_base[i], max_ops, os, og, ok, ob, true, lane);
  }
  if (tid == 0) *n_ops = tot[0] < max_ops ? tot[0] : max_ops;
}

__global__ __launch_bounds__(WG) void k_anneal(DevState S, int n, const int32_t* seq_ids, int r0, int max_ops,
                                               int32_t* n_ops, int32_t* os, int32_t* og, int32_t* ok, uint8_t* ob) {
  anneal_body(S, n, seq_ids, r0, max_ops, n_ops, os, og, ok, ob);
}
// The annealing plan and the first part of the eviction in one work-group:
// the op list the plan writes (global memory) is read back by the same
// work-group after a barrier; then the eviction's apply and re-quantization
// kernels as in kv_evict_segment.
__global__ __launch_bounds__(WG) void k_anneal_evict(DevState S, int n, const int32_t* seq_ids, int r0, int max_ops,
                                                     int32_t* n_ops, int32_t* os, int32_t* og, int32_t* ok,
                                                     uint8_t* ob) {
  anneal_body(S, n, seq_ids, r0, max_ops, n_ops, os, og, ok, ob);
  __syncthreads();
  evict_plan_body(S, max_ops, n_ops, os, og, ok, ob);
}

int launch_anneal(tkv_cache* c, int n, const int32_t* seq_ids, int r0, int max_ops, int32_t* n_ops_dev,
                  int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits, hipStream_t st) {
  const int nt = n < 1 ? 64 : (n >= WG / 64 ? WG : 64 * n);
  TKV_TIMED(c, st, "k_anneal",
            k_anneal<<<1, nt, 0, st>>>(c->S, n, seq_ids, r0, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits));
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}
int launch_anneal_evict(tkv_cache* c, int n, const int32_t* seq_ids, int r0, int max_ops, int32_t* n_ops_dev,
                        int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits, hipStream_t st) {
  if (max_ops == 0) return launch_anneal(c, n, seq_ids, r0, 0, n_ops_dev, op_seq, op_seg, op_keep, op_bits, st);
  TKV_TIMED(c, st, "k_anneal_evict",
            k_anneal_evict<<<1, WG, 0, st>>>(c->S, n, seq_ids, r0, max_ops, n_ops_dev, op_seq, op_seg, op_keep,
                                             op_bits));
  TKV_TIMED(c, st, "k_evict_apply", k_evict_apply<<<c->S.max_seqs, EV_THREADS, 0, st>>>(c->S));
  launch_requant(c, st);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// Gather compaction, the baseline that in-place reuse avoids (abstract: the
// kernel reuses evicted tokens' slots, eliminating compaction; Continuous
// Thinking bullet).  For each listed sequence (first listing only) and class
// holding blocks, the m retained tokens are copied bit for bit, in position
// order, into ceil(m/16) blocks popped from the class's global stack (token i
// into slot i % 16 of the (i/16)-th popped block), which become its block
// list; its free-slot stack becomes the empty tail of the last one (lowest
// slot on top).  All pops of the call come first (list order), then every
// compacted sequence's old blocks go back (list order, classes in order,
// blocks in list order, records cleared).  A sequence that does not find all
// its blocks fails with ENOMEM, untouched; after the first such failure of a
// class, every later sequence needing blocks of that class fails too.
//   k_compact_plan: first listings, token counts (a wave per sequence), the
//     list-order pops (one thread: the failure rule is a chain), the pushes'
//     places, and the offsets of the copy tasks (one per new block).
//   k_compact_copy: a fixed grid of work-groups walks the tasks.  A task
//     ranks the class's retained tokens by position (a bitmap over their
//     positions and its prefix counts), takes the 16 of its block and writes
//     the block: K chunks hold one token each and are copied word for word; a
//     V word holds the codes of a token quad and is assembled field by field;
//     metadata words are per (token, group); then the new slots' and block's
//     records.  Sources are old blocks, destinations popped ones: no block is
//     both read and written, and the block lists are not touched yet.
//   k_compact_push: the new block lists and slot stacks, then the old blocks
//     onto the global stacks and the stack heights.
// Scratch: per item {seq or -1, pop top[3], push base[3]}; per (item, class)
// the task offsets; per sequence its old block lists [3][max_blocks], their
// lengths [3] and its token counts [3], in its move area.
// ---------------------------------------------------------------------------
#define CMP_BMW 2048          // position bitmap words of the ranking: spans up to 65536 positions
__device__ inline int32_t* cmp_old(const DevState& S, int s, int c) {
  return scr_moves(S.scratch, S.max_seqs) + (int64_t)s * S.max_blocks * TKV_BS * 2 + c * S.max_blocks;
}
__device__ inline int32_t* cmp_counts(const DevState& S, int s) {       // [0..2] old lengths, [3..5] tokens
  return scr_moves(S.scratch, S.max_seqs) + (int64_t)s * S.max_blocks * TKV_BS * 2 + 3 * S.max_blocks;
}
__device__ inline int32_t* cmp_tasks(const DevState& S) { return S.scratch + TKV_MAX_TOK; }   // [3 * MAX_TOK + 1]

__device__ inline int eff_count(int n_cap, const int32_t* n_dev) {
  if (!n_dev) return n_cap;
  const int m = *n_dev;
  return m < n_cap ? (m < 0 ? 0 : m) : n_cap;
}

__global__ __launch_bounds__(WG) void k_compact_plan(DevState S, int n_cap, const int32_t* n_dev,
                                                     const int32_t* seq_ids) {
  __shared__ int s_first[TKV_MAX_SEQS];
  __shared__ int16_t s_m[TKV_MAX_TOK][3];
  const int tid = threadIdx.x, NT = blockDim.x, wv = tid >> 6, lane = tid & 63, NW = NT >> 6;
  const int n = eff_count(n_cap, n_dev);
  for (int s = tid; s < S.max_seqs; s += NT) s_first[s] = TKV_INF;
  __syncthreads();
  for (int i = tid; i < n; i += NT) {
    const int s = seq_ids[i];
    if (s >= 0 && s < S.max_seqs) atomicMin(&s_first[s], i);
  }
  __syncthreads();
  // retained tokens per class of each first listing (a wave per item)
  for (int i = wv; i < n; i += NW) {
    const int s = __builtin_amdgcn_readfirstlane(seq_ids[i]);
    if (s < 0 || s >= S.max_seqs || s_first[s] != i) continue;
    const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
    for (int c = 0; c < 3; c++) {
      const int nb = q[Q_NBLK + c];
      int m = 0;
      for (int j = lane; j < nb; j += 64)
        m += __popc((uint32_t)pick3(S.blk, c)[(int64_t)S.btab[((int64_t)s * 3 + c) * S.max_blocks + j] * TKV_BLK_W] &
                    0xFFFFu);
      m = wave_total(wave_incl_scan(m));
      if (lane == 0) s_m[i][c] = (int16_t)m;
    }
  }
  int32_t* recs = scr_oprec(S.scratch);
  for (int i = tid; i < n_cap; i += NT) recs[8 * i] = -1;
  __syncthreads();
  if (tid == 0) {
    int avail[3], cum[3] = {0, 0, 0}, pushed[3] = {0, 0, 0}, tasks = 0;
    bool dry[3] = {false, false, false};
    for (int c = 0; c < 3; c++) avail[c] = S.hdr[H_FREE + c];
    int32_t* pre = cmp_tasks(S);
    for (int i = 0; i < n; i++) {
      const int s = seq_ids[i];
      int need[3] = {0, 0, 0};
      bool planned = false;
      if (s < 0 || s >= S.max_seqs) {
        record_error(S.hdr, TKV_EINVAL, s < 0 ? TKV_INF : s);
      } else if (s_first[s] == i) {
        bool ok = true;
        for (int c = 0; c < 3; c++) {
          need[c] = (s_m[i][c] + TKV_BS - 1) / TKV_BS;
          if (need[c] > 0 && (dry[c] || need[c] > avail[c] - cum[c])) { dry[c] = true; ok = false; }
        }
        if (!ok) record_error(S.hdr, TKV_ENOMEM, s);
        planned = ok;
      }
      if (planned) {
        recs[8 * i] = s;
        int32_t* cn = cmp_counts(S, s);
        for (int c = 0; c < 3; c++) {
          recs[8 * i + 1 + c] = avail[c] - 1 - cum[c];
          cum[c] += need[c];
          cn[3 + c] = s_m[i][c];
        }
      }
      for (int c = 0; c < 3; c++) {
        pre[3 * i + c] = tasks;
        tasks += planned ? need[c] : 0;
      }
    }
    pre[3 * n] = tasks;
    // pushes start where the pops ended
    for (int i = 0; i < n; i++) {
      const int s = recs[8 * i];
      if (s < 0) continue;
      const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
      int32_t* cn = cmp_counts(S, s);
      for (int c = 0; c < 3; c++) {
        recs[8 * i + 4 + c] = avail[c] - cum[c] + pushed[c];
        cn[c] = q[Q_NBLK + c];
        pushed[c] += q[Q_NBLK + c];
      }
    }
    int32_t* misc = scr_misc(S.scratch);
    for (int c = 0; c < 3; c++) misc[8 + c] = avail[c] - cum[c] + pushed[c];
  }
}

template <int BITS>
__device__ void compact_copy_block(const DevState& S, int c, int newb, int cnt, const int32_t* src_slot, int tid) {
  constexpr int W = 32 / BITS;
  const int D = S.D, g = S.g, NG = D / g, CB = D * BITS / 32, CW = CB / 4;
  const int nat = natural_order(S.fmt, c);
  const int64_t R = pick3(S.bh_bytes, c);
  uint8_t* pool = pick3(S.pool, c);
  const int nk = 16 * 4 * CW, nv = 4 * 16 * CW, nm = 16 * 2 * NG, per_head = nk + nv + nm;
  for (int x = tid; x < S.Hst * per_head; x += EV_THREADS) {
    const int h = x / per_head;
    int u = x % per_head;
    uint8_t* dst = pool + ((int64_t)newb * S.Hst + h) * R;
    if (u < nk) {                              // K chunk word: one token
      const int td = u / (4 * CW), lg = (u / CW) % 4, wc = u % CW;
      if (td >= cnt) continue;
      const int src = src_slot[td], ts = src % TKV_BS;
      const uint8_t* sr = pool + ((int64_t)(src / TKV_BS) * S.Hst + h) * R;
      *(uint32_t*)(dst + chunk_byte(CB, 16 * lg + td, 4 * wc)) = *(const uint32_t*)(sr + chunk_byte(CB, 16 * lg + ts, 4 * wc));
    } else if ((u -= nk) < nv) {               // V word: a token quad, field by field
      const int qd = u / (16 * CW), i = (u / CW) % 16, wc = u % CW;
      uint32_t out = 0;
      for (int r = 0; r < 4; r++) {
        const int td = 4 * qd + r;
        if (td >= cnt) break;
        const int src = src_slot[td], ts = src % TKV_BS, qs = ts >> 2, rs = ts & 3;
        const uint8_t* sr = pool + ((int64_t)(src / TKV_BS) * S.Hst + h) * R;
        const uint32_t w = *(const uint32_t*)(sr + 64 * CB + chunk_byte(CB, 16 * qs + i, 4 * wc));
        for (int nn = 0; nn < W / 4; nn++) {
          const int fs = 4 * nn + rs, fd = 4 * nn + r;
          const int ps = field_pos(fs, W, nat), pd = field_pos(fd, W, nat);
          out |= ((w >> (ps * BITS)) & ((1u << BITS) - 1u)) << (pd * BITS);
        }
      }
      *(uint32_t*)(dst + 64 * CB + chunk_byte(CB, 16 * qd + i, 4 * wc)) = out;
    } else {                                   // metadata word
      u -= nv;
      const int td = u / (2 * NG), kv = (u / NG) % 2, gi = u % NG;
      if (td >= cnt) continue;
      const int src = src_slot[td], ts = src % TKV_BS;
      const uint8_t* sr = pool + ((int64_t)(src / TKV_BS) * S.Hst + h) * R;
      *(uint32_t*)(dst + meta_byte(D, g, BITS, kv, td, gi)) = *(const uint32_t*)(sr + meta_byte(D, g, BITS, kv, ts, gi));
    }
  }
}

#define CMP_GRID 1024
__global__ __launch_bounds__(EV_THREADS) void k_compact_copy(DevState S, int n_cap, const int32_t* n_dev) {
  __shared__ uint32_t s_bm[CMP_BMW];
  __shared__ int32_t s_bpre[CMP_BMW];
  __shared__ int32_t s_pos[EV_MAXSLOT];        // the sort fallback (span above the bitmap)
  __shared__ int32_t s_slot[EV_MAXSLOT];
  __shared__ int32_t s_src[TKV_BS], s_spos[TKV_BS];
  __shared__ int s_tmp[48];
  __shared__ int s_lo, s_hi, s_cnt;
  const int tid = threadIdx.x;
  const int n = eff_count(n_cap, n_dev);
  const int32_t* pre = cmp_tasks(S);
  const int total = pre[3 * n];
  const int32_t* recs = scr_oprec(S.scratch);
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    // the (item, class) of task t: last k with pre[k] <= t (tasks exist only for planned items)
    int lo = 0, hi = 3 * n;
    while (hi - lo > 1) { const int mid = (lo + hi) >> 1; if (pre[mid] <= t) lo = mid; else hi = mid; }
    const int i = lo / 3, c = lo % 3, j = t - pre[lo];
    const int s = recs[8 * i];
    const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
    const int32_t* bt = S.btab + ((int64_t)s * 3 + c) * S.max_blocks;
    const int nold = q[Q_NBLK + c], m = cmp_counts(S, s)[3 + c];
    const int cnt = min(TKV_BS, m - TKV_BS * j);
    const int32_t* blkc = pick3(S.blk, c);
    const int32_t* slotc = pick3(S.slot, c);
    // position range of the class's retained tokens
    if (tid == 0) { s_lo = TKV_INF; s_hi = -1; s_cnt = 0; }
    __syncthreads();
    int my_lo = TKV_INF, my_hi = -1;
    for (int x = tid; x < nold * TKV_BS; x += EV_THREADS) {
      const int blk = bt[x / TKV_BS], tt = x % TKV_BS;
      if (!((blkc[(int64_t)blk * TKV_BLK_W] >> tt) & 1)) continue;
      const int p = slotc[((int64_t)blk * TKV_BS + tt) * 2];
      my_lo = min(my_lo, p); my_hi = max(my_hi, p);
    }
    if (my_hi >= 0) { atomicMin(&s_lo, my_lo); atomicMax(&s_hi, my_hi); }
    __syncthreads();
    const int P0 = s_lo, span = s_hi - s_lo + 1;
    if (span <= CMP_BMW * 32) {
      // rank by position: bitmap of the positions, prefix counts of its words
      const int nbw = (span + 31) >> 5;
      for (int w = tid; w < CMP_BMW; w += EV_THREADS) s_bm[w] = 0;
      __syncthreads();
      for (int x = tid; x < nold * TKV_BS; x += EV_THREADS) {
        const int blk = bt[x / TKV_BS], tt = x % TKV_BS;
        if (!((blkc[(int64_t)blk * TKV_BLK_W] >> tt) & 1)) continue;
        const int off = slotc[((int64_t)blk * TKV_BS + tt) * 2] - P0;
        atomicOr(&s_bm[off >> 5], 1u << (off & 31));
      }
      __syncthreads();
      {
        int pc[CMP_BMW / EV_THREADS], v[3] = {0, 0, 0}, ex[3], tot[3];
#pragma unroll
        for (int u = 0; u < CMP_BMW / EV_THREADS; u++) {
          const int w = tid * (CMP_BMW / EV_THREADS) + u;
          pc[u] = w < nbw ? __popc(s_bm[w]) : 0;
          v[0] += pc[u];
        }
        wg_scan3(v, ex, tot, s_tmp);
        int run = ex[0];
#pragma unroll
        for (int u = 0; u < CMP_BMW / EV_THREADS; u++) {
          s_bpre[tid * (CMP_BMW / EV_THREADS) + u] = run;
          run += pc[u];
        }
      }
      __syncthreads();
      for (int x = tid; x < nold * TKV_BS; x += EV_THREADS) {
        const int blk = bt[x / TKV_BS], tt = x % TKV_BS;
        if (!((blkc[(int64_t)blk * TKV_BLK_W] >> tt) & 1)) continue;
        const int p = slotc[((int64_t)blk * TKV_BS + tt) * 2], off = p - P0;
        const int rk = s_bpre[off >> 5] + __popc(s_bm[off >> 5] & ((1u << (off & 31)) - 1u)) - TKV_BS * j;
        if (rk >= 0 && rk < cnt) { s_src[rk] = blk * TKV_BS + tt; s_spos[rk] = p; }
      }
    } else {
      // a span above the bitmap: gather and sort
      for (int x = tid; x < nold * TKV_BS; x += EV_THREADS) {
        const int blk = bt[x / TKV_BS], tt = x % TKV_BS;
        if (!((blkc[(int64_t)blk * TKV_BLK_W] >> tt) & 1)) continue;
        const int at = atomicAdd(&s_cnt, 1);
        s_pos[at] = slotc[((int64_t)blk * TKV_BS + tt) * 2];
        s_slot[at] = blk * TKV_BS + tt;
      }
      __syncthreads();
      lds_sort_pairs(s_pos, s_slot, min(s_cnt, EV_MAXSLOT), tid, EV_THREADS);
      if (tid < cnt) { s_src[tid] = s_slot[TKV_BS * j + tid]; s_spos[tid] = s_pos[TKV_BS * j + tid]; }
    }
    __syncthreads();
    const int newb = pick3(S.freestk, c)[recs[8 * i + 1 + c] - j];
    if (c == 0) compact_copy_block<8>(S, c, newb, cnt, s_src, tid);
    else if (c == 1) compact_copy_block<4>(S, c, newb, cnt, s_src, tid);
    else compact_copy_block<2>(S, c, newb, cnt, s_src, tid);
    // the new slots' records and the new block's record
    int32_t* slotw = pick3(S.slot, c);
    if (tid < cnt) {
      slotw[((int64_t)newb * TKV_BS + tid) * 2] = s_spos[tid];
      slotw[((int64_t)newb * TKV_BS + tid) * 2 + 1] = slotc[(int64_t)s_src[tid] * 2 + 1];
    }
    if (tid == 0) {
      int32_t* r = pick3(S.blk, c) + (int64_t)newb * TKV_BLK_W;
      r[0] = (int)((1u << cnt) - 1u);
      r[1] = s_spos[cnt - 1];
      r[2] = s;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(WG) void k_compact_push(DevState S, int n_cap, const int32_t* n_dev) {
  const int tid = threadIdx.x, NT = blockDim.x;
  const int n = eff_count(n_cap, n_dev);
  const int32_t* recs = scr_oprec(S.scratch);
  // 1. save the old block lists
  for (int i = 0; i < n; i++) {
    const int s = recs[8 * i];
    if (s < 0) continue;
    const int32_t* cn = cmp_counts(S, s);
    for (int c = 0; c < 3; c++) {
      const int32_t* bt = S.btab + ((int64_t)s * 3 + c) * S.max_blocks;
      int32_t* oldl = cmp_old(S, s, c);
      for (int j = tid; j < cn[c]; j += NT) oldl[j] = bt[j];
    }
  }
  __syncthreads();
  // 2. the new block lists (popped entries, read before the pushes overwrite
  //    them) and slot stacks of the classes that held blocks
  for (int i = 0; i < n; i++) {
    const int s = recs[8 * i];
    if (s < 0) continue;
    const int32_t* cn = cmp_counts(S, s);
    int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
    for (int c = 0; c < 3; c++) {
      if (cn[c] == 0) continue;
      const int m = cn[3 + c], need = (m + TKV_BS - 1) / TKV_BS;
      const int used = m % TKV_BS, tail = used ? TKV_BS - used : 0;
      int32_t* bt = S.btab + ((int64_t)s * 3 + c) * S.max_blocks;
      const int32_t* fs = pick3(S.freestk, c);
      for (int j = tid; j < need; j += NT) bt[j] = fs[recs[8 * i + 1 + c] - j];
      if (tail) {
        const int last = fs[recs[8 * i + 1 + c] - (need - 1)];
        int32_t* st = S.sstk + ((int64_t)s * 3 + c) * S.max_blocks * TKV_BS;
        for (int k = tid; k < tail; k += NT) st[k] = last * TKV_BS + (TKV_BS - 1 - k);
      }
      if (tid == 0) { q[Q_NBLK + c] = need; q[Q_NSLOT + c] = tail; }
    }
  }
  __syncthreads();
  // 3. the old blocks back onto the global stacks, records cleared
  for (int i = 0; i < n; i++) {
    const int s = recs[8 * i];
    if (s < 0) continue;
    const int32_t* cn = cmp_counts(S, s);
    for (int c = 0; c < 3; c++) {
      const int32_t* oldl = cmp_old(S, s, c);
      for (int j = tid; j < cn[c]; j += NT) {
        const int b = oldl[j];
        int32_t* r = pick3(S.blk, c) + (int64_t)b * TKV_BLK_W;
        r[0] = 0; r[1] = -1; r[2] = -1;
        pick3(S.freestk, c)[recs[8 * i + 4 + c] + j] = b;
      }
    }
  }
  if (tid < 3) S.hdr[H_FREE + tid] = scr_misc(S.scratch)[8 + tid];
}

int launch_compact(tkv_cache* c, int n, const int32_t* n_dev, const int32_t* seq_ids, hipStream_t st) {
  if (n == 0) return TKV_OK;
  TKV_TIMED(c, st, "k_compact_plan", k_compact_plan<<<1, WG, 0, st>>>(c->S, n, n_dev, seq_ids));
  TKV_TIMED(c, st, "k_compact_copy", k_compact_copy<<<CMP_GRID, EV_THREADS, 0, st>>>(c->S, n, n_dev));
  TKV_TIMED(c, st, "k_compact_push", k_compact_push<<<1, WG, 0, st>>>(c->S, n, n_dev));
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
        int32_t* br = pick3(S.blk, c) + (int64_t)blk * TKV_BLK_W;
        br[0] = 0; br[1] = -1; br[2] = -1;
        pick3(S.freestk, c)[base_cnt[c] + ex[c]++] = blk;
      }
    }
    for (int w = 0; w < TKV_SEQ_W; w++) q[w] = 0;
  }
  __syncthreads();
  if (tid < 3) S.hdr[H_FREE + tid] = base_cnt[tid] + tot[tid];
}

int launch_seq_reset(tkv_cache* c, int n, const int32_t* seq_ids, hipStream_t st) {
  if (n == 0) return TKV_OK;
  TKV_TIMED(c, st, "k_seq_reset", k_seq_reset<<<1, WG, 0, st>>>(c->S, n, seq_ids));
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// thought_classify: one wave per batch entry; lane l reads the statistic of
// heads l, l + 64, ... (up to 16 such chunks read together), and the sum runs
// over the heads in head order (fp32, sequential), then the thresholds.
// ---------------------------------------------------------------------------
#define CL_NB 16
__global__ __launch_bounds__(256) void k_classify(int batch, int Hq, const float* stats, float tT, float tE, int kind,
                                                  uint8_t* labels) {
#pragma clang fp contract(off)
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= batch) return;
  float sum = 0.0f;
  for (int c0 = 0; c0 < Hq; c0 += 64 * CL_NB) {
    // (every lane reads, a head inside the row, so that no read waits under a branch)
    float v[CL_NB];
#pragma unroll
    for (int i = 0; i < CL_NB; i++) {
      const int h = c0 + 64 * i + lane;
      v[i] = stats[((int64_t)b * Hq + (h < Hq ? h : Hq - 1)) * 3 + (kind == 0 ? 1 : 2)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < CL_NB; i++) v[i] = kind == 0 ? v[i] : 1.0f - v[i];
    // the terms in head order: whole 64-head chunks by v_readlane with a
    // constant lane (no LDS round trip, no lane index in a register), then the
    // partial chunk, if any
    const int nfull = (Hq - c0) / 64 < CL_NB ? (Hq - c0) / 64 : CL_NB;
#pragma unroll
    for (int i = 0; i < CL_NB; i++) {
      if (i < nfull) {
        // eight lanes read out, then their eight terms added (the reads into
        // distinct scalar registers need no wait between read and add)
#pragma unroll
        for (int j0 = 0; j0 < 64; j0 += 8) {
          int t[8];
#pragma unroll
          for (int e = 0; e < 8; e++) t[e] = __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[i]), j0 + e);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int e = 0; e < 8; e++) sum = sum + __builtin_bit_cast(float, t[e]);
        }
      }
    }
    const int rem = Hq - c0 - 64 * nfull;
    if (nfull < CL_NB && rem > 0) {
      float vp = v[0];
#pragma unroll
      for (int i = 1; i < CL_NB; i++) vp = i == nfull ? v[i] : vp;
      for (int j = 0; j < rem; j++)
        sum = sum + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vp), j));
    }
  }
  const float score = sum / (float)Hq;
  if (lane == 0) labels[b] = (uint8_t)thought_label(score, tT, tE);
}

int launch_classify(int batch, int Hq, const float* stats, float tau_T, float tau_E, int kind, uint8_t* labels,
                    hipStream_t st) {
  if (batch == 0) return TKV_OK;
  k_classify<<<(batch + 3) / 4, 256, 0, st>>>(batch, Hq, stats, tau_T, tau_E, kind, labels);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}
