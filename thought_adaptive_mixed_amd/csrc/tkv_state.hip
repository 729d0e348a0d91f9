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
struct AppendWalk {
  // per-sequence running state
  int failed, fail_code, nblk[3], nslot[3], nseg, len, open_type, open_bits, nret, napp;
};

__device__ void append_walk(const DevState& S, int s, int n, const uint16_t* s_seq, const uint8_t* s_type,
                            uint8_t* s_need, const int32_t* pos, const int* dry_from, const int* avail,
                            const int32_t* idx, int32_t* info, int32_t* slot_out, bool commit) {
  int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
  AppendWalk w;
  w.failed = 0; w.fail_code = 0;
  for (int c = 0; c < 3; c++) { w.nblk[c] = q[Q_NBLK + c]; w.nslot[c] = q[Q_NSLOT + c]; }
  w.nseg = q[Q_NSEG]; w.len = q[Q_LEN]; w.nret = q[Q_NRET]; w.napp = q[Q_NAPP];
  w.open_type = -1; w.open_bits = -1;
  if (w.nseg > 0) {
    const int32_t* g = S.segt + ((int64_t)s * S.max_segs + w.nseg - 1) * TKV_SEG_W;
    w.open_type = g[G_TYPE]; w.open_bits = g[G_BITS];
  }
  int32_t* bt = S.btab + (int64_t)s * 3 * S.max_blocks;
  int32_t* st = S.sstk + (int64_t)s * 3 * S.max_blocks * TKV_BS;
  for (int i = 0; i < n; i++) {
    if (s_seq[i] != s) continue;
    if (!commit) s_need[i] = 0;
    if (w.failed) continue;
    int y = s_type[i];
    int p = pos[i];
    if (y > 2 || p < w.len) { w.failed = 1; w.fail_code = TKV_EINVAL; continue; }
    int c = S.type_class[y];
    int cb = class_bits(c);
    int new_seg = (w.nseg == 0) || (w.open_type != y) || (w.open_bits != cb);
    if (new_seg && w.nseg == S.max_segs) { w.failed = 1; w.fail_code = TKV_ENOMEM; continue; }
    int need = w.nslot[c] == 0;
    if (need) {
      if (w.nblk[c] == S.max_blocks || i >= dry_from[c]) { w.failed = 1; w.fail_code = TKV_ENOMEM; continue; }
    }
    if (!commit) {
      s_need[i] = (uint8_t)need;
      if (need) { w.nblk[c]++; w.nslot[c] += TKV_BS; }
      w.nslot[c]--;
      if (new_seg) { w.nseg++; w.open_type = y; w.open_bits = cb; }
      w.len = p + 1;
      continue;
    }
    // commit
    int32_t* btc = bt + c * S.max_blocks;
    int32_t* stc = st + (int64_t)c * S.max_blocks * TKV_BS;
    if (need && (idx[i] < 0 || idx[i] >= avail[c])) {   // cannot happen after the dry passes; keeps indexing in bounds
      w.failed = 1; w.fail_code = TKV_ENOMEM; continue;
    }
    if (need) {
      int blk = S.freestk[c][avail[c] - 1 - idx[i]];
      btc[w.nblk[c]++] = blk;
      S.blk[c][(int64_t)blk * TKV_BLK_W + 2] = s;
      for (int t = TKV_BS - 1; t >= 0; t--) stc[w.nslot[c]++] = blk * TKV_BS + t;
    }
    int slot = stc[--w.nslot[c]];
    if (new_seg) {
      int32_t* g = S.segt + ((int64_t)s * S.max_segs + w.nseg) * TKV_SEG_W;
      g[G_TYPE] = y; g[G_BITS] = cb; g[G_FIRST] = p; g[G_LAST] = p; g[G_NTOT] = 0; g[G_NRET] = 0;
      g[6] = 0; g[7] = 0;
      w.nseg++; w.open_type = y; w.open_bits = cb;
    }
    int32_t* g = S.segt + ((int64_t)s * S.max_segs + w.nseg - 1) * TKV_SEG_W;
    g[G_LAST] = p; g[G_NTOT] += 1; g[G_NRET] += 1;
    int blk = slot / TKV_BS, t = slot % TKV_BS;
    int32_t* br = S.blk[c] + (int64_t)blk * TKV_BLK_W;
    br[0] |= 1 << t;
    if (p > br[1]) br[1] = p;
    S.slot[c][(int64_t)slot * 2] = p;
    S.slot[c][(int64_t)slot * 2 + 1] = w.nseg - 1;
    w.len = p + 1; w.nret++; w.napp++;
    int code = (c << 28) | slot;
    info[i] = code;
    if (slot_out) slot_out[i] = code;
  }
  if (commit) {
    for (int c = 0; c < 3; c++) { q[Q_NBLK + c] = w.nblk[c]; q[Q_NSLOT + c] = w.nslot[c]; }
    q[Q_NSEG] = w.nseg; q[Q_LEN] = w.len; q[Q_NRET] = w.nret; q[Q_NAPP] = w.napp;
    if (w.failed) record_error(S.hdr, w.fail_code, s);
  }
}

__global__ __launch_bounds__(WG) void k_append_alloc(DevState S, int n, const int32_t* seq_ids, const int32_t* pos,
                                                     const uint8_t* thought, int32_t* slot_out) {
  __shared__ uint16_t s_seq[TKV_MAX_TOK];
  __shared__ uint8_t s_type[TKV_MAX_TOK];
  __shared__ uint8_t s_need[TKV_MAX_TOK];
  __shared__ int s_tmp[48];
  __shared__ int dry_from[3], avail[3], viol[3], total[3];
  const int tid = threadIdx.x;
  int32_t* idx = scr_idx(S.scratch);
  int32_t* info = scr_info(S.scratch);
  for (int i = tid; i < n; i += WG) {
    int s = seq_ids[i];
    info[i] = -1;
    if (slot_out) slot_out[i] = -1;
    if (s < 0 || s >= S.max_seqs) {
      s_seq[i] = 0xFFFF;
      record_error(S.hdr, TKV_EINVAL, s < 0 ? TKV_INF : s);
    } else {
      s_seq[i] = (uint16_t)s;
    }
    s_type[i] = thought[i];
    s_need[i] = 0;
  }
  if (tid < 3) { dry_from[tid] = TKV_INF; avail[tid] = S.hdr[H_FREE + tid]; }
  __syncthreads();
  const int per = (n + WG - 1) / WG;
  const int lo = tid * per, hi = min(n, lo + per);
  for (int iter = 0; iter < 4; iter++) {
    if (tid < S.max_seqs)
      append_walk(S, tid, n, s_seq, s_type, s_need, pos, dry_from, avail, idx, info, slot_out, false);
    __syncthreads();
    int v[3] = {0, 0, 0}, ex[3], tot[3];
    for (int i = lo; i < hi; i++)
      if (s_need[i]) v[S.type_class[s_type[i]]]++;
    wg_scan3(v, ex, tot, s_tmp);
    if (tid < 3) viol[tid] = TKV_INF;
    __syncthreads();
    for (int i = lo; i < hi; i++) {
      if (!s_need[i]) continue;
      int c = S.type_class[s_type[i]];
      idx[i] = ex[c]++;
      if (idx[i] >= avail[c]) atomicMin(&viol[c], i);
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
  if (tid < S.max_seqs)
    append_walk(S, tid, n, s_seq, s_type, s_need, pos, dry_from, avail, idx, info, slot_out, true);
  __syncthreads();
  if (tid < 3) S.hdr[H_FREE + tid] = avail[tid] - total[tid];
}

// ---------------------------------------------------------------------------
// Append, part 2: quantize and pack.  One thread per (token, KV head, tensor)
// row; K codes of a token fill whole words of its own chunks (plain stores);
// V codes of 4 tokens share bytes, so 4- and 2-bit V codes are merged with
// atomic AND/OR on their words.
// ---------------------------------------------------------------------------
template <class Get>
__device__ void store_row(const DevState& S, int c, int blk, int t, int h, int kv, Get get) {
  const int D = S.D, g = S.g, NG = S.NG, bits = class_bits(c);
  uint8_t* base = S.pool[c] + ((int64_t)blk * S.Hkv + h) * S.bh_bytes[c];
  uint8_t codes[128];
  for (int gi = 0; gi < NG; gi++) {
    float sf, zf; uint16_t sh, zh;
    auto gg = [&](int i) { return get(gi * g + i); };
    quant_scale_zero(gg, g, bits, sf, zf, sh, zh);
    for (int i = 0; i < g; i++) codes[gi * g + i] = (uint8_t)quant_code(get(gi * g + i), sf, zf, bits);
    *(uint32_t*)(base + meta_byte(D, g, bits, kv, t, gi)) = (uint32_t)sh | ((uint32_t)zh << 16);
  }
  const int W = 32 / bits;
  const int cw = D * bits / 32 / 4;            // words per chunk
  if (kv == 0) {
    // chunk 16*lg + t holds dims gi*g + lg*(g/4) + e' at element gi*(g/4) + e'
    const int q4 = g / 4;
    for (int lg = 0; lg < 4; lg++) {
      uint32_t* ch = (uint32_t*)(base + (16 * lg + t) * (D * bits / 32));
      for (int w = 0; w < cw; w++) {
        uint32_t word = 0;
        for (int f = 0; f < W; f++) {
          int e = w * W + f;
          int d = (e / q4) * g + lg * q4 + (e % q4);
          int p = (f >> 1) + (f & 1) * (W >> 1);
          word |= (uint32_t)codes[d] << (p * bits);
        }
        ch[w] = word;
      }
    }
  } else {
    // chunk 16*q + i, element 4n + r, for token t = 4q + r and dim d = 16n + i
    const int q = t >> 2, r = t & 3;
    uint8_t* vbase = base + 64 * (D * bits / 32);
    for (int i = 0; i < 16; i++) {
      uint8_t* ch = vbase + (16 * q + i) * (D * bits / 32);
      if (bits == 8) {
        for (int n = 0; n < D / 16; n++) {
          int e = 4 * n + r;
          int bit = elem_bit(e, 8);
          ch[bit >> 3] = codes[16 * n + i];
        }
      } else {
        for (int w = 0; w < cw; w++) {
          uint32_t mask = 0, val = 0;
          for (int f = 0; f < W; f++) {
            int e = w * W + f;
            if ((e & 3) != r) continue;
            int n = e >> 2;
            int p = (f >> 1) + (f & 1) * (W >> 1);
            mask |= ((1u << bits) - 1u) << (p * bits);
            val |= (uint32_t)codes[16 * n + i] << (p * bits);
          }
          uint32_t* wp = (uint32_t*)ch + w;
          atomicAnd(wp, ~mask);
          atomicOr(wp, val);
        }
      }
    }
  }
}

__global__ void k_append_store(DevState S, int n, const float* k, const float* v) {
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)n * S.Hkv * 2;
  if (gid >= total) return;
  int kv = (int)(gid & 1);
  int64_t th = gid >> 1;
  int h = (int)(th % S.Hkv);
  int i = (int)(th / S.Hkv);
  int info = scr_info(S.scratch)[i];
  if (info < 0) return;
  int c = info >> 28, slot = info & 0x0FFFFFFF;
  const float* row = (kv ? v : k) + ((int64_t)i * S.Hkv + h) * S.D;
  store_row(S, c, slot / TKV_BS, slot % TKV_BS, h, kv, [&](int d) { return row[d]; });
}

int launch_append(tkv_cache* c, int n, const int32_t* seq_ids, const int32_t* pos, const uint8_t* thought,
                  const float* k, const float* v, int32_t* slot_out, hipStream_t st) {
  if (n == 0) return TKV_OK;
  k_append_alloc<<<1, WG, 0, st>>>(c->S, n, seq_ids, pos, thought, slot_out);
  int64_t total = (int64_t)n * c->S.Hkv * 2;
  k_append_store<<<(int)((total + 255) / 256), 256, 0, st>>>(c->S, n, k, v);
  return hipGetLastError() == hipSuccess ? TKV_OK : TKV_EHIP;
}

// ---------------------------------------------------------------------------
// Evict, part 1: validation and reservation of fresh lower-class blocks for
// downgrades, in list order (same walk / scan / dry scheme as append).
// status[j]: 1 = apply, 0 = skipped or failed.  need[j] = fresh blocks,
// idx[j] = index of its first global pop.
// ---------------------------------------------------------------------------
__device__ void evict_walk(const DevState& S, int s, int n, const uint16_t* s_seq, const int32_t* seg_ids,
                           const int32_t* keep_n, const uint8_t* new_bits, uint8_t* s_cls, int32_t* need,
                           int32_t* status, const int* dry_from, bool final_pass) {
  const int32_t* q = S.seq + (int64_t)s * TKV_SEQ_W;
  int nslot[3], nblk[3];
  for (int c = 0; c < 3; c++) { nslot[c] = q[Q_NSLOT + c]; nblk[c] = q[Q_NBLK + c]; }
  int nseg = q[Q_NSEG];
  int failed = 0, code = 0;
  for (int j = 0; j < n; j++) {
    if (s_seq[j] != s) continue;
    need[j] = 0; status[j] = 0; s_cls[j] = 0;
    if (failed) continue;
    int k = seg_ids[j];
    if (k < 0 || k >= nseg) { failed = 1; code = TKV_ENOSEG; continue; }
    int dup = 0;
    for (int j2 = 0; j2 < j; j2++) if (s_seq[j2] == s && seg_ids[j2] == k) { dup = 1; break; }
    const int32_t* g = S.segt + ((int64_t)s * S.max_segs + k) * TKV_SEG_W;
    int nb = new_bits[j], gb = g[G_BITS];
    if (dup || keep_n[j] < 0 || !(nb == 0 || nb == 2 || nb == 4 || nb == 8) || (nb != 0 && nb > gb)) {
      failed = 1; code = TKV_EINVAL; continue;
    }
    int r = g[G_NRET];
    if (r == 0) { failed = 1; code = TKV_ENOSEG; continue; }
    int c = class_of_bits(gb);
    int keep = keep_n[j] < r ? keep_n[j] : r;
    int down = (nb != 0 && nb < gb && keep > 0);
    int c2 = down ? class_of_bits(nb) : c;
    int nd = 0;
    if (down) {
      int have = nslot[c2];
      nd = keep > have ? (keep - have + TKV_BS - 1) / TKV_BS : 0;
      if (nblk[c2] + nd > S.max_blocks) { failed = 1; code = TKV_ENOMEM; continue; }
      if (nd > 0 && j >= dry_from[c2]) { failed = 1; code = TKV_ENOMEM; continue; }
    }
    int ev = r - keep;
    nslot[c] += ev;
    if (down) {
      nblk[c2] += nd;
      nslot[c2] = nslot[c2] + TKV_BS * nd - keep;
      nslot[c] += keep;
    }
    need[j] = nd; status[j] = 1; s_cls[j] = (uint8_t)c2;
  }
  if (final_pass && failed) record_error(S.hdr, code, s);
}

__global__ __launch_bounds__(WG) void k_evict_plan(DevState S, int n_cap, const int32_t* n_dev, const int32_t* seq_ids,
                                                   const int32_t* seg_ids, const int32_t* keep_n,
                                                   const uint8_t* new_bits) {
  __shared__ uint16_t s_seq[TKV_MAX_TOK];
  __shared__ uint8_t s_cls[TKV_MAX_TOK];
  __shared__ int s_tmp[48];
  __shared__ int dry_from[3], avail[3], viol[3], total[3];
  const int tid = threadIdx.x;
  int n = n_cap;
  if (n_dev) { int m = *n_dev; n = m < n_cap ? (m < 0 ? 0 : m) : n_cap; }
  int32_t* idx = scr_idx(S.scratch);
  int32_t* status = scr_status(S.scratch);
  int32_t* need = scr_need(S.scratch);
  int32_t* misc = scr_misc(S.scratch);
  for (int j = tid; j < n; j += WG) {
    int s = seq_ids[j];
    status[j] = 0; need[j] = 0; idx[j] = 0;
    if (s < 0 || s >= S.max_seqs) { s_seq[j] = 0xFFFF; record_error(S.hdr, TKV_EINVAL, s < 0 ? TKV_INF : s); }
    else s_seq[j] = (uint16_t)s;
  }
  if (tid < 3) { dry_from[tid] = TKV_INF; avail[tid] = S.hdr[H_FREE + tid]; }
  if (tid == 0) misc[3] = n;
  __syncthreads();
  const int per = (n + WG - 1) / WG;
  const int lo = tid * per, hi = min(n, lo + per);
  for (int iter = 0; iter < 4; iter++) {
    if (tid < S.max_seqs)
      evict_walk(S, tid, n, s_seq, seg_ids, keep_n, new_bits, s_cls, need, status, dry_from, false);
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
    evict_walk(S, tid, n, s_seq, seg_ids, keep_n, new_bits, s_cls, need, status, dry_from, true);
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

__global__ __launch_bounds__(EV_THREADS) void k_evict_apply(DevState S, const int32_t* seq_ids, const int32_t* seg_ids,
                                                            const int32_t* keep_n, const uint8_t* new_bits) {
  __shared__ int32_t s_pos[EV_MAXSLOT];
  __shared__ int32_t s_slot[EV_MAXSLOT];
  __shared__ int32_t s_sorted[EV_MAXSLOT];
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
    for (int a = tid; a < m; a += EV_THREADS) {
      int pa = s_pos[a], rank = 0;
      for (int b = 0; b < m; b++) rank += s_pos[b] < pa;
      s_sorted[rank] = s_slot[a];
    }
    __syncthreads();
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
      for (int wi = tid; wi < keep * S.Hkv * 2; wi += EV_THREADS) {
        int kv = wi & 1, h = (wi >> 1) % S.Hkv, p = (wi >> 1) / S.Hkv;
        int old = s_sorted[ev + p];
        int ns;
        if (p < S0) ns = st2[S0 - 1 - p];
        else { int pp = p - S0; ns = bt[c2 * S.max_blocks + nbk2 + pp / TKV_BS] * TKV_BS + pp % TKV_BS; }
        int ob = old / TKV_BS, ot = old % TKV_BS;
        store_row(S, c2, ns / TKV_BS, ns % TKV_BS, h, kv,
                  [&](int d) { return deq_code(S, c, ob, ot, h, kv, d); });
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
}

int launch_evict(tkv_cache* c, int n_ops, const int32_t* n_ops_dev, const int32_t* seq_ids, const int32_t* seg_ids,
                 const int32_t* keep_n, const uint8_t* new_bits, hipStream_t st) {
  if (n_ops == 0) return TKV_OK;
  k_evict_plan<<<1, WG, 0, st>>>(c->S, n_ops, n_ops_dev, seq_ids, seg_ids, keep_n, new_bits);
  k_evict_apply<<<c->S.max_seqs, EV_THREADS, 0, st>>>(c->S, seq_ids, seg_ids, keep_n, new_bits);
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
