// Host side of libthinkv: argument checks, buffer sizing, handle life cycle,
// state export / import, the sticky error word, and the C-ABI entry points
// declared in tkv.h.  Every entry point validates what the host can check and
// only then enqueues kernels; nothing here allocates device memory.
#include <stdlib.h>
#include <string.h>
#include <new>
#include <string>
#include <vector>
#include "tkv_internal.h"

// ---------------------------------------------------------------------------
// Per-kernel timing (tkv_kernel_timing / tkv_kernel_times).  Events come from
// a pool and go back to it when their durations are read; at most
// kMaxPending launches are recorded between two reads (later ones are
// counted as dropped).
// ---------------------------------------------------------------------------
struct KernelTimes {
  struct Rec { const char* name; hipEvent_t e0, e1; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  std::vector<std::string> names;        // first-seen order
  std::vector<double> total_us;
  std::vector<int32_t> calls;
  int64_t dropped = 0;
  int failed = 0;
  static const size_t kMaxPending = 1 << 16;
  hipEvent_t take() {
    hipEvent_t e = nullptr;
    if (!pool.empty()) { e = pool.back(); pool.pop_back(); return e; }
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) { failed = 1; return nullptr; }
    return e;
  }
  void give(hipEvent_t e) { if (e) pool.push_back(e); }
  void add(const char* name, double us) {
    size_t i = 0;
    while (i < names.size() && names[i] != name) i++;
    if (i == names.size()) { names.push_back(name); total_us.push_back(0.0); calls.push_back(0); }
    total_us[i] += us;
    calls[i] += 1;
  }
  ~KernelTimes() {
    for (auto& r : pending) { if (r.e0) hipEventDestroy(r.e0); if (r.e1) hipEventDestroy(r.e1); }
    for (auto e : pool) hipEventDestroy(e);
  }
};

KernelScope::KernelScope(const tkv_cache* c, hipStream_t stream, const char* name)
    : kt(c ? c->kt : nullptr), slot(-1), st(stream) {
  if (!kt) return;
  if (kt->pending.size() >= KernelTimes::kMaxPending) { kt->dropped++; kt = nullptr; return; }
  hipEvent_t a = kt->take(), b = kt->take();
  if (!a || !b || hipEventRecord(a, st) != hipSuccess) { kt->give(a); kt->give(b); kt->failed = 1; kt = nullptr; return; }
  kt->pending.push_back({name, a, b});
  slot = (int)kt->pending.size() - 1;
}
KernelScope::~KernelScope() {
  if (kt && slot >= 0 && hipEventRecord(kt->pending[slot].e1, st) != hipSuccess) kt->failed = 1;
}

static int layout_ok(const tkv_layout* L) {
  if (!L) return 0;
  if (L->num_kv_heads < 1 || L->num_q_heads < L->num_kv_heads || L->num_q_heads % L->num_kv_heads) return 0;
  if (L->num_q_heads / L->num_kv_heads > 16) return 0;
  if (L->head_dim != 64 && L->head_dim != 128) return 0;
  if (L->group_size != 32 && L->group_size != 64) return 0;
  if (L->group_size > L->head_dim) return 0;
  for (int t = 0; t < 3; t++) {
    if (class_of_bits(L->bits[t]) < 0) return 0;
    if (L->pool_blocks[t] < 1 || L->pool_blocks[t] > TKV_MAX_POOL_BLOCKS) return 0;
  }
  if (L->max_seqs < 1 || L->max_seqs > TKV_MAX_SEQS) return 0;
  if (L->max_blocks_per_seq < 1 || L->max_blocks_per_seq > TKV_MAX_BLOCKS) return 0;
  if (L->max_segments_per_seq < 1) return 0;
  if (L->max_tokens_per_call < 1 || L->max_tokens_per_call > TKV_MAX_TOK) return 0;
  if (L->num_layers < 0 || L->num_layers > 64) return 0;
  if (L->code_format != 0 && L->code_format != 1) return 0;
  return 1;
}

static int64_t bh_bytes(const tkv_layout* L, int c) {
  return 4LL * L->head_dim * class_bits(c) + 128LL * (L->head_dim / L->group_size);
}

extern "C" int tkv_buffer_sizes(const tkv_layout* L, size_t sizes[TKV_NUM_BUFFERS]) {
  if (!layout_ok(L) || !sizes) return TKV_EINVAL;
  for (int c = 0; c < 3; c++) {
    const size_t P = (size_t)L->pool_blocks[c];
    sizes[TKV_BUF_POOL0 + c] = P * (size_t)(L->num_layers > 1 ? L->num_layers : 1) * L->num_kv_heads *
                               (size_t)bh_bytes(L, c);
    sizes[TKV_BUF_BLK0 + c] = P * TKV_BLK_W * 4;
    sizes[TKV_BUF_SLOT0 + c] = P * TKV_BS * TKV_SLOT_W * 4;
    sizes[TKV_BUF_FREE0 + c] = P * 4;
  }
  sizes[TKV_BUF_HDR] = 16 * 4;
  sizes[TKV_BUF_SEQ] = (size_t)L->max_seqs * TKV_SEQ_W * 4;
  sizes[TKV_BUF_BTAB] = (size_t)L->max_seqs * 3 * L->max_blocks_per_seq * 4;
  sizes[TKV_BUF_SSTK] = (size_t)L->max_seqs * 3 * L->max_blocks_per_seq * TKV_BS * 4;
  sizes[TKV_BUF_SEGT] = (size_t)L->max_seqs * L->max_segments_per_seq * TKV_SEG_W * 4;
  sizes[TKV_BUF_SCRATCH] = ((size_t)TKV_SCR_FIXED + (size_t)L->max_seqs +
                            (size_t)L->max_seqs * L->max_blocks_per_seq * TKV_BS * 2) * 4;
  return TKV_OK;
}

extern "C" int tkv_create(const tkv_layout* L, void* const bufs[TKV_NUM_BUFFERS], const int32_t* const order[3],
                          hipStream_t stream, tkv_cache** out) {
  if (!out) return TKV_EINVAL;
  *out = nullptr;
  size_t sizes[TKV_NUM_BUFFERS];
  if (tkv_buffer_sizes(L, sizes) != TKV_OK || !bufs) return TKV_EINVAL;
  for (int i = 0; i < TKV_NUM_BUFFERS; i++)
    if (!bufs[i]) return TKV_EINVAL;
  // the initial pop order must be a permutation of each pool
  std::vector<int32_t> stacks[3];
  for (int c = 0; c < 3; c++) {
    const int P = L->pool_blocks[c];
    stacks[c].resize(P);
    if (order && order[c]) {
      std::vector<char> seen(P, 0);
      for (int i = 0; i < P; i++) {
        int b = order[c][i];
        if (b < 0 || b >= P || seen[b]) return TKV_EINVAL;
        seen[b] = 1;
        stacks[c][P - 1 - i] = b;
      }
    } else {
      for (int i = 0; i < P; i++) stacks[c][P - 1 - i] = i;
    }
  }
  tkv_cache* c = (tkv_cache*)calloc(1, sizeof(tkv_cache));
  if (!c) return TKV_EINVAL;
  c->L = *L;
  for (int i = 0; i < TKV_NUM_BUFFERS; i++) { c->buf[i] = bufs[i]; c->size[i] = sizes[i]; }
  DevState& S = c->S;
  for (int k = 0; k < 3; k++) {
    S.pool[k] = (uint8_t*)bufs[TKV_BUF_POOL0 + k];
    S.blk[k] = (int32_t*)bufs[TKV_BUF_BLK0 + k];
    S.slot[k] = (int32_t*)bufs[TKV_BUF_SLOT0 + k];
    S.freestk[k] = (int32_t*)bufs[TKV_BUF_FREE0 + k];
    S.pool_blocks[k] = L->pool_blocks[k];
    S.type_class[k] = class_of_bits(L->bits[k]);
    S.bh_bytes[k] = bh_bytes(L, k);
    S.chunk_bytes[k] = L->head_dim * class_bits(k) / 32;
  }
  S.hdr = (int32_t*)bufs[TKV_BUF_HDR];
  S.seq = (int32_t*)bufs[TKV_BUF_SEQ];
  S.btab = (int32_t*)bufs[TKV_BUF_BTAB];
  S.sstk = (int32_t*)bufs[TKV_BUF_SSTK];
  S.segt = (int32_t*)bufs[TKV_BUF_SEGT];
  S.scratch = (int32_t*)bufs[TKV_BUF_SCRATCH];
  S.Hkv = L->num_kv_heads; S.Hq = L->num_q_heads; S.D = L->head_dim; S.g = L->group_size;
  S.NG = L->head_dim / L->group_size;
  S.NL = L->num_layers > 1 ? L->num_layers : 1;
  S.Hst = S.NL * S.Hkv;
  S.fmt = L->code_format;
  S.max_seqs = L->max_seqs; S.max_blocks = L->max_blocks_per_seq; S.max_segs = L->max_segments_per_seq;
  S.max_tokens = L->max_tokens_per_call;
  c->last_stream = stream;
  int r = hipGetDevice(&c->device) == hipSuccess ? static_workspace_setup(c->device) : TKV_EHIP;
  if (r == TKV_OK) r = launch_init(c, stream);
  for (int k = 0; r == TKV_OK && k < 3; k++)
    if (hipMemcpyAsync(S.freestk[k], stacks[k].data(), sizes[TKV_BUF_FREE0 + k], hipMemcpyHostToDevice, stream) !=
        hipSuccess)
      r = TKV_EHIP;
  if (r == TKV_OK && hipStreamSynchronize(stream) != hipSuccess) r = TKV_EHIP;
  if (r != TKV_OK) { free(c); return r; }
  *out = c;
  return TKV_OK;
}

extern "C" int tkv_destroy(tkv_cache* c) {
  if (!c) return TKV_EINVAL;
  delete c->kt;
  free(c);
  return TKV_OK;
}

extern "C" int tkv_kernel_timing(tkv_cache* c, int32_t enable) {
  if (!c) return TKV_EINVAL;
  delete c->kt;       // (waits for nothing: recorded events are destroyed with it)
  c->kt = nullptr;
  if (enable) {
    c->kt = new (std::nothrow) KernelTimes();
    if (!c->kt) return TKV_EHIP;
  }
  return TKV_OK;
}

extern "C" int tkv_kernel_times(tkv_cache* c, int32_t max_kernels, char* names, double* total_us, int32_t* calls,
                                int64_t* dropped) {
  if (!c || max_kernels < 0 || (max_kernels > 0 && (!names || !total_us || !calls))) return TKV_EINVAL;
  KernelTimes* kt = c->kt;
  if (!kt) return TKV_EINVAL;
  int r = TKV_OK;
  for (auto& rec : kt->pending) {
    float ms = 0.f;
    if (r == TKV_OK &&
        (hipEventSynchronize(rec.e1) != hipSuccess || hipEventElapsedTime(&ms, rec.e0, rec.e1) != hipSuccess))
      r = TKV_EHIP;
    if (r == TKV_OK) kt->add(rec.name, 1000.0 * ms);
    kt->give(rec.e0);
    kt->give(rec.e1);
  }
  kt->pending.clear();
  if (r != TKV_OK || kt->failed) return TKV_EHIP;
  const int n = (int)kt->names.size();
  for (int i = 0; i < n && i < max_kernels; i++) {
    strncpy(names + 32 * i, kt->names[i].c_str(), 31);
    names[32 * i + 31] = 0;
    total_us[i] = kt->total_us[i];
    calls[i] = kt->calls[i];
  }
  if (dropped) *dropped = kt->dropped;
  return n;
}

extern "C" int tkv_seq_reset(tkv_cache* c, int32_t n, const int32_t* seq_ids, hipStream_t stream) {
  if (!c || n < 0 || n > c->S.max_seqs || (n > 0 && !seq_ids)) return TKV_EINVAL;
  c->last_stream = stream;
  return launch_seq_reset(c, n, seq_ids, stream);
}

extern "C" int kv_append_quant(tkv_cache* c, int32_t n, const int32_t* seq_ids, const int32_t* positions,
                               const uint8_t* thought, const float* k, const float* v, int32_t* slot_out,
                               hipStream_t stream) {
  if (!c || n < 0 || n > c->S.max_tokens) return TKV_EINVAL;
  if (n > 0 && (!seq_ids || !positions || !thought || !k || !v)) return TKV_EINVAL;
  c->last_stream = stream;
  return launch_append(c, n, seq_ids, positions, thought, k, v, slot_out, stream);
}

// rows of at most this many heads are classified inside the allocation kernel
static const int kFusedClassifyHeads = 128;

extern "C" int kv_classify_append(tkv_cache* c, int32_t n, const int32_t* seq_ids, const int32_t* positions,
                                  const float* stats, int32_t num_q_heads, float tau_T, float tau_E,
                                  int32_t score_kind, uint8_t* labels_out, const float* k, const float* v,
                                  int32_t* slot_out, hipStream_t stream) {
  if (!c || n < 0 || n > c->S.max_tokens) return TKV_EINVAL;
  if (num_q_heads < 1 || (score_kind != 0 && score_kind != 1)) return TKV_EINVAL;
  if (n > 0 && (!seq_ids || !positions || !stats || !k || !v)) return TKV_EINVAL;
  c->last_stream = stream;
  if (num_q_heads > kFusedClassifyHeads && n > 0) {
    // many heads per row (several layers' statistics): a wave per row reads
    // the row in parallel, then the allocation takes the labels; the labels go
    // to an unused scratch region when the caller wants none
    uint8_t* lab = labels_out ? labels_out : (uint8_t*)scr_status(c->S.scratch);
    int r;
    TKV_TIMED(c, stream, "k_classify",
              r = launch_classify(n, num_q_heads, stats, tau_T, tau_E, score_kind, lab, stream));
    if (r != TKV_OK) return r;
    return launch_append(c, n, seq_ids, positions, lab, k, v, slot_out, stream);
  }
  const ClassifyIn cl = {stats, num_q_heads, score_kind, tau_T, tau_E, labels_out};
  return launch_append(c, n, seq_ids, positions, nullptr, k, v, slot_out, stream, &cl);
}

extern "C" int kv_evict_segment(tkv_cache* c, int32_t n_ops, const int32_t* n_ops_dev, const int32_t* seq_ids,
                                const int32_t* segment_ids, const int32_t* keep_n, const uint8_t* new_bits,
                                hipStream_t stream) {
  if (!c || n_ops < 0 || n_ops > c->S.max_tokens) return TKV_EINVAL;
  if (n_ops > 0 && (!seq_ids || !segment_ids || !keep_n || !new_bits)) return TKV_EINVAL;
  c->last_stream = stream;
  return launch_evict(c, n_ops, n_ops_dev, seq_ids, segment_ids, keep_n, new_bits, stream);
}

extern "C" int kv_plan_budget(tkv_cache* c, int32_t n, const int32_t* seq_ids, int32_t num, int32_t den,
                              int32_t max_ops, int32_t* n_ops_dev, int32_t* op_seq, int32_t* op_seg, int32_t* op_keep,
                              uint8_t* op_bits, hipStream_t stream) {
  if (!c || n < 0 || n > c->S.max_tokens || num < 0 || den <= 0 || max_ops < 0 || max_ops > c->S.max_tokens)
    return TKV_EINVAL;
  if (!n_ops_dev || (n > 0 && !seq_ids) || (max_ops > 0 && (!op_seq || !op_seg || !op_keep || !op_bits)))
    return TKV_EINVAL;
  c->last_stream = stream;
  return launch_plan(c, n, seq_ids, num, den, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits, stream);
}

extern "C" int kv_plan_budget_evict(tkv_cache* c, int32_t n, const int32_t* seq_ids, int32_t num, int32_t den,
                                    int32_t max_ops, int32_t* n_ops_dev, int32_t* op_seq, int32_t* op_seg,
                                    int32_t* op_keep, uint8_t* op_bits, hipStream_t stream) {
  if (!c || n < 0 || n > c->S.max_tokens || num < 0 || den <= 0 || max_ops < 0 || max_ops > c->S.max_tokens)
    return TKV_EINVAL;
  if (!n_ops_dev || (n > 0 && !seq_ids) || (max_ops > 0 && (!op_seq || !op_seg || !op_keep || !op_bits)))
    return TKV_EINVAL;
  c->last_stream = stream;
  return launch_plan_evict(c, n, seq_ids, num, den, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits, stream);
}

extern "C" int kv_plan_anneal(tkv_cache* c, int32_t n, const int32_t* seq_ids, int32_t r0, int32_t max_ops,
                              int32_t* n_ops_dev, int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits,
                              hipStream_t stream) {
  if (!c || n < 0 || n > c->S.max_tokens || r0 < 0 || max_ops < 0 || max_ops > c->S.max_tokens) return TKV_EINVAL;
  if (!n_ops_dev || (n > 0 && !seq_ids) || (max_ops > 0 && (!op_seq || !op_seg || !op_keep || !op_bits)))
    return TKV_EINVAL;
  c->last_stream = stream;
  return launch_anneal(c, n, seq_ids, r0, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits, stream);
}

extern "C" int kv_plan_anneal_evict(tkv_cache* c, int32_t n, const int32_t* seq_ids, int32_t r0, int32_t max_ops,
                                    int32_t* n_ops_dev, int32_t* op_seq, int32_t* op_seg, int32_t* op_keep,
                                    uint8_t* op_bits, hipStream_t stream) {
  if (!c || n < 0 || n > c->S.max_tokens || r0 < 0 || max_ops < 0 || max_ops > c->S.max_tokens) return TKV_EINVAL;
  if (!n_ops_dev || (n > 0 && !seq_ids) || (max_ops > 0 && (!op_seq || !op_seg || !op_keep || !op_bits)))
    return TKV_EINVAL;
  c->last_stream = stream;
  return launch_anneal_evict(c, n, seq_ids, r0, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits, stream);
}

extern "C" int tkv_compact(tkv_cache* c, int32_t n, const int32_t* n_dev, const int32_t* seq_ids, hipStream_t stream) {
  if (!c || n < 0 || n > c->S.max_tokens || (n > 0 && !seq_ids)) return TKV_EINVAL;
  c->last_stream = stream;
  return launch_compact(c, n, n_dev, seq_ids, stream);
}

extern "C" size_t tkv_attn_workspace(const tkv_cache* c, int32_t batch, int32_t num_splits) {
  if (!c || batch < 0) return 0;
  int nw, s;
  attn_plan(c, batch, num_splits, false, &nw, &s);
  return attn_workspace_bytes(c, batch, s);
}

static int attn_args_ok(const tkv_cache* c, const tkv_attn_args* a) {
  if (!c || !a) return 0;
  if (a->batch < 0 || a->batch > c->S.max_seqs) return 0;
  if (a->topk < 1 || a->topk > 8 || a->window < 0 || a->num_splits < 0 || a->num_splits > 64) return 0;
  if (a->layer < 0 || a->layer >= c->S.NL) return 0;
  if (a->stats_stride != 0 && a->stats_stride < c->S.Hq * 3) return 0;
  if (a->batch > 0 && (!a->seq_ids || !a->q_pos || !a->q || !a->out)) return 0;
  if ((a->k_self == nullptr) != (a->v_self == nullptr)) return 0;
  // the kernels move q, the self token, the outputs and the partial records in 16-byte units
  const auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!al16(a->q) || !al16(a->out) || !al16(a->k_self) || !al16(a->v_self) || !al16(a->workspace)) return 0;
  return 1;
}

extern "C" int tkv_attn_order(tkv_cache* c, int32_t batch, const int32_t* seq_ids, int32_t* order,
                              hipStream_t stream) {
  if (!c || batch < 0 || batch > c->S.max_seqs || (batch > 0 && (!seq_ids || !order))) return TKV_EINVAL;
  if (batch == 0) return TKV_OK;
  c->last_stream = stream;
  return launch_attn_order(c, batch, seq_ids, order, stream);
}

extern "C" int paged_decode_attn_noalloc(tkv_cache* c, const tkv_attn_args* a, hipStream_t stream) {
  if (!attn_args_ok(c, a)) return TKV_EINVAL;
  int nw, s;
  attn_plan(c, a->batch, a->num_splits, a->order != nullptr, &nw, &s);
  if (attn_workspace_bytes(c, a->batch, s) > (size_t)TKV_STATIC_WORKSPACE_BYTES) return TKV_ERANGE;
  void* ws = static_workspace(c->device);
  if (!ws) return TKV_EHIP;
  c->last_stream = stream;
  return launch_attention(c, a, nw, s, stream, ws);
}

extern "C" int paged_decode_attn(tkv_cache* c, const tkv_attn_args* a, hipStream_t stream) {
  if (!attn_args_ok(c, a)) return TKV_EINVAL;
  int nw, s;
  attn_plan(c, a->batch, a->num_splits, a->order != nullptr, &nw, &s);
  const size_t need = attn_workspace_bytes(c, a->batch, s);
  if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return TKV_EINVAL;
  c->last_stream = stream;
  return launch_attention(c, a, nw, s, stream);
}

extern "C" int thought_classify(int32_t batch, int32_t num_q_heads, const float* stats, float tau_T, float tau_E,
                                int32_t score_kind, uint8_t* labels_out, hipStream_t stream) {
  if (batch < 0 || num_q_heads < 1 || (score_kind != 0 && score_kind != 1)) return TKV_EINVAL;
  if (batch > 0 && (!stats || !labels_out)) return TKV_EINVAL;
  return launch_classify(batch, num_q_heads, stats, tau_T, tau_E, score_kind, labels_out, stream);
}

extern "C" int tkv_get_error(tkv_cache* c, int32_t* kinds, int32_t* min_seq, int32_t* count) {
  if (!c) return TKV_EINVAL;
  if (hipStreamSynchronize(c->last_stream) != hipSuccess) return TKV_EHIP;
  int32_t h[16];
  if (hipMemcpy(h, c->S.hdr, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return TKV_EHIP;
  if (kinds) *kinds = h[H_EKIND];
  if (min_seq) *min_seq = h[H_EMINSEQ];
  if (count) *count = h[H_ECOUNT];
  h[H_EKIND] = 0; h[H_EMINSEQ] = TKV_INF; h[H_ECOUNT] = 0;
  if (hipMemcpy(c->S.hdr + H_EKIND, h + H_EKIND, 3 * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess)
    return TKV_EHIP;
  return TKV_OK;
}

extern "C" int tkv_export_state(tkv_cache* c, void* const host[TKV_NUM_BUFFERS]) {
  if (!c || !host) return TKV_EINVAL;
  if (hipStreamSynchronize(c->last_stream) != hipSuccess) return TKV_EHIP;
  for (int i = 0; i < TKV_BUF_SCRATCH; i++)
    if (host[i] && hipMemcpy(host[i], c->buf[i], c->size[i], hipMemcpyDeviceToHost) != hipSuccess) return TKV_EHIP;
  return TKV_OK;
}

extern "C" int tkv_import_state(tkv_cache* c, void* const host[TKV_NUM_BUFFERS]) {
  if (!c || !host) return TKV_EINVAL;
  if (hipStreamSynchronize(c->last_stream) != hipSuccess) return TKV_EHIP;
  for (int i = 0; i < TKV_BUF_SCRATCH; i++)
    if (host[i] && hipMemcpy(c->buf[i], host[i], c->size[i], hipMemcpyHostToDevice) != hipSuccess) return TKV_EHIP;
  if (hipDeviceSynchronize() != hipSuccess) return TKV_EHIP;
  return TKV_OK;
}

extern "C" const char* tkv_strerror(int status) {
  switch (status) {
    case TKV_OK: return "ok";
    case TKV_EINVAL: return "invalid argument";
    case TKV_ENOMEM: return "out of cache memory (pool, block list or segment table)";
    case TKV_ENOSEG: return "unknown or evicted segment";
    case TKV_EHIP: return "HIP runtime error";
    case TKV_ERANGE: return "request exceeds the library's static workspace";
    default: return "unknown status";
  }
}
