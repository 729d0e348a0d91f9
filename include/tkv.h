/*
 * tkv.h -- C ABI of libthinkv.so: the ThinKV decode hot path on MI355X (gfx950).
 *
 * The method (pages: "ThinKV: Thought-Adaptive KV Cache Compression for
 * Efficient Reasoning Models" -- the arXiv abstract, and the technical summary
 * section "Methodologie" with its TBQ, TBE and Continuous Thinking bullets):
 * a reasoning model's decode attention is read for its sparsity to label each
 * generated token a Reasoning (R), Execution (E) or Transition (T) thought;
 * tokens are group-quantized at a precision set by the label (R > E > T);
 * whole thought segments are evicted as the trajectory moves on; and evicted
 * slots are refilled in place by new tokens through a block table that keeps
 * thought type, start index and eviction mask, so the cache is never compacted.
 *
 * Conventions for every call below
 *   - Pointers are DEVICE pointers unless the name ends in _h (host memory).
 *   - Every call validates what the host can check, enqueues its kernels on
 *     `stream`, and returns without synchronizing, except tkv_create,
 *     tkv_get_error, tkv_export_state and tkv_import_state, which synchronize.
 *   - Return value: TKV_OK or a negative TKV_E* code.  A call that returns an
 *     error code enqueued nothing.
 *   - The caller allocates and owns every device buffer (sizes from
 *     tkv_buffer_sizes) and every stream.  The library never allocates or
 *     frees device memory; a tkv_cache handle holds raw pointers only.
 *   - A handle is used from one stream at a time; it is not thread-safe.
 *     Calls that overlap on different streams against the same handle race.
 *   - Errors found on the device (pool exhausted, segment table or block list
 *     full, unknown segment, bad per-item argument) do not abort the call:
 *     the failing item is skipped, its sequence's state is left as it was,
 *     later items of that sequence in the same call are skipped, other
 *     sequences proceed, and a sticky error word records the kinds seen, the
 *     lowest sequence id involved and a count (tkv_get_error).
 *   - Inputs must be finite with magnitude below 2^15 (K/V rows, queries,
 *     sinks); outside that range results are undefined.
 *
 * State format (the buffers, all little-endian):
 *   Three precision classes c = 0, 1, 2 hold 8-, 4- and 2-bit codes.  Each
 *   class has a pool of `pool_blocks[c]` blocks; a block holds 16 token slots
 *   of every layer and KV head (the L layers share block tables, segments and
 *   eviction: a token is stored, evicted, moved for all layers at once).  Slot
 *   id = block * 16 + slot-in-block.
 *   POOLc  u8  [pool_blocks[c]][L][Hkv][R_c] with R_c = 4*D*bits_c + 128*(D/g):
 *          per (block, layer, KV head): K codes (64 chunks of D*bits/32 bytes), V
 *          codes (64 chunks), K meta, V meta.  Meta = fp16 (scale, zero) per
 *          (token, group), token-major.  K code of token t, dim d: chunk
 *          16*lg + t, element gi*(g/4) + e' with gi = d/g, lg = (d%g)/(g/4),
 *          e' = d%(g/4).  V code of token t = 4q+r, dim d = 16n+i: chunk 16*q+i,
 *          element 4n+r.  Within a chunk, codes sit in 32-bit words of 32/bits
 *          codes; the low half-word holds the word's even elements and the high
 *          half-word its odd elements, least significant field first.
 *          With code_format 1 the 8- and 4-bit (float) codes sit in element
 *          order instead (element j of a word in bits j*bits..).
 *   Code formats (ThinKV technical summary, "Methodology", TBQ bullet: FP8
 *   or NVFP4 for Reasoning tokens, ternary for Transition tokens).  Per
 *   (token, group) of g dims with fp16 scale s and zero z:
 *     code_format 0, every class: asymmetric integer, s = (max-min)/(2^b-1),
 *          z = min, code = round-to-nearest-even((x - z)/s) clamped; x^ = s*code + z.
 *     code_format 1, class 0: FP8 E4M3 (bias 7, subnormals, no infinities),
 *          s = amax/448, z = 0, code = E4M3(x/s) rounded to nearest even and
 *          saturated at +-448; x^ = s*value(code).
 *     code_format 1, class 1: FP4 E2M1 (values 0, .5, 1, 1.5, 2, 3, 4, 6),
 *          s = amax/6, z = 0, nearest with ties to the even code, saturated;
 *          x^ = s*value(code).
 *     code_format 1, class 2: ternary by the rule of Ternary Weight Networks
 *          (Li, Zhang, Liu 2016): threshold 0.7*mean|x|, t = sign(x) beyond it
 *          else 0, s = mean |x| over the nonzero t (the sums pairwise over
 *          index halves); stored as the integer code t + 1 with z = -s, so
 *          x^ = s*code + z as for integer codes.
 *     A zero scale stores all-zero codes and zero; a -0 scale or zero is stored as +0.
 *   BLKc   i32 [pool_blocks[c]][4]   {valid mask (bit t = slot t), max position
 *          ever stored, owner sequence, 0}; a free block is {0, -1, -1, 0}.
 *   SLOTc  i32 [pool_blocks[c]*16][2] {position, segment id} (valid slots).
 *   FREEc  i32 [pool_blocks[c]]  global free-block stack, bottom first; its
 *          depth is HDR[c].
 *   HDR    i32 [16]  {free depth[3], error kinds (bit -code), lowest error
 *          sequence, error count, 0...}.
 *   SEQ    i32 [max_seqs][16] {blocks[3], stack depth[3], segments, length
 *          (last position + 1), retained tokens, appended tokens, 0...}.
 *   BTAB   i32 [max_seqs][3][max_blocks_per_seq]   block list per class.
 *   SSTK   i32 [max_seqs][3][max_blocks_per_seq*16] free-slot stack per class.
 *   SEGT   i32 [max_seqs][max_segments_per_seq][8] {type, bits, first position,
 *          last position, appended, retained, 0, 0}.
 *   SCRATCH     per-call scratch of the library (not state).
 */
#ifndef TKV_H
#define TKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tkv_cache tkv_cache;

enum { TKV_R = 0, TKV_E = 1, TKV_T = 2 };            /* thought types */

enum {
  TKV_OK = 0,
  TKV_EINVAL = -1,      /* bad argument                                      */
  TKV_ENOMEM = -2,      /* pool exhausted, block list or segment table full  */
  TKV_ENOSEG = -3,      /* unknown or fully evicted segment                  */
  TKV_EHIP = -4,        /* a HIP runtime call failed                         */
  TKV_ERANGE = -5       /* request larger than the static workspace          */
};

enum {
  TKV_BUF_POOL0 = 0, TKV_BUF_POOL1, TKV_BUF_POOL2,
  TKV_BUF_BLK0, TKV_BUF_BLK1, TKV_BUF_BLK2,
  TKV_BUF_SLOT0, TKV_BUF_SLOT1, TKV_BUF_SLOT2,
  TKV_BUF_FREE0, TKV_BUF_FREE1, TKV_BUF_FREE2,
  TKV_BUF_HDR, TKV_BUF_SEQ, TKV_BUF_BTAB, TKV_BUF_SSTK, TKV_BUF_SEGT,
  TKV_BUF_SCRATCH,
  TKV_NUM_BUFFERS
};

typedef struct {
  int32_t num_kv_heads;           /* Hkv >= 1                                  */
  int32_t num_q_heads;            /* Hq, a multiple of Hkv, Hq/Hkv <= 16       */
  int32_t head_dim;               /* D: 64 or 128                              */
  int32_t group_size;             /* g: 32 or 64, g <= D                       */
  int32_t bits[3];                /* bits for types R, E, T, each 8, 4 or 2    */
  int32_t pool_blocks[3];         /* blocks in the 8-, 4-, 2-bit pools (>= 1)  */
  int32_t max_seqs;               /* 1..1024                                   */
  int32_t max_blocks_per_seq;     /* per class, 1..256                         */
  int32_t max_segments_per_seq;   /* >= 1                                      */
  int32_t max_tokens_per_call;    /* bound on items per append/evict/plan call, 1..4096 */
  int32_t num_layers;             /* L: layers sharing the block tables, 1..64 (0 counts as 1) */
  int32_t code_format;            /* 0: asymmetric integer codes; 1: the class's float or ternary
                                     format (8-bit FP8 E4M3, 4-bit FP4 E2M1, 2-bit ternary) */
} tkv_layout;

/* Byte sizes of the TKV_NUM_BUFFERS buffers for layout L_h.  EINVAL for a
   layout outside the ranges above. */
int tkv_buffer_sizes(const tkv_layout* L_h, size_t sizes_h[TKV_NUM_BUFFERS]);

/* Bind the caller's buffers and write the empty state: zeroed pools, all
   blocks free, no sequences.  block_order_h[c] (nullable, or a NULL entry)
   lists pool c's blocks in the order they will be popped; NULL means
   0, 1, 2, ...  Synchronizes `stream`.  The handle is host memory owned by
   the library until tkv_destroy. */
int tkv_create(const tkv_layout* L_h, void* const bufs_h[TKV_NUM_BUFFERS],
               const int32_t* const block_order_h[3], hipStream_t stream, tkv_cache** out_h);

/* Free the handle (not the buffers). */
int tkv_destroy(tkv_cache* c);

/* Return every block of the listed sequences to the global stacks (list
   order, classes in order, blocks in block-list order) and clear their
   records.  seq_ids: i32[n]; repeated ids after the first are no-ops. */
int tkv_seq_reset(tkv_cache* c, int32_t n, const int32_t* seq_ids, hipStream_t stream);

/* kv_append_quant -- TBQ bullet (tokens buffered, then group-quantized by
 * their identified thought category) and Continuous Thinking bullet (a new
 * token overwrites an evicted slot of its precision class in place).
 *   seq_ids i32[n], positions i32[n] (strictly increasing per sequence, at
 *   least the sequence's length), thought u8[n] (TKV_R/E/T), k and v fp32
 *   [n][L][Hkv][D] rows (every layer's rows of the token).  Tokens are
 *   applied in list order: each pops its (sequence, class) free-slot stack,
 *   refilled with a fresh block from the class's global stack when empty;
 *   each (token, layer, head, tensor, group of g dims) is quantized to bits_c asymmetric codes with an fp16 scale
 *   (max-min)/(2^bits-1) and fp16 zero-point min, codes rounded half-even and
 *   clamped.  A token opens a new segment when its type differs from the open
 *   segment's (or that segment was downgraded).
 *   slot_out (nullable) i32[n]: (class << 28) | slot, or -1 if not stored.
 *   EINVAL: n < 0 or n > max_tokens_per_call, or a required pointer is NULL. */
int kv_append_quant(tkv_cache* c, int32_t n, const int32_t* seq_ids, const int32_t* positions,
                    const uint8_t* thought, const float* k, const float* v, int32_t* slot_out,
                    hipStream_t stream);

/* kv_classify_append -- thought decomposition bullets (the attention
 * sparsity of a decode step assigns the type of the token it produces) with
 * the TBQ bullet (that token is then quantized at its type's precision): the
 * same result as thought_classify(n, num_q_heads, stats, tau_T, tau_E,
 * score_kind, labels) followed by kv_append_quant(c, n, seq_ids, positions,
 * labels, k, v, slot_out), with the classification done inside the append's
 * allocation kernel (one launch fewer) when num_q_heads <= 128; longer rows
 * (several layers' statistics) are classified by the thought_classify kernel,
 * a wave per row reading the row in parallel, whose labels the allocation then
 * takes (labels_out, or a region of the cache's scratch memory when it is
 * NULL: two calls on one cache must not overlap).  Token i takes the label of row i of
 * stats fp32 [n][num_q_heads][3] (the attention batch in token order; with
 * several layers num_q_heads = L*Hq).  labels_out (nullable) u8[n] receives
 * the labels taken.
 *   EINVAL: n < 0 or n > max_tokens_per_call, num_q_heads < 1, score_kind
 *   not 0 or 1, or a required pointer NULL. */
int kv_classify_append(tkv_cache* c, int32_t n, const int32_t* seq_ids, const int32_t* positions,
                       const float* stats, int32_t num_q_heads, float tau_T, float tau_E, int32_t score_kind,
                       uint8_t* labels_out, const float* k, const float* v, int32_t* slot_out,
                       hipStream_t stream);

/* kv_evict_segment -- TBE bullet (progressive eviction at thought-segment
 * granularity; the retention schedule shrinks a segment step by step).
 *   Op i = (seq_ids[i], segment_ids[i], keep_n[i], new_bits[i]): keep the
 *   keep_n newest retained tokens of the segment (0 keeps none), clear the
 *   others' valid bits and push their slots on the sequence's stack in
 *   ascending position order.  new_bits below the segment's bits (8->4/2,
 *   4->2) re-quantizes the kept tokens from their dequantized fp32 values
 *   into slots of the lower class (popped in ascending position order), then
 *   frees the old slots.  new_bits 0 keeps the precision.
 *   A segment may appear in one op per call.  Arrays have n_ops entries; when
 *   n_ops_dev (device i32, nullable) is given, only its first *n_ops_dev <=
 *   n_ops ops are applied (for op lists written by kv_plan_budget or
 *   kv_plan_anneal).
 *   Device errors: ENOSEG (unknown or fully evicted segment), EINVAL (bad
 *   keep_n/new_bits, repeated segment), ENOMEM (no room for the downgrade). */
int kv_evict_segment(tkv_cache* c, int32_t n_ops, const int32_t* n_ops_dev, const int32_t* seq_ids,
                     const int32_t* segment_ids, const int32_t* keep_n, const uint8_t* new_bits,
                     hipStream_t stream);

/* kv_plan_budget -- the eviction ladder for a token budget (TBE bullet; the
 * lay summary's "Astuce B": a small safety net of Transition thoughts is
 * always kept).  For each listed sequence with budget B = floor(length *
 * budget_num / budget_den): while its retained count exceeds B, evict whole T
 * segments oldest first, never the open (last) segment nor the newest
 * retained T segment; if still over, downgrade the oldest non-open E segment
 * above 2 bits to 2 bits.  Writes at most max_ops ops (list order of the
 * sequences) to op_* (device arrays of max_ops entries) and their count to
 * *n_ops_dev; feed them to kv_evict_segment with n_ops_dev. */
int kv_plan_budget(tkv_cache* c, int32_t n, const int32_t* seq_ids, int32_t budget_num,
                   int32_t budget_den, int32_t max_ops, int32_t* n_ops_dev, int32_t* op_seq,
                   int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits, hipStream_t stream);

/* kv_plan_budget_evict -- the same result as kv_plan_budget(c, n, seq_ids,
 * budget_num, budget_den, max_ops, n_ops_dev, op_*) followed by
 * kv_evict_segment(c, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits),
 * in one call; the ladder's work-group is kept to 8 waves so that, in a
 * decode loop, it can start beside another batch's attention call.  The op
 * list is written to op_* and *n_ops_dev as by kv_plan_budget.  Errors as the
 * two calls'. */
int kv_plan_budget_evict(tkv_cache* c, int32_t n, const int32_t* seq_ids, int32_t budget_num, int32_t budget_den,
                         int32_t max_ops, int32_t* n_ops_dev, int32_t* op_seq, int32_t* op_seg, int32_t* op_keep,
                         uint8_t* op_bits, hipStream_t stream);

/* kv_plan_anneal -- the annealing schedule of TBE (TBE bullet: once a
 * Transition thought is detected, the earlier Reasoning/Execution segments are
 * evicted progressively, the retention shrinking on a schedule such as 64, 32,
 * 16; segment granularity; the lay summary's "Astuce B" keeps a small safety
 * net of Transition thoughts).  For each listed sequence (ids outside
 * [0, max_seqs) are skipped) and each of its R or E segments with retained
 * tokens: e = the number of T segments opened after it; when e >= 1 its cap
 * is r0 halved e-1 times (integer halving: 64, 32, 16, ..., 1, 0 for r0 =
 * 64), and a segment holding more retained tokens than its cap gets the op
 * (seq, segment, keep_n = cap, new_bits = 0).  T segments are never planned.
 * The plan depends only on the segment tables, so planning again after
 * applying it gives no ops.  Ops in list order of the sequences, segments in
 * order; at most max_ops (<= max_tokens_per_call) are written to op_*
 * (device arrays of max_ops entries) and their count to *n_ops_dev; feed them
 * to kv_evict_segment with n_ops_dev.  A sequence listed twice is planned
 * twice (kv_evict_segment then rejects the repeated segments).
 *   EINVAL: n or max_ops out of range, r0 < 0, or a required pointer is NULL. */
int kv_plan_anneal(tkv_cache* c, int32_t n, const int32_t* seq_ids, int32_t r0, int32_t max_ops,
                   int32_t* n_ops_dev, int32_t* op_seq, int32_t* op_seg, int32_t* op_keep,
                   uint8_t* op_bits, hipStream_t stream);

/* kv_plan_anneal_evict -- the same result as kv_plan_anneal(c, n, seq_ids,
 * r0, max_ops, n_ops_dev, op_*) followed by kv_evict_segment(c, max_ops,
 * n_ops_dev, op_seq, op_seg, op_keep, op_bits), with the plan and the
 * eviction's planning in one work-group (one launch fewer).  Errors as the
 * two calls'. */
int kv_plan_anneal_evict(tkv_cache* c, int32_t n, const int32_t* seq_ids, int32_t r0, int32_t max_ops,
                         int32_t* n_ops_dev, int32_t* op_seq, int32_t* op_seg, int32_t* op_keep,
                         uint8_t* op_bits, hipStream_t stream);

/* tkv_compact -- gather compaction, the baseline that in-place slot reuse
 * makes unnecessary (abstract: the kernel reuses evicted tokens' slots and so
 * eliminates compaction; Continuous Thinking bullet).  For each listed
 * sequence (an id listed again is compacted once; with n_dev, device i32,
 * nullable, only the first *n_dev <= n ids are read, so the seq_ids of an op
 * list written by a planner can be passed as they are) and each class it
 * holds blocks of: its m retained tokens are copied bit for bit, in position
 * order, into ceil(m/16) blocks popped from the class's global stack (token i
 * into slot i % 16 of the (i/16)-th popped block), which become its block
 * list; its free-slot stack becomes the empty tail of the last of them (lowest
 * slot on top).  All pops of the call come first (list order), then the old
 * blocks of every compacted sequence return to the global stacks (list
 * order, classes in order, blocks in list order).  Segments, lengths and
 * counts are unchanged; attention over the compacted cache reads the same
 * tokens.  Scratch (inside the cache's scratch buffer) carries the plan
 * between the three kernels of the call.
 *   Device errors: EINVAL (id outside [0, max_seqs)), ENOMEM (a sequence that
 *   does not find all its blocks is left untouched; after the first such
 *   failure of a class every later sequence needing that class fails too).
 *   EINVAL: n < 0 or n > max_tokens_per_call, or seq_ids NULL with n > 0. */
int tkv_compact(tkv_cache* c, int32_t n, const int32_t* n_dev, const int32_t* seq_ids, hipStream_t stream);

/* paged_decode_attn -- one decode step of attention over the mixed-precision,
 * hole-bearing cache (abstract: a kernel extending PagedAttention that reuses
 * evicted slots), with the sparsity statistics that assign the thought type
 * (thought decomposition bullets).  One layer per call (`layer`): for batch
 * entry b and query head h (KV head h / (Hq/Hkv) of that layer): attend every valid slot of sequence seq_ids[b] in all
 * three classes (with position >= q_pos[b] - window + 1 when window > 0) plus
 * the unquantized self token when k_self is given; logits q.k/sqrt(D);
 * out = sum e^(l-m) v / (sum e^(l-m) + [sinks] e^(sinks[h]-m)).
 * Statistics over the tokens only (sink excluded): H = -sum p ln p, H/ln n
 * (0 if n < 2), and the mass of the min(topk, n) largest p.  With
 * stats_stride = L*Hq*3 and stats advanced by layer*Hq*3, the L calls of a
 * step fill one [batch][L][Hq][3] array that thought_classify can average
 * over all layers (num_q_heads = L*Hq).
 *   EINVAL (besides the shapes): layer outside [0, L), stats_stride neither 0
 *   nor >= Hq*3, q, k_self, v_self, out or workspace not 16-byte aligned. */
typedef struct {
  int32_t batch;              /* entries, <= max_seqs                              */
  const int32_t* seq_ids;     /* i32[batch]                                        */
  const int32_t* q_pos;       /* i32[batch]: position t of each query              */
  const uint16_t* q;          /* bf16 bits [batch][Hq][D]                          */
  const float* k_self;        /* nullable fp32 [batch][Hkv][D]: staged token at t  */
  const float* v_self;        /* required with k_self                              */
  const float* sinks;         /* nullable fp32 [Hq]: extra logit per query head    */
  int32_t window;             /* 0 = full attention; W > 0: positions >= t-W+1     */
  int32_t topk;               /* 1..8                                              */
  int32_t num_splits;         /* 0 = library choice; else splits per (seq, KV head) */
  float* out;                 /* fp32 [batch][Hq][D]                               */
  float* stats;               /* nullable fp32 [batch][Hq][3] = {H, H/ln n, M_k}   */
  int32_t* n_attended;        /* nullable i32[batch]                               */
  void* workspace;            /* >= tkv_attn_workspace(c, batch, num_splits) bytes; nullable when that is 0 */
  size_t workspace_bytes;
  int32_t layer;              /* 0..L-1: the layer whose K/V are attended                  */
  int32_t stats_stride;       /* floats between batch entries of stats; 0 = Hq*3, else >= Hq*3 */
  const int32_t* order;       /* nullable i32[1 + batch] from tkv_attn_order over this batch:
                                 the dispatch order of the entries (results do not depend on it);
                                 ignored unless order[0] == batch                             */
} tkv_attn_args;

/* Workspace bytes paged_decode_attn needs for `batch` entries and the given
   num_splits (0 = the library's choice). */
size_t tkv_attn_workspace(const tkv_cache* c, int32_t batch, int32_t num_splits);

/* tkv_attn_order -- dispatch order for paged_decode_attn (not part of the
 * method; its results are the same in any order): writes order[0] = batch and
 * order[1..batch] = the batch entries, longest first (by the code bytes per KV
 * head the sequences hold now, in 256 length buckets; the order inside a bucket
 * is not fixed).  Passed as tkv_attn_args.order, it makes the attention deal
 * its work-groups so that every compute unit gets a similar mix of long and
 * short sequences (random lengths otherwise leave some compute units with
 * several long ones), and a grid of >= 2048 (entry, KV head) units then runs as
 * two-wave work-groups.  Lengths change slowly in decode, so one order can
 * serve many steps over the same seq_ids; an order made for another batch size
 * is ignored.  seq_ids: i32[batch] (the attention's); order: device i32
 * [1 + batch], caller-owned.  One small kernel on `stream`.
 *   EINVAL: c NULL, batch < 0 or > max_seqs, or a needed pointer NULL. */
int tkv_attn_order(tkv_cache* c, int32_t batch, const int32_t* seq_ids, int32_t* order, hipStream_t stream);
int paged_decode_attn(tkv_cache* c, const tkv_attn_args* a_h, hipStream_t stream);

/* paged_decode_attn_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same result as paged_decode_attn(c, a_h, stream), with
 * a_h->workspace and a_h->workspace_bytes ignored.  The split-K partial
 * records go to a device array of TKV_STATIC_WORKSPACE_BYTES inside the
 * library (one per device, held until the process ends, its address looked up
 * by tkv_create); no memory is allocated or freed by the call.  Every call on
 * one device shares that array: calls that overlap on one device (different
 * streams, threads or handles) race and must be serialized by the caller.
 *   ERANGE: tkv_attn_workspace(c, batch, num_splits) exceeds
 *   TKV_STATIC_WORKSPACE_BYTES (nothing is enqueued; pass fewer splits or a
 *   smaller batch).  Other errors as paged_decode_attn's. */
#define TKV_STATIC_WORKSPACE_BYTES (32u << 20)
int paged_decode_attn_noalloc(tkv_cache* c, const tkv_attn_args* a_h, hipStream_t stream);

/* thought_classify -- thought decomposition bullets: T shows the most
 * concentrated (sparse) attention, R less, E the least.  score_b = fp32 mean
 * over the Hq heads, in head order, of H/ln n (score_kind 0) or 1 - M_k
 * (score_kind 1) from stats fp32 [batch][Hq][3]; label T if score <= tau_T,
 * E if score >= tau_E, else R.  labels_out u8[batch]. */
int thought_classify(int32_t batch, int32_t num_q_heads, const float* stats, float tau_T, float tau_E,
                     int32_t score_kind, uint8_t* labels_out, hipStream_t stream);

/* Synchronize the handle's last stream, read and clear the sticky error
   word: kinds_h = OR of (1 << -code), min_seq_h = lowest sequence id
   involved, count_h = errors recorded.  Returns TKV_OK or TKV_EHIP. */
int tkv_get_error(tkv_cache* c, int32_t* kinds_h, int32_t* min_seq_h, int32_t* count_h);

/* Synchronous copies of every state buffer (SCRATCH excluded) to or from host
   memory; NULL entries are skipped.  Usable as a checkpoint. */
int tkv_export_state(tkv_cache* c, void* const host_bufs_h[TKV_NUM_BUFFERS]);
int tkv_import_state(tkv_cache* c, void* const host_bufs_h[TKV_NUM_BUFFERS]);

const char* tkv_strerror(int status);

/* tkv_kernel_timing -- measurement aid, not part of the method: with enable
 * != 0, every kernel the library launches for cache c from then on is
 * bracketed by two HIP events on the stream of its call (events without the
 * system-scope fence, so the L2 is not flushed), and tkv_kernel_times adds up
 * the durations per kernel name; enable == 0 turns it off.  Either call drops
 * every record so far (events recorded and not yet read are destroyed: call
 * it when the cache's streams are idle).  The events add a small gap between
 * the kernels of a call; nothing else changes.  The library allocates the
 * host-side records and events; they are freed by tkv_kernel_timing(c, 0)
 * or tkv_destroy.  EINVAL: c NULL.  EHIP: out of host memory. */
int tkv_kernel_timing(tkv_cache* c, int32_t enable);

/* tkv_kernel_times -- measurement aid: waits for the events recorded since the
 * last read, adds their durations to the per-kernel totals and writes, for the
 * first max_kernels kernel names in first-launch order, names (char[32] each,
 * NUL-terminated, caller-owned [max_kernels][32]), total_us (f64) and calls
 * (i32); *dropped (nullable) receives the launches left unrecorded because
 * more than 65536 were waiting to be read.  Returns the number of distinct
 * kernels timed so far (may exceed max_kernels), or EINVAL (c NULL, timing
 * off, max_kernels < 0 or a needed pointer NULL) or EHIP (an event call
 * failed). */
int tkv_kernel_times(tkv_cache* c, int32_t max_kernels, char* names, double* total_us, int32_t* calls,
                     int64_t* dropped);

/* tkv_stream_read -- measurement aid, not part of the method: read `bytes`
 * (a multiple of 16) of the device buffer `src` with 128-bit loads at a grid
 * stride and fold them into a value that is stored to the device word `sink`
 * only in a case that does not arise in practice.  Timing it on a buffer
 * larger than the 256 MB Infinity Cache gives the streaming-read ceiling of
 * HBM on this machine.  EINVAL: src or sink NULL, or bytes % 16 != 0. */
int tkv_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* TKV_H */
