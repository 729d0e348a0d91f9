// Internal declarations of libthinkv: the handle, the device view of the
// cache state, and device helpers shared by the state and attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "tkv.h"

#define TKV_BS 16                 // tokens per block
#define TKV_SEQ_W 16              // words per sequence record
#define TKV_SEG_W 8               // words per segment record
#define TKV_BLK_W 4               // words per block record
#define TKV_SLOT_W 2              // words per slot record
#define TKV_MAX_TOK 4096          // items per append / evict / plan call
#define TKV_MAX_SEQS 1024
#define TKV_MAX_BLOCKS 256        // per sequence and class
#define TKV_MAX_POOL_BLOCKS (1 << 22)   // per class (global pop indices are packed in 23 bits)
#define TKV_INF 0x7fffffff

// SEQ record words
enum { Q_NBLK = 0, Q_NSLOT = 3, Q_NSEG = 6, Q_LEN = 7, Q_NRET = 8, Q_NAPP = 9 };
// SEGT record words
enum { G_TYPE = 0, G_BITS = 1, G_FIRST = 2, G_LAST = 3, G_NTOT = 4, G_NRET = 5 };
// HDR words
enum { H_FREE = 0, H_EKIND = 3, H_EMINSEQ = 4, H_ECOUNT = 5 };

// Device view of the state: raw pointers plus geometry, passed by value.
struct DevState {
  uint8_t* pool[3];
  int32_t* blk[3];
  int32_t* slot[3];
  int32_t* freestk[3];
  int32_t* hdr;
  int32_t* seq;
  int32_t* btab;
  int32_t* sstk;
  int32_t* segt;
  int32_t* scratch;
  int Hkv, Hq, D, g, NG;
  int NL, Hst;                    // layers; KV heads stored per block (NL * Hkv)
  int fmt;                        // code format: 0 integer, 1 FP8 / FP4 / ternary
  int type_class[3];              // class index for thought type R, E, T
  int pool_blocks[3];
  int max_seqs, max_blocks, max_segs, max_tokens;
  int64_t bh_bytes[3];            // bytes per (block, KV head) record
  int chunk_bytes[3];             // bytes per lane chunk = D*bits/32
};

struct KernelTimes;               // per-kernel timing records (tkv_kernel_timing)
struct tkv_cache {
  tkv_layout L;
  void* buf[TKV_NUM_BUFFERS];
  size_t size[TKV_NUM_BUFFERS];
  DevState S;
  hipStream_t last_stream;
  int device;                     // the device current when the cache was created
  KernelTimes* kt;                // null unless per-kernel timing is on
};

// Per-kernel timing (off by default): with it on, every kernel the library
// launches for a cache is bracketed by two HIP events on its stream (created
// without the system-scope fence), and tkv_kernel_times adds up the measured
// durations per kernel name.  KernelScope brackets one launch.
struct KernelScope {
  KernelTimes* kt;
  int slot;
  hipStream_t st;
  KernelScope(const tkv_cache* c, hipStream_t stream, const char* name);
  ~KernelScope();
};
#define TKV_TIMED(c, st, name, ...)     \
  do {                                   \
    KernelScope ks_((c), (st), (name));  \
    __VA_ARGS__;                         \
  } while (0)

// Per-class fields of DevState indexed by a run-time class: select among the
// three kernel-argument values (held in scalar registers) instead of indexing
// the by-value argument, which would turn into a load from the kernel-argument
// segment on every use.
template <class T>
__device__ __forceinline__ T pick3(const T (&a)[3], int c) {
  return c == 0 ? a[0] : (c == 1 ? a[1] : a[2]);
}

__host__ __device__ inline int class_bits(int c) { return c == 0 ? 8 : (c == 1 ? 4 : 2); }
__host__ __device__ inline int class_of_bits(int b) { return b == 8 ? 0 : (b == 4 ? 1 : (b == 2 ? 2 : -1)); }

// Scratch carve-up (int32 words), sized by tkv_buffer_sizes as TKV_SCR_FIXED +
// max_seqs (per-sequence move counts) + max_seqs*max_blocks*16*2 (moves).
#define TKV_SCR_FIXED (14 * TKV_MAX_TOK + 64)
__host__ __device__ inline int32_t* scr_idx(int32_t* s) { return s; }                       // [MAX_TOK]
__host__ __device__ inline int32_t* scr_info(int32_t* s) { return s + TKV_MAX_TOK; }        // [MAX_TOK]
__host__ __device__ inline int32_t* scr_status(int32_t* s) { return s + 2 * TKV_MAX_TOK; }  // [MAX_TOK] (u8 labels of kv_classify_append)
__host__ __device__ inline int32_t* scr_need(int32_t* s) { return s + 3 * TKV_MAX_TOK; }    // [MAX_TOK]
__host__ __device__ inline int32_t* scr_list(int32_t* s) { return s + 4 * TKV_MAX_TOK; }    // [MAX_TOK] ops by sequence
__host__ __device__ inline int32_t* scr_grp(int32_t* s) { return s + 5 * TKV_MAX_TOK; }     // [3][max_seqs] off, count, downgrades
__host__ __device__ inline int32_t* scr_oprec(int32_t* s) { return s + 6 * TKV_MAX_TOK; }   // [MAX_TOK][8] op records
__host__ __device__ inline int32_t* scr_misc(int32_t* s) { return s + 14 * TKV_MAX_TOK; }   // [64]
__host__ __device__ inline int32_t* scr_mcnt(int32_t* s) { return s + TKV_SCR_FIXED; }      // [max_seqs]
__host__ __device__ inline int32_t* scr_moves(int32_t* s, int max_seqs) {                    // [max_seqs][max_blocks*16][2]
  return s + TKV_SCR_FIXED + max_seqs;
}

// ---------------------------------------------------------------------------
// Code placement inside a (block, KV head) record.  Each of the K and V code
// regions holds 64 lane chunks of CB = D*bits/32 bytes.  Codes of a chunk sit
// in 32-bit words of W = 32/bits codes: even elements in the low half-word,
// odd elements in the high half-word, so that a shift and mask (or a byte
// permute) puts a pair of codes into the two halves of an MFMA operand word.
// A chunk is stored in units of U = min(CB, 16) bytes, unit u of chunk k at
// byte (64u + k) U of its region: lane l's u-th 16-byte load then reads one
// contiguous kilobyte across the 64 lanes.  Float codes (format 1, the 8- and
// 4-bit classes) sit in element order instead: the hardware's packed
// conversions take consecutive fields of a word.  Ternary codes are integers.
// ---------------------------------------------------------------------------
__host__ __device__ inline int natural_order(int fmt, int c) { return fmt && c < 2; }
__host__ __device__ inline int field_pos(int f, int W, int nat) {
  return nat ? f : (f >> 1) + (f & 1) * (W >> 1);
}
__host__ __device__ inline int elem_bit(int e, int bits, int nat) {
  int W = 32 / bits, w = e / W, f = e % W;
  return w * 32 + field_pos(f, W, nat) * bits;
}
// byte b of chunk k of a region of chunks of CB bytes -> byte within the region
__host__ __device__ inline int chunk_byte(int CB, int k, int b) {
  const int U = CB < 16 ? CB : 16;
  return (64 * (b / U) + k) * U + b % U;
}
// K: token t, dim d -> chunk 16*lg + t, element gi*(g/4) + e'
__host__ __device__ inline int k_code_bit(int D, int g, int bits, int nat, int t, int d) {
  int q4 = g >> 2, gi = d / g, w = d % g, lg = w / q4, ep = w % q4;
  int chunk = 16 * lg + t, eb = elem_bit(gi * q4 + ep, bits, nat);
  return chunk_byte(D * bits / 32, chunk, eb >> 3) * 8 + (eb & 7);
}
// V: token t = 4q + r, dim d = 16n + i -> chunk 16*q + i, element 4n + r
__host__ __device__ inline int v_code_bit(int D, int bits, int nat, int t, int d) {
  int q = t >> 2, r = t & 3, n = d >> 4, i = d & 15;
  int chunk = 16 * q + i, eb = elem_bit(4 * n + r, bits, nat);
  return 64 * (D * bits / 32) * 8 + chunk_byte(D * bits / 32, chunk, eb >> 3) * 8 + (eb & 7);
}
__host__ __device__ inline int meta_byte(int D, int g, int bits, int kv, int t, int gi) {
  int NG = D / g;
  return 2 * 64 * (D * bits / 32) + kv * (16 * NG * 4) + (t * NG + gi) * 4;
}

// Sticky error word.
// ---------------------------------------------------------------------------
// Exact cross-lane butterflies on VALU (no LDS round trip).  xchg<K> (K = 1,
// 2, 4, 8) is the value of lane i ^ K: DPP quad permutations, a pair of
// bank-masked row shifts, a row rotation by 8.  For K = 16, 32 swap_pair hands
// every lane both values of its pair (even row / lower half first) through
// the gfx950 v_permlane16_swap / v_permlane32_swap, written as one asm block
// with the copy: given the same value as both operands, the compiler's builtin
// folds its two results into one.  The block also holds the two wait states a
// permlane needs after a VALU write.  Sums, minima, maxima and top-k merges of
// a pair do not depend on operand order, so both partners get the same bits.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int K>
__device__ inline float xchg(float v) {
  if constexpr (K == 1) return dpp_f<0xB1>(v);                   // quad_perm [1,0,3,2]
  if constexpr (K == 2) return dpp_f<0x4E>(v);                   // quad_perm [2,3,0,1]
  if constexpr (K == 4) {
    int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x104, 0xf, 0x5, false);   // row_shl:4, banks 0, 2
    t = __builtin_amdgcn_update_dpp(t, __builtin_bit_cast(int, v), 0x114, 0xf, 0xA, false);       // row_shr:4, banks 1, 3
    return __builtin_bit_cast(float, t);
  }
  if constexpr (K == 8) return dpp_f<0x128>(v);                  // row_ror:8
}
template <int K>
__device__ inline void swap_pair(float v, float& a, float& b) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y;
  if constexpr (K == 16) asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "=&v"(y));
  else asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "=&v"(y));
  a = __builtin_bit_cast(float, x);
  b = __builtin_bit_cast(float, y);
}

template <int K>
__device__ inline float pair_sum(float v) {
  if constexpr (K <= 8) {
    return v + xchg<K>(v);
  } else {
    float a, b;
    swap_pair<K>(v, a, b);
    return a + b;
  }
}
template <int K>
__device__ inline float pair_max(float v) {
  if constexpr (K <= 8) {
    return fmaxf(v, xchg<K>(v));
  } else {
    float a, b;
    swap_pair<K>(v, a, b);
    return fmaxf(a, b);
  }
}

__device__ inline void record_error(int32_t* hdr, int code, int seq) {
  atomicOr(&hdr[H_EKIND], 1 << (-code));
  atomicMin(&hdr[H_EMINSEQ], seq);
  atomicAdd(&hdr[H_ECOUNT], 1);
}

// ---------------------------------------------------------------------------
// Group quantizer, bit-exact IEEE fp32 (no contraction): scale =
// fp16((max-min)/(2^bits-1)), zero = fp16(min), -0 -> +0, codes =
// clamp(rint-half-even((x - zero)/scale)); zero scale -> all codes 0.
// `get(i)` yields the group's i-th fp32 value.
// ---------------------------------------------------------------------------
__device__ inline uint16_t f16_bits_rne(float x) {
  _Float16 h = (_Float16)x;   // v_cvt_f16_f32, round to nearest even
  uint16_t b = __builtin_bit_cast(uint16_t, h);
  return b == 0x8000u ? (uint16_t)0 : b;
}
__device__ inline float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

template <class Get>
__device__ inline void quant_scale_zero(Get get, int n, int bits, float& sf, float& zf, uint16_t& sh, uint16_t& zh) {
#pragma clang fp contract(off)
  float mn = get(0), mx = mn;
  for (int i = 1; i < n; i++) {
    float x = get(i);
    mn = x < mn ? x : mn;
    mx = x > mx ? x : mx;
  }
  float levels = (float)((1 << bits) - 1);
  float range = mx - mn;
  float s32 = range / levels;
  sh = f16_bits_rne(s32);
  zh = f16_bits_rne(mn);
  sf = f16_bits_to_f32(sh);
  zf = f16_bits_to_f32(zh);
}
__device__ inline unsigned quant_code(float x, float sf, float zf, int bits) {
#pragma clang fp contract(off)
  if (sf == 0.0f) return 0u;
  float diff = x - zf;
  float q = diff / sf;
  float r = __builtin_rintf(q);
  float top = (float)((1 << bits) - 1);
  r = r < 0.0f ? 0.0f : r;
  r = r > top ? top : r;
  return (unsigned)r;
}

// ---------------------------------------------------------------------------
// Float and ternary codes (format 1), per (token, group) with one fp16 scale:
// class 0 FP8 E4M3 (scale amax/448), class 1 FP4 E2M1 (scale amax/6), both
// rounded to nearest even and saturated, zero-point 0; class 2 ternary by the
// Ternary Weight Networks rule (threshold 0.7 mean|x|, scale the mean |x| of
// the entries beyond it), stored as the integer code t + 1 with zero-point
// -scale.
// The encoders work on the fp32 bit pattern: a value below the smallest
// normal of the format is a multiple of its subnormal step, rounded as an
// integer; above, the mantissa is cut to the format's width with round to
// nearest even (a carry into the exponent is the integer add itself).
// ---------------------------------------------------------------------------
__device__ inline unsigned e4m3_encode(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t a = u & 0x7FFFFFFFu, sgn = (u >> 24) & 0x80u;
  unsigned mag;
  if (a >= 0x43E00000u) mag = 0x7E;                                   // |y| >= 448
  else if (a < 0x3C800000u) {                                         // |y| < 2^-6: steps of 2^-9
    mag = (unsigned)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
  } else {
    // rebias 127 -> 7 and keep 3 mantissa bits, rounding the 20 dropped bits to nearest even
    const uint32_t r = a - (120u << 23);
    const uint32_t keep = r >> 20, rest = r & 0xFFFFFu;
    mag = keep + ((rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ? 1u : 0u);
  }
  return mag ? (mag | sgn) : 0u;
}
__device__ inline unsigned e2m1_encode(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t a = u & 0x7FFFFFFFu, sgn = (u >> 28) & 0x8u;
  unsigned mag;
  if (a >= 0x40C00000u) mag = 7;                                      // |y| >= 6
  else if (a < 0x3F800000u) {                                         // |y| < 1: steps of 1/2
    mag = (unsigned)__builtin_rintf(__builtin_bit_cast(float, a) * 2.0f);
  } else {
    const uint32_t r = a - (126u << 23);                              // rebias 127 -> 1
    const uint32_t keep = r >> 22, rest = r & 0x3FFFFFu;
    mag = keep + ((rest > 0x200000u || (rest == 0x200000u && (keep & 1u))) ? 1u : 0u);
  }
  return mag ? (mag | sgn) : 0u;
}
// value of a float code of class c (0 or 1) in format 1, before the scale
__device__ inline float fmt_value(int c, unsigned code) {
  if (c == 0) {
    const unsigned e = (code >> 3) & 15u, m = code & 7u;
    const float v = e ? __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (code & 0x80u) ? -v : v;
  }
  if (c == 1) {
    const unsigned e = (code >> 1) & 3u, m = code & 1u;
    const float v = e ? __builtin_bit_cast(float, ((e + 126u) << 23) | (m << 22)) : (float)m * 0.5f;
    return (code & 8u) ? -v : v;
  }
  return (float)code;
}

// ---------------------------------------------------------------------------
// Thought label of one batch entry from its statistics row (heads x {H,
// H/ln n, M_k}): fp32 sum in head order of H/ln n (kind 0) or 1 - M_k (kind
// 1), divided by the head count; T at or below tT, E at or above tE, else R.
// ---------------------------------------------------------------------------
struct ClassifyIn {
  const float* stats;           // [n][heads][3]; null: the thought labels are an input
  int heads, kind;
  float tT, tE;
  uint8_t* labels;              // nullable: the labels taken, [n]
};
__device__ inline uint32_t thought_label(float score, float tT, float tE) {
  return score <= tT ? (uint32_t)TKV_T : (score >= tE ? (uint32_t)TKV_E : (uint32_t)TKV_R);
}
// Launchers (state kernels)
int launch_init(tkv_cache* c, hipStream_t st);
int launch_append(tkv_cache* c, int n, const int32_t* seq_ids, const int32_t* pos, const uint8_t* thought,
                  const float* k, const float* v, int32_t* slot_out, hipStream_t st, const ClassifyIn* cl = nullptr);
int launch_evict(tkv_cache* c, int n_ops, const int32_t* n_ops_dev, const int32_t* seq_ids, const int32_t* seg_ids,
                 const int32_t* keep_n, const uint8_t* new_bits, hipStream_t st);
int launch_plan(tkv_cache* c, int n, const int32_t* seq_ids, int num, int den, int max_ops, int32_t* n_ops_dev,
                int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits, hipStream_t st);
int launch_plan_evict(tkv_cache* c, int n, const int32_t* seq_ids, int num, int den, int max_ops, int32_t* n_ops_dev,
                      int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits, hipStream_t st);
int launch_anneal(tkv_cache* c, int n, const int32_t* seq_ids, int r0, int max_ops, int32_t* n_ops_dev,
                  int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits, hipStream_t st);
int launch_anneal_evict(tkv_cache* c, int n, const int32_t* seq_ids, int r0, int max_ops, int32_t* n_ops_dev,
                        int32_t* op_seq, int32_t* op_seg, int32_t* op_keep, uint8_t* op_bits, hipStream_t st);
int launch_compact(tkv_cache* c, int n, const int32_t* n_dev, const int32_t* seq_ids, hipStream_t st);
int launch_seq_reset(tkv_cache* c, int n, const int32_t* seq_ids, hipStream_t st);
int launch_classify(int batch, int Hq, const float* stats, float tau_T, float tau_E, int kind, uint8_t* labels,
                    hipStream_t st);
// Attention
void attn_plan(const tkv_cache* c, int batch, int num_splits, bool ordered, int* nw, int* splits);
int launch_attn_order(tkv_cache* c, int batch, const int32_t* seq_ids, int32_t* order, hipStream_t st);
size_t attn_workspace_bytes(const tkv_cache* c, int batch, int splits);
int launch_attention(tkv_cache* c, const tkv_attn_args* a, int nw, int splits, hipStream_t st,
                     void* workspace = nullptr);
// the allocation-free attention call's device array: address lookup (once per
// device, with that device current) and the address found
int static_workspace_setup(int device);
void* static_workspace(int device);
