"""CPU oracle for the ThinKV decode hot path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code
with them.

The oracle's C source (``tkv_oracle.c``) is plain and sequential; this module
builds it with gcc, owns the cache state as numpy arrays in the documented
state format, and exposes the same operations as the HIP library under
``OracleCache``.  See the header of ``tkv_oracle.c`` for the method passages
each function follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tkv_oracle.c")
_LIB = os.path.join(_HERE, "libtkv_oracle.so")

BS = 16
SEQ_W, HDR_W, SEG_W, BLK_W, SLOT_W = 16, 16, 8, 4, 2
CLASS_BITS = (8, 4, 2)
R, E, T = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction, so fp32 is plain IEEE)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Layout(C.Structure):
    _fields_ = [("num_kv_heads", C.c_int32), ("num_q_heads", C.c_int32), ("head_dim", C.c_int32),
                ("group_size", C.c_int32), ("bits", C.c_int32 * 3), ("pool_blocks", C.c_int32 * 3),
                ("max_seqs", C.c_int32), ("max_blocks_per_seq", C.c_int32),
                ("max_segments_per_seq", C.c_int32), ("num_layers", C.c_int32), ("code_format", C.c_int32)]


class _State(C.Structure):
    _fields_ = [("pool", C.c_void_p * 3), ("blk", C.c_void_p * 3), ("slot", C.c_void_p * 3),
                ("freestk", C.c_void_p * 3), ("hdr", C.c_void_p), ("seq", C.c_void_p),
                ("btab", C.c_void_p), ("sstk", C.c_void_p), ("segt", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        L.ora_f32_to_f16.argtypes = [C.c_float]; L.ora_f32_to_f16.restype = C.c_uint16
        L.ora_f16_to_f64.argtypes = [C.c_uint16]; L.ora_f16_to_f64.restype = C.c_double
        L.ora_block_head_bytes.argtypes = [P, C.c_int]; L.ora_block_head_bytes.restype = C.c_int64
        L.ora_quantize_group.argtypes = [P, C.c_int, C.c_int, P, P, P]; L.ora_quantize_group.restype = None
        L.ora_quantize_group_fmt.argtypes = [C.c_int, P, C.c_int, P, P, P]
        L.ora_quantize_group_fmt.restype = None
        L.ora_code_value.argtypes = [C.c_int, C.c_int, C.c_uint]; L.ora_code_value.restype = C.c_double
        L.ora_init.argtypes = [P, P, P]; L.ora_init.restype = None
        L.ora_append.argtypes = [P, P, C.c_int, P, P, P, P, P, P]; L.ora_append.restype = None
        L.ora_evict.argtypes = [P, P, C.c_int, P, P, P, P]; L.ora_evict.restype = None
        L.ora_plan_budget.argtypes = [P, P, C.c_int, P, C.c_int, C.c_int, C.c_int, P, P, P, P]
        L.ora_plan_budget.restype = C.c_int
        L.ora_plan_anneal.argtypes = [P, P, C.c_int, P, C.c_int, C.c_int, P, P, P, P]
        L.ora_plan_anneal.restype = C.c_int
        L.ora_compact.argtypes = [P, P, C.c_int, P]; L.ora_compact.restype = None
        L.ora_token_rows.argtypes = [P, P, C.c_int, C.c_int, C.c_int, P, P]; L.ora_token_rows.restype = None
        L.ora_seq_reset.argtypes = [P, P, C.c_int, P]; L.ora_seq_reset.restype = None
        L.ora_attention.argtypes = [P, P, C.c_int, P, P, P, P, P, P, C.c_int, C.c_int, C.c_int, P, P, P]
        L.ora_attention.restype = None
        L.ora_classify.argtypes = [C.c_int, C.c_int, P, C.c_float, C.c_float, C.c_int, P]
        L.ora_classify.restype = None
        L.ora_f32_to_f16_vec.argtypes = [P, P, C.c_int64]; L.ora_f32_to_f16_vec.restype = None
        L.ora_code_bit.argtypes = [P, C.c_int, C.c_int, C.c_int, C.c_int]; L.ora_code_bit.restype = C.c_int64
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _arr(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
# element-level helpers (used by the oracle's own pins)
# ---------------------------------------------------------------------------
def f32_to_f16_bits(x: float) -> int:
    return int(lib().ora_f32_to_f16(C.c_float(x)))


def f32_to_f16_bits_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32).ravel()
    h = np.empty(x.size, np.uint16)
    lib().ora_f32_to_f16_vec(_p(x), _p(h), x.size)
    return h


def quantize_group(x: np.ndarray, bits: int):
    x = np.ascontiguousarray(x, np.float32)
    codes = np.zeros(x.size, np.uint32)
    s = np.zeros(1, np.uint16); z = np.zeros(1, np.uint16)
    lib().ora_quantize_group(_p(x), x.size, bits, _p(codes), _p(s), _p(z))
    return codes, int(s[0]), int(z[0])


def quantize_group_fmt(x: np.ndarray, c: int):
    """Float / ternary quantizer of class c (0 FP8 E4M3, 1 FP4 E2M1, 2 ternary):
    codes and the fp16 scale and zero-point bits (zero-point 0 for the float
    classes, -scale for ternary, whose codes are t + 1)."""
    x = np.ascontiguousarray(x, np.float32)
    codes = np.zeros(x.size, np.uint32)
    s = np.zeros(1, np.uint16); z = np.zeros(1, np.uint16)
    lib().ora_quantize_group_fmt(c, _p(x), x.size, _p(codes), _p(s), _p(z))
    return codes, int(s[0]), int(z[0])


def code_value(code_format: int, c: int, code: int) -> float:
    """The value a stored code stands for, before scale and zero-point."""
    return float(lib().ora_code_value(code_format, c, code))


# ---------------------------------------------------------------------------
# state
# ---------------------------------------------------------------------------
class OracleLayout:
    def __init__(self, num_kv_heads, num_q_heads, head_dim, group_size, pool_blocks,
                 max_seqs, max_blocks_per_seq, max_segments_per_seq, bits=(8, 4, 2), num_layers=1,
                 code_format=0):
        self.num_kv_heads, self.num_q_heads = int(num_kv_heads), int(num_q_heads)
        self.head_dim, self.group_size = int(head_dim), int(group_size)
        self.bits = tuple(int(b) for b in bits)
        self.pool_blocks = tuple(int(p) for p in pool_blocks)
        self.max_seqs, self.max_blocks_per_seq = int(max_seqs), int(max_blocks_per_seq)
        self.max_segments_per_seq = int(max_segments_per_seq)
        self.num_layers = max(1, int(num_layers))
        self.stored_heads = self.num_kv_heads * self.num_layers
        self.code_format = int(code_format)
        self._c = _Layout(self.num_kv_heads, self.num_q_heads, self.head_dim, self.group_size,
                          (C.c_int32 * 3)(*self.bits), (C.c_int32 * 3)(*self.pool_blocks),
                          self.max_seqs, self.max_blocks_per_seq, self.max_segments_per_seq, self.num_layers,
                          self.code_format)

    def block_head_bytes(self, c: int) -> int:
        return int(lib().ora_block_head_bytes(C.byref(self._c), c))

    def code_bit(self, c: int, kv: int, t: int, d: int) -> int:
        return int(lib().ora_code_bit(C.byref(self._c), c, kv, t, d))


class OracleCache:
    """The oracle's cache: numpy arrays in the documented state format."""

    def __init__(self, layout: OracleLayout, block_order=None):
        self.L = layout
        L = layout
        self.bufs = {}
        for c in range(3):
            P = L.pool_blocks[c]
            self.bufs[f"pool{c}"] = np.zeros(P * L.stored_heads * L.block_head_bytes(c), np.uint8)
            self.bufs[f"blk{c}"] = np.zeros(P * BLK_W, np.int32)
            self.bufs[f"slot{c}"] = np.zeros(P * BS * SLOT_W, np.int32)
            self.bufs[f"free{c}"] = np.zeros(P, np.int32)
        self.bufs["hdr"] = np.zeros(HDR_W, np.int32)
        self.bufs["seq"] = np.zeros(L.max_seqs * SEQ_W, np.int32)
        self.bufs["btab"] = np.zeros(L.max_seqs * 3 * L.max_blocks_per_seq, np.int32)
        self.bufs["sstk"] = np.zeros(L.max_seqs * 3 * L.max_blocks_per_seq * BS, np.int32)
        self.bufs["segt"] = np.zeros(L.max_seqs * L.max_segments_per_seq * SEG_W, np.int32)
        self._state = _State()
        self._bind()
        orders = None
        keep = []
        if block_order is not None:
            orders = (C.c_void_p * 3)()
            for c in range(3):
                if block_order[c] is not None:
                    a = np.ascontiguousarray(block_order[c], np.int32)
                    keep.append(a)
                    orders[c] = a.ctypes.data
        lib().ora_init(C.byref(L._c), C.byref(self._state), orders)

    def _bind(self):
        st = self._state
        for c in range(3):
            st.pool[c] = self.bufs[f"pool{c}"].ctypes.data
            st.blk[c] = self.bufs[f"blk{c}"].ctypes.data
            st.slot[c] = self.bufs[f"slot{c}"].ctypes.data
            st.freestk[c] = self.bufs[f"free{c}"].ctypes.data
        for n in ("hdr", "seq", "btab", "sstk", "segt"):
            setattr(st, n, self.bufs[n].ctypes.data)

    # -- operations ----------------------------------------------------------
    def append(self, seq_ids, positions, thought, k, v):
        seq_ids = _arr(seq_ids, np.int32); positions = _arr(positions, np.int32)
        thought = _arr(thought, np.uint8); k = _arr(k, np.float32); v = _arr(v, np.float32)
        n = seq_ids.size
        slot_out = np.zeros(n, np.int32)
        lib().ora_append(C.byref(self.L._c), C.byref(self._state), n, _p(seq_ids), _p(positions),
                         _p(thought), _p(k), _p(v), _p(slot_out))
        return slot_out

    def evict(self, seq_ids, seg_ids, keep_n, new_bits):
        seq_ids = _arr(seq_ids, np.int32); seg_ids = _arr(seg_ids, np.int32)
        keep_n = _arr(keep_n, np.int32); new_bits = _arr(new_bits, np.uint8)
        lib().ora_evict(C.byref(self.L._c), C.byref(self._state), seq_ids.size, _p(seq_ids),
                        _p(seg_ids), _p(keep_n), _p(new_bits))

    def plan_budget(self, seq_ids, num, den, max_ops):
        seq_ids = _arr(seq_ids, np.int32)
        os_ = np.zeros(max_ops, np.int32); og = np.zeros(max_ops, np.int32)
        ok = np.zeros(max_ops, np.int32); ob = np.zeros(max_ops, np.uint8)
        m = lib().ora_plan_budget(C.byref(self.L._c), C.byref(self._state), seq_ids.size, _p(seq_ids),
                                  int(num), int(den), int(max_ops), _p(os_), _p(og), _p(ok), _p(ob))
        return os_[:m], og[:m], ok[:m], ob[:m]

    def plan_anneal(self, seq_ids, r0, max_ops):
        seq_ids = _arr(seq_ids, np.int32)
        os_ = np.zeros(max_ops, np.int32); og = np.zeros(max_ops, np.int32)
        ok = np.zeros(max_ops, np.int32); ob = np.zeros(max_ops, np.uint8)
        m = lib().ora_plan_anneal(C.byref(self.L._c), C.byref(self._state), seq_ids.size, _p(seq_ids),
                                  int(r0), int(max_ops), _p(os_), _p(og), _p(ok), _p(ob))
        return os_[:m], og[:m], ok[:m], ob[:m]

    def compact(self, seq_ids):
        seq_ids = _arr(seq_ids, np.int32)
        lib().ora_compact(C.byref(self.L._c), C.byref(self._state), seq_ids.size, _p(seq_ids))

    def seq_reset(self, seq_ids):
        seq_ids = _arr(seq_ids, np.int32)
        lib().ora_seq_reset(C.byref(self.L._c), C.byref(self._state), seq_ids.size, _p(seq_ids))

    def attention(self, seq_ids, q_pos, q_bf16, k_self=None, v_self=None, sinks=None, window=0, topk=8, layer=0):
        L = self.L
        seq_ids = _arr(seq_ids, np.int32); q_pos = _arr(q_pos, np.int32)
        q_bf16 = _arr(q_bf16, np.uint16)
        k_self = _arr(k_self, np.float32); v_self = _arr(v_self, np.float32); sinks = _arr(sinks, np.float32)
        B = seq_ids.size
        out = np.zeros((B, L.num_q_heads, L.head_dim), np.float64)
        stats = np.zeros((B, L.num_q_heads, 3), np.float64)
        n_att = np.zeros(B, np.int32)
        lib().ora_attention(C.byref(L._c), C.byref(self._state), B, _p(seq_ids), _p(q_pos), _p(q_bf16),
                            _p(k_self), _p(v_self), _p(sinks), int(window), int(topk), int(layer), _p(out),
                            _p(stats), _p(n_att))
        return out, stats, n_att

    # -- state views -----------------------------------------------------------
    def export(self):
        return {k: v.copy() for k, v in self.bufs.items()}

    def import_(self, bufs):
        for k, v in bufs.items():
            if k in self.bufs:
                self.bufs[k][...] = np.asarray(v).view(self.bufs[k].dtype).reshape(self.bufs[k].shape)

    def seq_record(self, s):
        return self.bufs["seq"][s * SEQ_W:(s + 1) * SEQ_W]

    def segments(self, s):
        L = self.L
        n = int(self.seq_record(s)[6])
        base = s * L.max_segments_per_seq * SEG_W
        return self.bufs["segt"][base:base + n * SEG_W].reshape(n, SEG_W)

    def token_rows(self, s):
        """{position: fp32 [2][Hkv][D] K and V rows} of the retained tokens of sequence s."""
        L = self.L
        q = self.seq_record(s)
        H, D = L.stored_heads, L.head_dim
        out = {}
        for c in range(3):
            bt = self.bufs["btab"][(s * 3 + c) * L.max_blocks_per_seq:][:int(q[c])]
            for blk in bt:
                mask = int(self.bufs[f"blk{c}"][int(blk) * 4])
                for t in range(16):
                    if not (mask >> t) & 1:
                        continue
                    slot = int(blk) * 16 + t
                    rows = np.zeros((2, H, D), np.float32)
                    for h in range(H):
                        k = np.zeros(D, np.float32); v = np.zeros(D, np.float32)
                        lib().ora_token_rows(C.byref(L._c), C.byref(self._state), c, slot, h, _p(k), _p(v))
                        rows[0, h], rows[1, h] = k, v
                    out[int(self.bufs[f"slot{c}"][slot * 2])] = rows
        return out

    def error(self):
        h = self.bufs["hdr"]
        return int(h[3]), int(h[4]), int(h[5])

    def clear_error(self):
        h = self.bufs["hdr"]
        h[3] = 0; h[4] = 0x7FFFFFFF; h[5] = 0


def classify(stats_f32, tau_T, tau_E, kind=0):
    stats_f32 = np.ascontiguousarray(stats_f32, np.float32)
    B, Hq = stats_f32.shape[0], stats_f32.shape[1]
    labels = np.zeros(B, np.uint8)
    lib().ora_classify(B, Hq, _p(stats_f32), C.c_float(tau_T), C.c_float(tau_E), int(kind), _p(labels))
    return labels
