"""ctypes binding of libthinkv.so (argument marshalling only).

Every step of the hot path runs in the HIP library; this module allocates the
caller-owned device buffers with torch (``torch.empty(..., device="cuda")``),
passes raw pointers and the current HIP stream, and reads results back.  It
raises if the library is missing or no GPU is present -- there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libthinkv.so")

TKV_OK, TKV_EINVAL, TKV_ENOMEM, TKV_ENOSEG, TKV_EHIP, TKV_ERANGE = 0, -1, -2, -3, -4, -5
STATIC_WORKSPACE_BYTES = 32 << 20
BUFFER_NAMES = ["pool0", "pool1", "pool2", "blk0", "blk1", "blk2", "slot0", "slot1", "slot2",
                "free0", "free1", "free2", "hdr", "seq", "btab", "sstk", "segt", "scratch"]
NUM_BUFFERS = len(BUFFER_NAMES)
BUFFER_DTYPES = {n: (np.uint8 if n.startswith("pool") else np.int32) for n in BUFFER_NAMES}

# Entry points declared in include/tkv.h
SYMBOLS = ["tkv_buffer_sizes", "tkv_create", "tkv_destroy", "tkv_seq_reset", "kv_append_quant", "kv_classify_append",
           "kv_evict_segment", "kv_plan_budget", "kv_plan_budget_evict", "kv_plan_anneal", "kv_plan_anneal_evict", "tkv_compact", "tkv_attn_workspace", "paged_decode_attn",
           "paged_decode_attn_noalloc",
           "thought_classify", "tkv_get_error", "tkv_export_state", "tkv_import_state", "tkv_strerror",
           "tkv_stream_read", "tkv_kernel_timing", "tkv_kernel_times", "tkv_attn_order"]


class Layout(C.Structure):
    _fields_ = [("num_kv_heads", C.c_int32), ("num_q_heads", C.c_int32), ("head_dim", C.c_int32),
                ("group_size", C.c_int32), ("bits", C.c_int32 * 3), ("pool_blocks", C.c_int32 * 3),
                ("max_seqs", C.c_int32), ("max_blocks_per_seq", C.c_int32),
                ("max_segments_per_seq", C.c_int32), ("max_tokens_per_call", C.c_int32),
                ("num_layers", C.c_int32), ("code_format", C.c_int32)]


class AttnArgs(C.Structure):
    _fields_ = [("batch", C.c_int32), ("seq_ids", C.c_void_p), ("q_pos", C.c_void_p), ("q", C.c_void_p),
                ("k_self", C.c_void_p), ("v_self", C.c_void_p), ("sinks", C.c_void_p),
                ("window", C.c_int32), ("topk", C.c_int32), ("num_splits", C.c_int32),
                ("out", C.c_void_p), ("stats", C.c_void_p), ("n_attended", C.c_void_p),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t), ("layer", C.c_int32),
                ("stats_stride", C.c_int32), ("order", C.c_void_p)]


class TkvError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


_lib = None


def load(path: str = LIB_PATH):
    """Load the library (no GPU needed to load; calls need one)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with `python -m thought_adaptive_mixed_amd.build`")
    # torch first: the library then binds to the HIP runtime torch has loaded
    # (the same soname), so one runtime serves both in the process
    import torch  # noqa: F401
    L = C.CDLL(path)
    P, I, U = C.c_void_p, C.c_int32, C.c_uint8
    L.tkv_buffer_sizes.argtypes = [P, P]
    L.tkv_create.argtypes = [P, P, P, P, P]
    L.tkv_destroy.argtypes = [P]
    L.tkv_seq_reset.argtypes = [P, I, P, P]
    L.kv_append_quant.argtypes = [P, I, P, P, P, P, P, P, P]
    L.kv_classify_append.argtypes = [P, I, P, P, P, I, C.c_float, C.c_float, I, P, P, P, P, P]
    L.kv_evict_segment.argtypes = [P, I, P, P, P, P, P, P]
    L.kv_plan_budget.argtypes = [P, I, P, I, I, I, P, P, P, P, P, P]
    L.kv_plan_budget_evict.argtypes = [P, I, P, I, I, I, P, P, P, P, P, P]
    L.kv_plan_anneal.argtypes = [P, I, P, I, I, P, P, P, P, P, P]
    L.kv_plan_anneal_evict.argtypes = [P, I, P, I, I, P, P, P, P, P, P]
    L.tkv_compact.argtypes = [P, I, P, P, P]
    L.tkv_attn_workspace.argtypes = [P, I, I]; L.tkv_attn_workspace.restype = C.c_size_t
    L.paged_decode_attn.argtypes = [P, P, P]
    L.paged_decode_attn_noalloc.argtypes = [P, P, P]
    L.thought_classify.argtypes = [I, I, P, C.c_float, C.c_float, I, P, P]
    L.tkv_get_error.argtypes = [P, P, P, P]
    L.tkv_export_state.argtypes = [P, P]
    L.tkv_import_state.argtypes = [P, P]
    L.tkv_strerror.argtypes = [C.c_int]; L.tkv_strerror.restype = C.c_char_p
    L.tkv_stream_read.argtypes = [P, C.c_size_t, P, P]
    L.tkv_kernel_timing.argtypes = [P, I]
    L.tkv_kernel_times.argtypes = [P, I, P, P, P, P]
    L.tkv_attn_order.argtypes = [P, I, P, P, P]
    _lib = L
    return L


def strerror(code: int) -> str:
    try:
        return load().tkv_strerror(int(code)).decode()
    except FileNotFoundError:
        return str(code)


def _check(rc, what):
    if rc != TKV_OK:
        raise TkvError(rc, what)


_torch_mod = None


def _torch():
    global _torch_mod
    if _torch_mod is None:
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("thought_adaptive_mixed_amd needs a ROCm GPU (torch.cuda.is_available() is False)")
        _torch_mod = torch
    return _torch_mod


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return C.c_void_p(int(stream))
    return C.c_void_p(_torch().cuda.current_stream().cuda_stream)


class Prepared:
    """One library call with its C arguments converted once; calling it
    re-issues the call (for launch loops where argument marshalling would
    otherwise dominate).  The referenced buffers must outlive it."""

    __slots__ = ("fn", "args", "what", "keep")

    def __init__(self, fn, args, what, keep=None):
        self.fn, self.args, self.what, self.keep = fn, tuple(args), what, keep

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != TKV_OK:
            raise TkvError(rc, self.what)


def _issue(fn, args, what, prepare, keep=None):
    if prepare:
        return Prepared(fn, args, what, keep)
    _check(fn(*args), what)
    return None


def make_layout(num_kv_heads, num_q_heads, head_dim, group_size, pool_blocks, max_seqs, max_blocks_per_seq,
                max_segments_per_seq, max_tokens_per_call=4096, bits=(8, 4, 2), num_layers=1,
                code_format=0) -> Layout:
    return Layout(num_kv_heads, num_q_heads, head_dim, group_size, (C.c_int32 * 3)(*bits),
                  (C.c_int32 * 3)(*pool_blocks), max_seqs, max_blocks_per_seq, max_segments_per_seq,
                  max_tokens_per_call, num_layers, code_format)


def buffer_sizes(layout: Layout):
    sizes = (C.c_size_t * NUM_BUFFERS)()
    _check(load().tkv_buffer_sizes(C.byref(layout), sizes), "tkv_buffer_sizes")
    return [int(s) for s in sizes]


class Cache:
    """A cache state on the current GPU: caller-owned buffers + library handle."""

    def __init__(self, layout: Layout, block_order: Optional[Sequence[np.ndarray]] = None, device="cuda"):
        torch = _torch()
        self.layout = layout
        self.L = load()
        self.sizes = buffer_sizes(layout)
        self.bufs = [torch.empty(max(s, 16), dtype=torch.uint8, device=device) for s in self.sizes]
        ptrs = (C.c_void_p * NUM_BUFFERS)(*[_ptr(b) for b in self.bufs])
        orders = None
        self._orders = []
        if block_order is not None:
            orders = (C.c_void_p * 3)()
            for c in range(3):
                if block_order[c] is not None:
                    a = np.ascontiguousarray(block_order[c], np.int32)
                    self._orders.append(a)
                    orders[c] = a.ctypes.data
        h = C.c_void_p()
        _check(self.L.tkv_create(C.byref(layout), ptrs, orders, _stream(), C.byref(h)), "tkv_create")
        self.h = h
        self.Hkv, self.Hq, self.D = layout.num_kv_heads, layout.num_q_heads, layout.head_dim

    def close(self):
        if getattr(self, "h", None):
            self.L.tkv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- calls ----------------------------------------------------------------
    # Each call enqueues on `stream` (a raw HIP stream handle; default: torch's
    # current stream).  With prepare=True nothing is enqueued: a Prepared call
    # is returned instead.
    def append(self, seq_ids, positions, thought, k, v, slot_out=None, *, stream=None, prepare=False):
        n = int(seq_ids.numel())
        args = (self.h, n, _ptr(seq_ids), _ptr(positions), _ptr(thought), _ptr(k), _ptr(v), _ptr(slot_out),
                _stream(stream))
        return _issue(self.L.kv_append_quant, args, "kv_append_quant", prepare)

    def classify_append(self, seq_ids, positions, stats, tau_T, tau_E, k, v, labels_out=None, score_kind=0,
                        slot_out=None, *, stream=None, prepare=False):
        """thought_classify of `stats` rows followed by kv_append_quant with those
        labels, in one launch sequence (kv_classify_append)."""
        n = int(seq_ids.numel())
        heads = int(stats.numel()) // (3 * n) if n else 1     # every head of every layer in a row
        args = (self.h, n, _ptr(seq_ids), _ptr(positions), _ptr(stats), heads, C.c_float(tau_T), C.c_float(tau_E),
                int(score_kind), _ptr(labels_out), _ptr(k), _ptr(v), _ptr(slot_out), _stream(stream))
        return _issue(self.L.kv_classify_append, args, "kv_classify_append", prepare)

    def evict(self, seq_ids, seg_ids, keep_n, new_bits, n_ops_dev=None, n_ops=None, *, stream=None, prepare=False):
        n = int(seq_ids.numel()) if n_ops is None else int(n_ops)
        args = (self.h, n, _ptr(n_ops_dev), _ptr(seq_ids), _ptr(seg_ids), _ptr(keep_n), _ptr(new_bits),
                _stream(stream))
        return _issue(self.L.kv_evict_segment, args, "kv_evict_segment", prepare)

    def plan_budget(self, seq_ids, num, den, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits, *, stream=None,
                    prepare=False):
        args = (self.h, int(seq_ids.numel()), _ptr(seq_ids), int(num), int(den), int(max_ops), _ptr(n_ops_dev),
                _ptr(op_seq), _ptr(op_seg), _ptr(op_keep), _ptr(op_bits), _stream(stream))
        return _issue(self.L.kv_plan_budget, args, "kv_plan_budget", prepare)

    def plan_budget_evict(self, seq_ids, num, den, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits, *,
                          stream=None, prepare=False):
        """plan_budget followed by evict of the planned ops (kv_plan_budget_evict)."""
        args = (self.h, int(seq_ids.numel()), _ptr(seq_ids), int(num), int(den), int(max_ops), _ptr(n_ops_dev),
                _ptr(op_seq), _ptr(op_seg), _ptr(op_keep), _ptr(op_bits), _stream(stream))
        return _issue(self.L.kv_plan_budget_evict, args, "kv_plan_budget_evict", prepare)

    def plan_anneal_evict(self, seq_ids, r0, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits, *, stream=None,
                          prepare=False):
        """plan_anneal followed by evict of the planned ops (kv_plan_anneal_evict)."""
        args = (self.h, int(seq_ids.numel()), _ptr(seq_ids), int(r0), int(max_ops), _ptr(n_ops_dev), _ptr(op_seq),
                _ptr(op_seg), _ptr(op_keep), _ptr(op_bits), _stream(stream))
        return _issue(self.L.kv_plan_anneal_evict, args, "kv_plan_anneal_evict", prepare)

    def compact(self, seq_ids, n_dev=None, n=None, *, stream=None, prepare=False):
        k = int(seq_ids.numel()) if n is None else int(n)
        args = (self.h, k, _ptr(n_dev), _ptr(seq_ids), _stream(stream))
        return _issue(self.L.tkv_compact, args, "tkv_compact", prepare)

    def plan_anneal(self, seq_ids, r0, max_ops, n_ops_dev, op_seq, op_seg, op_keep, op_bits, *, stream=None,
                    prepare=False):
        args = (self.h, int(seq_ids.numel()), _ptr(seq_ids), int(r0), int(max_ops), _ptr(n_ops_dev),
                _ptr(op_seq), _ptr(op_seg), _ptr(op_keep), _ptr(op_bits), _stream(stream))
        return _issue(self.L.kv_plan_anneal, args, "kv_plan_anneal", prepare)

    def seq_reset(self, seq_ids, *, stream=None):
        _check(self.L.tkv_seq_reset(self.h, int(seq_ids.numel()), _ptr(seq_ids), _stream(stream)), "tkv_seq_reset")

    def workspace_bytes(self, batch, num_splits=0):
        return int(self.L.tkv_attn_workspace(self.h, int(batch), int(num_splits)))

    def attention(self, seq_ids, q_pos, q, out, workspace, stats=None, n_attended=None, k_self=None, v_self=None,
                  sinks=None, window=0, topk=8, num_splits=0, layer=0, stats_stride=0, order=None, *, stream=None,
                  prepare=False):
        a = AttnArgs(int(seq_ids.numel()), _ptr(seq_ids), _ptr(q_pos), _ptr(q), _ptr(k_self), _ptr(v_self),
                     _ptr(sinks), int(window), int(topk), int(num_splits), _ptr(out), _ptr(stats), _ptr(n_attended),
                     _ptr(workspace), int(workspace.numel() * workspace.element_size()), int(layer),
                     int(stats_stride), _ptr(order))
        args = (self.h, C.byref(a), _stream(stream))
        return _issue(self.L.paged_decode_attn, args, "paged_decode_attn", prepare, keep=a)

    def attention_noalloc(self, seq_ids, q_pos, q, out, stats=None, n_attended=None, k_self=None, v_self=None,
                          sinks=None, window=0, topk=8, num_splits=0, layer=0, stats_stride=0, order=None, *,
                          stream=None, prepare=False):
        """paged_decode_attn_noalloc: the split-K partials in the library's static
        device array instead of a caller workspace."""
        a = AttnArgs(int(seq_ids.numel()), _ptr(seq_ids), _ptr(q_pos), _ptr(q), _ptr(k_self), _ptr(v_self),
                     _ptr(sinks), int(window), int(topk), int(num_splits), _ptr(out), _ptr(stats), _ptr(n_attended),
                     None, 0, int(layer), int(stats_stride), _ptr(order))
        args = (self.h, C.byref(a), _stream(stream))
        return _issue(self.L.paged_decode_attn_noalloc, args, "paged_decode_attn_noalloc", prepare, keep=a)

    def attn_order(self, seq_ids, order, *, stream=None, prepare=False):
        """tkv_attn_order: the attention's dispatch order for this batch (order:
        device int32 [1 + batch]), to pass as attention(..., order=order)."""
        args = (self.h, int(seq_ids.numel()), _ptr(seq_ids), _ptr(order), _stream(stream))
        return _issue(self.L.tkv_attn_order, args, "tkv_attn_order", prepare)

    def kernel_timing(self, enable: bool):
        """tkv_kernel_timing: bracket every kernel launched for this cache with
        events (on), or stop (off); either drops the records so far."""
        _check(self.L.tkv_kernel_timing(self.h, 1 if enable else 0), "tkv_kernel_timing")

    def kernel_times(self, max_kernels: int = 32):
        """tkv_kernel_times: {kernel name: (total us, launches)} since timing was
        turned on, and the launches left unrecorded."""
        names = C.create_string_buffer(32 * max_kernels)
        tot = (C.c_double * max_kernels)()
        calls = (C.c_int32 * max_kernels)()
        dropped = C.c_int64()
        n = self.L.tkv_kernel_times(self.h, max_kernels, names, tot, calls, C.byref(dropped))
        if n < 0:
            _check(n, "tkv_kernel_times")
        raw = names.raw
        out = {raw[32 * i:32 * i + 32].split(b"\0", 1)[0].decode(): (tot[i], calls[i]) for i in range(min(n, max_kernels))}
        return out, dropped.value

    def get_error(self):
        k, m, n = C.c_int32(), C.c_int32(), C.c_int32()
        _check(self.L.tkv_get_error(self.h, C.byref(k), C.byref(m), C.byref(n)), "tkv_get_error")
        return k.value, m.value, n.value

    def export(self) -> Dict[str, np.ndarray]:
        host = [np.zeros(s, np.uint8) for s in self.sizes]
        ptrs = (C.c_void_p * NUM_BUFFERS)(*([h.ctypes.data for h in host[:-1]] + [None]))
        _check(self.L.tkv_export_state(self.h, ptrs), "tkv_export_state")
        return {n: host[i].view(BUFFER_DTYPES[n]) for i, n in enumerate(BUFFER_NAMES[:-1])}

    def import_(self, bufs: Dict[str, np.ndarray]):
        host = []
        for i, n in enumerate(BUFFER_NAMES[:-1]):
            a = np.ascontiguousarray(bufs[n]).view(np.uint8).ravel()
            assert a.size == self.sizes[i], (n, a.size, self.sizes[i])
            host.append(a)
        ptrs = (C.c_void_p * NUM_BUFFERS)(*([h.ctypes.data for h in host] + [None]))
        _check(self.L.tkv_import_state(self.h, ptrs), "tkv_import_state")


def classify(stats, tau_T, tau_E, labels_out, score_kind=0, *, stream=None, prepare=False):
    B = int(stats.shape[0])
    Hq = int(stats.numel()) // (3 * B) if B else 0          # every head of every layer in the rows
    args = (B, Hq, _ptr(stats), C.c_float(tau_T), C.c_float(tau_E), int(score_kind), _ptr(labels_out),
            _stream(stream))
    return _issue(load().thought_classify, args, "thought_classify", prepare)


def stream_read(buf, sink, *, stream=None, prepare=False):
    """Streaming 128-bit read of a whole device tensor (the HBM read ceiling)."""
    nbytes = int(buf.numel() * buf.element_size())
    args = (_ptr(buf), C.c_size_t(nbytes), _ptr(sink), _stream(stream))
    return _issue(load().tkv_stream_read, args, "tkv_stream_read", prepare)
