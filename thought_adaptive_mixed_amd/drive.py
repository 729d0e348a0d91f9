"""Drive the C-ABI from a seeded workload description: build a cache state on
the GPU through kv_append_quant / kv_evict_segment calls, and move numpy
arrays to the device.  Argument marshalling only (every step of the path runs
in libthinkv.so)."""
from __future__ import annotations

import numpy as np

from . import binding, synth


def gpu_layout(L: synth.Layout) -> binding.Layout:
    """The C layout struct of a workload's layout."""
    return binding.make_layout(L.num_kv_heads, L.num_q_heads, L.head_dim, L.group_size, L.pool_blocks,
                               L.max_seqs, L.max_blocks_per_seq, L.max_segments_per_seq, L.max_tokens_per_call,
                               L.bits, L.num_layers, L.code_format)


def dev(a, dtype=None):
    """A contiguous device copy of a numpy array (optionally cast first)."""
    import torch
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype))
    return torch.from_numpy(a).cuda()


def build_gpu(w: synth.Workload, cache: binding.Cache = None) -> binding.Cache:
    """Replay a workload's append and evict calls through the C-ABI on a new
    (or the given) cache."""
    gc = cache or binding.Cache(gpu_layout(w.layout), w.block_order)
    for call in w.calls:
        if isinstance(call, synth.AppendCall):
            k, v = w.kv(call)
            gc.append(dev(call.seq_ids), dev(call.positions), dev(call.thought), dev(k), dev(v))
        else:
            gc.evict(dev(call.seq_ids), dev(call.seg_ids), dev(call.keep_n), dev(call.new_bits))
    return gc
