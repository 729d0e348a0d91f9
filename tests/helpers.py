"""Shared test helpers: build a workload's cache state on the oracle and on the
HIP path from the same seeded calls, and compare exported states."""
from __future__ import annotations

import numpy as np

from thought_adaptive_mixed_amd import synth

BS = 16


def oracle_layout(L: synth.Layout):
    import oracle
    return oracle.OracleLayout(L.num_kv_heads, L.num_q_heads, L.head_dim, L.group_size, L.pool_blocks,
                               L.max_seqs, L.max_blocks_per_seq, L.max_segments_per_seq, L.bits)


def build_oracle(w: synth.Workload):
    import oracle
    oc = oracle.OracleCache(oracle_layout(w.layout), w.block_order)
    for call in w.calls:
        if isinstance(call, synth.AppendCall):
            k, v = w.kv(call)
            oc.append(call.seq_ids, call.positions, call.thought, k, v)
        else:
            oc.evict(call.seq_ids, call.seg_ids, call.keep_n, call.new_bits)
    return oc
