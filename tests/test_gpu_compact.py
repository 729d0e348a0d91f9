"""GPU parity of the gather-compaction baseline (tkv_compact) against the oracle.

Method passages: ThinKV abstract (the kernel reuses evicted tokens' slots and
so eliminates compaction) and the technical summary's Continuous Thinking
bullet.  The compacted state must match the oracle's bit for bit (valid
tokens' bits, block and slot records, block lists, stacks, free stacks, error
word); attention over it must match the oracle's.
"""
import dataclasses

import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import check_attention, gpu_attention, say

pytestmark = pytest.mark.gpu


def roomy(w, factor=2):
    """The workload with its pools enlarged (compaction pops before it returns)."""
    w.layout = dataclasses.replace(w.layout, pool_blocks=tuple(factor * p for p in w.layout.pool_blocks))
    w.block_order = None
    return w


def compact_both(gc, oc, L, ids, tag):
    import torch
    gc.compact(helpers.dev(np.array(ids, np.int32), np.int32))
    oc.compact(np.array(ids, np.int32))
    torch.cuda.synchronize()
    helpers.compare_states(L, gc.export(), oc.export(), tag)
    err = oc.error()
    assert gc.get_error() == err, tag               # reading the device word clears it
    oc.clear_error()
    return err


@pytest.mark.parametrize("D,g", [(128, 64), (64, 32)])
def test_compact_small(D, g):
    """Every sequence compacted (list with repeats and bad ids), then attention
    over the compacted cache, then a second compaction (a no-op move of dense
    blocks into fresh ones)."""
    w = roomy(synth.small_static(seed=86, B=4, Hq=8, Hkv=2, D=D, g=g, permute=False))
    L = w.layout
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    ids = [int(s) for s in w.seq_ids]
    say(f"[compact] D{D} g{g} first")
    compact_both(gc, oc, L, [ids[2], -1, ids[0], ids[2], L.max_seqs, ids[1], ids[3], ids[0]], "first")
    got = gpu_attention(gc, w.seq_ids, w.q_pos, w.q_bf16)
    check_attention(f"D{D} compacted", got, oc.attention(w.seq_ids, w.q_pos, w.q_bf16))
    say(f"[compact] D{D} g{g} again")
    compact_both(gc, oc, L, ids, "again")


def test_compact_out_of_blocks():
    """Pools with little room: some sequences fail with ENOMEM (and every later
    one needing the dry class), the others are compacted."""
    w = synth.small_static(seed=87, B=4, Hq=8, Hkv=2, D=64, g=32, permute=False)
    L = w.layout
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    say("[compact] out of blocks")
    err = compact_both(gc, oc, L, [int(s) for s in w.seq_ids], "dry")
    assert err[0] & (1 << 2), "the pools were expected to run dry"


@pytest.mark.parametrize("name", ["llama8b", "qwen14b"])
def test_compact_full_size(name):
    """Full-size states (permuted block order for qwen14b): all sequences in
    reverse list order, then sampled attention against the oracle."""
    w = synth.WORKLOADS[name]()
    w = roomy(w) if name == "llama8b" else w
    L = w.layout
    say(f"[compact] build {name}")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    say(f"[compact] {name} compact")
    compact_both(gc, oc, L, [int(s) for s in w.seq_ids[::-1]], name)
    sel = np.arange(0, w.seq_ids.size, max(1, w.seq_ids.size // 8))
    got = gpu_attention(gc, w.seq_ids[sel], w.q_pos[sel], w.q_bf16[sel])
    check_attention(f"{name} compacted", got, oc.attention(w.seq_ids[sel], w.q_pos[sel], w.q_bf16[sel]))


def test_compact_after_evictions_lockstep():
    """Decode loop with the budget ladder and, after every eviction, the
    compaction of the sequences the op list names (read from the device op
    count): outputs every step, state every 8 steps."""
    import torch
    import oracle
    ch = synth.small_churn(seed=92)
    w = roomy(ch.base)
    L = w.layout
    say("[compact-loop] build")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    dv = helpers.dev
    seq_d = dv(w.seq_ids, np.int32)
    max_ops = 64
    n_ops = torch.zeros(1, dtype=torch.int32, device="cuda")
    o_seq = torch.zeros(max_ops, dtype=torch.int32, device="cuda")
    o_seg = torch.zeros_like(o_seq); o_keep = torch.zeros_like(o_seq)
    o_bits = torch.zeros(max_ops, dtype=torch.uint8, device="cuda")
    tT, tE = ch.tau
    n_compacted = 0
    for s in range(ch.steps):
        q, k, v, pos = ch.step_inputs(s)
        go, gs, gn = gpu_attention(gc, w.seq_ids, pos, q, k_self=k, v_self=v)
        ro, rs, rn = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
        if s % 8 == 0:
            check_attention(f"step {s}", (go, gs, gn), (ro, rs, rn))
        lab_o = oracle.classify(rs.astype(np.float32), tT, tE)
        gc.append(seq_d, dv(pos, np.int32), dv(lab_o, np.uint8), dv(k, np.float32), dv(v, np.float32))
        oc.append(w.seq_ids, pos, lab_o, k, v)
        gc.plan_budget(seq_d, ch.budget[0], ch.budget[1], max_ops, n_ops, o_seq, o_seg, o_keep, o_bits)
        ops = oc.plan_budget(w.seq_ids, ch.budget[0], ch.budget[1], max_ops)
        gc.evict(o_seq, o_seg, o_keep, o_bits, n_ops_dev=n_ops, n_ops=max_ops)
        gc.compact(o_seq, n_dev=n_ops, n=max_ops)
        if ops[0].size:
            oc.evict(*ops)
            oc.compact(ops[0])
            n_compacted += len(set(ops[0].tolist()))
        if s % 8 == 7 or s == ch.steps - 1:
            helpers.compare_states(L, gc.export(), oc.export(), f"compact step {s}")
            assert gc.get_error() == oc.error(), s
            oc.clear_error()
    say(f"[compact-loop] steps={ch.steps} compactions={n_compacted}")
    assert n_compacted > 0
