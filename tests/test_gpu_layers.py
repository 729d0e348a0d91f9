"""GPU parity of the layered cache (several layers sharing block tables,
segments and eviction) against the oracle.

Method passages: ThinKV technical summary, "Methodologie": thought types and
eviction belong to tokens (TBQ, TBE bullets) and the block table with
eviction masks is per sequence (Continuous Thinking bullet), so every
layer's K/V of a token share one slot.  State bit for bit; attention of every
layer within the attention tolerances; the statistics of all layers written
into one array through stats_stride, and the labels classified over all of
them.
"""
import dataclasses

import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import TOL_ABS, TOL_L2, TOL_STAT, _check_labels, say

pytestmark = pytest.mark.gpu


def layered_attention(gc, w, NL, **kw):
    """Every layer's attention on the device; statistics into one [B][NL][Hq][3] array."""
    import torch
    L = w.layout
    B, Hq, D = w.seq_ids.size, L.num_q_heads, L.head_dim
    dv = helpers.dev
    stats = torch.full((B, NL, Hq, 3), -1.0, dtype=torch.float32, device="cuda")
    outs = []
    ws = torch.empty(max(gc.workspace_bytes(B, 0), 16), dtype=torch.uint8, device="cuda")
    for l in range(NL):
        out = torch.empty(B, Hq, D, dtype=torch.float32, device="cuda")
        gc.attention(dv(w.seq_ids, np.int32), dv(w.q_pos, np.int32), dv(synth.layer_queries(w, l), np.uint16), out,
                     ws, stats=stats[:, l], layer=l, stats_stride=NL * Hq * 3, **kw)
        outs.append(out)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs], stats.cpu().numpy()


def check_layers(gc, oc, w, NL, tag, **kw):
    outs, stats = layered_attention(gc, w, NL, **kw)
    ref_stats = []
    for l in range(NL):
        ro, rs, rn = oc.attention(w.seq_ids, w.q_pos, synth.layer_queries(w, l), layer=l, **kw)
        mabs, rl2 = helpers.attn_metrics(outs[l], ro)
        assert mabs <= TOL_ABS and rl2 <= TOL_L2, f"{tag} layer {l}: {mabs:.2e} {rl2:.2e}"
        assert np.abs(stats[:, l, :, 1:] - rs[..., 1:]).max() <= TOL_STAT, f"{tag} layer {l} stats"
        ref_stats.append(rs)
    return stats, np.stack(ref_stats, axis=1)


@pytest.mark.parametrize("D,g,NL", [(128, 64, 3), (64, 32, 2)])
def test_layers_small(D, g, NL):
    """Build, every layer's attention (with the self token: each layer's own
    rows), labels over all layers, then a downgrade, an eviction and a
    compaction, and every layer again."""
    import torch
    import oracle
    from thought_adaptive_mixed_amd import binding
    w = synth.small_static(seed=90, B=3, Hq=8, Hkv=2, D=D, g=g, permute=False)
    w.layout = dataclasses.replace(w.layout, pool_blocks=tuple(2 * p for p in w.layout.pool_blocks))
    w = synth.layered(w, NL)
    L = w.layout
    say(f"[layers] D{D} NL{NL} build")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    helpers.compare_states(L, gc.export(), oc.export(), "layered build")
    stats, rstats = check_layers(gc, oc, w, NL, "build")
    # labels over every layer's heads (mean of H/ln n over NL*Hq heads)
    B, Hq = w.seq_ids.size, L.num_q_heads
    labels = torch.zeros(B, dtype=torch.uint8, device="cuda")
    tT, tE = 0.6, 0.9
    binding.classify(helpers.dev(stats.reshape(B, NL * Hq, 3), np.float32), tT, tE, labels)
    lab_o = oracle.classify(rstats.reshape(B, NL * Hq, 3).astype(np.float32), tT, tE)
    _check_labels(labels.cpu().numpy(), lab_o, rstats.reshape(B, NL * Hq, 3), tT, tE, 0)
    # downgrade every layer's rows of an E segment, evict part of an R segment, compact
    s = int(w.seq_ids[0])
    segs = oc.segments(s)
    e = [k for k in range(len(segs) - 1) if segs[k][0] == 1 and segs[k][1] == 4 and segs[k][5] > 2]
    r = [k for k in range(len(segs) - 1) if segs[k][0] == 0 and segs[k][5] > 1]
    ops = [np.array(x, np.int32) for x in ([s, s], [e[0], r[0]], [int(segs[e[0]][5]) - 1, 1])] + \
          [np.array([2, 0], np.uint8)]
    say(f"[layers] D{D} NL{NL} evict + compact")
    dv = helpers.dev
    gc.evict(dv(ops[0]), dv(ops[1]), dv(ops[2]), dv(ops[3]))
    oc.evict(*ops)
    gc.compact(dv(w.seq_ids, np.int32))
    oc.compact(w.seq_ids)
    torch.cuda.synchronize()
    helpers.compare_states(L, gc.export(), oc.export(), "layered after evict + compact")
    assert gc.get_error() == oc.error()
    check_layers(gc, oc, w, NL, "after evict + compact")


def test_layers_full_size():
    """The llama8b-like layer's state with 2 layers: sampled attention of each layer."""
    w = synth.layered(synth.WORKLOADS["llama8b"](), 2)
    L = w.layout
    say("[layers] llama8b x2 build")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    helpers.compare_states(L, gc.export(), oc.export(), "llama8b x2")
    sel = np.arange(0, w.seq_ids.size, 4)
    ws = dataclasses.replace(w, seq_ids=w.seq_ids[sel], q_pos=w.q_pos[sel], q_bf16=w.q_bf16[sel])
    check_layers(gc, oc, ws, 2, "llama8b x2")


def test_layers_lockstep():
    """Decode loop over 2 layers: every layer's attention (with its own self
    token rows), labels over both layers, one append of both layers' rows,
    the budget ladder and evictions; state every 8 steps."""
    import torch
    import oracle
    from thought_adaptive_mixed_amd import binding
    NL = 2
    ch = synth.small_churn(seed=93, steps=48)
    ch.base = synth.layered(ch.base, NL)
    w = ch.base
    L = w.layout
    B, Hq, Hkv, D = w.seq_ids.size, L.num_q_heads, L.num_kv_heads, L.head_dim
    say("[layers-loop] build")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    dv = helpers.dev
    seq_d = dv(w.seq_ids, np.int32)
    max_ops = 64
    n_ops = torch.zeros(1, dtype=torch.int32, device="cuda")
    o_seq = torch.zeros(max_ops, dtype=torch.int32, device="cuda")
    o_seg = torch.zeros_like(o_seq); o_keep = torch.zeros_like(o_seq)
    o_bits = torch.zeros(max_ops, dtype=torch.uint8, device="cuda")
    labels = torch.zeros(B, dtype=torch.uint8, device="cuda")
    tT, tE = ch.tau
    for s in range(ch.steps):
        q, k, v, pos = ch.step_inputs(s)            # k, v: [B][NL*Hkv][D], every layer's rows
        stats = torch.zeros((B, NL, Hq, 3), dtype=torch.float32, device="cuda")
        rstats = np.zeros((B, NL, Hq, 3))
        for l in range(NL):
            kl, vl = k[:, l * Hkv:(l + 1) * Hkv], v[:, l * Hkv:(l + 1) * Hkv]
            ql = q if l == 0 else synth.layer_queries(dataclasses.replace(w, q_bf16=q), l)
            out = torch.empty(B, Hq, D, dtype=torch.float32, device="cuda")
            ws = torch.empty(max(gc.workspace_bytes(B, 0), 16), dtype=torch.uint8, device="cuda")
            gc.attention(seq_d, dv(pos, np.int32), dv(ql, np.uint16), out, ws, stats=stats[:, l],
                         k_self=dv(kl, np.float32), v_self=dv(vl, np.float32), layer=l, stats_stride=NL * Hq * 3)
            ro, rs, rn = oc.attention(w.seq_ids, pos, ql, k_self=kl, v_self=vl, layer=l)
            torch.cuda.synchronize()
            mabs, rl2 = helpers.attn_metrics(out.cpu().numpy(), ro)
            assert mabs <= TOL_ABS and rl2 <= TOL_L2, (s, l)
            rstats[:, l] = rs
        binding.classify(stats.reshape(B, NL * Hq, 3), tT, tE, labels)
        lab_o = oracle.classify(rstats.reshape(B, NL * Hq, 3).astype(np.float32), tT, tE)
        _check_labels(labels.cpu().numpy(), lab_o, rstats.reshape(B, NL * Hq, 3), tT, tE, s)
        gc.append(seq_d, dv(pos, np.int32), dv(lab_o, np.uint8), dv(k, np.float32), dv(v, np.float32))
        oc.append(w.seq_ids, pos, lab_o, k, v)
        gc.plan_budget(seq_d, ch.budget[0], ch.budget[1], max_ops, n_ops, o_seq, o_seg, o_keep, o_bits)
        ops = oc.plan_budget(w.seq_ids, ch.budget[0], ch.budget[1], max_ops)
        gc.evict(o_seq, o_seg, o_keep, o_bits, n_ops_dev=n_ops, n_ops=max_ops)
        if ops[0].size:
            oc.evict(*ops)
        if s % 8 == 7 or s == ch.steps - 1:
            helpers.compare_states(L, gc.export(), oc.export(), f"layers step {s}")
    assert gc.get_error() == oc.error()
