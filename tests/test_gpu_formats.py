"""GPU parity of the float / ternary code formats (code_format 1) against
the oracle.

Method passage: ThinKV technical summary, "Methodology", TBQ bullet: 8-bit
FP8 or 4-bit NVFP4 for Reasoning tokens, 2-bit ternary for Transition tokens,
by group quantization.  Codes, scales and zero-points bit for bit after the
appends, the downgrades (8 -> 4, 8 -> 2, 4 -> 2 re-quantize the
reconstruction), evictions and compactions; attention within the attention
tolerances.
"""
import dataclasses

import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import _check_labels, check_attention, gpu_attention, say, TOL_ABS, TOL_L2, TOL_STAT

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "llama8b", "gptoss20b"])
def test_formats_build_and_attention(name):
    """Built state (appends, downgrades and evictions of the workload's call
    list) bit for bit, then attention with and without the self token, with
    the workload's windows and sinks, at 1 and 3 splits (sampled entries for
    the large caches)."""
    w = synth.page_formats(synth.WORKLOADS[name]())
    L = w.layout
    say(f"[formats] build {name}")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    helpers.compare_states(L, gc.export(), oc.export(), f"formats {name}")
    assert gc.get_error() == oc.error()
    B = w.seq_ids.size
    sel = np.arange(B) if B <= 8 else np.arange(0, B, B // 8)
    ws = dataclasses.replace(w, seq_ids=w.seq_ids[sel], q_pos=w.q_pos[sel], q_bf16=w.q_bf16[sel])
    rng = np.random.default_rng(6)
    ks = rng.standard_normal((sel.size, L.num_kv_heads, L.head_dim)).astype(np.float32)
    vs = rng.standard_normal((sel.size, L.num_kv_heads, L.head_dim)).astype(np.float32)
    for window in w.windows:
        for self_tok in (False, True):
            for splits in (0, 3):
                tag = f"formats {name} W={window} self={self_tok} splits={splits}"
                say(f"[attn] {tag}")
                kw = dict(window=window, sinks=w.sinks)
                if self_tok:
                    kw.update(k_self=ks, v_self=vs)
                got = gpu_attention(gc, ws.seq_ids, ws.q_pos, ws.q_bf16, splits=splits, **kw)
                check_attention(tag, got, oc.attention(ws.seq_ids, ws.q_pos, ws.q_bf16, **kw))


@pytest.mark.parametrize("D,g,NL", [(128, 64, 1), (64, 32, 1), (128, 32, 2)])
def test_formats_downgrade_evict_compact(D, g, NL):
    """Explicit downgrades of every kind (FP8 -> FP4, FP8 -> ternary, FP4 ->
    ternary), an eviction, then a compaction of every sequence; state and
    attention (every layer) after each stage."""
    import torch
    w = synth.small_static(seed=94, B=4, Hq=8, Hkv=2, D=D, g=g, L=2400, permute=False)
    w.layout = dataclasses.replace(w.layout, pool_blocks=tuple(5 * p for p in w.layout.pool_blocks))
    w = synth.page_formats(synth.layered(w, NL) if NL > 1 else w)
    L = w.layout
    say(f"[formats] D{D} g{g} NL{NL} build")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    helpers.compare_states(L, gc.export(), oc.export(), "formats small build")
    dv = helpers.dev

    def attention_all(tag):
        for l in range(NL):
            q = synth.layer_queries(w, l)
            Hq = L.num_q_heads
            out = torch.empty(w.seq_ids.size, Hq, D, dtype=torch.float32, device="cuda")
            st = torch.empty(w.seq_ids.size, Hq, 3, dtype=torch.float32, device="cuda")
            na = torch.empty(w.seq_ids.size, dtype=torch.int32, device="cuda")
            ws = torch.empty(max(gc.workspace_bytes(w.seq_ids.size, 0), 16), dtype=torch.uint8, device="cuda")
            gc.attention(dv(w.seq_ids, np.int32), dv(w.q_pos, np.int32), dv(q, np.uint16), out, ws, stats=st,
                         n_attended=na, layer=l)
            torch.cuda.synchronize()
            check_attention(f"{tag} layer {l}", (out.cpu().numpy(), st.cpu().numpy(), na.cpu().numpy()),
                            oc.attention(w.seq_ids, w.q_pos, q, layer=l))

    attention_all("built")
    # 8-bit segments in turn: to 4 bits, to 2 bits, evicted down to one token;
    # 4-bit segments: to 2 bits.  Each keeps all but its oldest token.
    ops = ([], [], [], [])
    r_plan, n_r = (4, 2, 0), 0
    for s in w.seq_ids:
        segs = oc.segments(int(s))
        for k in range(len(segs)):
            if segs[k][5] < 2:
                continue
            if segs[k][1] == 8:
                nb = r_plan[n_r % 3]; n_r += 1
            elif segs[k][1] == 4:
                nb = 2
            else:
                continue
            ops[0].append(int(s)); ops[1].append(k); ops[2].append(int(segs[k][5]) - 1); ops[3].append(nb)
    ops = [np.array(ops[0], np.int32), np.array(ops[1], np.int32), np.array(ops[2], np.int32),
           np.array(ops[3], np.uint8)]
    assert (ops[3] == 2).sum() >= 2 and (ops[3] == 4).sum() >= 1 and (ops[3] == 0).sum() >= 1
    say(f"[formats] D{D} g{g} NL{NL} {ops[0].size} ops")
    gc.evict(*[dv(a) for a in ops])
    oc.evict(*ops)
    torch.cuda.synchronize()
    helpers.compare_states(L, gc.export(), oc.export(), "formats after downgrades")
    assert gc.get_error() == oc.error() and oc.error()[0] == 0
    attention_all("downgraded")
    gc.compact(dv(w.seq_ids, np.int32))
    oc.compact(w.seq_ids)
    torch.cuda.synchronize()
    helpers.compare_states(L, gc.export(), oc.export(), "formats after compaction")
    assert gc.get_error() == oc.error() and oc.error()[0] == 0
    attention_all("compacted")


def test_formats_churn_lockstep():
    """Decode loop in the page formats: attention with the self token ->
    classify -> append -> budget ladder (FP4 -> ternary downgrades, T
    evictions), lockstep with the oracle; state every 8 steps."""
    import torch
    import oracle
    from thought_adaptive_mixed_amd import binding
    ch = synth.small_churn(seed=95, steps=64)
    ch.base = synth.page_formats(ch.base)
    w = ch.base
    L = w.layout
    say("[formats-churn] build")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    B = w.seq_ids.size
    dv = helpers.dev
    seq_d = dv(w.seq_ids, np.int32)
    max_ops = 64
    n_ops = torch.zeros(1, dtype=torch.int32, device="cuda")
    o_seq = torch.zeros(max_ops, dtype=torch.int32, device="cuda")
    o_seg = torch.zeros_like(o_seq); o_keep = torch.zeros_like(o_seq)
    o_bits = torch.zeros(max_ops, dtype=torch.uint8, device="cuda")
    labels_d = torch.zeros(B, dtype=torch.uint8, device="cuda")
    tT, tE = ch.tau
    n_down = 0
    for s in range(ch.steps):
        q, k, v, pos = ch.step_inputs(s)
        go, gs, gn = gpu_attention(gc, w.seq_ids, pos, q, k_self=k, v_self=v)
        ro, rs, rn = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
        mabs, rl2 = helpers.attn_metrics(go, ro)
        assert mabs <= TOL_ABS and rl2 <= TOL_L2 and np.abs(gs[..., 1:] - rs[..., 1:]).max() <= TOL_STAT, s
        lab_o = oracle.classify(rs.astype(np.float32), tT, tE)
        binding.classify(dv(gs, np.float32), tT, tE, labels_d)
        _check_labels(labels_d.cpu().numpy(), lab_o, rs, tT, tE, s)
        gc.append(seq_d, dv(pos, np.int32), dv(lab_o, np.uint8), dv(k, np.float32), dv(v, np.float32))
        oc.append(w.seq_ids, pos, lab_o, k, v)
        gc.plan_budget(seq_d, ch.budget[0], ch.budget[1], max_ops, n_ops, o_seq, o_seg, o_keep, o_bits)
        ops = oc.plan_budget(w.seq_ids, ch.budget[0], ch.budget[1], max_ops)
        gc.evict(o_seq, o_seg, o_keep, o_bits, n_ops_dev=n_ops, n_ops=max_ops)
        if ops[0].size:
            oc.evict(*ops)
            n_down += int((ops[3] == 2).sum())
        if s % 8 == 7 or s == ch.steps - 1:
            helpers.compare_states(L, gc.export(), oc.export(), f"formats churn step {s}")
    say(f"[formats-churn] steps={ch.steps} downgrades={n_down}")
    assert n_down > 0
    assert gc.get_error() == oc.error()
