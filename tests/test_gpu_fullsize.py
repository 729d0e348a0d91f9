"""GPU parity at the full sizes of the measured workloads, in the launch
configuration the bench uses (library-chosen waves and splits).

The whole cache state built through the C-ABI must equal the oracle's bit
for bit, and every attention row (every batch entry and query head) is
compared with the oracle's: outputs within max-abs 2e-3 and relative L2
1e-3, normalized entropy and top-k mass within 1e-4, attended counts exact.
"""
import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import _check_labels, check_attention, gpu_attention, say

pytestmark = pytest.mark.gpu


def _properties(w, got, window):
    out, stats, n_att = got
    assert np.isfinite(out).all() and np.isfinite(stats).all()
    assert (stats[..., 1] >= -1e-6).all() and (stats[..., 1] <= 1 + 1e-5).all()
    assert (stats[..., 2] > 0).all() and (stats[..., 2] <= 1 + 1e-5).all()
    if window == 0:
        assert np.array_equal(n_att, w.retained.astype(np.int32)), "attended = retained tokens"
    else:
        assert (n_att <= min(window, int(w.retained.max()))).all() and (n_att >= 1).all()


def _worst_row(go, ro):
    d = np.abs(go.astype(np.float64) - ro).reshape(go.shape[0], -1).max(axis=1)
    return int(d.argmax()), float(d.max())


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama8b", "qwen14b", "gptoss20b"])
def test_fullsize_state_and_attention(name):
    say(f"[fullsize] {name}: building")
    w = synth.WORKLOADS[name]()
    gc = helpers.build_gpu(w)
    oc = helpers.build_oracle(w)
    say(f"[fullsize] {name}: comparing state")
    helpers.compare_states(w.layout, gc.export(), oc.export(), name)
    for window in w.windows:
        say(f"[fullsize] {name}: attention W={window}")
        got = gpu_attention(gc, w.seq_ids, w.q_pos, w.q_bf16, window=window, sinks=w.sinks)
        _properties(w, got, window)
        ref = oc.attention(w.seq_ids, w.q_pos, w.q_bf16, window=window, sinks=w.sinks)
        b, worst = _worst_row(got[0], ref[0])
        say(f"[fullsize] {name} W={window}: worst batch entry {b} max-abs {worst:.2e}")
        check_attention(f"{name} W={window} all {w.seq_ids.size} rows", got, ref)


@pytest.mark.timeout(900)
def test_fullshape_churn():
    """The churn loop at full shape (B256, Hq32/Hkv8, D128, starting lengths
    U{4k..32k}, 5% budget) for 128 decode steps in the calls the bench times:
    attention with the self token (in the dispatch order of tkv_attn_order,
    renewed every 16 steps), kv_classify_append, kv_plan_budget_evict.
    Every step: all 256 attention rows against the oracle, the GPU's own
    labels against the oracle's outside the threshold ambiguity band, the
    fused call's labels (fed the oracle's fp32 statistics) equal to the
    oracle's, op lists equal.  The whole state bit for bit at steps 64 and
    128 (and after the build)."""
    import torch
    import oracle
    from thought_adaptive_mixed_amd import binding
    steps = 128
    ch = synth.churn(steps=steps)
    w = ch.base
    L = w.layout
    say("[churn-full] build")
    gc = helpers.build_gpu(w)
    oc = helpers.build_oracle(w)
    helpers.compare_states(L, gc.export(), oc.export(), "churn-full build")
    B = w.seq_ids.size
    dv = helpers.dev
    seq_d = dv(w.seq_ids, np.int32)
    max_ops = 1024
    n_ops = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = [torch.zeros(max_ops, dtype=torch.int32, device="cuda") for _ in range(3)]
    o_bits = torch.zeros(max_ops, dtype=torch.uint8, device="cuda")
    labels_g = torch.zeros(B, dtype=torch.uint8, device="cuda")
    labels_f = torch.zeros(B, dtype=torch.uint8, device="cuda")
    tT, tE = ch.tau
    amb = n_ev = n_down = 0
    worst = 0.0
    order = torch.zeros(1 + B, dtype=torch.int32, device="cuda")
    for s in range(steps):
        q, k, v, pos = ch.step_inputs(s)
        if s % 16 == 0:                       # the dispatch order, renewed as the bench does
            gc.attn_order(seq_d, order)
        go, gs, gn = gpu_attention(gc, w.seq_ids, pos, q, k_self=k, v_self=v, order=order)
        ro, rs, rn = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
        check_attention(f"step {s} all rows", (go, gs, gn), (ro, rs, rn)) if s % 16 == 0 else None
        mabs, rl2 = helpers.attn_metrics(go, ro)
        worst = max(worst, mabs)
        assert np.array_equal(gn, rn), f"n_attended step {s}"
        assert mabs <= 2e-3 and rl2 <= 1e-3, (s, mabs, rl2)
        assert np.abs(gs[..., 1:] - rs[..., 1:]).max() <= 1e-4, s
        rs32 = rs.astype(np.float32)
        lab_o = oracle.classify(rs32, tT, tE)
        # the GPU's labels from its own statistics, outside the ambiguity band
        binding.classify(dv(gs, np.float32), tT, tE, labels_g)
        amb += _check_labels(labels_g.cpu().numpy(), lab_o, rs, tT, tE, s)
        # the fused classification + append, fed the oracle's statistics:
        # labels bit for bit, and both sides append at them
        pos_d = dv(pos, np.int32)
        gc.classify_append(seq_d, pos_d, dv(rs32), tT, tE, dv(k, np.float32), dv(v, np.float32),
                           labels_out=labels_f)
        oc.append(w.seq_ids, pos, lab_o, k, v)
        assert np.array_equal(labels_f.cpu().numpy(), lab_o), f"fused labels step {s}"
        gc.plan_budget_evict(seq_d, ch.budget[0], ch.budget[1], max_ops, n_ops, *o, o_bits)
        ops = oc.plan_budget(w.seq_ids, ch.budget[0], ch.budget[1], max_ops)
        m = int(n_ops.item())
        assert m == ops[0].size, f"op count step {s}"
        for a, b in zip([x.cpu().numpy()[:m] for x in (*o, o_bits)], ops):
            assert np.array_equal(a, b), f"ops step {s}"
        if m:
            oc.evict(*ops)
            n_down += int((ops[3] == 2).sum()); n_ev += int((ops[3] == 0).sum())
        if (s + 1) % 64 == 0:
            say(f"[churn-full] step {s + 1}: whole state")
            helpers.compare_states(L, gc.export(), oc.export(), f"churn-full after step {s + 1}")
    say(f"[churn-full] {steps} steps x {B} sequences: worst max-abs {worst:.2e}, {amb} labels in the "
        f"ambiguity band, {n_ev} segment evictions, {n_down} downgrades")
    assert gc.get_error() == oc.error()
    assert n_ev > 0


@pytest.mark.timeout(900)
def test_fullshape_churn_1024_steps():
    """The churn loop at full shape for 1024 decode steps (B256, Hq32/Hkv8,
    D128, starting lengths U{4k..32k}, 5% budget): every step appends each
    sequence's new token at its planted thought type (kv_append_quant, the
    same labels on both sides, so the oracle needs no attention between
    checks) and runs kv_plan_budget_evict; the op lists equal the oracle's at
    every step, the whole state is bit for bit the oracle's every 64 steps,
    and every 128 steps all 256 attention rows are checked against the
    oracle's.  This is the long horizon over which allocator drift (free
    stacks, block lists, segment tables) would show."""
    import torch
    steps = 1024
    ch = synth.churn(steps=steps)
    w = ch.base
    L = w.layout
    say("[churn-1024] build")
    gc = helpers.build_gpu(w)
    oc = helpers.build_oracle(w)
    B = w.seq_ids.size
    dv = helpers.dev
    seq_d = dv(w.seq_ids, np.int32)
    max_ops = 1024
    n_ops = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = [torch.zeros(max_ops, dtype=torch.int32, device="cuda") for _ in range(3)]
    o_bits = torch.zeros(max_ops, dtype=torch.uint8, device="cuda")
    n_ev = n_down = 0
    for s in range(steps):
        q, k, v, pos = ch.step_inputs(s)
        lab = ch.target_types[s].astype(np.uint8)
        if s % 128 == 0:
            got = gpu_attention(gc, w.seq_ids, pos, q, k_self=k, v_self=v)
            ref = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
            check_attention(f"churn-1024 step {s} all {B} rows", got, ref)
        gc.append(seq_d, dv(pos, np.int32), dv(lab), dv(k, np.float32), dv(v, np.float32))
        oc.append(w.seq_ids, pos, lab, k, v)
        gc.plan_budget_evict(seq_d, ch.budget[0], ch.budget[1], max_ops, n_ops, *o, o_bits)
        ops = oc.plan_budget(w.seq_ids, ch.budget[0], ch.budget[1], max_ops)
        m = int(n_ops.item())
        assert m == ops[0].size, f"op count step {s}"
        for a, b in zip([x.cpu().numpy()[:m] for x in (*o, o_bits)], ops):
            assert np.array_equal(a, b), f"ops step {s}"
        if m:
            oc.evict(*ops)
            n_down += int((ops[3] == 2).sum()); n_ev += int((ops[3] == 0).sum())
        if (s + 1) % 64 == 0:
            say(f"[churn-1024] step {s + 1}: whole state ({n_ev} evictions, {n_down} downgrades so far)")
            helpers.compare_states(L, gc.export(), oc.export(), f"churn-1024 after step {s + 1}")
    assert gc.get_error() == oc.error()
    assert n_ev > 0 and n_down > 0
