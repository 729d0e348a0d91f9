"""GPU parity at the full sizes of the measured workloads, in the launch
configuration the bench uses (library-chosen waves and splits).

The whole cache state built through the C-ABI must equal the oracle's bit
for bit; attention is checked against the oracle on sampled batch entries
(the oracle computes them one by one) and by properties on every entry.
"""
import sys

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


@pytest.mark.parametrize("name", ["llama8b", "qwen14b", "gptoss20b"])
def test_fullsize_state_and_attention(name):
    say(f"[fullsize] {name}: building")
    w = synth.WORKLOADS[name]()
    gc = helpers.build_gpu(w)
    oc = helpers.build_oracle(w)
    say(f"[fullsize] {name}: comparing state")
    helpers.compare_states(w.layout, gc.export(), oc.export(), name)
    B = w.seq_ids.size
    rng = np.random.default_rng(11)
    sample = np.sort(rng.choice(B, min(4, B), replace=False))
    for window in w.windows:
        say(f"[fullsize] {name}: attention W={window}")
        got = gpu_attention(gc, w.seq_ids, w.q_pos, w.q_bf16, window=window, sinks=w.sinks)
        _properties(w, got, window)
        ref = oc.attention(w.seq_ids[sample], w.q_pos[sample], w.q_bf16[sample], window=window, sinks=w.sinks)
        check_attention(f"{name} W={window} rows {sample.tolist()}",
                        tuple(a[sample] for a in got), ref)


def test_fullshape_churn():
    """The churn loop at full shape (B256, Hq32/Hkv8, D128, starting lengths
    U{4k..32k}, 5% budget) for a bounded number of steps, in lockstep with
    the oracle: labels and sampled outputs every step, full state every 8."""
    import torch
    import oracle
    from thought_adaptive_mixed_amd import binding
    steps = 24
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
    labels_d = torch.zeros(B, dtype=torch.uint8, device="cuda")
    tT, tE = ch.tau
    rng = np.random.default_rng(3)
    amb = 0
    for s in range(steps):
        q, k, v, pos = ch.step_inputs(s)
        go, gs, gn = gpu_attention(gc, w.seq_ids, pos, q, k_self=k, v_self=v)
        ro, rs, rn = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
        sample = rng.choice(B, 8, replace=False)
        check_attention(f"step {s} rows", (go[sample], gs[sample], gn[sample]), (ro[sample], rs[sample], rn[sample]))
        lab_o = oracle.classify(rs.astype(np.float32), tT, tE)
        binding.classify(dv(gs, np.float32), tT, tE, labels_d)
        amb += _check_labels(labels_d.cpu().numpy(), lab_o, rs, tT, tE, s)
        # both sides append at the oracle's labels (they agree outside the band)
        gc.append(seq_d, dv(pos, np.int32), dv(lab_o, np.uint8), dv(k, np.float32), dv(v, np.float32))
        oc.append(w.seq_ids, pos, lab_o, k, v)
        gc.plan_budget(seq_d, ch.budget[0], ch.budget[1], max_ops, n_ops, *o, o_bits)
        ops = oc.plan_budget(w.seq_ids, ch.budget[0], ch.budget[1], max_ops)
        m = int(n_ops.item())
        assert m == ops[0].size
        for a, b in zip([x.cpu().numpy()[:m] for x in (*o, o_bits)], ops):
            assert np.array_equal(a, b), f"ops step {s}"
        gc.evict(o[0], o[1], o[2], o_bits, n_ops_dev=n_ops, n_ops=max_ops)
        if m:
            oc.evict(*ops)
        if s % 8 == 7:
            say(f"[churn-full] step {s}: state")
            helpers.compare_states(L, gc.export(), oc.export(), f"churn-full step {s}")
    say(f"[churn-full] {steps} steps x {B} sequences: {amb} labels in the ambiguity band")
