"""GPU parity of kv_classify_append (classification inside the append's
allocation kernel) against thought_classify followed by kv_append_quant, and
against the oracle.

Method passages: ThinKV technical summary, "Methodology": thought
decomposition bullets (the decode step's attention sparsity assigns the type
of its token) and TBQ bullet (the token is then stored at its type's
precision).  Labels must equal the two-call path's bit for bit (the same fp32
sum in head order), and the state must stay bit for bit equal to the
two-call path's and to the oracle's.
"""
import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import _check_labels, gpu_attention, say, TOL_ABS, TOL_L2

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("formats", [False, True])
def test_classify_append_lockstep(formats):
    """Decode loop on three caches: fused classify + append, the two-call path,
    and the oracle; ladder and evictions on all three; labels every step,
    states every 8 steps."""
    import torch
    import oracle
    from thought_adaptive_mixed_amd import binding
    ch = synth.small_churn(seed=96, steps=48)
    if formats:
        ch.base = synth.page_formats(ch.base)
    w = ch.base
    L = w.layout
    B = w.seq_ids.size
    say(f"[fused] build formats={formats}")
    oc = helpers.build_oracle(w)
    ga = helpers.build_gpu(w)
    gb = helpers.build_gpu(w)
    dv = helpers.dev
    seq_d = dv(w.seq_ids, np.int32)
    max_ops = 64
    bufs = {}
    for tag in ("a", "b"):
        bufs[tag] = [torch.zeros(1, dtype=torch.int32, device="cuda")] + \
                    [torch.zeros(max_ops, dtype=torch.int32, device="cuda") for _ in range(3)] + \
                    [torch.zeros(max_ops, dtype=torch.uint8, device="cuda")]
    lab_a = torch.zeros(B, dtype=torch.uint8, device="cuda")
    lab_b = torch.zeros(B, dtype=torch.uint8, device="cuda")
    tT, tE = ch.tau
    in_sync = True
    for s in range(ch.steps):
        q, k, v, pos = ch.step_inputs(s)
        oa, sa, na = gpu_attention(ga, w.seq_ids, pos, q, k_self=k, v_self=v)
        ob, sb, nb = gpu_attention(gb, w.seq_ids, pos, q, k_self=k, v_self=v)
        assert np.array_equal(sa, sb) and np.array_equal(oa, ob), f"step {s}: the two caches diverged"
        pos_d, k_d, v_d = dv(pos, np.int32), dv(k, np.float32), dv(v, np.float32)
        ga.classify_append(seq_d, pos_d, dv(sa, np.float32), tT, tE, k_d, v_d, labels_out=lab_a)
        binding.classify(dv(sb, np.float32), tT, tE, lab_b)
        gb.append(seq_d, pos_d, lab_b, k_d, v_d)
        la = lab_a.cpu().numpy()
        assert np.array_equal(la, lab_b.cpu().numpy()), f"labels step {s}"
        if in_sync:
            ro, rs, rn = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
            mabs, rl2 = helpers.attn_metrics(oa, ro)
            assert mabs <= TOL_ABS and rl2 <= TOL_L2, s
            lab_o = oracle.classify(rs.astype(np.float32), tT, tE)
            if _check_labels(la, lab_o, rs, tT, tE, s):
                in_sync = False            # a label inside the ambiguity band: the oracle stops here
                say(f"[fused] oracle comparison stops at step {s} (label in the ambiguity band)")
            else:
                oc.append(w.seq_ids, pos, lab_o, k, v)
        for tag, g in (("a", ga), ("b", gb)):
            n_ops, o_seq, o_seg, o_keep, o_bits = bufs[tag]
            g.plan_budget(seq_d, ch.budget[0], ch.budget[1], max_ops, n_ops, o_seq, o_seg, o_keep, o_bits)
            g.evict(o_seq, o_seg, o_keep, o_bits, n_ops_dev=n_ops, n_ops=max_ops)
        if in_sync:
            ops = oc.plan_budget(w.seq_ids, ch.budget[0], ch.budget[1], max_ops)
            if ops[0].size:
                oc.evict(*ops)
        if s % 8 == 7 or s == ch.steps - 1:
            ea = ga.export()
            helpers.compare_states(L, ea, gb.export(), f"fused vs two calls, step {s}")
            if in_sync:
                helpers.compare_states(L, ea, oc.export(), f"fused vs oracle, step {s}")
    assert ga.get_error() == gb.get_error()


def test_classify_append_layers_and_kind():
    """Rows of several layers' statistics (num_q_heads = L * Hq) and the
    top-k score kind: labels equal to thought_classify's, states equal."""
    import torch
    from thought_adaptive_mixed_amd import binding
    rng = np.random.default_rng(97)
    w = synth.small_static(seed=97, B=6, Hq=8, Hkv=2, D=64, g=32)
    L = w.layout
    B = w.seq_ids.size
    ga = helpers.build_gpu(w)
    gb = helpers.build_gpu(w)
    dv = helpers.dev
    for kind, NL in ((0, 3), (1, 1), (1, 4)):
        st = rng.uniform(0, 1, (B, NL * L.num_q_heads, 3)).astype(np.float32)
        pos = w.q_pos.astype(np.int32) + kind * 10 + NL
        k = rng.standard_normal((B, L.num_kv_heads, L.head_dim)).astype(np.float32)
        v = rng.standard_normal((B, L.num_kv_heads, L.head_dim)).astype(np.float32)
        la = torch.zeros(B, dtype=torch.uint8, device="cuda")
        lb = torch.zeros(B, dtype=torch.uint8, device="cuda")
        ga.classify_append(dv(w.seq_ids, np.int32), dv(pos), dv(st), 0.48, 0.52, dv(k), dv(v), labels_out=la,
                           score_kind=kind)
        binding.classify(dv(st), 0.48, 0.52, lb, score_kind=kind)
        gb.append(dv(w.seq_ids, np.int32), dv(pos), lb, dv(k), dv(v))
        torch.cuda.synchronize()
        assert np.array_equal(la.cpu().numpy(), lb.cpu().numpy()), (kind, NL)
        assert len(set(la.cpu().numpy().tolist())) > 1
    helpers.compare_states(L, ga.export(), gb.export(), "fused vs two calls")


@pytest.mark.parametrize("max_ops", [64, 1])
def test_plan_budget_evict_lockstep(max_ops):
    """Decode loop on three caches: kv_plan_budget_evict, kv_plan_budget then
    kv_evict_segment, and the oracle; op lists equal every step (device and
    oracle; with max_ops 1 the lists are cut to their first op), states every
    8 steps, error words at the end."""
    import torch
    import oracle
    ch = synth.small_churn(seed=98, steps=64)
    w = ch.base
    L = w.layout
    say("[fused-plan] build")
    oc = helpers.build_oracle(w)
    ga = helpers.build_gpu(w)
    gb = helpers.build_gpu(w)
    dv = helpers.dev
    seq_d = dv(w.seq_ids, np.int32)
    bufs = {tag: [torch.zeros(1, dtype=torch.int32, device="cuda")] +
                 [torch.zeros(max_ops, dtype=torch.int32, device="cuda") for _ in range(3)] +
                 [torch.zeros(max_ops, dtype=torch.uint8, device="cuda")] for tag in ("a", "b")}
    tT, tE = ch.tau
    n_evict = n_down = 0
    for s in range(ch.steps):
        q, k, v, pos = ch.step_inputs(s)
        ro, rs, rn = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
        lab = oracle.classify(rs.astype(np.float32), tT, tE)
        for g in (ga, gb):
            g.append(seq_d, dv(pos, np.int32), dv(lab, np.uint8), dv(k, np.float32), dv(v, np.float32))
        oc.append(w.seq_ids, pos, lab, k, v)
        ga.plan_budget_evict(seq_d, ch.budget[0], ch.budget[1], max_ops, *bufs["a"])
        gb.plan_budget(seq_d, ch.budget[0], ch.budget[1], max_ops, *bufs["b"])
        gb.evict(*bufs["b"][1:], n_ops_dev=bufs["b"][0], n_ops=max_ops)
        ops = oc.plan_budget(w.seq_ids, ch.budget[0], ch.budget[1], max_ops)
        torch.cuda.synchronize()
        m = int(bufs["a"][0].item())
        assert m == int(bufs["b"][0].item()) == ops[0].size, f"op count step {s}"
        for xa, xb, xo in zip(bufs["a"][1:], bufs["b"][1:], ops):
            assert np.array_equal(xa.cpu().numpy()[:m], xo) and np.array_equal(xb.cpu().numpy()[:m], xo), s
        if m:
            oc.evict(*ops)
            n_down += int((ops[3] == 2).sum()); n_evict += int((ops[3] == 0).sum())
        if s % 8 == 7 or s == ch.steps - 1:
            ea = ga.export()
            helpers.compare_states(L, ea, gb.export(), f"fused plan vs two calls, step {s}")
            helpers.compare_states(L, ea, oc.export(), f"fused plan vs oracle, step {s}")
    say(f"[fused-plan] max_ops={max_ops} steps={ch.steps} evictions={n_evict} downgrades={n_down}")
    assert n_evict > 0 and (n_down > 0 or max_ops == 1)
    assert ga.get_error() == gb.get_error() == oc.error()


def test_plan_anneal_evict_lockstep():
    """Decode loop with the TBE annealing policy on three caches:
    kv_plan_anneal_evict, kv_plan_anneal then kv_evict_segment, and the
    oracle; op lists every step, states every 8 steps."""
    import torch
    import oracle
    ch = synth.small_churn(seed=100, steps=64)
    w = ch.base
    L = w.layout
    say("[fused-anneal] build")
    oc = helpers.build_oracle(w)
    ga = helpers.build_gpu(w)
    gb = helpers.build_gpu(w)
    dv = helpers.dev
    seq_d = dv(w.seq_ids, np.int32)
    max_ops = L.max_tokens_per_call
    bufs = {tag: [torch.zeros(1, dtype=torch.int32, device="cuda")] +
                 [torch.zeros(max_ops, dtype=torch.int32, device="cuda") for _ in range(3)] +
                 [torch.zeros(max_ops, dtype=torch.uint8, device="cuda")] for tag in ("a", "b")}
    tT, tE = ch.tau
    n_ops_total = 0
    for s in range(ch.steps):
        q, k, v, pos = ch.step_inputs(s)
        ro, rs, rn = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
        lab = oracle.classify(rs.astype(np.float32), tT, tE)
        for g in (ga, gb):
            g.append(seq_d, dv(pos, np.int32), dv(lab, np.uint8), dv(k, np.float32), dv(v, np.float32))
        oc.append(w.seq_ids, pos, lab, k, v)
        ga.plan_anneal_evict(seq_d, 64, max_ops, *bufs["a"])
        gb.plan_anneal(seq_d, 64, max_ops, *bufs["b"])
        gb.evict(*bufs["b"][1:], n_ops_dev=bufs["b"][0], n_ops=max_ops)
        ops = oc.plan_anneal(w.seq_ids, 64, max_ops)
        torch.cuda.synchronize()
        m = int(bufs["a"][0].item())
        assert m == int(bufs["b"][0].item()) == ops[0].size, f"op count step {s}"
        for xa, xb, xo in zip(bufs["a"][1:], bufs["b"][1:], ops):
            assert np.array_equal(xa.cpu().numpy()[:m], xo) and np.array_equal(xb.cpu().numpy()[:m], xo), s
        if m:
            oc.evict(*ops)
            n_ops_total += m
        if s % 8 == 7 or s == ch.steps - 1:
            ea = ga.export()
            helpers.compare_states(L, ea, gb.export(), f"fused anneal vs two calls, step {s}")
            helpers.compare_states(L, ea, oc.export(), f"fused anneal vs oracle, step {s}")
    say(f"[fused-anneal] steps={ch.steps} ops={n_ops_total}")
    assert n_ops_total > 0
    assert ga.get_error() == gb.get_error() == oc.error()
