"""GPU parity of the TBE annealing planner (kv_plan_anneal) against the oracle.

Method passages: ThinKV technical summary, "Methodologie" > TBE bullet (on a
Transition thought, the earlier Reasoning/Execution segments are evicted
progressively on an annealing schedule of the retention, 64 -> 32 -> 16, at
segment granularity); lay summary "Astuce B" (Transition thoughts kept as a
safety net).  Op lists must match bit for bit; after applying them the state
must match bit for bit.
"""
import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import _check_labels, check_attention, gpu_attention, say, TOL_ABS, TOL_L2, TOL_STAT

pytestmark = pytest.mark.gpu


class Ops:
    """Device op buffers of one planner call."""

    def __init__(self, max_ops):
        import torch
        self.max_ops = max_ops
        self.n = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.seq = torch.zeros(max_ops, dtype=torch.int32, device="cuda")
        self.seg = torch.zeros_like(self.seq)
        self.keep = torch.zeros_like(self.seq)
        self.bits = torch.zeros(max_ops, dtype=torch.uint8, device="cuda")

    def plan(self, gc, seq_ids, r0, max_ops=None):
        import torch
        m = self.max_ops if max_ops is None else max_ops
        self.n.fill_(-7)
        gc.plan_anneal(helpers.dev(seq_ids, np.int32), r0, m, self.n, self.seq, self.seg, self.keep, self.bits)
        torch.cuda.synchronize()
        k = int(self.n.item())
        return k, [a.cpu().numpy()[:k] for a in (self.seq, self.seg, self.keep, self.bits)]

    def apply(self, gc):
        gc.evict(self.seq, self.seg, self.keep, self.bits, n_ops_dev=self.n, n_ops=self.max_ops)


def same_ops(got, want, tag):
    k, arrs = got
    assert k == want[0].size, f"{tag}: {k} ops against {want[0].size}"
    for a, b in zip(arrs, want):
        assert np.array_equal(a, b), tag


@pytest.mark.parametrize("name", ["llama8b", "qwen14b"])
def test_anneal_full_size(name):
    """The planner on a full-size built state (hundreds of segments per
    sequence), at several starting retentions and with capped op lists; the
    capped list is applied and the states compared."""
    w = synth.WORKLOADS[name]()
    L = w.layout
    say(f"[anneal] build {name}")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    ops = Ops(L.max_tokens_per_call)
    for r0 in (64, 8, 1, 0, 1 << 30):
        for m in (L.max_tokens_per_call, 37, 1, 0):
            say(f"[anneal] {name} r0={r0} max_ops={m}")
            same_ops(ops.plan(gc, w.seq_ids, r0, m), oc.plan_anneal(w.seq_ids, r0, m), f"{name} r0={r0} m={m}")
    # apply the schedule at 64 (capped at the call size) and compare the states
    want = oc.plan_anneal(w.seq_ids, 64, L.max_tokens_per_call)
    same_ops(ops.plan(gc, w.seq_ids, 64), want, f"{name} apply")
    assert want[0].size > 0
    ops.apply(gc)
    oc.evict(*want)
    helpers.compare_states(L, gc.export(), oc.export(), f"{name} after anneal")
    assert gc.get_error() == oc.error()
    # attention over the annealed state
    got = gpu_attention(gc, w.seq_ids, w.q_pos, w.q_bf16)
    check_attention(f"{name} annealed", got, oc.attention(w.seq_ids, w.q_pos, w.q_bf16))


def test_anneal_list_edge_cases():
    """Empty list, ids outside the table (skipped), a sequence listed twice
    (planned twice), reset sequences (no segments)."""
    w = synth.small_static(seed=83, B=4, Hq=8, Hkv=2, D=64, g=32)
    L = w.layout
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    ops = Ops(64)
    s0, s1 = int(w.seq_ids[0]), int(w.seq_ids[1])
    gc.seq_reset(helpers.dev([s1], np.int32))
    oc.seq_reset([s1])
    cases = [[], [s0], [s0, s0], [-1, s0, L.max_seqs, s1], list(w.seq_ids)]
    for lst in cases:
        for r0 in (0, 2, 64):
            say(f"[anneal] list {lst} r0={r0}")
            same_ops(ops.plan(gc, np.array(lst, np.int32), r0), oc.plan_anneal(np.array(lst, np.int32), r0, 64),
                     f"list {lst} r0={r0}")
    assert gc.get_error() == oc.error()


def test_anneal_lockstep():
    """Decode loop with the TBE policy: attention (with the self token) ->
    classify -> append at the label's precision -> annealing plan -> evict, on
    both sides; ops every step, full state every 8 steps; planning again after
    applying a plan gives no ops."""
    import torch
    import oracle
    from thought_adaptive_mixed_amd import binding
    ch = synth.small_churn(seed=91)
    w = ch.base
    L = w.layout
    say("[anneal-loop] build")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    B = w.seq_ids.size
    dv = helpers.dev
    seq_d = dv(w.seq_ids, np.int32)
    ops = Ops(L.max_tokens_per_call)
    labels_d = torch.zeros(B, dtype=torch.uint8, device="cuda")
    tT, tE = ch.tau
    n_ops_total = 0
    for s in range(ch.steps):
        q, k, v, pos = ch.step_inputs(s)
        go, gs, gn = gpu_attention(gc, w.seq_ids, pos, q, k_self=k, v_self=v)
        ro, rs, rn = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
        mabs, rl2 = helpers.attn_metrics(go, ro)
        assert mabs <= TOL_ABS and rl2 <= TOL_L2 and np.abs(gs[..., 1:] - rs[..., 1:]).max() <= TOL_STAT, s
        lab_o = oracle.classify(rs.astype(np.float32), tT, tE)
        binding.classify(dv(gs, np.float32), tT, tE, labels_d)
        lab_g = labels_d.cpu().numpy()
        labels_in = labels_d if _check_labels(lab_g, lab_o, rs, tT, tE, s) == 0 else dv(lab_o, np.uint8)
        gc.append(seq_d, dv(pos, np.int32), labels_in, dv(k, np.float32), dv(v, np.float32))
        oc.append(w.seq_ids, pos, lab_o, k, v)
        want = oc.plan_anneal(w.seq_ids, 64, L.max_tokens_per_call)
        same_ops(ops.plan(gc, w.seq_ids, 64), want, f"step {s}")
        ops.apply(gc)
        if want[0].size:
            oc.evict(*want)
            n_ops_total += want[0].size
            if want[0].size < L.max_tokens_per_call:
                assert ops.plan(gc, w.seq_ids, 64)[0] == 0, f"replan step {s}"
        if s % 8 == 7 or s == ch.steps - 1:
            helpers.compare_states(L, gc.export(), oc.export(), f"anneal step {s}")
    say(f"[anneal-loop] steps={ch.steps} ops={n_ops_total}")
    assert n_ops_total > 0
    assert gc.get_error() == oc.error()
