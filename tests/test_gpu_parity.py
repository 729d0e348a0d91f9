"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

State (codes, packing, scales, allocator stacks, block tables, masks,
positions, segments, error word) must match bit for bit; attention outputs
within max-abs 2e-3 and relative L2 1e-3 over [B, Hq, D]; normalized entropy
and top-k mass within 1e-4.
"""
import os
import sys

import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth

pytestmark = pytest.mark.gpu

TOL_ABS, TOL_L2, TOL_STAT = 2e-3, 1e-3, 1e-4


PROGRESS = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out",
                        "gpu_test_progress.log")


def say(*a):
    """A progress line of a long GPU test: to stdout (captured by pytest) and
    appended to gpurun_out/gpu_test_progress.log, so that a run whose output
    pytest holds back until a test ends still shows each step it finishes."""
    line = " ".join(str(x) for x in a)
    print(line, flush=True)
    sys.stdout.flush()
    try:
        os.makedirs(os.path.dirname(PROGRESS), exist_ok=True)
        with open(PROGRESS, "a") as f:
            f.write(line + "\n")
    except OSError:
        pass


def gpu_attention(gc, seq_ids, q_pos, q, window=0, sinks=None, k_self=None, v_self=None, splits=0, topk=8,
                  order=None):
    import torch
    B = len(seq_ids)
    Hq, D = gc.Hq, gc.D
    out = torch.empty(B, Hq, D, dtype=torch.float32, device="cuda")
    stats = torch.empty(B, Hq, 3, dtype=torch.float32, device="cuda")
    n_att = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(gc.workspace_bytes(B, splits), 16), dtype=torch.uint8, device="cuda")
    dv = helpers.dev
    gc.attention(dv(seq_ids, np.int32), dv(q_pos, np.int32), dv(q, np.uint16), out, ws, stats=stats,
                 n_attended=n_att, k_self=None if k_self is None else dv(k_self, np.float32),
                 v_self=None if v_self is None else dv(v_self, np.float32),
                 sinks=None if sinks is None else dv(sinks, np.float32), window=window, topk=topk,
                 num_splits=splits, order=order)
    torch.cuda.synchronize()
    return out.cpu().numpy(), stats.cpu().numpy(), n_att.cpu().numpy()


AMBIGUITY = 1e-4     # half-width of the band around a threshold where either label is accepted


def _check_labels(lab_g, lab_o, rs, tT, tE, step):
    """GPU labels equal the oracle's wherever the oracle's score is farther
    than AMBIGUITY from both thresholds; returns the number of in-band cases."""
    score = rs[..., 1].astype(np.float32).mean(axis=1)
    band = (np.abs(score - tT) <= AMBIGUITY) | (np.abs(score - tE) <= AMBIGUITY)
    assert np.array_equal(lab_g[~band], lab_o[~band]), f"labels step {step}"
    return int(band.sum())


def check_attention(tag, got, ref, tol_stat=TOL_STAT):
    (go, gs, gn), (ro, rs, rn) = got, ref
    mabs, rl2 = helpers.attn_metrics(go, ro)
    dh = float(np.abs(gs[..., 1] - rs[..., 1]).max()) if gs.size else 0.0
    dm = float(np.abs(gs[..., 2] - rs[..., 2]).max()) if gs.size else 0.0
    say(f"  {tag}: max_abs={mabs:.2e} rel_l2={rl2:.2e} dHn={dh:.2e} dMk={dm:.2e}")
    assert np.array_equal(gn, rn), f"{tag}: n_attended {gn} vs {rn}"
    assert np.isfinite(go).all()
    assert mabs <= TOL_ABS and rl2 <= TOL_L2, tag
    assert dh <= tol_stat and dm <= tol_stat, tag
    np.testing.assert_allclose(gs[..., 0], rs[..., 0], rtol=1e-3, atol=2e-4)


WORKLOADS = {
    "tiny_g1_d64": lambda: synth.tiny(),
    "g4_d128": lambda: synth.small_static(seed=77, B=3, Hq=8, Hkv=2, D=128, g=64),
    "g5_d128": lambda: synth.small_static(seed=79, B=3, Hq=10, Hkv=2, D=128, g=64),
    "g8_d64_sink_swa": lambda: synth.small_static(seed=78, B=4, Hq=16, Hkv=2, D=64, g=32, sinks=True,
                                                  windows=(32, 0)),
    "g4_d128_g32": lambda: synth.small_static(seed=80, B=2, Hq=8, Hkv=2, D=128, g=32),
}


@pytest.fixture(scope="module")
def built():
    cache = {}

    def get(name):
        if name not in cache:
            say(f"[build] {name}")
            w = WORKLOADS[name]()
            oc = helpers.build_oracle(w)
            gc = helpers.build_gpu(w)
            cache[name] = (w, oc, gc)
        return cache[name]
    return get


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_build_state_bit_exact(built, name):
    w, oc, gc = built(name)
    say(f"[state] {name}")
    helpers.compare_states(w.layout, gc.export(), oc.export(), name)
    assert gc.get_error() == oc.error()


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_attention_parity(built, name):
    w, oc, gc = built(name)
    rng = np.random.default_rng(5)
    L = w.layout
    B = w.seq_ids.size
    ks = rng.standard_normal((B, L.num_kv_heads, L.head_dim)).astype(np.float32)
    vs = rng.standard_normal((B, L.num_kv_heads, L.head_dim)).astype(np.float32)
    for window in w.windows:
        for self_tok in (False, True):
            for splits in (0, 1, 3):
                tag = f"{name} W={window} self={self_tok} splits={splits}"
                say(f"[attn] {tag}")
                kw = dict(window=window, sinks=w.sinks)
                if self_tok:
                    kw.update(k_self=ks, v_self=vs)
                got = gpu_attention(gc, w.seq_ids, w.q_pos, w.q_bf16, splits=splits, **kw)
                ref = oc.attention(w.seq_ids, w.q_pos, w.q_bf16, **kw)
                check_attention(tag, got, ref)


def test_churn_lockstep():
    """Decode loop: attention (with the self token) -> classify -> append at
    the label's precision -> budget ladder -> evict/downgrade, on both sides;
    labels and outputs every step, full state every 8 steps."""
    import torch
    import oracle
    ch = synth.small_churn()
    w = ch.base
    L = w.layout
    say("[churn] build")
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    helpers.compare_states(L, gc.export(), oc.export(), "churn build")
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
    n_down = n_evict = 0
    for s in range(ch.steps):
        q, k, v, pos = ch.step_inputs(s)
        go, gs, gn = gpu_attention(gc, w.seq_ids, pos, q, k_self=k, v_self=v)
        ro, rs, rn = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
        check_attention(f"step {s}", (go, gs, gn), (ro, rs, rn)) if s % 16 == 0 else None
        mabs, rl2 = helpers.attn_metrics(go, ro)
        assert mabs <= TOL_ABS and rl2 <= TOL_L2 and np.abs(gs[..., 1:] - rs[..., 1:]).max() <= TOL_STAT, s
        # labels: the oracle classifies its own statistics; the GPU's labels
        # must agree wherever the oracle's score is outside the ambiguity band
        lab_o = oracle.classify(rs.astype(np.float32), tT, tE)
        from thought_adaptive_mixed_amd import binding
        binding.classify(dv(gs, np.float32), tT, tE, labels_d)
        lab_g = labels_d.cpu().numpy()
        if _check_labels(lab_g, lab_o, rs, tT, tE, s) == 0:
            labels_in = labels_d          # the device labels drive the append directly
        else:
            labels_in = dv(lab_o, np.uint8)
        # append at the label's precision
        gc.append(seq_d, dv(pos, np.int32), labels_in, dv(k, np.float32), dv(v, np.float32))
        oc.append(w.seq_ids, pos, lab_o, k, v)
        # ladder + evict
        gc.plan_budget(seq_d, ch.budget[0], ch.budget[1], max_ops, n_ops, o_seq, o_seg, o_keep, o_bits)
        ops = oc.plan_budget(w.seq_ids, ch.budget[0], ch.budget[1], max_ops)
        m = int(n_ops.item())
        assert m == ops[0].size
        got_ops = [a.cpu().numpy()[:m] for a in (o_seq, o_seg, o_keep, o_bits)]
        for a, b in zip(got_ops, ops):
            assert np.array_equal(a, b), f"ops step {s}"
        gc.evict(o_seq, o_seg, o_keep, o_bits, n_ops_dev=n_ops, n_ops=max_ops)
        if m:
            oc.evict(*ops)
            n_down += int((ops[3] == 2).sum()); n_evict += int((ops[3] == 0).sum())
        if s % 8 == 7 or s == ch.steps - 1:
            helpers.compare_states(L, gc.export(), oc.export(), f"churn step {s}")
    say(f"[churn] steps={ch.steps} evictions={n_evict} downgrades={n_down}")
    assert n_evict > 0 and n_down > 0
    assert gc.get_error() == oc.error()
