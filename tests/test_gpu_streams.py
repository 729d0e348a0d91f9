"""Two caches stepped at once on two streams, in the bench's pipelined form:
copy j's steps on stream j, each attention launch waiting (an event) for the
previous step's attention on the other stream, so one copy's state calls
(classification + append, ladder + eviction) run beside the other copy's
attention.  Handles share nothing, so each copy must end exactly where one
cache stepped alone through the same decode sequence ends: every step's
attention rows against the oracle's, the whole state bit for bit after the
last step (both copies fed the oracle's fp32 statistics for their labels, so
the labels and every later state are the oracle's)."""
import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import check_attention, say

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_two_batches_in_flight():
    import torch
    import oracle
    steps = 32
    ch = synth.churn(seed=1105, B=64, steps=steps, lo=4096, hi=16384)
    w = ch.base
    L = w.layout
    B = w.seq_ids.size
    tT, tE = ch.tau
    max_ops = 512
    say("[streams] oracle lockstep")
    oc = helpers.build_oracle(w)
    ref = []
    for i in range(steps):
        q, k, v, pos = ch.step_inputs(i)
        ro, rs, rn = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
        rs32 = rs.astype(np.float32)
        oc.append(w.seq_ids, pos, oracle.classify(rs32, tT, tE), k, v)
        ops = oc.plan_budget(w.seq_ids, ch.budget[0], ch.budget[1], max_ops)
        if ops[0].size:
            oc.evict(*ops)
        ref.append((ro, rs, rn, rs32))
    final = oc.export()

    say("[streams] two GPU copies")
    dv = helpers.dev
    g0 = helpers.build_gpu(w)
    g1 = helpers.build_gpu(w)
    gcs = [g0, g1]
    Hq, D = L.num_q_heads, L.head_dim
    seq_d = dv(w.seq_ids, np.int32)
    inputs = []
    for i in range(steps):
        q, k, v, pos = ch.step_inputs(i)
        inputs.append((dv(q, np.uint16), dv(k, np.float32), dv(v, np.float32), dv(pos, np.int32), dv(ref[i][3])))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty(steps, B, Hq, D, dtype=torch.float32, device="cuda") for _ in range(2)]
    stats = [torch.empty(steps, B, Hq, 3, dtype=torch.float32, device="cuda") for _ in range(2)]
    n_att = [torch.zeros(steps, B, dtype=torch.int32, device="cuda") for _ in range(2)]
    ws = [torch.empty(max(g0.workspace_bytes(B), 16), dtype=torch.uint8, device="cuda") for _ in range(2)]
    labels = [torch.empty(B, dtype=torch.uint8, device="cuda") for _ in range(2)]
    n_ops = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(2)]
    ops = [[torch.zeros(max_ops, dtype=torch.int32, device="cuda") for _ in range(3)] for _ in range(2)]
    bits = [torch.zeros(max_ops, dtype=torch.uint8, device="cuda") for _ in range(2)]
    orders = [torch.zeros(1 + B, dtype=torch.int32, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    attn_done = [torch.cuda.Event() for _ in range(2 * steps)]
    for s in range(2 * steps):
        j, i = s % 2, s // 2                     # copy j takes its i-th decode step
        st = streams[j]
        h = st.cuda_stream
        q, k, v, pos, rs32 = inputs[i]
        if s > 0:
            st.wait_event(attn_done[s - 1])
        if i % 16 == 0:
            gcs[j].attn_order(seq_d, orders[j], stream=h)
        gcs[j].attention(seq_d, pos, q, outs[j][i], ws[j], stats=stats[j][i], n_attended=n_att[j][i], k_self=k,
                         v_self=v, order=orders[j], stream=h)
        attn_done[s].record(st)
        gcs[j].classify_append(seq_d, pos, rs32, tT, tE, k, v, labels_out=labels[j], stream=h)
        gcs[j].plan_budget_evict(seq_d, ch.budget[0], ch.budget[1], max_ops, n_ops[j], *ops[j], bits[j], stream=h)
    torch.cuda.synchronize()
    for j in range(2):
        assert gcs[j].get_error() == oc.error(), f"copy {j} error word"
        o, sa, na = outs[j].cpu().numpy(), stats[j].cpu().numpy(), n_att[j].cpu().numpy()
        for i in range(steps):
            ro, rs, rn, _ = ref[i]
            if i % 8 == 0 or i == steps - 1:
                check_attention(f"copy {j} step {i}", (o[i], sa[i], na[i]), (ro, rs, rn))
            else:
                mabs, rl2 = helpers.attn_metrics(o[i], ro)
                assert np.array_equal(na[i], rn) and mabs <= 2e-3 and rl2 <= 1e-3, (j, i, mabs, rl2)
        helpers.compare_states(L, gcs[j].export(), final, f"copy {j} after {steps} steps")
    say(f"[streams] 2 copies x {steps} steps x {B} sequences: attention and final states match the oracle")
