"""Per-kernel timing (tkv_kernel_timing / tkv_kernel_times): a small decode
loop on two copies of one cache, one timed and one not, gives identical
outputs, statistics and states; the timed one reports every kernel of the
step, launched once per step, with positive durations."""
import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import say

pytestmark = pytest.mark.gpu


def test_kernel_timing_changes_nothing_and_names_every_kernel():
    import torch
    from thought_adaptive_mixed_amd import binding, drive
    ch = synth.churn(seed=77, B=16, steps=6, lo=1024, hi=4096)
    w = ch.base
    L = w.layout
    B, Hq, D = w.seq_ids.size, L.num_q_heads, L.head_dim
    a = drive.build_gpu(w)
    st0 = a.export()
    b = binding.Cache(drive.gpu_layout(L), w.block_order)
    b.import_(st0)
    dv = drive.dev
    seq = dv(w.seq_ids, np.int32)
    max_ops = 256
    bufs = {}
    for name, c in (("a", a), ("b", b)):
        bufs[name] = dict(out=torch.empty(B, Hq, D, dtype=torch.float32, device="cuda"),
                          stats=torch.empty(B, Hq, 3, dtype=torch.float32, device="cuda"),
                          ws=torch.empty(max(c.workspace_bytes(B, 2), 16), dtype=torch.uint8, device="cuda"),
                          n_ops=torch.zeros(1, dtype=torch.int32, device="cuda"),
                          ops=[torch.zeros(max_ops, dtype=torch.int32, device="cuda") for _ in range(3)],
                          bits=torch.zeros(max_ops, dtype=torch.uint8, device="cuda"))
    assert a.workspace_bytes(B, 2) > 0          # two splits: the combine kernel is timed too
    a.kernel_timing(True)
    for s in range(ch.steps):
        q, k, v, pos = ch.step_inputs(s)
        qd, kd, vd, pd = dv(q, np.uint16), dv(k, np.float32), dv(v, np.float32), dv(pos, np.int32)
        res = []
        for name, c in (("a", a), ("b", b)):
            x = bufs[name]
            c.attention(seq, pd, qd, x["out"], x["ws"], stats=x["stats"], k_self=kd, v_self=vd, num_splits=2)
            c.classify_append(seq, pd, x["stats"], ch.tau[0], ch.tau[1], kd, vd)
            c.plan_budget_evict(seq, ch.budget[0], ch.budget[1], max_ops, x["n_ops"], *x["ops"], x["bits"])
            torch.cuda.synchronize()
            res.append((x["out"].cpu().numpy(), x["stats"].cpu().numpy()))
        assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1]), s
    helpers.compare_states(L, a.export(), b.export(), "timed vs untimed")
    times, dropped = a.kernel_times()
    assert dropped == 0
    for name in ("k_attn", "k_combine", "k_append_alloc", "k_append_store", "k_plan", "k_evict_plan",
                 "k_evict_apply", "k_requant"):
        assert name in times, (name, times)
        us, calls = times[name]
        assert calls == ch.steps and us > 0, (name, us, calls)
    say("[timing] " + ", ".join(f"{n} {us / c:.1f} us x{c}" for n, (us, c) in times.items()))
    # reading again adds nothing new; turning timing off drops the records
    again, _ = a.kernel_times()
    assert again == times
    a.kernel_timing(False)
    with pytest.raises(binding.TkvError):
        a.kernel_times()
