"""Dispatch order of the attention (tkv_attn_order / tkv_attn_args.order): the
order is a permutation of the batch, longest first by 256 length buckets of
the code bytes each sequence holds per KV head; the ordered call (which at
>= 2048 units also runs two-wave work-groups) matches the oracle on every row
and the unordered call within rounding, and is bit-reproducible; an order made
for another batch size is ignored."""
import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import check_attention, say

pytestmark = pytest.mark.gpu


def _attn(gc, seq, pd, qd, kd, vd, B, Hq, D, order=None):
    import torch
    out = torch.empty(B, Hq, D, dtype=torch.float32, device="cuda")
    stats = torch.empty(B, Hq, 3, dtype=torch.float32, device="cuda")
    n_att = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(gc.workspace_bytes(B), 16), dtype=torch.uint8, device="cuda")
    gc.attention(seq, pd, qd, out, ws, stats=stats, n_attended=n_att, k_self=kd, v_self=vd, order=order)
    torch.cuda.synchronize()
    return out.cpu().numpy(), stats.cpu().numpy(), n_att.cpu().numpy()


def test_dispatch_order():
    import torch
    ch = synth.churn(seed=41, B=256, steps=4, lo=512, hi=4096)      # 256 x 8 = 2048 units
    w = ch.base
    L = w.layout
    B, Hq, Hkv, D = w.seq_ids.size, L.num_q_heads, L.num_kv_heads, L.head_dim
    gc = helpers.build_gpu(w)
    oc = helpers.build_oracle(w)
    q, k, v, pos = ch.step_inputs(0)
    dv = helpers.dev
    seq, pd, qd, kd, vd = dv(w.seq_ids, np.int32), dv(pos, np.int32), dv(q, np.uint16), dv(k), dv(v)
    order = torch.full((1 + B,), -7, dtype=torch.int32, device="cuda")
    gc.attn_order(seq, order)
    torch.cuda.synchronize()
    o = order.cpu().numpy()
    assert o[0] == B and np.array_equal(np.sort(o[1:]), np.arange(B))
    # longest first, by buckets of the code bytes per KV head
    rec = gc.export()["seq"].view(np.int32).reshape(-1, 16)
    bh = [4 * D * b + 128 * (D // L.group_size) for b in (8, 4, 2)]
    wb = (rec[w.seq_ids, 0:3].astype(np.int64) * np.array(bh)).sum(axis=1)
    bucket = 255 - (wb * 255) // max(int(wb.max()), 1)
    assert np.all(np.diff(bucket[o[1:]]) >= 0)
    ro = oc.attention(w.seq_ids, pos, q, k_self=k, v_self=v)
    plain = _attn(gc, seq, pd, qd, kd, vd, B, Hq, D)
    ordered = _attn(gc, seq, pd, qd, kd, vd, B, Hq, D, order=order)
    check_attention("ordered vs oracle", ordered, ro)
    check_attention("plain vs oracle", plain, ro)
    assert np.array_equal(ordered[2], plain[2])
    # (two waves per work-group merge their records: rounding differs from one wave)
    assert np.abs(ordered[0] - plain[0]).max() <= 2e-4
    again = _attn(gc, seq, pd, qd, kd, vd, B, Hq, D, order=order)
    assert all(np.array_equal(x, y) for x, y in zip(ordered, again)), "ordered call not reproducible"
    # an order whose header is another batch size is ignored (batch order, same launch shape)
    bad = order.clone()
    bad[0] = B - 1
    ignored = _attn(gc, seq, pd, qd, kd, vd, B, Hq, D, order=bad)
    assert all(np.array_equal(x, y) for x, y in zip(ordered, ignored))
    say(f"[order] B{B}: buckets {int(bucket.min())}..{int(bucket.max())}, ordered call within rounding of batch order")
