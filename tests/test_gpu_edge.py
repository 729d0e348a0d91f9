"""GPU attention on degenerate inputs, against the oracle: a sequence with
nothing cached (with and without the staged self token), a window that admits
no cached token, windows shorter than the top-k size, top-k of 1, a batch that
names one sequence several times, and an empty batch."""
import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import check_attention, gpu_attention, say

pytestmark = pytest.mark.gpu


def test_attention_degenerate_inputs():
    import torch
    w = synth.small_static(seed=81, B=3, Hq=8, Hkv=2, D=128, g=64)
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    empty = int(w.seq_ids[1])
    gc.seq_reset(helpers.dev([empty], np.int32))
    oc.seq_reset([empty])
    helpers.compare_states(w.layout, gc.export(), oc.export(), "after reset")
    L = w.layout
    B = w.seq_ids.size
    rng = np.random.default_rng(9)
    ks = rng.standard_normal((B, L.num_kv_heads, L.head_dim)).astype(np.float32)
    vs = rng.standard_normal((B, L.num_kv_heads, L.head_dim)).astype(np.float32)
    slf = dict(k_self=ks, v_self=vs)
    cases = [
        ("nothing cached in one sequence", {}),
        ("nothing cached + self token", slf),
        ("window 1 (no cached token)", dict(window=1)),
        ("window 1 + self token", dict(window=1, **slf)),
        ("window 3 + self, top-8 over <= 3 tokens", dict(window=3, **slf)),
        ("top-1", dict(topk=1, **slf)),
    ]
    for tag, kw in cases:
        for splits in (0, 3):
            say(f"[edge] {tag} splits={splits}")
            got = gpu_attention(gc, w.seq_ids, w.q_pos, w.q_bf16, splits=splits, **kw)
            ref = oc.attention(w.seq_ids, w.q_pos, w.q_bf16, **kw)
            check_attention(f"{tag} splits={splits}", got, ref)
            out, stats, n_att = got
            if "self" not in tag and "top-1" not in tag:
                assert n_att[1] == 0 and np.all(out[1] == 0) and np.all(stats[1] == 0), tag
    # the self token alone: weight 1, zero entropy, all the mass in the top-k
    out, stats, n_att = gpu_attention(gc, w.seq_ids, w.q_pos, w.q_bf16, **slf)
    G = L.num_q_heads // L.num_kv_heads
    assert n_att[1] == 1
    np.testing.assert_allclose(out[1], np.repeat(vs[1], G, axis=0), rtol=0, atol=1e-6)
    np.testing.assert_allclose(stats[1], np.tile([0.0, 0.0, 1.0], (L.num_q_heads, 1)), rtol=0, atol=1e-6)

    # one sequence named by every batch entry (different queries)
    ids = np.full(B, int(w.seq_ids[0]), np.int32)
    pos = np.full(B, int(w.q_pos[0]), np.int32)
    say("[edge] repeated sequence")
    check_attention("repeated sequence", gpu_attention(gc, ids, pos, w.q_bf16, **slf),
                    oc.attention(ids, pos, w.q_bf16, **slf))

    # an empty batch enqueues nothing and reports success
    say("[edge] empty batch")
    none = torch.empty(0, dtype=torch.int32, device="cuda")
    out0 = torch.empty(0, L.num_q_heads, L.head_dim, dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    gc.attention(none, none, torch.empty(0, dtype=torch.int16, device="cuda"), out0, ws)
    torch.cuda.synchronize()
    assert gc.get_error() == oc.error()
