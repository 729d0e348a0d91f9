"""paged_decode_attn_noalloc (the split-K partials in the library's static
device array, for callers that cannot allocate) against paged_decode_attn
with a caller workspace: two calls in a row, the second with a smaller batch
and fewer splits, outputs and statistics bit for bit equal, and both within
the oracle bounds; a request beyond the static array is refused with ERANGE
before anything is enqueued."""
import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import check_attention, gpu_attention, say

pytestmark = pytest.mark.gpu


def _noalloc(gc, seq_ids, q_pos, q, splits, **kw):
    import torch
    B = len(seq_ids)
    out = torch.full((B, gc.Hq, gc.D), float("nan"), dtype=torch.float32, device="cuda")
    stats = torch.full((B, gc.Hq, 3), float("nan"), dtype=torch.float32, device="cuda")
    n_att = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    dv = helpers.dev
    ks, vs = kw.get("k_self"), kw.get("v_self")
    gc.attention_noalloc(dv(seq_ids, np.int32), dv(q_pos, np.int32), dv(q, np.uint16), out, stats=stats,
                         n_attended=n_att, k_self=None if ks is None else dv(ks, np.float32),
                         v_self=None if vs is None else dv(vs, np.float32), num_splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), stats.cpu().numpy(), n_att.cpu().numpy()


def test_noalloc_matches_workspace_call():
    w = synth.small_static(seed=141, B=6, Hq=8, Hkv=2, D=128, g=64, L=1400)
    L = w.layout
    gc = helpers.build_gpu(w)
    oc = helpers.build_oracle(w)
    rng = np.random.default_rng(141)
    ks = rng.standard_normal((w.seq_ids.size, L.num_kv_heads, L.head_dim)).astype(np.float32)
    vs = rng.standard_normal((w.seq_ids.size, L.num_kv_heads, L.head_dim)).astype(np.float32)
    for tag, sel, splits in (("first call", np.arange(6), 4), ("second, smaller call", np.array([4, 1]), 2)):
        assert gc.workspace_bytes(sel.size, splits) > 0
        kw = dict(k_self=ks[sel], v_self=vs[sel])
        say(f"[noalloc] {tag}: batch {sel.size}, splits {splits}")
        ref = gpu_attention(gc, w.seq_ids[sel], w.q_pos[sel], w.q_bf16[sel], splits=splits, **kw)
        got = _noalloc(gc, w.seq_ids[sel], w.q_pos[sel], w.q_bf16[sel], splits, **kw)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), tag
        check_attention(f"noalloc {tag}", got, oc.attention(w.seq_ids[sel], w.q_pos[sel], w.q_bf16[sel], **kw))


def test_noalloc_refuses_beyond_static_workspace():
    import torch
    from thought_adaptive_mixed_amd import binding
    # a layout with room for a batch whose partials exceed the static array
    L = synth.Layout(2, 16, 128, 64, (8, 8, 8), 1024, 8, 8, 64)
    big = binding.Cache(helpers.gpu_layout(L))
    need = big.workspace_bytes(1024, 64)
    assert need > binding.STATIC_WORKSPACE_BYTES
    seq = torch.zeros(1024, dtype=torch.int32, device="cuda")
    q = torch.zeros(1024, 16, 128, dtype=torch.int16, device="cuda")
    out = torch.zeros(1024, 16, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.TkvError) as e:
        big.attention_noalloc(seq, seq, q, out, num_splits=64)
    assert e.value.code == binding.TKV_ERANGE
    torch.cuda.synchronize()
    assert big.get_error()[0] == 0
