"""GPU robustness: random append / evict / downgrade / ladder / reset programs
on a tiny pool (exhaustion, full tables, bad ids, repeated segments), applied
to the HIP path and the oracle call by call with the whole state compared
after every call; determinism of builds and attention."""
import numpy as np
import pytest

import helpers
from thought_adaptive_mixed_amd import synth
from test_gpu_parity import gpu_attention, say
from test_oracle_state import random_program

pytestmark = pytest.mark.gpu


def _run_gpu_program(prog, pools, max_seqs, max_blocks, max_segs, order, seed):
    import torch
    import oracle
    from thought_adaptive_mixed_amd import binding
    dv = helpers.dev
    lay = synth.Layout(1, 1, 64, 32, pools, max_seqs, max_blocks, max_segs, 64)
    oc = oracle.OracleCache(helpers.oracle_layout(lay), order)
    gc = binding.Cache(helpers.gpu_layout(lay), order)
    rng = np.random.default_rng(seed)
    n_ops = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs = [torch.zeros(16, dtype=torch.int32, device="cuda") for _ in range(3)]
    bits = torch.zeros(16, dtype=torch.uint8, device="cuda")
    for si, step in enumerate(prog):
        kind = step[0]
        if kind == "A":
            toks = step[1]
            n = len(toks)
            kv = rng.standard_normal((2, n, 1, 64)).astype(np.float32)
            sl = torch.zeros(n, dtype=torch.int32, device="cuda")
            gc.append(dv([t[0] for t in toks], np.int32), dv([t[1] for t in toks], np.int32),
                      dv([t[2] for t in toks], np.uint8), dv(kv[0]), dv(kv[1]), slot_out=sl)
            want = oc.append([t[0] for t in toks], [t[1] for t in toks], [t[2] for t in toks], kv[0], kv[1])
            assert np.array_equal(sl.cpu().numpy(), want), f"slots at call {si}"
        elif kind == "X":
            ops = step[1]
            cols = list(zip(*ops))
            gc.evict(dv(cols[0], np.int32), dv(cols[1], np.int32), dv(cols[2], np.int32), dv(cols[3], np.uint8))
            oc.evict(*[list(c) for c in cols])
        elif kind == "P":
            seqs, num, den = step[1], step[2], step[3]
            gc.plan_budget(dv(seqs, np.int32), num, den, 16, n_ops, *bufs, bits)
            want = oc.plan_budget(seqs, num, den, 16)
            m = int(n_ops.item())
            got = [b.cpu().numpy()[:m] for b in (*bufs, bits)]
            assert m == want[0].size and all(np.array_equal(a, b) for a, b in zip(got, want)), f"plan at call {si}"
            gc.evict(bufs[0], bufs[1], bufs[2], bits, n_ops_dev=n_ops, n_ops=16)
            if m:
                oc.evict(*want)
        else:
            gc.seq_reset(dv(step[1], np.int32))
            oc.seq_reset(step[1])
        helpers.compare_states(lay, gc.export(), oc.export(), f"call {si} ({kind})")


@pytest.mark.parametrize("seed", range(6))
def test_random_programs_match_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    pools = (2, 3, 2) if seed % 2 else (3, 2, 3)
    order = [rng.permutation(p).astype(np.int32) for p in pools] if seed % 3 == 0 else None
    for rep in range(4):
        prog = random_program(rng, 2, 10)
        _run_gpu_program(prog, pools, 2, 2, 5, order, seed * 100 + rep)


def test_error_word_and_tkv_get_error():
    """Errors are sticky until tkv_get_error, which reports and clears them."""
    import oracle
    from thought_adaptive_mixed_amd import binding
    dv = helpers.dev
    lay = synth.Layout(1, 1, 64, 32, (1, 1, 1), 2, 4, 8, 64)
    gc = binding.Cache(helpers.gpu_layout(lay))
    oc = oracle.OracleCache(helpers.oracle_layout(lay))
    kv = np.zeros((20, 1, 64), np.float32)
    seqs, pos = [0] * 16 + [1, 0, 1, 1], list(range(16)) + [0, 16, 1, 2]
    gc.append(dv(seqs, np.int32), dv(pos, np.int32), dv([0] * 20, np.uint8), dv(kv), dv(kv))
    oc.append(seqs, pos, [0] * 20, kv, kv)
    assert gc.get_error() == oc.error() == (1 << 2, 0, 2)
    assert gc.get_error() == (0, 0x7FFFFFFF, 0)            # cleared
    gc.evict(dv([0], np.int32), dv([9], np.int32), dv([0], np.int32), dv([0], np.uint8))
    assert gc.get_error() == (1 << 3, 0, 1)                 # unknown segment
    with pytest.raises(binding.TkvError):                   # host-detectable: nothing enqueued
        gc.append(dv(np.zeros(65, np.int32)), dv(np.arange(65, dtype=np.int32)), dv(np.zeros(65, np.uint8)),
                  dv(np.zeros((65, 1, 64), np.float32)), dv(np.zeros((65, 1, 64), np.float32)))


def test_build_and_attention_are_deterministic():
    w = synth.small_static(seed=90, B=4, Hq=16, Hkv=4, D=128, g=64)
    a = helpers.build_gpu(w)
    b = helpers.build_gpu(w)
    ea, eb = a.export(), b.export()
    for k in ea:
        assert np.array_equal(ea[k], eb[k]), k
    ra = gpu_attention(a, w.seq_ids, w.q_pos, w.q_bf16)
    rb = gpu_attention(a, w.seq_ids, w.q_pos, w.q_bf16)
    for x, y in zip(ra, rb):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("formats", [False, True])
@pytest.mark.parametrize("scale_k", [False, True])
def test_input_range_edge(formats, scale_k):
    """K/V rows at the top of the stated input range (magnitudes up to ~2^14.9,
    below 2^15): the synthetic rows scaled so that their largest element is
    30000 (V always, K too when scale_k), with the build's downgrade and
    eviction history; state bit for bit, and attention with and without the
    self token and splits against the oracle.  Outputs scale with V, so they
    are compared after dividing both sides by the V scale factor lam, under
    the usual bounds (max-abs 2e-3, relative L2 1e-3).  The statistics keep
    the 1e-4 bound, except that with K scaled the logits reach thousands:
    their fp32 rounding (a few units of 2^-24 of the sum of |q_d k_d| / sqrt(D)
    over a row's terms) then perturbs the weights of the near-ties at the top,
    so the bound becomes 2^-22 times the largest such sum (computed in fp64
    from the oracle's dequantized rows)."""
    from test_gpu_parity import check_attention
    w = synth.small_static(seed=99, B=4, Hq=8, Hkv=2, D=128, g=64, L=1600)
    if formats:
        w = synth.page_formats(w)
    base_kv = w.kv
    biggest = max(max(np.abs(x).max() for x in base_kv(c)) for c in w.calls if isinstance(c, synth.AppendCall))
    lam = np.float32(30000.0 / biggest)
    lam_k = lam if scale_k else np.float32(1.0)
    w.kv = lambda call: (base_kv(call)[0] * lam_k, base_kv(call)[1] * lam)
    L = w.layout
    oc = helpers.build_oracle(w)
    gc = helpers.build_gpu(w)
    helpers.compare_states(L, gc.export(), oc.export(), "input range edge")
    top = max(max(np.abs(x).max() for x in w.kv(c)) for c in w.calls if isinstance(c, synth.AppendCall))
    assert 2.0 ** 14 < top < 2.0 ** 15, top
    rng = np.random.default_rng(7)
    ks = (rng.standard_normal((w.seq_ids.size, L.num_kv_heads, L.head_dim)) * 4).astype(np.float32) * lam_k
    vs = (rng.standard_normal((w.seq_ids.size, L.num_kv_heads, L.head_dim)) * 4).astype(np.float32) * lam
    # the largest sum of |q_d k_d| / sqrt(D) over the attended tokens (cached
    # and staged) of any query head
    G = L.num_q_heads // L.num_kv_heads
    q = synth.bf16_bits_to_f32(w.q_bf16).astype(np.float64)
    s1 = 0.0
    for i, s in enumerate(w.seq_ids):
        rows = oc.token_rows(int(s))
        kr = np.stack([r[0] for r in rows.values()] + [ks[i]]).astype(np.float64)    # [n][Hkv][D]
        for h in range(L.num_q_heads):
            s1 = max(s1, float((np.abs(kr[:, h // G, :]) @ np.abs(q[i, h])).max()) / np.sqrt(L.head_dim))
    tol_stat = max(1e-4, s1 * 2.0 ** -22) if scale_k else 1e-4
    say(f"[range] scale_k={scale_k}: largest |q||k| logit sum {s1:.1f}, statistics bound {tol_stat:.1e}")
    for self_tok in (False, True):
        for splits in (0, 3):
            kw = dict(k_self=ks, v_self=vs) if self_tok else {}
            tag = f"range formats={formats} scale_k={scale_k} self={self_tok} splits={splits}"
            say(f"[range] {tag}")
            go, gs, gn = gpu_attention(gc, w.seq_ids, w.q_pos, w.q_bf16, splits=splits, **kw)
            ro, rs, rn = oc.attention(w.seq_ids, w.q_pos, w.q_bf16, **kw)
            assert np.isfinite(go).all() and np.isfinite(gs).all(), tag
            check_attention(tag, (go / lam, gs, gn), (ro / float(lam), rs, rn), tol_stat=tol_stat)
