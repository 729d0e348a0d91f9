"""Pins for the oracle's float and ternary code formats (CPU only).

Method passage: ThinKV technical summary, "Methodology", TBQ bullet: higher
precision for Reasoning tokens (8-bit FP8 or 4-bit NVFP4 given as examples),
lower for Transition tokens (2-bit ternary), by group quantization.  The
element formats have definitions of their own (OCP FP8 E4M3, the E2M1 element
of the OCP microscaling formats, the ternary rule of Ternary Weight Networks);
these tests pin the oracle against those definitions by independent routes:
torch's float8_e4m3fn dtype, brute-force nearest search over the value
tables, the closed-form least-squares scale and a hand-derived example.
"""
import math

import numpy as np
import pytest

import oracle
from thought_adaptive_mixed_amd import synth

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def torch_e4m3_bits(y):
    import torch
    b = torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    b = b.astype(np.uint32)
    b[b == 0x80] = 0                # the oracle stores a signed zero as +0
    return b


def f16(bits):
    return float(np.uint16(bits).view(np.float16))


def test_e4m3_decode_every_code():
    """All 254 non-NaN E4M3 codes decode to torch's float8_e4m3fn values."""
    import torch
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.code_value(1, 0, int(c)) for c in codes])
    assert np.array_equal(got, want)


def test_e2m1_decode_every_code():
    for c in range(16):
        v = E2M1[c & 7] * (-1 if c & 8 else 1)
        assert oracle.code_value(1, 1, c) == v
    # ternary codes are integers (t + 1, with zero-point -scale), as are code_format 0 codes
    assert [oracle.code_value(1, 2, c) for c in range(3)] == [0.0, 1.0, 2.0]
    assert oracle.code_value(0, 0, 200) == 200.0


def e4m3_midpoints():
    """Every value halfway between adjacent positive E4M3 values up to 448."""
    import torch
    v = np.sort(np.unique(torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()))
    return ((v[1:] + v[:-1]) / 2).astype(np.float32)


@pytest.mark.parametrize("kind", ["random", "ties", "subnormal"])
def test_e4m3_encode_matches_torch_at_unit_scale(kind):
    """With 448 in the group the scale is exactly 1, so the codes are the
    E4M3 encodings of x itself: compare with torch's rounding."""
    rng = np.random.default_rng(11)
    if kind == "random":
        y = (rng.standard_normal(4095) * 10.0 ** rng.uniform(-3, 2, 4095)).astype(np.float32)
    elif kind == "ties":
        m = e4m3_midpoints()
        y = np.concatenate([m, -m])
    else:
        y = (rng.uniform(-2.0 ** -6, 2.0 ** -6, 4095)).astype(np.float32)
    y = np.clip(y, -448, 448)
    for i in range(0, y.size, 63):
        x = np.concatenate([[448.0], y[i:i + 63]]).astype(np.float32)
        x = np.pad(x, (0, 64 - x.size))
        codes, s, z = oracle.quantize_group_fmt(x, 0)
        assert s == 0x3C00 and z == 0
        assert np.array_equal(codes, torch_e4m3_bits(x)), kind


def test_e4m3_scaled_groups_match_torch():
    """Groups at arbitrary scales: codes = torch's E4M3 of fp32 x / s with
    s the fp16 of amax/448 (saturating where s rounded down)."""
    rng = np.random.default_rng(12)
    for trial in range(300):
        n = (32, 64)[trial % 2]
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 3)).astype(np.float32)
        codes, s, z = oracle.quantize_group_fmt(x, 0)
        assert z == 0
        sf = np.float32(f16(s))
        assert s == oracle.f32_to_f16_bits(float(np.float32(np.abs(x).max()) / np.float32(448)))
        y = (x / sf).astype(np.float32)
        want = torch_e4m3_bits(np.clip(y, -448, 448))
        assert np.array_equal(codes, want), trial


def test_e4m3_saturates_when_scale_rounds_down():
    """amax/448 rounded down to fp16 puts amax/s above 448: the code is the
    largest finite one (0x7E, 448), not NaN."""
    amax = np.float32(0.9007)                      # amax/448 rounds down in fp16
    s = f16(oracle.f32_to_f16_bits(float(amax / np.float32(448))))
    assert amax / np.float32(s) > 448
    x = np.zeros(32, np.float32); x[3] = amax; x[4] = -amax
    codes, _, _ = oracle.quantize_group_fmt(x, 0)
    assert codes[3] == 0x7E and codes[4] == 0xFE


def brute_e2m1(y):
    """Nearest E2M1 value by search; ties to the even code (mantissa bit 0)."""
    a = min(abs(float(y)), 6.0)
    d = [abs(a - v) for v in E2M1]
    best = min(d)
    cands = [c for c in range(8) if d[c] == best]
    c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return 0 if c == 0 else c | (8 if y < 0 else 0)


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(13)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    for trial in range(400):
        n = (32, 64)[trial % 2]
        if trial < 50:
            x = np.concatenate([[6.0], rng.choice(np.concatenate([ties, -ties]), n - 1)]).astype(np.float32)
        else:
            x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 3)).astype(np.float32)
        codes, s, z = oracle.quantize_group_fmt(x, 1)
        assert z == 0
        sf = np.float32(f16(s))
        assert s == oracle.f32_to_f16_bits(float(np.float32(np.abs(x).max()) / np.float32(6)))
        want = [brute_e2m1(np.float32(v / sf)) for v in x]
        assert codes.tolist() == want, trial


@pytest.mark.parametrize("c", [0, 1])
def test_float_grid_roundtrip(c):
    """Values s * (format value) with the largest magnitude present come
    back bit for bit: same codes, same scale, exact reconstruction."""
    rng = np.random.default_rng(14 + c)
    top = 448.0 if c == 0 else 6.0
    nbits = 8 if c == 0 else 4
    vals = np.array([oracle.code_value(1, c, k) for k in range(1 << nbits)
                     if not (c == 0 and k & 0x7F == 0x7F)])
    for trial in range(100):
        g = (32, 64)[trial % 2]
        s = 2.0 ** int(rng.integers(-12, 4))
        v = rng.choice(vals, g)
        v[rng.integers(g)] = top * (1 if rng.integers(2) else -1)
        x = (s * v).astype(np.float32)
        codes, sh, _ = oracle.quantize_group_fmt(x, c)
        assert f16(sh) == s
        back = np.array([f16(sh) * oracle.code_value(1, c, int(k)) for k in codes])
        assert np.array_equal(back, x.astype(np.float64)), trial


def test_ternary_hand_example():
    """By hand: mean |x| = 8.3/8 = 1.0375, threshold 0.72625; the four
    entries beyond it keep their signs; s = (2 + 1.5 + 3 + 1)/4 = 1.875;
    codes t + 1, zero-point -1.875."""
    x = np.array([0.1, -2.0, 0.5, 1.5, -0.2, 0.0, 3.0, -1.0], np.float32)
    codes, s, z = oracle.quantize_group_fmt(x, 2)
    assert codes.tolist() == [1, 0, 1, 2, 1, 1, 2, 0]
    assert f16(s) == 1.875 and f16(z) == -1.875


def test_ternary_rule_and_least_squares_scale():
    """On random groups (no entry near the threshold): t is sign(x) beyond
    0.7 * mean |x| and 0 inside; the scale is the least-squares optimum of
    ||x - s t|| for that t (fp64 lstsq), up to the fp16 rounding."""
    rng = np.random.default_rng(15)
    for trial in range(200):
        g = (32, 64)[trial % 2]
        x = (rng.standard_normal(g) * 10.0 ** rng.uniform(-3, 2)).astype(np.float32)
        thr = 0.7 * np.abs(x.astype(np.float64)).mean()
        if np.min(np.abs(np.abs(x) - thr)) < 1e-4 * thr:
            continue
        codes, s, z = oracle.quantize_group_fmt(x, 2)
        t = np.where(x > thr, 1, np.where(x < -thr, -1, 0))
        assert codes.tolist() == (t + 1).tolist(), trial
        assert z == s ^ 0x8000
        opt = np.linalg.lstsq(t[:, None].astype(np.float64), x.astype(np.float64), rcond=None)[0][0]
        assert abs(f16(s) - opt) <= 2.0 ** -11 * abs(opt) * 1.01, trial


def test_ternary_symmetry_and_degenerate_groups():
    rng = np.random.default_rng(16)
    x = rng.standard_normal(64).astype(np.float32)
    c1, s1, _ = oracle.quantize_group_fmt(x, 2)
    c2, s2, _ = oracle.quantize_group_fmt(-x, 2)
    assert s1 == s2 and c2.tolist() == (2 - c1).tolist()
    for c in range(3):
        z = np.zeros(32, np.float32)
        codes, sh, zh = oracle.quantize_group_fmt(z, c)
        assert sh == 0 and zh == 0 and not codes.any()
        z[7] = -0.0
        assert oracle.quantize_group_fmt(z, c)[1:] == (0, 0)


@pytest.mark.parametrize("D,g", [(64, 32), (128, 64)])
def test_page_format_packing_is_natural_and_a_bijection(D, g):
    """code_format 1 keeps the chunk layout of code_format 0 (the same chunk
    and word for every code) and orders the fields of a word by element for
    the float classes; ternary codes keep the integer order."""
    L0 = oracle.OracleLayout(1, 1, D, g, (1, 1, 1), 1, 1, 1)
    L1 = oracle.OracleLayout(1, 1, D, g, (1, 1, 1), 1, 1, 1, code_format=1)
    for c, bits in enumerate((8, 4, 2)):
        used = np.zeros(2 * 16 * D * bits, np.int32)
        for kv in range(2):
            for t in range(16):
                for d in range(D):
                    b0, b1 = L0.code_bit(c, kv, t, d), L1.code_bit(c, kv, t, d)
                    assert b0 // 32 == b1 // 32 and (c < 2 or b0 == b1)
                    used[b1:b1 + bits] += 1
        assert np.all(used == 1)
        # K codes of one token: consecutive dims of a quarter-group in consecutive fields
        q4 = g // 4
        for d in range(0, D, q4) if c < 2 else []:
            bs = [L1.code_bit(c, 0, 0, d + e) for e in range(q4)]
            per_word = 32 // bits
            for e in range(1, q4):
                if e % per_word:
                    assert bs[e] == bs[e - 1] + bits


def format_rows(rng, types, H, D, g, c_of_type):
    """Rows exactly representable in each token's page format (grid values
    times a power-of-two scale, the largest magnitude present per group)."""
    out = np.zeros((len(types), H, D), np.float32)
    tabs = {c: np.array([oracle.code_value(1, c, k) for k in range(1 << (8, 4)[c])
                         if not (c == 0 and k & 0x7F == 0x7F)]) for c in range(2)}
    tabs[2] = np.array([-1.0, 0.0, 1.0])         # the ternary grid in units of the scale
    tops = {0: 448.0, 1: 6.0, 2: 1.0}
    for i, y in enumerate(types):
        c = c_of_type[int(y)]
        for h in range(H):
            for gi in range(D // g):
                v = rng.choice(tabs[c], g)
                v[rng.integers(g)] = tops[c]
                out[i, h, gi * g:(gi + 1) * g] = 2.0 ** int(rng.integers(-8, -2)) * v
    return out


@pytest.mark.parametrize("D,g,Hq,H", [(64, 32, 4, 2), (128, 64, 8, 2)])
def test_page_format_cache_attention_equals_dense_softmax(D, g, Hq, H):
    """A code_format 1 cache holding format-exact rows attends exactly like
    textbook softmax attention over the rows themselves; rows read back
    through token_rows are the rows stored."""
    from test_oracle_attention import dense_attention
    rng = np.random.default_rng(D + 3)
    n = 120
    types = rng.integers(0, 3, n)
    K = format_rows(rng, types, H, D, g, {0: 0, 1: 1, 2: 2})
    V = format_rows(rng, types, H, D, g, {0: 0, 1: 1, 2: 2})
    L = oracle.OracleLayout(H, Hq, D, g, (16, 16, 16), 2, 16, 256, code_format=1)
    oc = oracle.OracleCache(L)
    oc.append(np.zeros(n, np.int32), np.arange(n), types, K, V)
    q = synth.queries(rng, 1, Hq, D)
    out, st, na = oc.attention([0], [n], q)
    qf = synth.bf16_bits_to_f32(q)[0]
    G = Hq // H
    assert na[0] == n
    for h in range(Hq):
        ref, _ = dense_attention(qf[h], K[:, h // G], V[:, h // G], 1 / math.sqrt(D))
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-12, atol=1e-12)
    rows = oc.token_rows(0)
    for pos, r in rows.items():
        assert np.array_equal(r[0], K[pos]) and np.array_equal(r[1], V[pos])


def test_page_format_downgrade_requantizes_reconstruction():
    """A 4 -> 2 bit downgrade in code_format 1: the ternary codes of the
    FP4 reconstruction."""
    L = oracle.OracleLayout(1, 1, 64, 32, (1, 2, 2), 1, 2, 4, code_format=1)
    oc = oracle.OracleCache(L)
    rng = np.random.default_rng(17)
    x = rng.standard_normal((3, 1, 64)).astype(np.float32)
    oc.append([0] * 3, [0, 1, 2], [1, 1, 1], x, x)
    oc.evict([0], [0], [3], [2])
    rows = oc.token_rows(0)
    for pos in range(3):
        for gi in range(2):
            c4, s4, _ = oracle.quantize_group_fmt(x[pos, 0, gi * 32:(gi + 1) * 32], 1)
            xr = np.array([np.float32(f16(s4)) * np.float32(oracle.code_value(1, 1, int(k))) for k in c4],
                          np.float32)
            c2, s2, z2 = oracle.quantize_group_fmt(xr, 2)
            want = np.array([np.float32(f16(s2)) * np.float32(k) + np.float32(f16(z2)) for k in c2], np.float32)
            assert np.array_equal(rows[pos][0][0, gi * 32:(gi + 1) * 32], want)
