"""Pins for the oracle's quantizer and fp16 conversion (CPU only).

Method passage: ThinKV technical summary, "Methodologie" > TBQ bullet (group
quantization of buffered tokens by thought category); the integer format with
per-group fp16 scale and zero-point is the reading the oracle follows (the page
formats are pinned in test_oracle_formats.py).
"""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "quantizer_cases.txt")


def _golden():
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        bits, xs, s, z, codes = [p.strip() for p in line.split("|")]
        yield int(bits), np.array([float(v) for v in xs.split()], np.float32), int(s, 16), int(z, 16), \
            [int(c) for c in codes.split()]


@pytest.mark.parametrize("case", list(_golden()), ids=lambda c: f"{c[0]}bit-{c[1].tolist()}")
def test_hand_derived_cases(case):
    bits, x, s, z, codes = case
    got, gs, gz = oracle.quantize_group(x, bits)
    assert (gs, gz) == (s, z)
    assert got.tolist() == codes


def test_f16_conversion_against_numpy_strided():
    # Every exponent and sign, with a stride over the mantissa plus the
    # round-half cases (low 13 bits = 0x1000) and their neighbours.  (The full
    # 2^32 sweep matched numpy's binary16 conversion bit for bit when run once.)
    hi = np.arange(1 << 9, dtype=np.uint32) << 23
    lo = np.concatenate([np.arange(0, 1 << 23, 4099, dtype=np.uint32),
                         (np.arange(0, 1 << 10, dtype=np.uint32) << 13) + 0x1000,
                         (np.arange(0, 1 << 10, dtype=np.uint32) << 13) + 0x0FFF,
                         (np.arange(0, 1 << 10, dtype=np.uint32) << 13) + 0x1001])
    u = (hi[:, None] | lo[None, :]).ravel()
    f = u.view(np.float32)
    got = oracle.f32_to_f16_bits_array(f)
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("g", [32, 64])
def test_exact_grid_roundtrip(bits, g):
    """x = z + s*code with s a power of two and z on the fp16 grid: the
    quantizer must return exactly s, z and the codes."""
    rng = np.random.default_rng(bits * 100 + g)
    top = (1 << bits) - 1
    for _ in range(200):
        codes = rng.integers(0, top + 1, g)
        i0, i1 = rng.choice(g, 2, replace=False)
        codes[i0] = 0
        codes[i1] = top
        e = int(rng.integers(-8, 3))
        s = 2.0 ** e
        z = float(rng.integers(-64, 64)) / 16.0
        x = (z + s * codes).astype(np.float32)
        got, gs, gz = oracle.quantize_group(x, bits)
        assert np.array_equal(got, codes)
        assert np.float16(s).view(np.uint16) == gs
        assert np.float16(z if z != 0 else 0.0).view(np.uint16) == gz


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_codes_are_nearest_grid_point(bits):
    """Every code is the argmin over all 2^bits codes of |x - (s*c + z)|
    (computed in fp64), except near ties within 2 ulp of the quotient."""
    rng = np.random.default_rng(7 + bits)
    top = (1 << bits) - 1
    allc = np.arange(top + 1, dtype=np.float64)
    for _ in range(300):
        x = (rng.standard_normal(64) * rng.choice([0.01, 1.0, 8.0])).astype(np.float32)
        codes, sh, zh = oracle.quantize_group(x, bits)
        s = float(np.uint16(sh).view(np.float16)); z = float(np.uint16(zh).view(np.float16))
        assert s >= 0
        err = np.abs(x.astype(np.float64)[:, None] - (s * allc[None, :] + z))
        best = err.argmin(axis=1)
        q = (x.astype(np.float64) - z) / s
        near_tie = np.abs(q - np.floor(q) - 0.5) < 4 * np.finfo(np.float32).eps * np.maximum(1, np.abs(q))
        ok = (codes == best) | near_tie
        assert ok.all()
        # min maps to 0 and max to the top code, give or take one for fp16 rounding
        assert codes[x.argmin()] <= 1 and codes[x.argmax()] >= top - 1


def test_reconstruction_error_bound():
    """|x - x_hat| <= s/2 (+ fp16 rounding of z) for every element."""
    rng = np.random.default_rng(3)
    for bits in (8, 4, 2):
        for _ in range(200):
            x = rng.standard_normal(32).astype(np.float32) * 3
            codes, sh, zh = oracle.quantize_group(x, bits)
            s = float(np.uint16(sh).view(np.float16)); z = float(np.uint16(zh).view(np.float16))
            xh = s * codes + z
            zerr = abs(z - float(x.min()))
            assert np.all(np.abs(xh - x) <= s / 2 + zerr + 1e-6)
