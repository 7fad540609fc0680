"""Pins of the NF4 codec oracle against what mathematics and the construction fix.

None of these retypes the oracle's formula: each checks it against an
independent routine (bisection inverse CDF, exact rationals, torch's bf16
conversion), a closed form, or an invariant.
"""

import math

import numpy as np
import pytest
import torch

from oracle import nf4


def f32_bits(v):
    return np.asarray(v, np.float32).view(np.uint32)


def test_codebook_invariants():
    c = nf4.codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert c[0] == np.float32(-1.0) and c[7] == np.float32(0.0) and c[15] == np.float32(1.0)
    assert np.all(np.diff(c) > 0)
    assert np.sum(c < 0) == 7 and np.sum(c > 0) == 8
    assert f32_bits(c[7]) == 0  # +0, not -0


def test_codebook_independent_inverse_cdf():
    # SciPy's ndtri against a bisection on math.erfc: same float32 bits.
    a = nf4.codebook()
    b = nf4.codebook(inv_cdf=nf4.inv_normal_cdf_bisect)
    assert np.array_equal(f32_bits(a), f32_bits(b))


def test_codebook_levels_are_evenly_spaced_quantiles():
    # Closed form of the construction: Phi(level) of the 8 positive levels is
    # evenly spaced from the offset probability down to (not including) 1/2 in
    # 8 steps; of the 7 negative levels in 7 steps.
    v = nf4.codebook_unnormalised()
    phi = lambda x: 0.5 * math.erfc(-x / math.sqrt(2.0))
    pos = sorted(v[v > 0], reverse=True)
    neg = sorted(-v[v < 0], reverse=True)
    p0 = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    for i, x in enumerate(pos):
        assert abs(phi(x) - (p0 - i * (p0 - 0.5) / 8)) < 1e-13
    for i, x in enumerate(neg):
        assert abs(phi(x) - (p0 - i * (p0 - 0.5) / 7)) < 1e-13


def test_codebook_rounding_is_robust():
    # Each normalised float64 level sits well away from a float32 rounding
    # boundary, so no float64 evaluation order can change the float32 table.
    v = nf4.codebook_unnormalised()
    v = v / np.max(np.abs(v))
    for x in v:
        if x == 0 or abs(x) == 1:
            continue
        f = np.float32(x)
        ulp = float(np.spacing(np.float32(abs(f))))
        frac = abs(float(f) - x) / ulp
        assert frac < 0.5 - 0.01, (x, frac)


def _quant_single_scale(values):
    """Quantise values with absmax forced to 1 (a 1.0 at the end of each block)."""
    vals = np.asarray(values, np.float32)
    n = len(vals)
    per = 63
    nb = (n + per - 1) // per
    w = np.zeros(nb * 64, np.float32)
    w.reshape(nb, 64)[:, 63] = 1.0
    flat = w.reshape(nb, 64)[:, :63].reshape(-1)
    flat[:n] = vals
    w.reshape(nb, 64)[:, :63] = flat.reshape(nb, 63)
    codes, absmax = nf4.quantize(w, codes_out=True)
    assert np.all(absmax == 1.0)
    return codes.reshape(nb, 64)[:, :63].reshape(-1)[:n]


def test_threshold_brute_force_exact_rationals():
    # Every float32 within +-300 ulp of each midpoint between adjacent levels:
    # the oracle's code equals the nearest level in exact rational arithmetic,
    # ties going to the lower index.
    c = nf4.codebook().astype(np.float64)
    vals = []
    for j in range(15):
        m = np.float32((c[j] + c[j + 1]) / 2)
        x = m
        down, up = [m], []
        for _ in range(300):
            x = np.nextafter(x, np.float32(-2))
            down.append(x)
        x = m
        for _ in range(300):
            x = np.nextafter(x, np.float32(2))
            up.append(x)
        vals += down + up
    vals = np.array(vals, np.float32)
    got = _quant_single_scale(vals)
    want = np.array([nf4.nearest_code_exact(float(v)) for v in vals], np.uint8)
    assert np.array_equal(got, want)


def test_exact_midpoint_ties_go_to_lower_index():
    c = nf4.codebook().astype(np.float64)
    ties = []
    for j in range(15):
        m = (c[j] + c[j + 1]) / 2
        if float(np.float32(m)) == m:
            ties.append(j)
            assert _quant_single_scale([np.float32(m)])[0] == j
    assert len(ties) >= 1


def test_round_trip_of_codebook_valued_blocks():
    # Blocks made of fl32(c_j * a) with one element at +-a quantise back to
    # the same codes and scale, and dequantise to the same float32 values.
    g = np.random.default_rng(1)
    c = nf4.codebook()
    scales = [np.float32(2.0 ** e) for e in range(-120, 122, 7)]
    scales += list(np.float32(g.uniform(1e-3, 10.0, 40)))
    scales += [np.float32(0.02 * 2.4), np.float32(3.0e-38 * 4), np.float32(1.7e38)]
    nb = len(scales)
    codes = g.integers(0, 16, size=(nb, 64)).astype(np.uint8)
    codes[:, g.integers(0, 64, size=nb)] = 0
    for b in range(nb):
        codes[b, b % 64] = 15 if b % 2 else 0
    a = np.array(scales, np.float32)
    w = (c[codes] * a[:, None]).astype(np.float32)
    got_codes, got_absmax = nf4.quantize(w.reshape(-1), codes_out=True)
    assert np.array_equal(got_absmax, a)
    assert np.array_equal(got_codes.reshape(nb, 64), codes)
    packed, absmax = nf4.quantize(w.reshape(-1))
    assert np.array_equal(f32_bits(nf4.dequant_f32(packed, absmax)), f32_bits(w.reshape(-1)))


def test_block_extreme_maps_to_end_codes():
    g = np.random.default_rng(2)
    w = g.standard_normal(64 * 500).astype(np.float32) * np.float32(0.02)
    codes, absmax = nf4.quantize(w, codes_out=True)
    wb = w.reshape(-1, 64)
    cb = codes.reshape(-1, 64)
    i = np.argmax(np.abs(wb), axis=1)
    ext = cb[np.arange(len(i)), i]
    sign = wb[np.arange(len(i)), i] > 0
    assert np.all(ext[sign] == 15) and np.all(ext[~sign] == 0)
    assert np.array_equal(absmax, np.max(np.abs(wb), axis=1))


def test_zero_block():
    w = np.zeros(128, np.float32)
    w[64:] = -0.0
    codes, absmax = nf4.quantize(w, codes_out=True)
    assert np.all(codes == 7) and np.all(absmax == 0)
    out = nf4.dequant_f32(nf4.pack(codes), absmax)
    assert np.all(f32_bits(out) == 0)


def test_nonfinite_refused():
    for bad in (np.nan, np.inf, -np.inf):
        w = np.zeros(64, np.float32)
        w[5] = bad
        with pytest.raises(ValueError):
            nf4.quantize(w)


def test_pack_nibble_order_and_all_bytes():
    # codes 0..7 -> bytes (c0 | c4 << 4, c1 | c5 << 4, c2 | c6 << 4, c3 | c7 << 4)
    assert nf4.pack(list(range(8))).tolist() == [0x40, 0x51, 0x62, 0x73]
    assert nf4.pack([1, 2, 3, 4, 5, 6, 7, 8]).view(np.uint32).tolist() == [0x84736251]
    assert nf4.unpack(np.array([0xA5, 0, 0, 0x3C], np.uint8)).tolist() == [5, 0, 0, 0xC, 0xA, 0, 0, 3]
    allb = np.arange(256, dtype=np.uint8)
    assert np.array_equal(nf4.pack(nf4.unpack(allb)), allb)
    codes = np.random.default_rng(0).integers(0, 16, 4096).astype(np.uint8)
    assert np.array_equal(nf4.unpack(nf4.pack(codes)), codes)


def test_quantisation_error_bound():
    # |dequant(quant(w)) - w| <= absmax * (largest half-gap of the codebook) + 1 ulp.
    g = np.random.default_rng(3)
    w = g.standard_normal(64 * 2000).astype(np.float32) * np.float32(0.02)
    packed, absmax = nf4.quantize(w)
    d = nf4.dequant_f32(packed, absmax).astype(np.float64)
    c = nf4.codebook().astype(np.float64)
    half_gap = np.max(np.diff(c)) / 2
    a = np.repeat(absmax.astype(np.float64), 64)
    assert np.all(np.abs(d - w) <= a * half_gap * (1 + 1e-6) + 1e-12)


def test_round_bf16_matches_torch():
    # torch's float32 -> bfloat16 conversion (round to nearest even) is an
    # independent routine.
    g = np.random.default_rng(4)
    v = np.concatenate([
        g.standard_normal(20000).astype(np.float32),
        (g.standard_normal(2000) * 1e-39).astype(np.float32),      # bf16 subnormals
        np.float32([3.3895e38, 3.4e38, -3.39e38, 1e-45, -1e-45, 0.0, -0.0]),
    ])
    # exact ties: 8 significant bits followed by a single 1 bit
    m = g.integers(128, 256, size=500)
    ties = np.ldexp((2 * m + 1).astype(np.float64), g.integers(-20, 20, size=500)).astype(np.float32)
    v = np.concatenate([v, ties, -ties])
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = nf4.round_bf16(v.astype(np.float64))
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert np.array_equal(got, want)


def test_dequant_bf16_power_of_two_scales_commute():
    c = nf4.codebook().astype(np.float64)
    for e in (-20, -7, 0, 3, 11):
        a = np.float32(2.0 ** e)
        codes = np.arange(16, dtype=np.uint8).repeat(4)
        out = nf4.dequant_bf16(nf4.pack(codes), np.array([a], np.float32))
        want = np.ldexp(torch.from_numpy(c.astype(np.float32)).to(torch.bfloat16).double().numpy(), e)
        assert np.array_equal(out, want[codes])


def test_row_and_column_dequant_match_full_dequant():
    g = np.random.default_rng(5)
    N, K = 48, 256
    w = (g.standard_normal(N * K) * 0.02).astype(np.float32)
    packed, absmax = nf4.quantize(w)
    full = nf4.dequant_bf16(packed, absmax).reshape(N, K)
    rows = np.array([0, 7, 47])
    cols = np.array([0, 1, 63, 64, 130, 255])
    assert np.array_equal(nf4.dequant_rows_bf16(packed, absmax, K, rows), full[rows])
    assert np.array_equal(nf4.dequant_cols_bf16(packed, absmax, N, K, cols), full[:, cols])


def test_dequant_bf16_table_form_equals_elementwise_definition():
    g = np.random.default_rng(6)
    n = 64 * 3000
    packed = g.integers(0, 256, n // 2).astype(np.uint8)
    absmax = np.concatenate([g.uniform(0, 1, 2990), [0.0, 1e-40, 3.4e38, 1.0, 2.0 ** -126, 7.0, 1e-3, 0.05,
                                                     1e20, 1e-20]]).astype(np.float32)
    want = nf4.round_bf16(nf4.dequant_f32(packed, absmax).astype(np.float64))
    got = nf4.dequant_bf16(packed, absmax)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert np.array_equal(got, want)


def test_dequant_exact_is_the_exact_product():
    # dequant_exact is the float64 reference behind the exact-mode stack: it
    # must hold c[code] * absmax with no rounding at all, element by element,
    # in the packed element order. Exact rationals decide, independently of
    # float64: random codes and scales, plus zero, subnormal, smallest normal
    # and the largest finite float32 scales.
    from fractions import Fraction
    g = np.random.default_rng(21)
    nb = 48
    codes = g.integers(0, 16, size=nb * nf4.BLOCK).astype(np.uint8)
    codes[: 16] = np.arange(16)
    absmax = (np.abs(g.standard_normal(nb)) * 0.05).astype(np.float32)
    specials = np.array([0.0, 1e-45, 2.0 ** -140, 2.0 ** -126, 1.0, 3.4028235e38, 7.0e-3, 0.0271],
                        np.float32)
    absmax[: specials.size] = specials
    got = nf4.dequant_exact(nf4.pack(codes), absmax)
    assert got.dtype == np.float64 and got.shape == (codes.size,)
    c = [Fraction(float(v)) for v in nf4.codebook()]
    for i in range(codes.size):
        want = c[codes[i]] * Fraction(float(absmax[i // nf4.BLOCK]))
        assert Fraction(float(got[i])) == want, (i, codes[i], absmax[i // nf4.BLOCK])


def test_dequant_exact_rounds_to_the_float32_and_bf16_dequants():
    # a float32 x float32 product is exact in float64 (48 significant bits,
    # exponents far inside float64's range), so rounding the exact product once
    # gives the float32 dequant bitwise, and once more the bf16 one
    g = np.random.default_rng(22)
    n = 64 * 4096
    packed = g.integers(0, 256, size=n // 2).astype(np.uint8)
    absmax = np.abs(g.standard_normal(n // 64)).astype(np.float32) * np.float32(0.02)
    absmax[::97] = np.float32(2.0 ** -130)   # subnormal products
    ex = nf4.dequant_exact(packed, absmax)
    f32 = nf4.dequant_f32(packed, absmax)
    assert np.array_equal(ex.astype(np.float32).view(np.uint32), f32.view(np.uint32))
    assert np.array_equal(nf4.round_bf16(ex.astype(np.float32).astype(np.float64)), nf4.dequant_bf16(packed, absmax))
