"""Pins of the double-quantised absmax oracle (oracle/dq.py) against things
fixed outside it: the pages' store sizes, the OCP FP8 E4M3 definition, brute
force, exact rational arithmetic and the quantiser's error bound."""

from fractions import Fraction
import math

import numpy as np
import pytest

from oracle import dq
from oracle import stack as ostack


def stack_store_bytes(L, H, I, KV):
    per = 0
    for N, K in ostack.proj_shapes(H, I, KV).values():
        per += dq.store_bytes_per_weight(N, K)
        per = (per + 255) // 256 * 256
    return per, per * L


def test_store_sizes_match_the_pages():
    # README header figure: 3.60 GB base store, two 113 MB layer buffers
    # (Llama-3.1-8B); CHANGELOG [0.72.2] / docs "NF4 streaming": 1.43 GB (Qwen2.5-3B)
    per8, total8 = stack_store_bytes(32, 4096, 14336, 1024)
    assert round(total8 / 1e9, 2) == 3.60
    assert round(per8 / 1e6) == 113
    _, total3 = stack_store_bytes(36, 2048, 11008, 256)
    assert round(total3 / 1e9, 2) == 1.43
    # and float32 absmax would not give them
    assert round(ostack.nf4_store_bytes(32, 4096, 14336, 1024) / 1e9, 2) != 3.60


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
    (0x3F, 1.875), (0x40, 2.0), (0x77, 240.0), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0)])
def test_e4m3_values_from_the_ocp_definition(code, value):
    assert dq.e4m3_decode(code) == value


def test_e4m3_nan_codes_and_roundtrip():
    assert math.isnan(dq.e4m3_decode(0x7F)) and math.isnan(dq.e4m3_decode(0xFF))
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        v = dq.e4m3_decode(c)
        assert dq.e4m3_encode(v) == c, hex(c)


def test_e4m3_encode_is_nearest_with_ties_to_even_by_brute_force():
    finite = [c for c in range(256) if c not in (0x7F, 0xFF) and c != 0x80]  # -0 aside
    vals = {c: Fraction(dq.e4m3_decode(c)) for c in finite}
    rng = np.random.default_rng(5)
    xs = list(rng.uniform(-460, 460, 3000)) + list(rng.uniform(-0.05, 0.05, 3000))
    # exact midpoints between neighbours (ties) and values just around them
    pos = sorted(v for v in vals.values() if v >= 0)
    for a, b in zip(pos, pos[1:]):
        mid = (a + b) / 2
        xs += [float(mid), -float(mid), float(mid) * (1 + 2 ** -20), float(mid) * (1 - 2 ** -20)]
    for x in xs:
        fx = Fraction(x)
        if abs(fx) >= 448:
            assert dq.e4m3_encode(x) & 0x7F == 0x7E
            continue
        best = min(abs(fx - v) for v in vals.values())
        cands = [c for c, v in vals.items() if abs(fx - v) == best]
        got = dq.e4m3_encode(x)
        if Fraction(dq.e4m3_decode(got)) == 0:
            assert best == abs(fx)          # rounds to a zero of either sign
            continue
        assert got in cands, (x, hex(got), [hex(c) for c in cands])
        if len(cands) == 2:                 # a tie: the even mantissa
            assert got & 1 == 0, x


def test_mean_is_the_exactly_rounded_mean_when_sums_are_exact():
    # values on a 2^-24 grid below 2^-4: every float64 partial sum is exact,
    # so the fixed-order sum is the exact sum
    rng = np.random.default_rng(1)
    for n in (1, 255, 256, 257, 1000, 4096 + 17):
        k = rng.integers(0, 2 ** 20, n)
        c = (k * 2.0 ** -24).astype(np.float32)
        exact = Fraction(int(k.sum()), 2 ** 24) / n
        assert dq.mean_scale(c) == np.float32(float(exact)), n


def test_roundtrip_error_bound_and_codes():
    rng = np.random.default_rng(2)
    # absmax of 64 N(0, 0.02) draws, as the NF4 quantiser produces them
    c = np.max(np.abs(rng.normal(0, 0.02, (3000, 64))), axis=1).astype(np.float32)
    codes, scales, mu = dq.double_quant(c)
    got = dq.expand(codes, scales, mu)
    assert codes.dtype == np.uint8 and scales.size == dq.runs(c.size)
    assert not np.any((codes & 0x7F) == 0x7F)
    d = (c - mu).astype(np.float64)
    for b in range(dq.runs(c.size)):
        sl = slice(b * 256, (b + 1) * 256)
        m = np.max(np.abs(d[sl]))
        # E4M3 keeps 3 fraction bits: |error| <= 2^-4 of the value (normals),
        # 2^-10 of 448 s (subnormals), plus the float32 roundings
        err = np.abs(got[sl].astype(np.float64) - c[sl].astype(np.float64))
        bound = 2.0 ** -4 * np.abs(d[sl]) + 2.0 ** -10 * m + 4 * 2.0 ** -24 * np.abs(c[sl])
        assert np.all(err <= bound + 1e-12)


def test_values_on_the_grid_come_back_exactly():
    # c = mu + e4m3(k) * s with s a power of two, mu = 0.5 and a run max of 448 s:
    # every step of the quantiser is exact
    rng = np.random.default_rng(3)
    s = np.float32(2.0 ** -12)
    ks = [c for c in range(256) if (c & 0x7F) not in (0x7F,)]
    for _ in range(5):
        pick = rng.choice(ks, 256)
        pick[0], pick[1] = 0x7E, 0xFE                 # the run max is 448 s
        # 0.5 + e4m3 * s is exact in float32; the mirrored run 1 - c makes the
        # (exact) float64 mean exactly 0.5
        c = (0.5 + np.array([dq.e4m3_decode(k) for k in pick]) * float(s)).astype(np.float32)
        c = np.concatenate([c, (1.0 - c.astype(np.float64)).astype(np.float32)])
        codes, scales, mu = dq.double_quant(c)
        assert mu == np.float32(0.5)
        got = dq.expand(codes, scales, mu)
        assert np.array_equal(got, c)


def test_constant_runs_and_zero_scales_are_exact():
    c = np.full(700, 0.0431, np.float32)
    codes, scales, mu = dq.double_quant(c)
    assert np.all(scales == 0) and np.all(codes == 0)
    assert np.array_equal(dq.expand(codes, scales, mu), c)
    z = np.zeros(300, np.float32)
    assert np.array_equal(dq.expand(*dq.double_quant(z)), z)


def test_block_pack_layout():
    rng = np.random.default_rng(4)
    c = rng.uniform(0.01, 0.08, 1000).astype(np.float32)
    codes, scales, mu = dq.double_quant(c)
    blk = dq.pack_block(codes, scales, mu)
    so, mo, total = dq.block_layout(1000)
    assert (so, mo, total) == (1024, 1280, 1536) and blk.size == total
    c2, s2, m2 = dq.unpack_block(blk, 1000)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales) and m2 == mu
