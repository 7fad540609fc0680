"""NF4 codec oracle: codebook, block quantiser, packing, dequantiser, bf16 rounding.

Test infrastructure only (see the package docstring).

What the pages fix: the frozen base is stored as NF4 and dequantised from it
on the fly, per layer (Soup README, "Citing Soup", v3 retraction bullet on the
per-layer NF4 dequantisation cost; soup-cli diff, docs "NF4 streaming
(quantization: 4bit)": quantised once, offline, one tensor at a time, with the
quantisation state travelling with the bytes). What they leave open, and the
reading taken here:

* codebook values - QLoRA section 3 construction (below), normalised in
  float64 and rounded once to float32. Parity against the pages: UNPINNED
  (the pages print no value); pinned to the construction by an independent
  inverse normal CDF and by its invariants.
* block = 64 consecutive elements of the row-major flattened weight; since
  K % 64 == 0 a block never crosses a row. One float32 absmax per block.
* scale = max |w| over the block; normalised value n = fl32(w / absmax)
  (IEEE correctly rounded division); code = index of the nearest codebook
  value, ties to the lower index; a block of zeros gets code 7 (the exact
  zero) and absmax 0; non-finite input is refused.
* packing: 8 consecutive codes per 32-bit little-endian word (bytes 4w..4w+3
  hold elements 8w..8w+7); byte j of the word holds element 8w+j in its low
  nibble and element 8w+j+4 in its high nibble.
* dequant: w_hat = fl32(c[code] * absmax) (one float32 multiply); the bf16
  form is that value rounded to nearest even.
"""

from fractions import Fraction
import math

import numpy as np
from scipy.special import ndtri

BLOCK = 64

# QLoRA, section 3: the probability offset that keeps the outermost quantile
# finite, 1 - (1/30 + 1/32) / 2, for 15 and 16 quantile bins of the two halves.
P_OFFSET = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)


def codebook_unnormalised(inv_cdf=ndtri) -> np.ndarray:
    """The 16 NF4 levels before normalisation, float64, ascending.

    Asymmetric construction of QLoRA section 3: evenly spaced probabilities
    from P_OFFSET down to 1/2, 9 points for the positive half and 8 for the
    negative half; the point at 1/2 (quantile 0) is dropped from both halves
    and a single exact zero is added, giving 8 positive, 7 negative levels.
    """
    pos = np.array([inv_cdf(p) for p in np.linspace(P_OFFSET, 0.5, 9)[:-1]], np.float64)
    neg = -np.array([inv_cdf(p) for p in np.linspace(P_OFFSET, 0.5, 8)[:-1]], np.float64)
    v = np.sort(np.concatenate([neg, [0.0], pos]))
    return v


def codebook(inv_cdf=ndtri) -> np.ndarray:
    """The NF4 codebook as float32[16]: levels divided by the largest, in float64, rounded once."""
    v = codebook_unnormalised(inv_cdf)
    v = v / np.max(np.abs(v))
    return v.astype(np.float32)


def _check_finite(w):
    if not np.all(np.isfinite(w)):
        raise ValueError("nf4 quantize: non-finite input")


def quantize(w, codes_out=False):
    """Block-wise NF4 quantisation of a float32 array (row-major flattened).

    Returns (packed uint8[n/2], absmax float32[n/64]) or, with codes_out,
    (codes uint8[n], absmax).

    Nearest-level search: the distance |n - c_j| is evaluated in float64. For
    n and c_j float32 values in [-1, 1] the subtraction is exact whenever
    |n| >= 2^-29 |c_j|; below that n lies within 2^-28 of zero, where level 7
    (exactly 0) is nearer than any other level by a margin far above any
    rounding, so the float64 argmin equals the exact one. np.argmin returns the
    first minimum, which is the lower index on a tie.
    """
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    if w.size % BLOCK:
        raise ValueError("nf4 quantize: element count must be a multiple of 64")
    _check_finite(w)
    c = codebook().astype(np.float64)
    blocks = w.reshape(-1, BLOCK)
    absmax = np.max(np.abs(blocks), axis=1).astype(np.float32)
    codes = np.empty(blocks.shape, np.uint8)
    step = 1 << 16  # blocks per chunk, bounds the float64 distance table
    for b0 in range(0, blocks.shape[0], step):
        blk = blocks[b0:b0 + step]
        a = absmax[b0:b0 + step]
        nz = a != 0
        safe = np.where(nz, a, np.float32(1.0))
        n = (blk / safe[:, None]).astype(np.float32)          # IEEE float32 division
        d = np.abs(n.astype(np.float64)[..., None] - c)        # [.., 64, 16]
        idx = np.argmin(d, axis=-1).astype(np.uint8)
        idx[~nz] = 7
        codes[b0:b0 + step] = idx
    codes = codes.reshape(-1)
    if codes_out:
        return codes, absmax
    return pack(codes), absmax


def pack(codes) -> np.ndarray:
    """Two 4-bit codes per byte, in words of 8 codes: within each group of 8
    consecutive codes c0..c7 (4 bytes), byte j = c_j | (c_{j+4} << 4)."""
    codes = np.asarray(codes, np.uint8).reshape(-1)
    if codes.size % 8:
        raise ValueError("pack: code count must be a multiple of 8")
    g = codes.reshape(-1, 8)
    return ((g[:, :4] & 0xF) | (g[:, 4:] << 4)).astype(np.uint8).reshape(-1)


def unpack(packed) -> np.ndarray:
    packed = np.asarray(packed, np.uint8).reshape(-1)
    if packed.size % 4:
        raise ValueError("unpack: byte count must be a multiple of 4")
    b = packed.reshape(-1, 4)
    out = np.empty((b.shape[0], 8), np.uint8)
    out[:, :4] = b & 0xF
    out[:, 4:] = b >> 4
    return out.reshape(-1)


def dequant_f32(packed, absmax) -> np.ndarray:
    """w_hat = fl32(c[code] * absmax), float32, flat."""
    codes = unpack(packed)
    absmax = np.asarray(absmax, np.float32).reshape(-1)
    c = codebook()
    a = np.repeat(absmax, BLOCK)
    if a.size != codes.size:
        raise ValueError("dequant: absmax count does not match the packed size")
    return (c[codes] * a).astype(np.float32)   # one float32 multiply, correctly rounded


def dequant_exact(packed, absmax) -> np.ndarray:
    """c[code] * absmax without rounding (float64 holds the product of two float32 exactly)."""
    codes = unpack(packed)
    c = codebook().astype(np.float64)
    a = np.repeat(np.asarray(absmax, np.float32).astype(np.float64), BLOCK)
    return c[codes] * a


def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range; below
    2^-126 it is subnormal with spacing 2^-133. Values whose rounded magnitude
    reaches 2^128 become infinite. NaN stays NaN.
    """
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)                        # v = m 2^e, 1/2 <= |m| < 1
    q = np.maximum(e - 8, -133)               # exponent of one unit in the last place
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)  # np.rint rounds half to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
    return np.where(np.isnan(v), v, r)


def bf16_bits(v) -> np.ndarray:
    """uint16 bit patterns of values that are already bfloat16-representable."""
    f = np.asarray(v, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def dequant_bf16(packed, absmax) -> np.ndarray:
    """bf16(fl32(c[code] * absmax)) as float64 values.

    The value depends only on (code, absmax), so it is evaluated once per
    block for each of the 16 codes and then looked up by code.
    """
    codes = unpack(packed).reshape(-1, BLOCK)
    absmax = np.asarray(absmax, np.float32).reshape(-1)
    if absmax.size != codes.shape[0]:
        raise ValueError("dequant: absmax count does not match the packed size")
    table = round_bf16((codebook()[None, :] * absmax[:, None]).astype(np.float32).astype(np.float64))
    return np.take_along_axis(table, codes.astype(np.intp), axis=1).reshape(-1)


def dequant_rows_bf16(packed, absmax, K, rows) -> np.ndarray:
    """Rows `rows` of the bf16 dequantised [N x K] weight, as float64 [len(rows) x K]."""
    rows = np.asarray(rows)
    p = np.asarray(packed, np.uint8).reshape(-1, K // 2)[rows]
    a = np.asarray(absmax, np.float32).reshape(-1, K // BLOCK)[rows]
    return dequant_bf16(p.reshape(-1), a.reshape(-1)).reshape(len(rows), K)


def dequant_cols_bf16(packed, absmax, N, K, cols) -> np.ndarray:
    """Columns `cols` of the bf16 dequantised [N x K] weight, as float64 [N x len(cols)].

    Element (n, k): word k // 8 of row n, byte (k % 8) % 4 of it, low nibble
    when k % 8 < 4, high nibble otherwise.
    """
    cols = np.asarray(cols)
    byte = (cols // 8) * 4 + (cols % 8) % 4
    p = np.asarray(packed, np.uint8).reshape(N, K // 2)[:, byte]
    codes = np.where(cols % 8 < 4, p & 15, p >> 4)
    a = np.asarray(absmax, np.float32).reshape(N, K // BLOCK)[:, cols // BLOCK]
    w32 = (codebook()[codes] * a).astype(np.float32)
    return round_bf16(w32.astype(np.float64))


def nearest_code_exact(n: float) -> int:
    """Reference nearest-level rule in exact rational arithmetic (for small brute-force checks)."""
    c = [Fraction(float(x)) for x in codebook()]
    fn = Fraction(float(n))
    best, bestd = 0, None
    for j, cj in enumerate(c):
        d = abs(fn - cj)
        if bestd is None or d < bestd:
            best, bestd = j, d
    return best


def inv_normal_cdf_bisect(p: float) -> float:
    """An inverse standard-normal CDF independent of SciPy: bisection on math.erfc.

    Phi(x) = erfc(-x / sqrt 2) / 2 is increasing; 200 halvings of [-40, 40]
    reach the float64 resolution. Used only to pin the codebook construction.
    """
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid == lo or mid == hi:
            break
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)
