"""Double-quantised absmax oracle: the 8-bit second-level quantisation of the
NF4 block scales.

Test infrastructure only (see the package docstring).

What the pages fix: the page-locked NF4 base store of Llama-3.1-8B is 3.60 GB
with two 113 MB layer buffers (Soup README, header figure caption), and
Qwen2.5-3B's is 1.43 GB (soup-cli 0.72.0 -> 0.72.2 diff: CHANGELOG [0.72.2]
measured table, and the docs' "Layer Streaming", "NF4 streaming" table). With
one float32 absmax per 64 weights the decoder stacks would be 3.93 GB and
1.54 GB; the pages' sizes are those of NF4 codes plus 8-bit block scales with a
float32 scale per 256 of them, about 0.516 bytes per weight (the tests pin the
layout below to the pages' three figures).

What they leave open, and the reading taken here (QLoRA, Dettmers et al.
2023, section 3, "Double Quantization"):

* the first-level scales c (the float32 absmax of each 64-weight block, as
  nf4.quantize computes them) are centred by their mean mu over the whole
  tensor, then quantised with 8-bit floats in blocks of 256;
* the 8-bit float is OCP FP8 E4M3 (bias 7, three mantissa bits, largest
  finite value 448, no infinities; 0x7F and 0xFF are NaN and never produced);
* mu = fl32(S / n) with S the float64 sum taken in a fixed order: each run of
  256 consecutive scales summed left to right, then the run sums left to
  right (so any implementation can reproduce it bit for bit);
* per run B of 256 scales: d = fl32(c - mu); m = max |d| over the run;
  s_B = fl32(m / 448); code = E4M3(fl32(d / s_B)) by round-to-nearest-even,
  saturating to +-448 (s_B = 0 gives code 0);
* dequantised scale: c' = fl32(fl32(e4m3(code) * s_B) + mu); the NF4 codes
  themselves are those of the float32 absmax (only the scale storage changes).

Stored block (one per weight tensor), byte offsets from its start: the codes
(n bytes), then at the next multiple of 256 the run scales (float32,
ceil(n / 256) of them), then at the next multiple of 256 mu (one float32);
the block is padded to a multiple of 256.
"""

from fractions import Fraction
import math

import numpy as np

RUN = 256
E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of an OCP FP8 E4M3 code (exact, as a Python float)."""
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m, -9)          # subnormal: 2^-6 * m / 8
    return s * math.ldexp(8 + m, e - 10)      # 2^(e-7) * (1 + m / 8)


def e4m3_encode(x: float) -> int:
    """Round-to-nearest-even E4M3 code of a finite float, saturating to +-448."""
    if not math.isfinite(x):
        raise ValueError("non-finite input")
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = Fraction(abs(x))
    if a >= E4M3_MAX:
        return sign | 0x7E
    if a < Fraction(1, 64):                    # subnormal range: multiples of 2^-9
        q = a * 512
        m = _rne(q)
        return sign | m                         # m == 8 is the smallest normal, code 0x08
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    frac = (a / Fraction(2) ** e - 1) * 8       # in [0, 8)
    m = _rne(frac)
    if m == 8:
        e, m = e + 1, 0
    code = ((e + 7) << 3) | m
    return sign | min(code, 0x7E)


def _rne(q: Fraction) -> int:
    """Round a non-negative rational to the nearest integer, ties to even."""
    f = math.floor(q)
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def runs(n: int) -> int:
    return (n + RUN - 1) // RUN


def block_layout(n: int):
    """(scale offset, mean offset, total bytes) of the stored block for n scales."""
    a256 = lambda v: (v + 255) // 256 * 256
    so = a256(n)
    mo = so + a256(4 * runs(n))
    return so, mo, mo + 256


def mean_scale(c) -> np.float32:
    """mu = fl32(S / n), S the float64 sum of the runs' left-to-right sums taken left to right."""
    c = np.asarray(c, np.float32).astype(np.float64)
    n = c.size
    pad = np.zeros(runs(n) * RUN, np.float64)
    pad[:n] = c
    pad = pad.reshape(-1, RUN)
    run_sums = np.zeros(pad.shape[0], np.float64)
    for i in range(RUN):            # elementwise float64 adds: each run summed left to right
        run_sums = run_sums + pad[:, i]
    total = 0.0
    for v in run_sums:
        total = total + float(v)
    return np.float32(total / n)


def double_quant(c, only_runs=None):
    """float32 scales [n] -> (codes uint8 [n], run scales float32 [ceil(n/256)], mu float32).

    only_runs: quantise just these runs (the others stay zero), for sampled
    checks of large tensors; mu is always that of the whole tensor.
    """
    c = np.asarray(c, np.float32).ravel()
    if not np.all(np.isfinite(c)):
        raise ValueError("non-finite scale")
    n = c.size
    mu = mean_scale(c)
    d = (c - mu).astype(np.float32)                       # float32 subtraction
    codes = np.zeros(n, np.uint8)
    scales = np.zeros(runs(n), np.float32)
    for b in (range(runs(n)) if only_runs is None else only_runs):
        db = d[b * RUN:(b + 1) * RUN]
        m = np.float32(np.max(np.abs(db)))
        s = np.float32(m / np.float32(E4M3_MAX))           # float32 division
        scales[b] = s
        if s == 0:
            continue
        q = (db / s).astype(np.float32)                    # float32 division
        codes[b * RUN:b * RUN + db.size] = [e4m3_encode(float(v)) for v in q]
    return codes, scales, mu


def expand(codes, scales, mu) -> np.ndarray:
    """Dequantised scales c' = fl32(fl32(e4m3(code) * s_run) + mu), float32 [n]."""
    codes = np.asarray(codes, np.uint8).ravel()
    table = np.array([e4m3_decode(k) for k in range(256)], np.float64).astype(np.float32)
    v = table[codes]
    s = np.repeat(np.asarray(scales, np.float32), RUN)[:codes.size]
    prod = (v * s).astype(np.float32)                       # float32 multiply
    return (prod + np.float32(mu)).astype(np.float32)       # float32 add


def pack_block(codes, scales, mu) -> np.ndarray:
    """The stored block as bytes (layout of block_layout)."""
    n = len(codes)
    so, mo, total = block_layout(n)
    out = np.zeros(total, np.uint8)
    out[:n] = codes
    out[so:so + 4 * len(scales)] = np.asarray(scales, np.float32).view(np.uint8)
    out[mo:mo + 4] = np.array([mu], np.float32).view(np.uint8)
    return out


def unpack_block(block, n):
    so, mo, _ = block_layout(n)
    b = np.asarray(block, np.uint8)
    return (b[:n].copy(), b[so:so + 4 * runs(n)].view(np.float32).copy(), b[mo:mo + 4].view(np.float32)[0])


def store_bytes_per_weight(N, K):
    """Stored bytes of one N x K weight: packed codes plus its double-quantised scale block."""
    n = N * K // 64
    return N * K // 2 + block_layout(n)[2]
