"""Pins of the NF4 + LoRA linear oracle: loops, exact rationals, finite differences, adjoints."""

from fractions import Fraction

import numpy as np

from oracle import linear, nf4


def _rand_layer(M, K, N, r, seed, sigma_w=0.02):
    g = np.random.default_rng(seed)
    x = nf4.round_bf16(g.standard_normal((M, K)))
    W = (g.standard_normal((N, K)) * sigma_w).astype(np.float32)
    packed, absmax = nf4.quantize(W.reshape(-1))
    A = nf4.round_bf16(g.standard_normal((r, K)) * 0.01)
    B = nf4.round_bf16(g.standard_normal((N, r)) * 0.01)
    dy = nf4.round_bf16(g.standard_normal((M, N)))
    return x, packed, absmax, A, B, dy


def test_fwd_bwd_match_python_loops():
    M, K, N, r, alpha = 3, 64, 5, 2, 4.0
    x, packed, absmax, A, B, dy = _rand_layer(M, K, N, r, 10)
    W = linear.weight(packed, absmax, N, K, "exact")
    y, U = linear.fwd(x, packed, absmax, N, K, A, B, alpha, mode="exact")
    yl, Ul = linear.fwd_loops(x.tolist(), W.tolist(), A.tolist(), B.tolist(), alpha)
    assert np.allclose(y, yl, rtol=1e-12, atol=1e-14)
    assert np.allclose(U, Ul, rtol=1e-12, atol=1e-14)
    dX, dA, dB, _ = linear.bwd(dy, x, U, packed, absmax, N, K, A, B, alpha, mode="exact")
    dXl, dAl, dBl = linear.bwd_loops(dy.tolist(), x.tolist(), W.tolist(), A.tolist(), B.tolist(), alpha)
    assert np.allclose(dX, dXl, rtol=1e-12, atol=1e-14)
    assert np.allclose(dA, dAl, rtol=1e-12, atol=1e-14)
    assert np.allclose(dB, dBl, rtol=1e-12, atol=1e-14)


def _exact_construction(M, K, N, r, seed):
    """Integer-grid operands: every partial sum is exactly representable.

    absmax 1 makes the bf16 weight bf16(c[code]) (on the 2^-11 grid, |w| <= 1);
    x in {-2..2}; A rows one-hot times 2^-4; B columns one-hot times 2^-3.
    """
    g = np.random.default_rng(seed)
    codes = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    codes[:, 0] = 15  # block extreme -> absmax 1 when quantised from values
    packed = nf4.pack(codes.reshape(-1))
    absmax = np.ones(N * K // 64, np.float32)
    x = g.integers(-2, 3, size=(M, K)).astype(np.float64)
    A = np.zeros((r, K))
    A[np.arange(r), g.integers(0, K, size=r)] = 2.0 ** -4
    B = np.zeros((N, r))
    B[np.arange(N), g.integers(0, r, size=N)] = 2.0 ** -3
    dy = g.integers(-2, 3, size=(M, N)).astype(np.float64)
    return codes, packed, absmax, x, A, B, dy


def test_exact_construction_against_rationals():
    M, K, N, r, alpha = 4, 128, 6, 2, 4.0
    codes, packed, absmax, x, A, B, dy = _exact_construction(M, K, N, r, 11)
    s = Fraction(alpha) / r
    cb = [Fraction(float(v)) for v in nf4.round_bf16(nf4.codebook().astype(np.float64))]
    Wf = [[cb[codes[n, k]] for k in range(K)] for n in range(N)]
    xf = [[Fraction(int(v)) for v in row] for row in x]
    Af = [[Fraction(float(v)) for v in row] for row in A]
    Bf = [[Fraction(float(v)) for v in row] for row in B]
    dyf = [[Fraction(int(v)) for v in row] for row in dy]
    U = [[sum(xf[m][k] * Af[j][k] for k in range(K)) for j in range(r)] for m in range(M)]
    y = [[sum(xf[m][k] * Wf[n][k] for k in range(K)) + s * sum(U[m][j] * Bf[n][j] for j in range(r))
          for n in range(N)] for m in range(M)]
    G = [[sum(dyf[m][n] * Bf[n][j] for n in range(N)) for j in range(r)] for m in range(M)]
    dX = [[sum(dyf[m][n] * Wf[n][k] for n in range(N)) + s * sum(G[m][j] * Af[j][k] for j in range(r))
           for k in range(K)] for m in range(M)]
    yo, Uo = linear.fwd(x, packed, absmax, N, K, A, B, alpha, mode="faithful")
    assert np.array_equal(Uo, np.array([[float(v) for v in row] for row in U]))
    assert np.array_equal(yo, nf4.round_bf16(np.array([[float(v) for v in row] for row in y])))
    dXo, _, _, Go = linear.bwd(dy, x, Uo, packed, absmax, N, K, A, B, alpha, mode="faithful")
    assert np.array_equal(Go, np.array([[float(v) for v in row] for row in G]))
    assert np.array_equal(dXo, nf4.round_bf16(np.array([[float(v) for v in row] for row in dX])))


def test_finite_differences_of_exact_forward():
    M, K, N, r, alpha = 3, 64, 4, 3, 6.0
    x, packed, absmax, A, B, dy = _rand_layer(M, K, N, r, 12)
    loss = lambda x_, A_, B_: float(np.sum(dy * linear.fwd(x_, packed, absmax, N, K, A_, B_, alpha, mode="exact")[0]))
    _, U = linear.fwd(x, packed, absmax, N, K, A, B, alpha, mode="exact")
    dX, dA, dB, _ = linear.bwd(dy, x, U, packed, absmax, N, K, A, B, alpha, mode="exact")
    g = np.random.default_rng(5)
    h = 1e-3
    for _ in range(6):
        m, k = g.integers(0, M), g.integers(0, K)
        e = np.zeros_like(x); e[m, k] = h
        fd = (loss(x + e, A, B) - loss(x - e, A, B)) / (2 * h)
        assert abs(fd - dX[m, k]) <= 1e-7 * max(1.0, abs(fd))
        j, k = g.integers(0, r), g.integers(0, K)
        e = np.zeros_like(A); e[j, k] = h
        fd = (loss(x, A + e, B) - loss(x, A - e, B)) / (2 * h)
        assert abs(fd - dA[j, k]) <= 1e-7 * max(1.0, abs(fd))
        n, j = g.integers(0, N), g.integers(0, r)
        e = np.zeros_like(B); e[n, j] = h
        fd = (loss(x, A, B + e) - loss(x, A, B - e)) / (2 * h)
        assert abs(fd - dB[n, j]) <= 1e-7 * max(1.0, abs(fd))


def test_adjoint_identity():
    # y is linear in x for fixed A, B: <dY, y(v)> = <dX(dY), v>.
    M, K, N, r, alpha = 5, 128, 7, 4, 8.0
    _, packed, absmax, A, B, dy = _rand_layer(M, K, N, r, 13)
    v = np.random.default_rng(6).standard_normal((M, K))
    yv, U = linear.fwd(v, packed, absmax, N, K, A, B, alpha, mode="exact")
    dX, _, _, _ = linear.bwd(dy, v, U, packed, absmax, N, K, A, B, alpha, mode="exact")
    lhs, rhs = np.sum(dy * yv), np.sum(dX * v)
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + 1)


def test_zero_factor_special_cases():
    M, K, N, r, alpha = 4, 64, 6, 2, 4.0
    x, packed, absmax, A, B, dy = _rand_layer(M, K, N, r, 14)
    _, U = linear.fwd(x, packed, absmax, N, K, A, B, alpha)
    _, dA, _, _ = linear.bwd(dy, x, U, packed, absmax, N, K, A, np.zeros_like(B), alpha)
    assert np.all(dA == 0)
    Az = np.zeros_like(A)
    _, Uz = linear.fwd(x, packed, absmax, N, K, Az, B, alpha)
    _, _, dB, _ = linear.bwd(dy, x, Uz, packed, absmax, N, K, Az, B, alpha)
    assert np.all(dB == 0)


def test_one_hot_rows_select_weight_columns():
    M, K, N, r, alpha = 4, 128, 6, 2, 4.0
    _, packed, absmax, A, B, _ = _rand_layer(M, K, N, r, 15)
    x = np.zeros((M, K))
    cols = [0, 17, 64, 127]
    x[np.arange(M), cols] = 1.0
    y, _ = linear.fwd(x, packed, absmax, N, K, A, np.zeros_like(B), alpha)
    Wb = nf4.dequant_bf16(packed, absmax).reshape(N, K)
    assert np.array_equal(y, Wb[:, cols].T)
