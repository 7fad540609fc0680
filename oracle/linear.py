"""Frozen NF4 linear + LoRA adapter, forward and backward (oracle).

Test infrastructure only (see the package docstring).

The pages: only the LoRA adapter trains, the quantised base is frozen (blog
post, "How does Soup train an 8B model on a 4 GB GPU?" and "The trick: layer
streaming"); streaming only reorders the copies and leaves the gradients unchanged
("Why the evidence is better than usual"). The adapter formula is the
standard LoRA one, y = x W^T + (alpha / r) (x A^T) B^T, with W the dequantised
NF4 weight [N x K], A [r x K], B [N x r], s = alpha / r. The backward needs dX
through the frozen W plus the adapter path, and dA, dB; there is no dW.

Two evaluation modes over the same exact inputs (x, A, B, dY are bf16 values,
carried as float64):

* ``exact``    - every product and sum in float64 with W = c[code] * absmax
                 unrounded; nothing is rounded between steps.
* ``faithful`` - the tensors the method stores are bf16 (the activations, the
                 adapter's rank-r intermediates U = x A^T and G = dY B, and
                 every activation gradient); the frozen weight is the bf16
                 dequant bf16(fl32(c[code] * absmax)); each stored tensor is
                 one float64 evaluation of its definition rounded once to bf16.
                 dA and dB are float32 outputs (rounded once from float64).

Pins (tests/test_oracle_linear.py): pure-Python loops on tiny shapes,
an exact integer-grid construction, central finite differences of the exact
forward, the adjoint identity, and the zero-factor special cases.
"""

import numpy as np

from . import nf4


def weight(packed, absmax, N, K, mode):
    if mode == "exact":
        w = nf4.dequant_exact(packed, absmax)
    elif mode == "faithful":
        w = nf4.dequant_bf16(packed, absmax)
    else:
        raise ValueError(mode)
    return w.reshape(N, K)


def _r(v, mode):
    return nf4.round_bf16(v) if mode == "faithful" else v


def _f32(v, mode):
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float64) if mode == "faithful" else v


def lora_down(x, A, mode="faithful"):
    """U = x A^T (bf16 in faithful mode)."""
    return _r(np.asarray(x, np.float64) @ np.asarray(A, np.float64).T, mode)


def fwd(x, packed, absmax, N, K, A, B, alpha, mode="faithful", W=None):
    """Returns (y [M x N], U [M x r]).

    U = x A^T (bf16 in faithful mode, it is stored for the backward);
    y = x W^T + s U B^T, rounded once to bf16 in faithful mode.
    """
    x = np.asarray(x, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    r = A.shape[0]
    s = alpha / r
    if W is None:
        W = weight(packed, absmax, N, K, mode)
    U = lora_down(x, A, mode)
    y = _r(x @ W.T + s * (U @ B.T), mode)
    return y, U


def bwd(dy, x, U, packed, absmax, N, K, A, B, alpha, mode="faithful", W=None, need_dx=True):
    """Returns (dX [M x K] or None, dA [r x K], dB [N x r], G [M x r]).

    G  = dY B                 (bf16 in faithful mode)
    dX = dY W + s G A         (bf16 in faithful mode)
    dB = s dY^T U             (float32 in faithful mode)
    dA = s G^T x              (float32 in faithful mode)
    """
    dy = np.asarray(dy, np.float64)
    x = np.asarray(x, np.float64)
    U = np.asarray(U, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    r = A.shape[0]
    s = alpha / r
    G = _r(dy @ B, mode)
    dX = None
    if need_dx:
        if W is None:
            W = weight(packed, absmax, N, K, mode)
        dX = _r(dy @ W + s * (G @ A), mode)
    dB = _f32(s * (dy.T @ U), mode)
    dA = _f32(s * (G.T @ x), mode)
    return dX, dA, dB, G


def fwd_loops(x, W, A, B, alpha):
    """Pure-Python triple loops of the exact forward (tiny shapes only)."""
    M, K = len(x), len(x[0])
    N, r = len(W), len(A)
    s = alpha / r
    U = [[sum(x[m][k] * A[j][k] for k in range(K)) for j in range(r)] for m in range(M)]
    y = [[sum(x[m][k] * W[n][k] for k in range(K)) + s * sum(U[m][j] * B[n][j] for j in range(r))
          for n in range(N)] for m in range(M)]
    return y, U


def bwd_loops(dy, x, W, A, B, alpha):
    """Pure-Python loops of the exact backward (tiny shapes only)."""
    M, K = len(x), len(x[0])
    N, r = len(W), len(A)
    s = alpha / r
    U = [[sum(x[m][k] * A[j][k] for k in range(K)) for j in range(r)] for m in range(M)]
    G = [[sum(dy[m][n] * B[n][j] for n in range(N)) for j in range(r)] for m in range(M)]
    dX = [[sum(dy[m][n] * W[n][k] for n in range(N)) + s * sum(G[m][j] * A[j][k] for j in range(r))
           for k in range(K)] for m in range(M)]
    dB = [[s * sum(dy[m][n] * U[m][j] for m in range(M)) for j in range(r)] for n in range(N)]
    dA = [[s * sum(G[m][j] * x[m][k] for m in range(M)) for k in range(K)] for j in range(r)]
    return dX, dA, dB
