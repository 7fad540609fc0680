"""Helpers shared by the GPU tests: library loading and the comparison rule."""

import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import nf4_layer_streamed_amd as ql  # noqa: E402

DEV = "cuda:0"
TOL = 2e-2  # relative tolerance for GEMM outputs and gradients (bf16 in, fp32 accumulate)


def lib():
    if not os.path.exists(ql.LIB_PATH):
        from nf4_layer_streamed_amd import build
        build.build()
    return ql.load()


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    lib()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def close(got, want, tol=TOL, what="", summand=None):
    """Element-wise |g - o| <= tol |o| + tol rms(o); also returns the normwise error.

    summand: for an output that is a bf16-rounded sum whose first term is
    itself a stored bf16 value (a residual add, h + f(h)), that term's values.
    Where the term is larger than the sum (cancellation), one bf16 unit of it
    exceeds tol |o|, so tol |term| is added to the element's bound.
    """
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(want * want))) if want.size else 0.0
    err = np.abs(got - want)
    bound = tol * np.abs(want) + tol * rms
    if summand is not None:
        bound = bound + tol * np.abs(np.asarray(summand, np.float64))
    bad = err > bound
    nrm = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    if np.any(bad):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} elements out of tolerance; worst at {i}: "
                             f"got {got[i]!r} want {want[i]!r} (rms {rms:.3g}); normwise {nrm:.3g}")
    return nrm


def bf16_bits_t(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_bits_t(t):
    return t.detach().cpu().view(torch.int32).numpy().view(np.uint32)


def close_norm(got, want, tol=TOL, what=""):
    """Normwise ||g - o|| / ||o|| <= tol (for outputs at the end of deep stacks)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    nrm = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    assert nrm <= tol, f"{what}: normwise error {nrm:.3g} > {tol}"
    return nrm
