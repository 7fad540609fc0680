"""GPU check of qlora_linear_bwd_noalloc, the allocation-free form of
qlora_linear_bwd (its temporaries in the library's fixed per-device scratch).

Two calls in a row on different shapes, the second smaller, each compared
bitwise with qlora_linear_bwd on the same inputs (same kernels, so the same
bits), and the second call must not see anything the first left in the
scratch. A shape whose workspace exceeds the scratch is refused.
"""

import ctypes

import pytest
import torch

import synth
from gpu_util import DEV, ql, require_gpu

pytestmark = pytest.mark.gpu


def _noalloc(dy, x, U, M, W, L, dx, dA, dB, accumulate):
    return ql.qlora_linear_bwd_noalloc(dy, x, U, M, W, L, dx, dA, dB, accumulate)


class Lin:
    def __init__(self, M, N, K, r, alpha, key):
        self.M, self.N, self.K, self.r = M, N, K, r
        packed, absmax = synth.nf4_store(N * K, *key, device=DEV)
        self.W = ql.NF4Weight(packed, absmax, N, K)
        self.L = ql.Lora(synth.normal_bf16((r, K), synth.LORA_SIGMA, *key, "A", device=DEV),
                         synth.normal_bf16((N, r), synth.LORA_SIGMA, *key, "B", device=DEV), r, alpha)
        self.x = synth.normal_bf16((M, K), 1.0, *key, "x", device=DEV)
        self.dy = synth.normal_bf16((M, N), 1.0, *key, "dy", device=DEV)
        fw, bw = ql.qlora_linear_workspace(M, N, K, r)
        self.bw = bw
        self.ws = torch.empty(max(fw, bw), dtype=torch.uint8, device=DEV)
        self.U = torch.empty(M, r, dtype=torch.bfloat16, device=DEV)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        ql.qlora_linear_fwd(self.x, M, self.W, self.L, y, self.U, self.ws)
        torch.cuda.synchronize()

    def outputs(self):
        return (torch.empty(self.M, self.K, dtype=torch.bfloat16, device=DEV),
                torch.full((self.r, self.K), 0.25, device=DEV), torch.full((self.N, self.r), -0.5, device=DEV))

    def with_ws(self, accumulate=0):
        dx, dA, dB = self.outputs()
        ql.qlora_linear_bwd(self.dy, self.x, self.U, self.M, self.W, self.L, dx, dA, dB, accumulate, self.ws)
        torch.cuda.synchronize()
        return dx, dA, dB

    def without_ws(self, accumulate=0):
        dx, dA, dB = self.outputs()
        _noalloc(self.dy, self.x, self.U, self.M, self.W, self.L, dx, dA, dB, accumulate)
        torch.cuda.synchronize()
        return dx, dA, dB


def _bitwise(a, b):
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


def test_noalloc_backward_equals_workspace_backward_twice():
    require_gpu()
    # first: an 8B gate projection at M = 2048 (split dX GEMM: the float32
    # partials, the transposed B and G all in the scratch); second, smaller:
    # ragged rows, a rank that is not a multiple of 8, no split
    big = Lin(2048, 14336, 4096, 16, 32.0, ("noalloc", "big"))
    small = Lin(77, 208, 320, 5, 7.0, ("noalloc", "small"))
    assert big.bw <= ql.QL_NOALLOC_SCRATCH_BYTES
    ref_big, ref_small = big.with_ws(), small.with_ws()
    got_big = big.without_ws()
    got_small = small.without_ws()
    assert _bitwise(got_big, ref_big)
    assert _bitwise(got_small, ref_small)
    # accumulate, and the big shape again after the small one
    assert _bitwise(small.without_ws(accumulate=1), small.with_ws(accumulate=1))
    assert _bitwise(big.without_ws(), ref_big)


def test_noalloc_allocates_nothing():
    require_gpu()
    lin = Lin(512, 4096, 4096, 16, 32.0, ("noalloc", "mem"))
    lin.without_ws()
    torch.cuda.synchronize()
    in_use = torch.cuda.memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    dx, dA, dB = lin.outputs()
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    torch.cuda.reset_peak_memory_stats()
    for _ in range(3):
        _noalloc(lin.dy, lin.x, lin.U, lin.M, lin.W, lin.L, dx, dA, dB, 0)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == torch.cuda.memory_allocated()
    assert torch.cuda.mem_get_info()[0] == free1, (free0, free1)


def test_noalloc_refuses_shapes_beyond_the_scratch():
    require_gpu()
    M, N, K, r = 16, 1 << 21, 64, 64    # transposed B alone is 256 MiB
    assert ql.qlora_linear_workspace(M, N, K, r)[1] > ql.QL_NOALLOC_SCRATCH_BYTES
    t = torch.empty(256, dtype=torch.uint8, device=DEV)
    W = ql.NF4Weight(t, t.view(torch.float32), N, K)
    L = ql.Lora(t, t, r, 128.0)
    before = t.clone()
    with pytest.raises(ql.QlError) as e:
        _noalloc(t, t, t, M, W, L, t, t.view(torch.float32), t.view(torch.float32), 0)
    assert e.value.status == ql.QL_ERR_WORKSPACE and "scratch" in ql.ql_last_error()
    torch.cuda.synchronize()
    assert torch.equal(t, before)
