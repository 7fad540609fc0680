"""GPU parity of the double-quantised block scales (nf4_double_quant,
nf4_dq_expand) and of the streamed stack with double-quantised records.

The GPU quantiser must reproduce the oracle bit for bit (codes, run scales and
the fixed-order mean), and the expansion too; the stack with compact records
must equal its resident run bitwise and the oracle stack whose scales are the
expanded ones within the GEMM tolerance.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, close, f64, ql, require_gpu
from oracle import dq as odq
from oracle import stack as ostack
from stack_util import GpuStack, identical

pytestmark = pytest.mark.gpu


def gpu_absmax(n_scales, seed):
    """Real scales: the absmax nf4_quantize computes for N(0, 0.02) weights."""
    w = synth.normal((n_scales * 64,), synth.W_SIGMA, "dq", seed, device=DEV)
    packed = torch.empty(n_scales * 32, dtype=torch.uint8, device=DEV)
    absmax = torch.empty(n_scales, dtype=torch.float32, device=DEV)
    ql.nf4_quantize(w, packed, absmax)
    return absmax


def gpu_dq(absmax):
    blk = torch.empty(ql.nf4_dq_layout(absmax.numel())[2], dtype=torch.uint8, device=DEV)
    ql.nf4_double_quant(absmax, blk)
    torch.cuda.synchronize()
    return blk


@pytest.mark.parametrize("n", [1, 255, 256, 257, 1000, 64 * 64 + 17])
def test_double_quant_bit_exact(n):
    require_gpu()
    a = gpu_absmax(n, n)
    blk = gpu_dq(a).cpu().numpy()
    codes, scales, mu = odq.double_quant(a.cpu().numpy())
    assert blk.size == odq.block_layout(n)[2]
    g_codes, g_scales, g_mu = odq.unpack_block(blk, n)
    assert g_mu.view(np.uint32) == np.float32(mu).view(np.uint32)
    assert np.array_equal(g_scales.view(np.uint32), scales.view(np.uint32))
    assert np.array_equal(g_codes, codes)
    # expansion
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    ql.nf4_dq_expand(torch.from_numpy(blk).to(DEV), n, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), odq.expand(codes, scales, mu).view(np.uint32))


def test_double_quant_full_size_sampled_runs():
    # the 8B gate|up projection's scale count; the mean over all of them, and
    # a sample of runs (first, last, ragged-free middle ones) bit for bit
    require_gpu()
    n = 14336 * 4096 // 64
    a = gpu_absmax(n, 7)
    blk = gpu_dq(a).cpu().numpy()
    c = a.cpu().numpy()
    runs = [0, 1, 2, 1000, 1791, odq.runs(n) - 1]
    codes, scales, mu = odq.double_quant(c, only_runs=runs)
    g_codes, g_scales, g_mu = odq.unpack_block(blk, n)
    assert g_mu == mu
    for b in runs:
        sl = slice(b * 256, (b + 1) * 256)
        assert np.array_equal(g_codes[sl], codes[sl]), b
        assert g_scales[b] == scales[b], b


def test_double_quant_special_cases():
    require_gpu()
    for c in (np.full(700, 0.0431, np.float32), np.zeros(300, np.float32),
              np.linspace(0.01, 0.2, 513).astype(np.float32)):
        blk = gpu_dq(torch.from_numpy(c).to(DEV)).cpu().numpy()
        codes, scales, mu = odq.double_quant(c)
        g = odq.unpack_block(blk, c.size)
        assert np.array_equal(g[0], codes) and np.array_equal(g[1], scales) and g[2] == mu


def test_double_quant_argument_errors():
    require_gpu()
    a = gpu_absmax(300, 1)
    small = torch.empty(512, dtype=torch.uint8, device=DEV)
    with pytest.raises(ql.QlError) as e:
        ql.nf4_double_quant(a, small)
    assert e.value.status == ql.QL_ERR_WORKSPACE


@pytest.fixture(scope="module")
def dqstack():
    require_gpu()
    return GpuStack("smollm2_stack", L=4, M=96, absmax_dq=1)


def test_dq_stack_streamed_equals_resident(dqstack):
    s = dqstack
    s.fwd()
    assert s.bwd(reuse=True) == ql.QL_OK
    assert s.fwd(reuse=True) == ql.QL_OK
    assert s.bwd(reuse=True) == ql.QL_OK
    got = s.results()
    s.step(resident=True)
    assert identical(got, s.results())


def test_dq_stack_matches_oracle_with_expanded_scales(dqstack):
    s = dqstack
    assert s.step(resident=False, reuse=True) == ql.QL_OK
    got = s.results()
    layers = s.oracle_layers()
    for lay in layers:   # the scales the stack uses: the oracle's expansion of its blocks
        for p, (packed, absmax) in list(lay.weights.items()):
            c, sc, mu = odq.double_quant(absmax)
            lay.weights[p] = (packed, odq.expand(c, sc, mu))
        lay.drop_cache()
    h, saved = ostack.stack_fwd(layers, f64(s.x))
    close(f64(got["y"]), h, what="y")
    dx0, grads = ostack.stack_bwd(layers, saved, f64(s.dy))
    close(f64(got["dx"]), dx0, what="dx0")
    for li in range(len(layers)):
        for p in ("v", "o", "gate", "up", "down"):
            close(f64(got["dA"][li][p]), grads[li][p][0], what=f"L{li}:{p}:dA")
            close(f64(got["dB"][li][p]), grads[li][p][1], what=f"L{li}:{p}:dB")


def test_dq_record_is_smaller(dqstack):
    s = dqstack
    offs_dq, _, _ = ql.stream_layer_stack_layout(s.cfg)
    plain = ql.StackCfg(**{**s.cfg.__dict__, "absmax_dq": 0})
    offs, _, _ = ql.stream_layer_stack_layout(plain)
    assert offs_dq[1] < offs[1]
