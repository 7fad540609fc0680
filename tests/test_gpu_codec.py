"""GPU parity of the NF4 codec: bit-exact against the oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import synth
from oracle import nf4 as onf4
from gpu_util import DEV, bf16_bits_t, f32_bits_t, ql, require_gpu

pytestmark = pytest.mark.gpu


def _quant_gpu(w_np):
    w = torch.from_numpy(np.ascontiguousarray(w_np, np.float32)).to(DEV)
    n = w.numel()
    packed = torch.empty(n // 2, dtype=torch.uint8, device=DEV)
    absmax = torch.empty(n // 64, dtype=torch.float32, device=DEV)
    ql.nf4_quantize(w, packed, absmax)
    return packed.cpu().numpy(), absmax.cpu().numpy()


def _special_weights():
    g = np.random.default_rng(7)
    c = onf4.codebook()
    blocks = []
    blocks.append(np.zeros(64, np.float32))                       # zero block
    z = np.zeros(64, np.float32); z[::2] = -0.0; blocks.append(z)  # negative zeros
    for e in (-126, -100, -20, 0, 20, 100, 126):                  # codebook-valued blocks
        a = np.float32(2.0 ** e * 1.37)
        codes = g.integers(0, 16, 64); codes[5] = 15
        blocks.append((c[codes] * a).astype(np.float32))
    mids = ((c[:-1].astype(np.float64) + c[1:]) / 2).astype(np.float32)
    b = np.zeros(64, np.float32); b[:15] = mids; b[63] = 1.0; blocks.append(b)   # exact ties
    b = np.zeros(64, np.float32); b[:15] = np.nextafter(mids, np.float32(2)); b[63] = 1.0; blocks.append(b)
    b = np.zeros(64, np.float32); b[:15] = np.nextafter(mids, np.float32(-2)); b[63] = -1.0; blocks.append(b)
    blocks.append((g.standard_normal(64) * 1e-40).astype(np.float32))   # subnormals
    blocks.append((g.standard_normal(64) * 1e37).astype(np.float32))    # large
    blocks.append(np.full(64, 3.0, np.float32))                        # constant block
    return np.concatenate(blocks)


def test_quantize_bitexact_pr1_and_special_cases():
    require_gpu()
    M, K, N, r = 64, 256, 512, 8
    W = synth.linear_inputs(M, K, N, r, ("linear_pr1",))["W"].numpy()
    w = np.concatenate([W.reshape(-1), _special_weights()])
    packed, absmax = _quant_gpu(w)
    op, oa = onf4.quantize(w)
    assert np.array_equal(packed, op)
    assert np.array_equal(absmax.view(np.uint32), oa.view(np.uint32))


def test_quantize_full_projection_sampled_blocks():
    # Llama-3.1-8B gate projection, 14336 x 4096, N(0, 0.02) drawn on the GPU.
    require_gpu()
    N, K = 14336, 4096
    w = synth.normal((N * K,), synth.W_SIGMA, "llama8b_layer", "gate", "W", device=DEV)
    packed = torch.empty(N * K // 2, dtype=torch.uint8, device=DEV)
    absmax = torch.empty(N * K // 64, dtype=torch.float32, device=DEV)
    ql.nf4_quantize(w, packed, absmax)
    nb = N * K // 64
    idx = np.unique(np.concatenate([[0, nb - 1], np.random.default_rng(8).integers(0, nb, 3000)]))
    ti = torch.from_numpy(idx).to(DEV)
    wb = w.view(nb, 64)[ti].cpu().numpy()
    pb = packed.view(nb, 32)[ti].cpu().numpy()
    ab = absmax[ti].cpu().numpy()
    op, oa = onf4.quantize(wb.reshape(-1))
    assert np.array_equal(pb.reshape(-1), op)
    assert np.array_equal(ab.view(np.uint32), oa.view(np.uint32))


@pytest.mark.parametrize("bad,at,n", [(float("nan"), 100, 256), (float("inf"), 0, 256),
                                      (float("-inf"), 255, 256), (float("nan"), 3 * 2 ** 20 + 7, 2 ** 22)])
def test_quantize_refuses_nonfinite(bad, at, n):
    # refused before anything is written: the outputs keep their contents; a
    # finite call right after (the device flag cleared) succeeds
    require_gpu()
    w = torch.zeros(n, dtype=torch.float32, device=DEV)
    w[at] = bad
    packed = torch.full((n // 2,), 0x5A, dtype=torch.uint8, device=DEV)
    absmax = torch.full((n // 64,), -2.5, dtype=torch.float32, device=DEV)
    with pytest.raises(ql.QlError) as e:
        ql.nf4_quantize(w, packed, absmax)
    assert e.value.status == ql.QL_ERR_NONFINITE
    torch.cuda.synchronize()
    assert bool((packed == 0x5A).all()) and bool((absmax == -2.5).all())
    w[at] = 1.0
    assert ql.nf4_quantize(w, packed, absmax) == ql.QL_OK
    torch.cuda.synchronize()
    assert float(absmax[at // 64]) == 1.0


def test_quantize_rejects_bad_sizes():
    require_gpu()
    w = torch.zeros(100, dtype=torch.float32, device=DEV)
    packed = torch.empty(50, dtype=torch.uint8, device=DEV)
    absmax = torch.empty(2, dtype=torch.float32, device=DEV)
    with pytest.raises(ql.QlError) as e:
        ql.nf4_quantize(w, packed, absmax)
    assert e.value.status == ql.QL_ERR_SHAPE


def _dequant_gpu(packed_np, absmax_np, dtype):
    p = torch.from_numpy(packed_np).to(DEV)
    a = torch.from_numpy(absmax_np).to(DEV)
    n = packed_np.size * 2
    out = torch.empty(n, dtype=dtype, device=DEV)
    ql.nf4_dequant(p, a, n, out)
    return out


def test_dequant_bitexact_all_codes_and_scales():
    require_gpu()
    g = np.random.default_rng(9)
    codes = np.tile(np.arange(16, dtype=np.uint8), 4 * 400)            # 400 blocks, all codes
    scales = np.concatenate([
        np.float32(2.0) ** np.arange(-149, 128, 3).astype(np.float32),   # powers of two incl. subnormal range
        g.uniform(0, 1, 200).astype(np.float32),
        np.float32([0.0, 3.4e38, 1e-45, 1.17549435e-38, 0.048, 0.02 * 2.4]),
    ])[:400].astype(np.float32)
    scales = np.resize(scales, 400).astype(np.float32)
    packed = onf4.pack(codes)
    want32 = onf4.dequant_f32(packed, scales)
    want16 = onf4.dequant_bf16(packed, scales)
    got32 = _dequant_gpu(packed, scales, torch.float32)
    got16 = _dequant_gpu(packed, scales, torch.bfloat16)
    assert np.array_equal(f32_bits_t(got32), want32.view(np.uint32))
    assert np.array_equal(bf16_bits_t(got16), onf4.bf16_bits(want16))


def test_dequant_full_projection_sampled():
    # Llama-3.1-8B down projection store, 4096 x 14336, synthetic codes and scales.
    require_gpu()
    n = 4096 * 14336
    packed, absmax = synth.nf4_store(n, "llama8b_layer", "down", device=DEV)
    out = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    ql.nf4_dequant(packed, absmax, n, out)
    out32 = torch.empty(n, dtype=torch.float32, device=DEV)
    ql.nf4_dequant(packed, absmax, n, out32)
    nb = n // 64
    idx = np.unique(np.concatenate([[0, nb - 1], np.random.default_rng(10).integers(0, nb, 4000)]))
    ti = torch.from_numpy(idx).to(DEV)
    pb = packed.view(nb, 32)[ti].cpu().numpy().reshape(-1)
    ab = absmax[ti].cpu().numpy()
    assert np.array_equal(bf16_bits_t(out.view(nb, 64)[ti]).reshape(-1), onf4.bf16_bits(onf4.dequant_bf16(pb, ab)))
    assert np.array_equal(f32_bits_t(out32.view(nb, 64)[ti]).reshape(-1), onf4.dequant_f32(pb, ab).view(np.uint32))


def test_codebook_bits_match_oracle():
    require_gpu()
    assert np.array_equal(ql.nf4_codebook().numpy().view(np.uint32), onf4.codebook().view(np.uint32))
