"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function the header declares, and refuses bad arguments before touching
the device."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

from gpu_util import ROOT, lib, ql
from oracle import nf4 as onf4
from oracle import stack as ostack
from oracle import dq as dq_oracle

HEADER = os.path.join(ROOT, "include", "nf4qlora.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names) - {"if", "while"})


def test_header_declares_the_abi():
    fns = header_functions()
    for name in ("nf4_quantize", "nf4_dequant", "qlora_linear_fwd", "qlora_linear_bwd",
                 "stream_layer_stack_fwd", "stream_layer_stack_bwd"):
        assert name in fns
    assert set(fns) == set(ql.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = lib()
    for name in header_functions():
        assert hasattr(L, name), name
    raw = ctypes.CDLL(ql.LIB_PATH)
    for name in header_functions():
        getattr(raw, name)


def test_abi_version_and_codebook():
    lib()
    assert ql.ql_abi_version() == 101
    assert np.array_equal(ql.nf4_codebook().numpy().view(np.uint32), onf4.codebook().view(np.uint32))


def test_workspace_shape_validation():
    lib()
    f, b = ql.qlora_linear_workspace(64, 512, 256, 8)
    assert f > 0 and b > 0
    for args, st in (((64, 512, 250, 8), ql.QL_ERR_SHAPE), ((64, 500, 256, 8), ql.QL_ERR_SHAPE),
                     ((64, 512, 256, 0), ql.QL_ERR_RANK), ((64, 512, 256, 65), ql.QL_ERR_RANK),
                     ((-1, 512, 256, 8), ql.QL_ERR_SHAPE),
                     ((64, (1 << 21) + 16, 256, 8), ql.QL_ERR_SHAPE),
                     ((64, 512, (1 << 21) + 64, 8), ql.QL_ERR_SHAPE)):
        with pytest.raises(ql.QlError) as e:
            ql.qlora_linear_workspace(*args)
        assert e.value.status == st
        assert ql.ql_last_error()


def test_linear_validation_refuses_before_device_work():
    # Shape and rank errors are reported before any HIP call is made.
    lib()
    x = torch.zeros(64, 256, dtype=torch.bfloat16)
    W = ql.NF4Weight(torch.zeros(100, dtype=torch.uint8), torch.zeros(4, dtype=torch.float32), 512, 250)
    L = ql.Lora(torch.zeros(8, 256, dtype=torch.bfloat16), torch.zeros(512, 8, dtype=torch.bfloat16), 8, 16.0)
    with pytest.raises(ql.QlError) as e:
        ql.qlora_linear_fwd(x, 64, W, L, x, x, x, stream=0)
    assert e.value.status == ql.QL_ERR_SHAPE and "W.K" in ql.ql_last_error()
    W = ql.NF4Weight(torch.zeros(100, dtype=torch.uint8), torch.zeros(4, dtype=torch.float32), 512, 256)
    L = ql.Lora(L.A, L.B, 0, 16.0)
    with pytest.raises(ql.QlError) as e:
        ql.qlora_linear_fwd(x, 64, W, L, x, x, x, stream=0)
    assert e.value.status == ql.QL_ERR_RANK


@pytest.mark.parametrize("N,K", [((1 << 21) + 16, 4096), (4096, (1 << 21) + 64), ((1 << 22), (1 << 22))])
def test_dimensions_above_the_limit_are_refused(N, K):
    # Every byte offset the GEMMs form within one row block (64 rows of codes,
    # 256 rows of activations) must fit in 32 bits; dimensions above
    # QL_MAX_DIM = 2^21 are refused before any device work, forward and backward.
    lib()
    x = torch.zeros(64, 256, dtype=torch.bfloat16)
    W = ql.NF4Weight(torch.zeros(256, dtype=torch.uint8), torch.zeros(4, dtype=torch.float32), N, K)
    L = ql.Lora(torch.zeros(8, 256, dtype=torch.bfloat16), torch.zeros(512, 8, dtype=torch.bfloat16), 8, 16.0)
    with pytest.raises(ql.QlError) as e:
        ql.qlora_linear_fwd(x, 64, W, L, x, x, x, stream=0)
    assert e.value.status == ql.QL_ERR_SHAPE and "QL_MAX_DIM" in ql.ql_last_error()
    dA = torch.zeros(8, 256)
    with pytest.raises(ql.QlError) as e:
        ql.qlora_linear_bwd(x, x, x, 64, W, L, x, dA, dA, 0, x, stream=0)
    assert e.value.status == ql.QL_ERR_SHAPE and "QL_MAX_DIM" in ql.ql_last_error()


def test_quantize_dequant_size_validation():
    lib()
    w = torch.zeros(100)
    with pytest.raises(ql.QlError) as e:
        ql.nf4_quantize(w, torch.zeros(50, dtype=torch.uint8), torch.zeros(2), stream=0)
    assert e.value.status == ql.QL_ERR_SHAPE
    with pytest.raises(ql.QlError) as e:
        ql._check(ql.load().nf4_dequant(None, None, 64, 7, None, None))
    assert e.value.status == ql.QL_ERR_ARG


@pytest.mark.parametrize("name,L,H,I,KV,d,r", [
    ("smollm2_stack", 30, 576, 1536, 192, 64, 8),
    ("qwen3b_stack", 36, 2048, 11008, 256, 128, 16),
    ("llama8b_stack", 32, 4096, 14336, 1024, 128, 16),
])
def test_stack_layout_sizes(name, L, H, I, KV, d, r):
    # The store is the algorithmic 0.5625 B/weight plus at most 256 B of
    # alignment per tensor; records and tensors are 256-byte aligned; two
    # slots hold exactly two records.
    lib()
    cfg = ql.StackCfg(L, H, I, KV, d, r, 2.0 * r)
    offs, proj, total = ql.stream_layer_stack_layout(cfg)
    alg = ostack.nf4_store_bytes(L, H, I, KV)
    assert alg <= total <= alg + L * 14 * 256
    assert offs[0] == 0 and offs[-1] == total
    rec = offs[1]
    assert all(o % 256 == 0 for o in offs)
    assert all(a % 256 == 0 and b % 256 == 0 for a, b in proj.values())
    for p, (po, ao) in proj.items():
        N, K = cfg.proj_shape(p)
        assert po + N * K // 2 <= rec and ao + N * K // 64 * 4 <= rec
    spans = sorted((po, po + cfg.proj_shape(p)[0] * cfg.proj_shape(p)[1] // 2) for p, (po, _) in proj.items())
    spans += sorted((ao, ao + cfg.proj_shape(p)[0] * cfg.proj_shape(p)[1] // 16) for p, (_, ao) in proj.items())
    spans.sort()
    assert all(spans[i][1] <= spans[i + 1][0] for i in range(len(spans) - 1))
    slots, saved, ws = ql.stream_layer_stack_workspace(cfg, 512)
    assert slots == 2 * rec
    for nb in (3, 8):   # n_buffers slots of one record each (docs: stream_buffers in [2, 8])
        c = ql.StackCfg(**{**cfg.__dict__, "n_buffers": nb})
        assert ql.stream_layer_stack_workspace(c, 512)[0] == nb * rec
    offs_s, per = ql.stream_layer_stack_saved_layout(cfg, 512)
    assert saved == per * L
    # recompute: only each layer's input is saved; the workspace gains one
    # layer of activations and one layer output
    rc = ql.StackCfg(**{**cfg.__dict__, "recompute": 1})
    offs_r, per_r = ql.stream_layer_stack_saved_layout(rc, 512)
    assert per_r == 512 * cfg.hidden * 2 and offs_r["h_in"] == 0
    assert all(v == -1 for k, v in offs_r.items() if k != "h_in")
    _, saved_r, ws_r = ql.stream_layer_stack_workspace(rc, 512)
    assert saved_r == per_r * L
    assert ws_r == ws + per + 512 * cfg.hidden * 2


@pytest.mark.parametrize("absmax_dq", [0, 1])
def test_stack_record_is_four_contiguous_weight_groups(absmax_dq):
    # A record holds q|k|v, o, gate|up, down in that order, each group its
    # projections' codes then their scales (float32 absmax, or the
    # double-quantised block), every tensor 256-byte aligned, so that a group
    # is one contiguous byte range (the streamer may copy a record group by
    # group).
    lib()
    cfg = ql.StackCfg(2, 4096, 14336, 1024, 128, 16, 32.0, absmax_dq=absmax_dq)
    offs, proj, _ = ql.stream_layer_stack_layout(cfg)

    def up256(n):
        return -(-n // 256) * 256

    pos = 0
    for group in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
        for p in group:  # codes, in order
            N, K = cfg.proj_shape(p)
            assert proj[p][0] == pos, p
            pos += up256(N * K // 2)
        for p in group:  # then scales, in order
            N, K = cfg.proj_shape(p)
            assert proj[p][1] == pos, p
            pos += ql.nf4_dq_layout(N * K // 64)[2] if absmax_dq else up256(N * K // 64 * 4)
    assert pos == offs[1]


def test_stack_cfg_validation():
    lib()
    bad = [ql.StackCfg(0, 576, 1536, 192, 64, 8, 16.0), ql.StackCfg(2, 577, 1536, 192, 64, 8, 16.0),
           ql.StackCfg(2, 576, 1536, 200, 64, 8, 16.0), ql.StackCfg(2, 576, 1536, 192, 64, 0, 16.0),
           ql.StackCfg(2, 576, 1536, 192, 64, 8, 16.0, n_buffers=1),
           ql.StackCfg(2, 576, 1536, 192, 64, 8, 16.0, n_buffers=9),
           ql.StackCfg(2, 576, 1536, 192, 64, 8, 16.0, recompute=2),
           ql.StackCfg(2, 576, (1 << 21) + 64, 192, 64, 8, 16.0)]
    want = [ql.QL_ERR_SHAPE, ql.QL_ERR_SHAPE, ql.QL_ERR_SHAPE, ql.QL_ERR_RANK, ql.QL_ERR_UNSUPPORTED,
            ql.QL_ERR_UNSUPPORTED, ql.QL_ERR_ARG, ql.QL_ERR_SHAPE]
    for cfg, st in zip(bad, want):
        with pytest.raises(ql.QlError) as e:
            ql.stream_layer_stack_layout(cfg)
        assert e.value.status == st, (cfg, ql.ql_last_error())


def test_double_quantised_store_is_the_pages_size():
    # with double-quantised scales the 8B stack's store is the pages' 3.60 GB
    # with 113 MB layer records (README header figure), Qwen2.5-3B's 1.43 GB
    lib()
    c8 = ql.StackCfg(32, 4096, 14336, 1024, 128, 16, 32.0, absmax_dq=1)
    offs, proj, total = ql.stream_layer_stack_layout(c8)
    assert total == 3600474112 and offs[1] == 112514816
    assert round(total / 1e9, 2) == 3.60 and round(offs[1] / 1e6) == 113
    c3 = ql.StackCfg(36, 2048, 11008, 256, 128, 16, 32.0, absmax_dq=1)
    assert round(ql.stream_layer_stack_layout(c3)[2] / 1e9, 2) == 1.43
    # and the block layout matches the oracle's
    for n in (1, 256, 1000, 917504):
        assert ql.nf4_dq_layout(n) == dq_oracle.block_layout(n)


def test_profile_read_refuses_unknown_kernel_ids():
    for k in (-1, 7):
        with pytest.raises(ql.QlError) as e:
            ql.ql_profile_read(k)
        assert e.value.status == ql.QL_ERR_ARG
    n, ms, work = ql.ql_profile_read(ql.QL_KERNEL_DEQUANT)   # nothing recorded: zeros, no GPU work
    assert n == 0 and ms == 0.0 and work == 0.0


def test_noalloc_backward_refuses_shapes_beyond_its_scratch():
    # qlora_linear_bwd_noalloc has a fixed scratch of QL_NOALLOC_SCRATCH_BYTES;
    # a shape needing more is refused before any device work (here: the
    # transposed B of a 2^21-row weight at r = 64 alone is 256 MiB)
    lib()
    M, N, K, r = 16, 1 << 21, 64, 64
    assert ql.qlora_linear_workspace(M, N, K, r)[1] > ql.QL_NOALLOC_SCRATCH_BYTES
    assert ql.qlora_linear_workspace(2048, 14336, 4096, 16)[1] <= ql.QL_NOALLOC_SCRATCH_BYTES
    t = torch.zeros(256, dtype=torch.uint8)
    W = ql.NF4Weight(t, t.view(torch.float32), N, K)
    L = ql.Lora(t, t, r, 128.0)
    with pytest.raises(ql.QlError) as e:
        ql.qlora_linear_bwd_noalloc(t, t, t, M, W, L, t, t.view(torch.float32), t.view(torch.float32), 0, stream=0)
    assert e.value.status == ql.QL_ERR_WORKSPACE and "scratch" in ql.ql_last_error()
