"""Kernel timing (ql_profile_enable / ql_profile_read) on one NF4 + LoRA linear:
every timed kernel id records its launches and the algorithmic work the
header states (FLOPs for the fused GEMMs, bytes for the HBM-bound kernels),
and results are the same with timing on."""

import pytest
import torch

from gpu_util import DEV, ql, require_gpu
import synth

pytestmark = pytest.mark.gpu


def _linear(M, K, N, r):
    inp = synth.linear_inputs(M, K, N, r, ("profile",))
    w = inp["W"].to(DEV).reshape(-1)
    packed = torch.empty(N * K // 2, dtype=torch.uint8, device=DEV)
    absmax = torch.empty(N * K // 64, dtype=torch.float32, device=DEV)
    ql.nf4_quantize(w, packed, absmax)
    W = ql.NF4Weight(packed, absmax, N, K)
    L = ql.Lora(inp["A"].to(DEV), inp["B"].to(DEV), r, 2.0 * r)
    fw, bw = ql.qlora_linear_workspace(M, N, K, r)
    ws = torch.empty(max(fw, bw), dtype=torch.uint8, device=DEV)
    x, dy = inp["x"].to(DEV), inp["dy"].to(DEV)
    out = dict(y=torch.empty(M, N, dtype=torch.bfloat16, device=DEV), U=torch.empty(M, r, dtype=torch.bfloat16, device=DEV),
               dx=torch.empty(M, K, dtype=torch.bfloat16, device=DEV), dA=torch.empty(r, K, device=DEV),
               dB=torch.empty(N, r, device=DEV), Wd=torch.empty(N * K, dtype=torch.bfloat16, device=DEV))

    def run():
        ql.qlora_linear_fwd(x, M, W, L, out["y"], out["U"], ws)
        ql.qlora_linear_bwd(dy, x, out["U"], M, W, L, out["dx"], out["dA"], out["dB"], 0, ws)
        ql.nf4_dequant(packed, absmax, N * K, out["Wd"])
        torch.cuda.synchronize()
        return {k: v.clone() for k, v in out.items()}
    return run


def test_profile_records_work_and_changes_no_result():
    require_gpu()
    M, K, N, r = 1100, 512, 640, 16
    run = _linear(M, K, N, r)
    plain = run()
    ql.ql_profile_enable(1)
    try:
        timed = run()
    finally:
        ql.ql_profile_enable(0)
    for k in plain:
        assert torch.equal(plain[k].view(torch.uint8), timed[k].view(torch.uint8)), k
    rec = {k: ql.ql_profile_read(k) for k in list(ql.KERNEL_SYMBOLS) + list(ql.HBM_KERNEL_SYMBOLS)}
    fwd = rec[ql.QL_KERNEL_GEMM_FWD][2] + rec[ql.QL_KERNEL_GEMM_FWD_NARROW][2]
    bwd = rec[ql.QL_KERNEL_GEMM_BWD][2] + rec[ql.QL_KERNEL_GEMM_BWD_NARROW][2]
    assert fwd == 2.0 * M * N * (K + r)
    assert bwd == 2.0 * M * K * (N + r)
    # the dequantisation reads codes and scales and writes bf16 once
    n, ms, b = rec[ql.QL_KERNEL_DEQUANT]
    assert n == 1 and ms > 0 and b == N * K * (0.5625 + 2.0)
    # U = x A^T and G = dY B: at least operands, Bt and outputs once each
    n, ms, b = rec[ql.QL_KERNEL_LORA_ROW]
    assert n == 2 and ms > 0
    base = (2 * M * K + 2 * r * K + 2 * M * r) + (2 * M * N + 2 * r * N + 2 * M * r)
    assert base <= b <= base + 2 * 8 * 8 * M * r
    # dB and dA in one launch; M = 1100 splits the rows, so partials count too
    n, ms, b = rec[ql.QL_KERNEL_LORA_COL]
    assert n == 1 and ms > 0
    base = (2 * M * N + 2 * M * r + 4 * N * r) + (2 * M * K + 2 * M * r + 4 * K * r)
    assert base < b <= base + 2 * 4 * 8 * (N + K) * r
