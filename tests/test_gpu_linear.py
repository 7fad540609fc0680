"""GPU parity of the NF4 + LoRA linear (qlora_linear_fwd / _bwd) through the C ABI."""

import numpy as np
import pytest
import torch

import synth
from oracle import linear as olin
from oracle import nf4 as onf4
from gpu_util import DEV, bf16_bits_t, close, f64, ql, require_gpu

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float64)).to(torch.float32).to(torch.bfloat16)


class Case:
    """Device tensors of one linear; packed/absmax either from the oracle or synthetic."""

    def __init__(self, M, K, N, r, alpha, key, x=None, packed=None, absmax=None, A=None, B=None, dy=None):
        inp = synth.linear_inputs(M, K, N, r, key)
        self.M, self.K, self.N, self.r, self.alpha = M, K, N, r, alpha
        self.x = (inp["x"] if x is None else x).contiguous()
        self.A = (inp["A"] if A is None else A).contiguous()
        self.B = (inp["B"] if B is None else B).contiguous()
        self.dy = (inp["dy"] if dy is None else dy).contiguous()
        if packed is None:
            packed, absmax = onf4.quantize(inp["W"].numpy().reshape(-1))
            packed, absmax = torch.from_numpy(packed), torch.from_numpy(absmax)
        self.packed, self.absmax = packed, absmax

    def run(self, need_dx=True, accumulate=False, dA0=None, dB0=None):
        M, K, N, r = self.M, self.K, self.N, self.r
        d = lambda t: t.to(DEV)
        W = ql.NF4Weight(d(self.packed), d(self.absmax), N, K)
        L = ql.Lora(d(self.A), d(self.B), r, self.alpha)
        fw, bw = ql.qlora_linear_workspace(M, N, K, r)
        ws = torch.empty(max(fw, bw, 1), dtype=torch.uint8, device=DEV)
        x, dy = d(self.x), d(self.dy)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        U = torch.empty(M, r, dtype=torch.bfloat16, device=DEV)
        ql.qlora_linear_fwd(x, M, W, L, y, U, ws)
        dx = torch.empty(M, K, dtype=torch.bfloat16, device=DEV) if need_dx else None
        dA = (torch.zeros(r, K, dtype=torch.float32) if dA0 is None else dA0.clone()).to(DEV)
        dB = (torch.zeros(N, r, dtype=torch.float32) if dB0 is None else dB0.clone()).to(DEV)
        ql.qlora_linear_bwd(dy, x, U, M, W, L, dx, dA, dB, accumulate, ws)
        torch.cuda.synchronize()
        return dict(y=y.cpu(), U=U.cpu(), dx=None if dx is None else dx.cpu(), dA=dA.cpu(), dB=dB.cpu())

    def oracle(self, mode="faithful"):
        p, a = self.packed.numpy(), self.absmax.numpy()
        x, A, B, dy = f64(self.x), f64(self.A), f64(self.B), f64(self.dy)
        y, U = olin.fwd(x, p, a, self.N, self.K, A, B, self.alpha, mode=mode)
        dX, dA, dB, _ = olin.bwd(dy, x, U, p, a, self.N, self.K, A, B, self.alpha, mode=mode)
        return dict(y=y, U=U, dx=dX, dA=dA, dB=dB)


def _compare(got, want, tag):
    for k in ("U", "y", "dx", "dA", "dB"):
        if got.get(k) is not None:
            close(f64(got[k]), want[k], what=f"{tag}:{k}")


def test_pr1_linear_matches_oracle():
    # M=64 tokens, K=256, N=512, r=8, alpha=16: the single-linear configuration.
    require_gpu()
    c = Case(64, 256, 512, 8, 16.0, ("linear_pr1",))
    _compare(c.run(), c.oracle(), "pr1")


@pytest.mark.parametrize("M,K,N,r,alpha", [
    (1, 64, 16, 1, 1.0),        # smallest legal shapes
    (77, 320, 208, 5, 7.0),     # ragged M, N not a tile multiple, r not a multiple of 8, s not a power of 2
    (130, 192, 144, 64, 64.0),  # r at its maximum, M just over one tile
    (300, 1024, 400, 16, 32.0), # several tiles each way with ragged tails
    (1100, 128, 80, 12, 24.0),  # the adapter-gradient reductions split over rows (float32 partials)
])
def test_ragged_shapes_match_oracle(M, K, N, r, alpha):
    require_gpu()
    c = Case(M, K, N, r, alpha, ("ragged", M, K, N, r))
    _compare(c.run(), c.oracle(), f"ragged{M}x{K}x{N}r{r}")


def test_wide_dx_tiles_ragged_rows_odd_rank():
    # K = 32768 output columns at M = 300 make 2 x 128 = 256 dX tiles of 256 x
    # 256, one whole round, so the dX runs unsplit on the wide 8-wave build:
    # its last row tile holds 44 rows, and r = 5 takes the LoRA step's
    # element-wise A-tile loads (done by half of its threads).
    require_gpu()
    c = Case(300, 32768, 256, 5, 7.0, ("wide-dx", 300, 32768, 256, 5))
    _compare(c.run(), c.oracle(), "wide-dx")


def test_accumulate_adds_to_existing_grads():
    require_gpu()
    c = Case(64, 256, 512, 8, 16.0, ("linear_pr1",))
    base = c.run()
    g = torch.Generator().manual_seed(3)
    dA0 = torch.randn(8, 256, generator=g)
    dB0 = torch.randn(512, 8, generator=g)
    acc = c.run(need_dx=False, accumulate=True, dA0=dA0, dB0=dB0)
    assert acc["dx"] is None
    # the same float32 addition on both sides
    assert torch.equal(acc["dA"], dA0 + base["dA"])
    assert torch.equal(acc["dB"], dB0 + base["dB"])


def test_accumulate_with_split_reductions():
    # M = 1100 splits the dA / dB row reductions; the second pass adds the
    # split sums, scales and accumulates
    require_gpu()
    c = Case(1100, 128, 80, 12, 24.0, ("ragged", 1100, 128, 80, 12))
    base = c.run()
    g = torch.Generator().manual_seed(4)
    dA0 = torch.randn(12, 128, generator=g)
    dB0 = torch.randn(80, 12, generator=g)
    acc = c.run(need_dx=False, accumulate=True, dA0=dA0, dB0=dB0)
    assert torch.equal(acc["dA"], dA0 + base["dA"])
    assert torch.equal(acc["dB"], dB0 + base["dB"])


def test_exact_construction_bitwise():
    # Integer-grid operands make every float32 partial sum exact in any order,
    # so y and dX must equal the exact result rounded once to bf16.
    require_gpu()
    M, K, N, r, alpha = 96, 512, 160, 4, 8.0
    g = np.random.default_rng(31)
    codes = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    packed = torch.from_numpy(onf4.pack(codes.reshape(-1)))
    absmax = torch.ones(N * K // 64, dtype=torch.float32)
    x = g.integers(-2, 3, size=(M, K)).astype(np.float64)
    A = np.zeros((r, K)); A[np.arange(r), g.integers(0, K, size=r)] = 2.0 ** -4
    B = np.zeros((N, r)); B[np.arange(N), g.integers(0, r, size=N)] = 2.0 ** -3
    dy = g.integers(-2, 3, size=(M, N)).astype(np.float64)
    c = Case(M, K, N, r, alpha, ("exact",), x=_bf16(x), packed=packed, absmax=absmax, A=_bf16(A), B=_bf16(B),
             dy=_bf16(dy))
    got, want = c.run(), c.oracle()
    assert np.array_equal(bf16_bits_t(got["y"]), onf4.bf16_bits(want["y"]))
    assert np.array_equal(bf16_bits_t(got["U"]), onf4.bf16_bits(want["U"]))
    assert np.array_equal(bf16_bits_t(got["dx"]), onf4.bf16_bits(want["dx"]))
    close(f64(got["dA"]), want["dA"], tol=1e-6, what="exact:dA")
    close(f64(got["dB"]), want["dB"], tol=1e-6, what="exact:dB")


@pytest.mark.parametrize("M,K,N", [(256, 14336, 4096), (256, 4096, 14336)])
def test_exact_construction_bitwise_split_reductions(M, K, N):
    # Shapes whose GEMMs split the reduction across workgroups (the forward
    # over K = 14336, the dX over N = 14336: three splits each at M = 256)
    # and sum float32 partials in a second pass. With operands in {-1, 0, 1},
    # at most 8192 non-zeros per row and absmax 1, every float32 partial sum is
    # exact in any order, so y and dX must equal the exact result rounded once.
    require_gpu()
    r, alpha = 4, 8.0
    g = np.random.default_rng(M + K + N)
    codes = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    packed = torch.from_numpy(onf4.pack(codes.reshape(-1)))
    absmax = torch.ones(N * K // 64, dtype=torch.float32)

    def sparse_pm1(rows, cols):
        v = g.integers(-1, 2, size=(rows, cols)).astype(np.float64)
        for i in range(rows):   # at most 8192 non-zeros per row
            nz = np.flatnonzero(v[i])
            if nz.size > 8192:
                v[i, g.choice(nz, nz.size - 8192, replace=False)] = 0.0
        return v

    x = sparse_pm1(M, K)
    dy = sparse_pm1(M, N)
    A = np.zeros((r, K)); A[np.arange(r), g.integers(0, K, size=r)] = 2.0 ** -4
    B = np.zeros((N, r)); B[np.arange(N), g.integers(0, r, size=N)] = 2.0 ** -3
    c = Case(M, K, N, r, alpha, ("exact-split", M, K, N), x=_bf16(x), packed=packed, absmax=absmax, A=_bf16(A),
             B=_bf16(B), dy=_bf16(dy))
    got, want = c.run(), c.oracle()
    assert np.array_equal(bf16_bits_t(got["y"]), onf4.bf16_bits(want["y"]))
    assert np.array_equal(bf16_bits_t(got["dx"]), onf4.bf16_bits(want["dx"]))


def test_one_hot_rows_read_weight_columns():
    # x rows one-hot, B = 0: each y row is a column of the bf16 dequantised W
    # (isolates the fused loader's decode), bitwise.
    require_gpu()
    M, K, N, r = 128, 256, 256, 8
    inp = synth.linear_inputs(M, K, N, r, ("onehot",))
    cols = np.random.default_rng(32).integers(0, K, size=M)
    x = np.zeros((M, K)); x[np.arange(M), cols] = 1.0
    c = Case(M, K, N, r, 16.0, ("onehot",), x=_bf16(x), B=torch.zeros(N, r, dtype=torch.bfloat16))
    got = c.run()
    Wb = onf4.dequant_bf16(c.packed.numpy(), c.absmax.numpy()).reshape(N, K)
    assert np.array_equal(bf16_bits_t(got["y"]), onf4.bf16_bits(Wb[:, cols].T))


def test_deterministic_runs():
    require_gpu()
    c = Case(300, 1024, 400, 16, 32.0, ("ragged", 300, 1024, 400, 16))
    a, b = c.run(), c.run()
    for k in a:
        assert torch.equal(a[k].view(torch.uint8) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.uint8) if b[k].dtype == torch.bfloat16 else b[k]), k


def test_zero_rows_is_noop_and_zeroes_grads():
    require_gpu()
    N, K, r = 64, 128, 4
    W = ql.NF4Weight(torch.zeros(N * K // 2, dtype=torch.uint8, device=DEV),
                     torch.zeros(N * K // 64, dtype=torch.float32, device=DEV), N, K)
    L = ql.Lora(torch.zeros(r, K, dtype=torch.bfloat16, device=DEV), torch.zeros(N, r, dtype=torch.bfloat16, device=DEV),
                r, 8.0)
    dA = torch.ones(r, K, device=DEV)
    dB = torch.ones(N, r, device=DEV)
    ql.qlora_linear_fwd(None, 0, W, L, None, None, None)
    ql.qlora_linear_bwd(None, None, None, 0, W, L, None, dA, dB, 0, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0


@pytest.mark.parametrize("what,status", [("K", ql.QL_ERR_SHAPE), ("N", ql.QL_ERR_SHAPE), ("r0", ql.QL_ERR_RANK),
                                         ("r65", ql.QL_ERR_RANK), ("align", ql.QL_ERR_ALIGN),
                                         ("ws", ql.QL_ERR_WORKSPACE), ("null", ql.QL_ERR_ARG)])
def test_errors_enqueue_nothing(what, status):
    require_gpu()
    M, N, K, r = 64, 128, 256, 8
    packed = torch.zeros(N * K // 2 + 16, dtype=torch.uint8, device=DEV)
    absmax = torch.zeros(N * K // 64, dtype=torch.float32, device=DEV)
    W = ql.NF4Weight(packed, absmax, N, K)
    A = torch.zeros(64, K, dtype=torch.bfloat16, device=DEV)
    B = torch.zeros(N, 64, dtype=torch.bfloat16, device=DEV)
    L = ql.Lora(A, B, r, 16.0)
    x = torch.zeros(M, K, dtype=torch.bfloat16, device=DEV)
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    U = torch.empty(M, 64, dtype=torch.bfloat16, device=DEV)
    fw, _ = ql.qlora_linear_workspace(M, N, K, r)
    ws = torch.empty(fw, dtype=torch.uint8, device=DEV)
    if what == "K":
        W = ql.NF4Weight(packed, absmax, N, 250)
    elif what == "N":
        W = ql.NF4Weight(packed, absmax, 120, K)
    elif what == "r0":
        L = ql.Lora(A, B, 0, 16.0)
    elif what == "r65":
        L = ql.Lora(A, B, 65, 16.0)
    elif what == "align":
        W = ql.NF4Weight(packed[1:], absmax, N, K)
    elif what == "ws":
        ws = ws[:16]
    elif what == "null":
        x = None
    with pytest.raises(ql.QlError) as e:
        ql.qlora_linear_fwd(x, M, W, L, y, U, ws)
    assert e.value.status == status
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_llama8b_layer_projections_full_size():
    # Projections of one Llama-3.1-8B-shaped layer at M=512, r=16, alpha=32,
    # with synthetic NF4 stores. U, dA and dB are checked in full; y and dX on
    # sampled rows (row m of y and dX needs only row m of x and dY).
    require_gpu()
    M, H, I, KV, r, alpha = 512, 4096, 14336, 1024, 16, 32.0
    rows = np.array([0, 1, 255, 511])
    for p, (N, K) in {"q": (H, H), "k": (KV, H), "gate": (I, H), "down": (H, I)}.items():
        packed, absmax = synth.nf4_store(N * K, "llama8b_layer", p, device=DEV)
        inp = synth.linear_inputs(M, K, N, r, ("llama8b_layer", p), device=DEV)
        W = ql.NF4Weight(packed, absmax, N, K)
        L = ql.Lora(inp["A"], inp["B"], r, alpha)
        fw, bw = ql.qlora_linear_workspace(M, N, K, r)
        ws = torch.empty(max(fw, bw), dtype=torch.uint8, device=DEV)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        U = torch.empty(M, r, dtype=torch.bfloat16, device=DEV)
        dx = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
        dA = torch.empty(r, K, device=DEV)
        dB = torch.empty(N, r, device=DEV)
        ql.qlora_linear_fwd(inp["x"], M, W, L, y, U, ws)
        ql.qlora_linear_bwd(inp["dy"], inp["x"], U, M, W, L, dx, dA, dB, 0, ws)
        torch.cuda.synchronize()
        x, A, B, dy = f64(inp["x"]), f64(inp["A"]), f64(inp["B"]), f64(inp["dy"])
        pk, am = packed.cpu().numpy(), absmax.cpu().numpy()
        Uo = olin.lora_down(x, A)
        close(f64(U), Uo, what=f"{p}:U")
        _, dAo, dBo, _ = olin.bwd(dy, x, Uo, pk, am, N, K, A, B, alpha, need_dx=False)
        close(f64(dA), dAo, what=f"{p}:dA")
        close(f64(dB), dBo, what=f"{p}:dB")
        Wf = olin.weight(pk, am, N, K, "faithful")
        yo, _ = olin.fwd(x[rows], pk, am, N, K, A, B, alpha, W=Wf)
        close(f64(y)[rows], yo, what=f"{p}:y")
        dXr, _, _, _ = olin.bwd(dy[rows], x[rows], Uo[rows], pk, am, N, K, A, B, alpha, W=Wf)
        close(f64(dx)[rows], dXr, what=f"{p}:dx")
        del Wf


def test_projection_beyond_2_gib_of_codes():
    # N x K = 65536 x 69632 = 4.56e9 weights: 2.28 GB of codes, past 2^31
    # bytes, the size above which the pages report a backward that went wrong
    # silently while the forward stayed right. The dX GEMM's weight loads are
    # based at each 64-row reduction step (64-bit base, 32-bit offsets within
    # the step), so rows past 2^31 bytes must read their own codes. Sampled
    # outputs: y[:, n] needs row n of W, dX[:, k] needs column k of W over all
    # 65536 rows.
    require_gpu()
    M, N, K, r, alpha = 16, 65536, 69632, 8, 16.0
    assert N * K // 2 > 2 ** 31
    packed, absmax = synth.nf4_store(N * K, "big", device=DEV)
    x = synth.normal_bf16((M, K), 1.0, "big", "x", device=DEV)
    dy = synth.normal_bf16((M, N), 1.0, "big", "dy", device=DEV)
    A = synth.normal_bf16((r, K), synth.LORA_SIGMA, "big", "A", device=DEV)
    B = synth.normal_bf16((N, r), synth.LORA_SIGMA, "big", "B", device=DEV)
    W = ql.NF4Weight(packed, absmax, N, K)
    L = ql.Lora(A, B, r, alpha)
    fw, bw = ql.qlora_linear_workspace(M, N, K, r)
    ws = torch.empty(max(fw, bw), dtype=torch.uint8, device=DEV)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    U = torch.empty(M, r, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    dA = torch.empty(r, K, device=DEV)
    dB = torch.empty(N, r, device=DEV)
    ql.qlora_linear_fwd(x, M, W, L, y, U, ws)
    ql.qlora_linear_bwd(dy, x, U, M, W, L, dx, dA, dB, 0, ws)
    torch.cuda.synchronize()
    g = np.random.default_rng(33)
    ns = np.unique(np.concatenate([[0, N - 1], g.integers(0, N, 24)]))
    ks = np.unique(np.concatenate([[0, 1, K - 1], g.integers(0, K, 24)]))
    x64, A64, B64, dy64 = f64(x), f64(A), f64(B), f64(dy)
    pk = packed.cpu().numpy()
    am = absmax.cpu().numpy()
    Wr = onf4.dequant_rows_bf16(pk, am, K, ns)                 # [len(ns) x K]
    yo, _ = olin.fwd(x64, None, None, len(ns), K, A64, B64[ns], alpha, W=Wr)
    close(f64(y)[:, ns], yo, what="big:y")
    Wc = onf4.dequant_cols_bf16(pk, am, N, K, ks)              # [N x len(ks)]
    Uo = olin.lora_down(x64, A64)
    dxo, _, _, _ = olin.bwd(dy64, x64[:, ks], Uo, None, None, N, len(ks), A64[:, ks], B64, alpha, W=Wc)
    close(f64(dx)[:, ks], dxo, what="big:dx")
