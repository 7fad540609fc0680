"""Pins of the decoder-stack oracle: finite differences, zero/non-zero gradients, page figures."""

import numpy as np

from oracle import nf4, stack


def _tiny_stack(L=2, H=128, I=256, KV=64, d=32, r=4, alpha=8.0, seed=20):
    g = np.random.default_rng(seed)
    layers = []
    for _ in range(L):
        weights, lora = {}, {}
        for p, (N, K) in stack.proj_shapes(H, I, KV).items():
            W = (g.standard_normal(N * K) * 0.05).astype(np.float32)
            weights[p] = nf4.quantize(W)
            lora[p] = (nf4.round_bf16(g.standard_normal((r, K)) * 0.05),
                       nf4.round_bf16(g.standard_normal((N, r)) * 0.05))
        layers.append(stack.Layer(H, I, KV, d, alpha, weights, lora))
    return layers


def test_stack_finite_differences_exact_mode():
    M, H = 3, 128
    layers = _tiny_stack()
    g = np.random.default_rng(21)
    x = g.standard_normal((M, H))
    dy = g.standard_normal((M, H))

    def loss():
        return float(np.sum(dy * stack.stack_fwd(layers, x, mode="exact", keep=False)[0]))

    h_L, saved = stack.stack_fwd(layers, x, mode="exact")
    dx0, grads = stack.stack_bwd(layers, saved, dy, mode="exact")
    eps = 1e-5
    for _ in range(4):
        m, k = g.integers(0, M), g.integers(0, H)
        x[m, k] += eps; lp = loss(); x[m, k] -= 2 * eps; lm = loss(); x[m, k] += eps
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - dx0[m, k]) <= 1e-5 * max(1.0, abs(fd)), (fd, dx0[m, k])
    for li in (0, 1):
        for p in ("v", "o", "gate", "up", "down"):
            A, B = layers[li].lora[p]
            for arr, grad in ((A, grads[li][p][0]), (B, grads[li][p][1])):
                i = tuple(g.integers(0, s) for s in arr.shape)
                arr[i] += eps; lp = loss(); arr[i] -= 2 * eps; lm = loss(); arr[i] += eps
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - grad[i]) <= 1e-5 * max(1.0, abs(fd)), (li, p, fd, grad[i])


def test_q_k_grads_zero_and_others_nonzero_at_layer0():
    M, H = 4, 128
    layers = _tiny_stack(seed=22)
    g = np.random.default_rng(23)
    x = nf4.round_bf16(g.standard_normal((M, H)))
    dy = nf4.round_bf16(g.standard_normal((M, H)))
    _, saved = stack.stack_fwd(layers, x)
    _, grads = stack.stack_bwd(layers, saved, dy)
    for p in ("q", "k"):
        assert np.all(grads[0][p][0] == 0) and np.all(grads[0][p][1] == 0)
    for p in ("v", "o", "gate", "up", "down"):
        assert np.any(grads[0][p][0] != 0) and np.any(grads[0][p][1] != 0)


def test_rmsnorm_scale_invariance_and_unit_rms():
    g = np.random.default_rng(24)
    h = g.standard_normal((5, 576))
    a = stack.rmsnorm(h, "exact")
    b = stack.rmsnorm(8.0 * h, "exact")
    assert np.allclose(a, b, rtol=1e-5)  # eps = 1e-5 perturbs by ~eps / (2 mean h^2)
    assert np.allclose(np.sqrt(np.mean(a * a, axis=-1)), 1.0, rtol=1e-5)


def test_rmsnorm_bwd_finite_differences():
    g = np.random.default_rng(25)
    h = g.standard_normal((2, 64))
    dn = g.standard_normal((2, 64))
    dh = stack.rmsnorm_bwd(h, dn)
    eps = 1e-6
    for _ in range(5):
        i = (g.integers(0, 2), g.integers(0, 64))
        hp = h.copy(); hp[i] += eps
        hm = h.copy(); hm[i] -= eps
        fd = (np.sum(dn * stack.rmsnorm(hp, "exact")) - np.sum(dn * stack.rmsnorm(hm, "exact"))) / (2 * eps)
        assert abs(fd - dh[i]) < 1e-7


def test_repeat_kv_adjoint():
    g = np.random.default_rng(26)
    v = g.standard_normal((3, 192))
    da = g.standard_normal((3, 576))
    lhs = np.sum(da * stack.repeat_kv(v, 576, 64))
    rhs = np.sum(stack.repeat_kv_bwd(da, 192, 64) * v)
    assert abs(lhs - rhs) < 1e-10
    a = stack.repeat_kv(v, 576, 64)
    # head h of a is kv head h // 3
    for h in range(9):
        assert np.array_equal(a[:, h * 64:(h + 1) * 64], v[:, (h // 3) * 64:(h // 3 + 1) * 64])


def test_silu_grad_finite_differences():
    g = np.linspace(-6, 6, 101)
    eps = 1e-6
    fd = (stack.silu(g + eps) - stack.silu(g - eps)) / (2 * eps)
    assert np.allclose(stack.silu_grad(g), fd, atol=1e-8)


def test_smollm2_parameter_count_matches_the_page():
    # The soup-cli 0.72.2 CHANGELOG gives SmolLM2-135M's true parameter count,
    # 134,515,008. Our 30-layer stack (hidden 576, intermediate 1536, kv 192)
    # plus a tied 49,152 x 576 embedding and 2 norms per layer + a final norm
    # (61 vectors of 576) reproduces it.
    w = stack.param_count(30, 576, 1536, 192)
    assert w == 106_168_320
    assert w + 49_152 * 576 + 61 * 576 == 134_515_008


def test_store_sizes():
    # 4 bits per weight + one float32 per 64 weights = 0.5625 B/weight.
    assert stack.param_count(32, 4096, 14336, 1024) == 6_979_321_856
    assert stack.nf4_store_bytes(32, 4096, 14336, 1024) == 3_925_868_544
    assert stack.nf4_store_bytes(36, 2048, 11008, 256) == 1_560_674_304
    # The pages' bf16 base for 8B is "~16 GB" against ~3.6 GB of NF4: the
    # decoder stack alone is 13.96 GB in bf16, and our NF4 store is 3.93 GB.
    assert abs(stack.param_count(32, 4096, 14336, 1024) * 2 / 1e9 - 13.96) < 0.01
