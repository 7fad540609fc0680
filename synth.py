"""Seeded synthetic inputs for the tests and the benchmark.

This module draws random numbers and converts dtypes; it holds none of the
method's arithmetic, and it is the only code that the oracle side and the
HIP side have in common.

Workloads (the pages measured real checkpoints on unnamed data; these
synthetic inputs take their shapes and stand in for them):

* ``linear_pr1``    one NF4 + LoRA linear, M=64, K=256, N=512, r=8, alpha=16
* ``llama8b_layer`` the seven projections of one Llama-3.1-8B-shaped layer,
                    M=512, r=16, alpha=32
* ``smollm2_stack`` 30 layers, hidden 576, intermediate 1536, kv 192,
                    head_dim 64, r=8, alpha=16, M=512
* ``qwen3b_stack``  36 layers, hidden 2048, intermediate 11008, kv 256,
                    head_dim 128, r=16, alpha=32, M=512
* ``llama8b_stack`` 32 layers, hidden 4096, intermediate 14336, kv 1024,
                    head_dim 128, r=16, alpha=32, M=2048 (batch 4 x seq 512)

Distributions: activations and upstream gradients N(0, 1) rounded to bf16;
frozen weights N(0, 0.02) float32 (then NF4-quantised); LoRA A and B
N(0, 0.01) rounded to bf16. Seeds: NumPy SeedSequence(0, spawn_key=key) on the
CPU; on a GPU, torch's generator seeded from the same key.

For the large stacks, drawing and quantising billions of float32 weights on
the host is too slow, so ``nf4_store`` draws the quantised form directly:
uniform 4-bit codes (the NF4 levels are normal quantiles, so codes of normal
data are close to uniform) and per-block scales distributed like the maximum
of 64 |N(0, 0.02)| draws (mean ~2.4 sigma).
"""

import hashlib

import numpy as np
import torch

WORKLOADS = {
    "linear_pr1": dict(M=64, K=256, N=512, r=8, alpha=16.0),
    "llama8b_layer": dict(M=512, H=4096, I=14336, KV=1024, head_dim=128, r=16, alpha=32.0),
    "smollm2_stack": dict(L=30, M=512, H=576, I=1536, KV=192, head_dim=64, r=8, alpha=16.0),
    "qwen3b_stack": dict(L=36, M=512, H=2048, I=11008, KV=256, head_dim=128, r=16, alpha=32.0),
    "llama8b_stack": dict(L=32, M=2048, H=4096, I=14336, KV=1024, head_dim=128, r=16, alpha=32.0),
}

W_SIGMA = 0.02
LORA_SIGMA = 0.01


def _key_ints(key):
    out = []
    for k in key:
        if isinstance(k, (int, np.integer)):
            out.append(int(k))
        else:
            out.append(int.from_bytes(hashlib.sha256(str(k).encode()).digest()[:4], "little"))
    return tuple(out)


def rng(*key):
    return np.random.default_rng(np.random.SeedSequence(0, spawn_key=_key_ints(key)))


def _torch_gen(device, key):
    g = torch.Generator(device=device)
    seed = int.from_bytes(hashlib.sha256(repr(_key_ints(key)).encode()).digest()[:8], "little") >> 1
    g.manual_seed(seed)
    return g


def normal(shape, sigma, *key, device="cpu"):
    """float32 tensor of N(0, sigma^2) draws."""
    dev = torch.device(device)
    if dev.type == "cpu":
        a = rng(*key).standard_normal(shape, dtype=np.float32)
        a *= np.float32(sigma)
        return torch.from_numpy(a)
    t = torch.randn(shape, generator=_torch_gen(dev, key), device=dev, dtype=torch.float32)
    return t.mul_(sigma)


def normal_bf16(shape, sigma, *key, device="cpu"):
    """bf16 tensor: N(0, sigma^2) float32 draws rounded to bf16 by torch."""
    return normal(shape, sigma, *key, device=device).to(torch.bfloat16)


def as_f64(t):
    """CPU float64 NumPy copy of a tensor (exact for bf16 and float32)."""
    return t.detach().to("cpu", torch.float64).numpy()


def nf4_store(n, *key, device="cpu"):
    """Synthetic NF4 bytes for n weights: (packed uint8 [n/2], absmax float32 [n/64])."""
    if n % 64:
        raise ValueError("n must be a multiple of 64")
    dev = torch.device(device)
    if dev.type == "cpu":
        g = rng(*key, "store")
        packed = torch.from_numpy(g.integers(0, 256, size=n // 2, dtype=np.uint8))
        z = g.standard_normal(n // 64, dtype=np.float32)
        absmax = torch.from_numpy(np.clip(W_SIGMA * (2.4 + 0.4 * z), 1.5 * W_SIGMA, 4.0 * W_SIGMA).astype(np.float32))
        return packed, absmax
    gen = _torch_gen(dev, key + ("store",))
    packed = torch.randint(0, 256, (n // 2,), generator=gen, device=dev, dtype=torch.uint8)
    z = torch.randn(n // 64, generator=gen, device=dev, dtype=torch.float32)
    absmax = (W_SIGMA * (2.4 + 0.4 * z)).clamp_(1.5 * W_SIGMA, 4.0 * W_SIGMA)
    return packed, absmax


def linear_inputs(M, K, N, r, key, device="cpu"):
    """Seeded inputs of one NF4 + LoRA linear: x, W (float32), A, B, dY."""
    return dict(
        x=normal_bf16((M, K), 1.0, *key, "x", device=device),
        W=normal((N, K), W_SIGMA, *key, "W", device=device),
        A=normal_bf16((r, K), LORA_SIGMA, *key, "A", device=device),
        B=normal_bf16((N, r), LORA_SIGMA, *key, "B", device=device),
        dy=normal_bf16((M, N), 1.0, *key, "dy", device=device),
    )


PROJ = ("q", "k", "v", "o", "gate", "up", "down")


def proj_shape(p, H, I, KV):
    return {"q": (H, H), "k": (KV, H), "v": (KV, H), "o": (H, H),
            "gate": (I, H), "up": (I, H), "down": (H, I)}[p]


def stack_inputs(L, M, H, I, KV, r, key, device="cpu"):
    """Seeded stack inputs: per-layer NF4 stores and LoRA factors, x0 and dY at the top."""
    layers = []
    for layer in range(L):
        d = {}
        for p in PROJ:
            N, K = proj_shape(p, H, I, KV)
            packed, absmax = nf4_store(N * K, *key, layer, p, device=device)
            d[p] = dict(packed=packed, absmax=absmax, N=N, K=K,
                        A=normal_bf16((r, K), LORA_SIGMA, *key, layer, p, "A", device=device),
                        B=normal_bf16((N, r), LORA_SIGMA, *key, layer, p, "B", device=device))
        layers.append(d)
    return dict(layers=layers,
                x=normal_bf16((M, H), 1.0, *key, "x", device=device),
                dy=normal_bf16((M, H), 1.0, *key, "dy", device=device))
