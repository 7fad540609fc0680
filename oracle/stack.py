"""Decoder-layer stand-in stacked over layers, forward and backward (oracle).

Test infrastructure only (see the package docstring).

The pages stream a decoder stack one layer at a time (Soup README intro and
"Citing Soup"; soup-cli diff, CHANGELOG [0.72.0]/[0.72.2]); the real models'
attention, embeddings and LM head lie outside the streamed path of interest
(the untied embed_tokens and lm_head stay resident, docs "NF4 streaming").
The layer used here is the attention-free stand-in of the benchmark recipe:

    n1 = RMSNorm(h)
    q = P_q(n1), k = P_k(n1), v = P_v(n1)
    a = repeat_kv(v)                        (grouped-query head replication)
    h = h + P_o(a)
    n2 = RMSNorm(h)
    g = P_gate(n2), u = P_up(n2)
    h = h + P_down(silu(g) * u)

with every P an NF4 + LoRA linear (oracle.linear). The output is h after the
last layer. Readings taken where the recipe is silent:

* RMSNorm has unit gain, eps = 1e-5, statistics over the hidden dimension.
* repeat_kv: with head_dim d and n_rep = H / kv_dim, head h of `a` is head
  h // n_rep of v.
* q and k feed nothing in the stand-in: their forward runs, their upstream
  gradient is exactly zero, so their dA and dB are exactly zero and their
  dX terms vanish.
* Rounding points in faithful mode (every stored activation and activation
  gradient is bf16): n1, q, k, v, U of each projection, h after each
  residual add (the add and the projection rounded once together), n2, g, u,
  act = silu(g) u, and the gradients dact, dg, du, dn2 (gate and up summed
  before rounding), dh after each residual, dv (the head-group sum rounded
  once), dn1. dA and dB are float32.
"""

import numpy as np

from . import linear, nf4

PROJ = ("q", "k", "v", "o", "gate", "up", "down")
RMS_EPS = 1e-5


def proj_shapes(H, I, KV):
    """(N, K) of each projection: out-features x in-features."""
    return {"q": (H, H), "k": (KV, H), "v": (KV, H), "o": (H, H),
            "gate": (I, H), "up": (I, H), "down": (H, I)}


def param_count(L, H, I, KV):
    return L * sum(n * k for n, k in proj_shapes(H, I, KV).values())


def nf4_store_bytes(L, H, I, KV):
    """Algorithmic NF4 store size: 4 bits per weight plus one float32 per 64 weights."""
    w = param_count(L, H, I, KV)
    return w // 2 + 4 * (w // nf4.BLOCK)


def _r(v, mode):
    return nf4.round_bf16(v) if mode == "faithful" else v


def rmsnorm(h, mode):
    h = np.asarray(h, np.float64)
    rms = np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + RMS_EPS)
    return _r(h / rms, mode)


def rmsnorm_bwd(h, dn):
    """d/dh of n = h / sqrt(mean(h^2) + eps), applied to dn (float64, unrounded)."""
    h = np.asarray(h, np.float64)
    dn = np.asarray(dn, np.float64)
    H = h.shape[-1]
    rinv = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + RMS_EPS)
    dot = np.sum(dn * h, axis=-1, keepdims=True)
    return rinv * dn - (rinv ** 3 / H) * h * dot


def repeat_kv(v, H, head_dim):
    kv = v.shape[-1]
    n_rep = H // kv
    heads = v.reshape(v.shape[0], kv // head_dim, 1, head_dim)
    return np.broadcast_to(heads, (v.shape[0], kv // head_dim, n_rep, head_dim)).reshape(v.shape[0], H)


def repeat_kv_bwd(da, kv, head_dim):
    """Sum of the gradient over the heads that share one kv head (float64, unrounded)."""
    M, H = da.shape
    n_rep = H // kv
    return da.reshape(M, kv // head_dim, n_rep, head_dim).sum(axis=2).reshape(M, kv)


def silu(g):
    return g / (1.0 + np.exp(-g))


def silu_grad(g):
    sg = 1.0 / (1.0 + np.exp(-g))
    return sg * (1.0 + g * (1.0 - sg))


class Layer:
    """One layer's frozen NF4 projections and LoRA factors.

    weights[p] = (packed uint8, absmax float32) for the projection's [N x K]
    weight; lora[p] = (A [r x K], B [N x r]) as float64 bf16 values.
    """

    def __init__(self, H, I, KV, head_dim, alpha, weights, lora):
        self.H, self.I, self.KV, self.head_dim, self.alpha = H, I, KV, head_dim, alpha
        self.shapes = proj_shapes(H, I, KV)
        self.weights = weights
        self.lora = lora
        self._w = {}

    def W(self, p, mode):
        key = (p, mode)
        if key not in self._w:
            N, K = self.shapes[p]
            packed, absmax = self.weights[p]
            self._w[key] = linear.weight(packed, absmax, N, K, mode)
        return self._w[key]

    def drop_cache(self):
        self._w = {}

    def _lin(self, p, x, mode):
        """Unrounded y = x W^T + s U B^T and the (rounded) U."""
        A, B = self.lora[p]
        s = self.alpha / A.shape[0]
        U = _r(x @ A.T, mode)
        return x @ self.W(p, mode).T + s * (U @ B.T), U

    def fwd(self, h, mode="faithful"):
        """Returns (h_out, saved dict)."""
        h = np.asarray(h, np.float64)
        sv = {"h_in": h}
        n1 = rmsnorm(h, mode)
        sv["n1"] = n1
        for p in ("q", "k", "v"):
            y, U = self._lin(p, n1, mode)
            sv[p] = _r(y, mode)
            sv["U_" + p] = U
        a = repeat_kv(sv["v"], self.H, self.head_dim)
        o, sv["U_o"] = self._lin("o", a, mode)
        h_mid = _r(h + o, mode)
        sv["h_mid"] = h_mid
        n2 = rmsnorm(h_mid, mode)
        sv["n2"] = n2
        for p in ("gate", "up"):
            y, U = self._lin(p, n2, mode)
            sv[p] = _r(y, mode)
            sv["U_" + p] = U
        act = _r(silu(sv["gate"]) * sv["up"], mode)
        sv["act"] = act
        d, sv["U_down"] = self._lin("down", act, mode)
        h_out = _r(h_mid + d, mode)
        return h_out, sv

    def _lin_bwd(self, p, dy, x, U, mode):
        """Unrounded dX contribution and (dA, dB)."""
        A, B = self.lora[p]
        s = self.alpha / A.shape[0]
        G = _r(dy @ B, mode)
        dx = dy @ self.W(p, mode) + s * (G @ A)
        dB = s * (dy.T @ U)
        dA = s * (G.T @ x)
        if mode == "faithful":
            dA = dA.astype(np.float32).astype(np.float64)
            dB = dB.astype(np.float32).astype(np.float64)
        return dx, dA, dB

    def bwd(self, dh, sv, mode="faithful", keep=None):
        """Returns (dh_in, grads) with grads[p] = (dA, dB). A dict `keep`
        receives the residual-path gradient dh_mid (for error bounds)."""
        dh = np.asarray(dh, np.float64)
        g = {}
        dact, dAd, dBd = self._lin_bwd("down", dh, sv["act"], sv["U_down"], mode)
        dact = _r(dact, mode)
        g["down"] = (dAd, dBd)
        gt, up = sv["gate"], sv["up"]
        dg = _r(dact * up * silu_grad(gt), mode)
        du = _r(dact * silu(gt), mode)
        dxg, dAg, dBg = self._lin_bwd("gate", dg, sv["n2"], sv["U_gate"], mode)
        dxu, dAu, dBu = self._lin_bwd("up", du, sv["n2"], sv["U_up"], mode)
        g["gate"], g["up"] = (dAg, dBg), (dAu, dBu)
        dn2 = _r(dxg + dxu, mode)
        dh_mid = _r(dh + rmsnorm_bwd(sv["h_mid"], dn2), mode)
        if keep is not None:
            keep["dh_mid"] = dh_mid
        a = repeat_kv(sv["v"], self.H, self.head_dim)
        da, dAo, dBo = self._lin_bwd("o", dh_mid, a, sv["U_o"], mode)
        g["o"] = (dAo, dBo)
        dv = _r(repeat_kv_bwd(da, self.KV, self.head_dim), mode)
        dn1, dAv, dBv = self._lin_bwd("v", dv, sv["n1"], sv["U_v"], mode)
        g["v"] = (dAv, dBv)
        dn1 = _r(dn1, mode)
        for p in ("q", "k"):
            A, B = self.lora[p]
            g[p] = (np.zeros_like(A), np.zeros_like(B))
        dh_in = _r(dh_mid + rmsnorm_bwd(sv["h_in"], dn1), mode)
        return dh_in, g


def stack_fwd(layers, x, mode="faithful", keep=True):
    """Runs the layers in order; returns (h_L, [saved per layer] or None)."""
    h = np.asarray(x, np.float64)
    saved = [] if keep else None
    for layer in layers:
        h, sv = layer.fwd(h, mode)
        if keep:
            saved.append(sv)
    return h, saved


def stack_bwd(layers, saved, dy, mode="faithful"):
    """Backward from dy at h_L through the layers in reverse; returns (dx0, grads per layer)."""
    dh = np.asarray(dy, np.float64)
    grads = [None] * len(layers)
    for i in range(len(layers) - 1, -1, -1):
        dh, grads[i] = layers[i].bwd(dh, saved[i], mode)
    return dh, grads
