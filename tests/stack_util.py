"""Builds a decoder stack for the GPU tests and the benchmark: inputs from
synth, the store assembled for the C ABI, buffers sized by the library."""

import numpy as np
import torch

import synth
from gpu_util import DEV, f64, ql


class GpuStack:
    def __init__(self, name, L=None, M=None, gen_device="cpu", pinned=True, resident_copy=True, n_buffers=2,
                 recompute=0, absmax_dq=0, r=None):
        w = dict(synth.WORKLOADS[name])
        if L is not None:
            w["L"] = L
        if M is not None:
            w["M"] = M
        if r is not None:  # another adapter rank, alpha = 2 r
            w["r"], w["alpha"] = r, 2.0 * r
        self.w = w
        self.name = name
        self.M = w["M"]
        self.cfg = ql.StackCfg(w["L"], w["H"], w["I"], w["KV"], w["head_dim"], w["r"], w["alpha"],
                               n_buffers=n_buffers, recompute=recompute, absmax_dq=absmax_dq)
        inp = synth.stack_inputs(w["L"], w["M"], w["H"], w["I"], w["KV"], w["r"], (name,), device=gen_device)
        self.inp = inp
        stores = [{p: (d[p]["packed"], d[p]["absmax"]) for p in ql.PROJ} for d in inp["layers"]]
        self.store = ql.build_store(self.cfg, stores, pinned=pinned)
        self.store_dev = self.store.to(DEV) if resident_copy else None
        self.lora = [{p: (d[p]["A"].to(DEV), d[p]["B"].to(DEV)) for p in ql.PROJ} for d in inp["layers"]]
        self.x = inp["x"].to(DEV)
        self.dy = inp["dy"].to(DEV)
        slots, saved, ws = ql.stream_layer_stack_workspace(self.cfg, self.M)
        self.slots = torch.empty(slots, dtype=torch.uint8, device=DEV)
        self.saved = torch.empty(saved, dtype=torch.uint8, device=DEV)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=DEV)
        self.y = torch.empty(self.M, w["H"], dtype=torch.bfloat16, device=DEV)
        self.dx = torch.empty(self.M, w["H"], dtype=torch.bfloat16, device=DEV)
        self.dA = [{p: torch.empty(w["r"], self.cfg.proj_shape(p)[1], device=DEV) for p in ql.PROJ}
                   for _ in range(w["L"])]
        self.dB = [{p: torch.empty(self.cfg.proj_shape(p)[0], w["r"], device=DEV) for p in ql.PROJ}
                   for _ in range(w["L"])]
        self.compute = torch.cuda.Stream(DEV)
        self.copy = torch.cuda.Stream(DEV)

    def cfg_mode(self, resident):
        c = ql.StackCfg(**{**self.cfg.__dict__, "resident": int(resident)})
        return c

    def set_buffers(self, n):
        """Use n device slots from now on (the slot memory must hold n records)."""
        offs, _, _ = ql.stream_layer_stack_layout(self.cfg)
        assert n * offs[1] <= self.slots.numel()
        self.cfg = ql.StackCfg(**{**self.cfg.__dict__, "n_buffers": n})

    def fwd(self, resident=False, store=None, reuse=False):
        cfg = self.cfg_mode(resident)
        st = store if store is not None else (self.store_dev if resident else self.store)
        return ql.stream_layer_stack_fwd(cfg, st, self.lora, self.x, self.M, self.y, self.saved,
                                         None if resident else self.slots, self.ws, self.compute, self.copy,
                                         reuse_bwd_slots=reuse)

    def bwd(self, resident=False, reuse=False, store=None, accumulate=False):
        cfg = self.cfg_mode(resident)
        st = store if store is not None else (self.store_dev if resident else self.store)
        return ql.stream_layer_stack_bwd(cfg, st, self.lora, self.dy, self.M, self.saved, self.dx, self.dA, self.dB,
                                         accumulate, reuse, None if resident else self.slots, self.ws,
                                         self.compute, self.copy)

    def step(self, resident=False, reuse=True):
        a = self.fwd(resident)
        b = self.bwd(resident, reuse=reuse and not resident)
        return max(a, b)

    def layer_stores(self):
        """Per-layer {proj: (packed, absmax)} host tensors of this stack's store."""
        return [{p: (d[p]["packed"], d[p]["absmax"]) for p in ql.PROJ} for d in self.inp["layers"]]

    def results(self):
        self.compute.synchronize()
        torch.cuda.synchronize()
        return dict(y=self.y.clone(), dx=self.dx.clone(),
                    dA=[{p: t.clone() for p, t in d.items()} for d in self.dA],
                    dB=[{p: t.clone() for p, t in d.items()} for d in self.dB],
                    saved=self.saved.clone())

    def saved_tensor(self, layer, name, buf=None):
        """Saved activation `name` of `layer` in buf (default: the live saved area)."""
        offs, per = ql.stream_layer_stack_saved_layout(self.cfg, self.M)
        H, I, KV, r = self.w["H"], self.w["I"], self.w["KV"], self.w["r"]
        cols = dict(h_in=H, n1=H, q=H, k=KV, v=KV, h_mid=H, n2=H, gate=I, up=I, act=I)
        c = cols.get(name, r)
        assert offs[name] >= 0, f"{name} is not kept in this mode"
        o = layer * per + offs[name]
        b = self.saved if buf is None else buf
        return b[o: o + self.M * c * 2].view(torch.bfloat16).view(self.M, c)

    def oracle_layer(self, l):
        """The oracle's layer l (host copies of its NF4 bytes and adapter)."""
        from oracle import stack as ostack
        w = self.w
        d = self.inp["layers"][l]
        weights = {p: (d[p]["packed"].cpu().numpy(), d[p]["absmax"].cpu().numpy()) for p in ql.PROJ}
        lora = {p: (f64(d[p]["A"]), f64(d[p]["B"])) for p in ql.PROJ}
        return ostack.Layer(w["H"], w["I"], w["KV"], w["head_dim"], w["alpha"], weights, lora)

    def oracle_layers(self):
        return [self.oracle_layer(l) for l in range(len(self.inp["layers"]))]


def identical(a, b):
    """Bitwise equality of two result dicts."""
    def eq(x, y):
        return torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    if not eq(a["y"], b["y"]) or not eq(a["dx"], b["dx"]) or not eq(a["saved"], b["saved"]):
        return False
    for la, lb in zip(a["dA"], b["dA"]):
        for p in la:
            if not eq(la[p], lb[p]):
                return False
    for la, lb in zip(a["dB"], b["dB"]):
        for p in la:
            if not eq(la[p], lb[p]):
                return False
    return True


# ------------------------------------------------------------ teacher forcing
#
# A deep bf16 stack is ill-conditioned end to end (a 30-layer random-weight
# stand-in amplifies |dx0| about 30x over |dy|), so its parity is checked
# layer by layer: the oracle layer l runs on the GPU's own input to l (h_in of
# l forward, the upstream gradient at l's output backward), and every output
# of the layer is compared element-wise at 2e-2.
#
# The GPU's per-layer upstream gradients are not kept by the stack call, so
# they are re-derived by running the same backward one layer at a time
# (1-layer stack calls on layer l's record, adapter and saved activations,
# chained from dy). The kernels and their launch geometry depend on shapes
# only, so each 1-layer call reproduces layer l of the full call; the chain
# asserts this bitwise (every dA, dB and the final dx0), so the gradients it
# exposes are the full call's own.

class LayerChain:
    """1-layer backward calls over the layers of a GpuStack's full run."""

    def __init__(self, s):
        self.s = s
        offs, _, _ = ql.stream_layer_stack_layout(s.cfg)
        self.rec = offs[1]
        _, self.per = ql.stream_layer_stack_saved_layout(s.cfg, s.M)
        self.cfg1 = ql.StackCfg(**{**s.cfg.__dict__, "n_layers": 1, "resident": 1})
        H = s.w["H"]
        self.dx = torch.empty(s.M, H, dtype=torch.bfloat16, device=DEV)
        self.dA = [{p: torch.empty_like(s.dA[0][p]) for p in ql.PROJ}]
        self.dB = [{p: torch.empty_like(s.dB[0][p]) for p in ql.PROJ}]

    def bwd(self, l, dy, saved):
        s = self.s
        store = s.store_dev[l * self.rec:(l + 1) * self.rec]
        sv = saved[l * self.per:(l + 1) * self.per]
        st = ql.stream_layer_stack_bwd(self.cfg1, store, s.lora[l:l + 1], dy, s.M, sv, self.dx, self.dA, self.dB,
                                       0, 0, None, s.ws, s.compute, s.copy)
        assert st == ql.QL_OK
        s.compute.synchronize()
        out = self.dx.clone()      # on torch's current stream; complete before the next call reads it
        torch.cuda.synchronize()
        return out

    def upstream(self, got):
        """dh[l]: the GPU's gradient at the output of layer l (dh[L-1] = dy), as device
        bf16 tensors. Asserts that the chain reproduces got's dA, dB and dx0 bitwise."""
        s = self.s
        L = s.cfg.n_layers
        dh = [None] * L
        d = s.dy
        torch.cuda.synchronize()   # got's copies (made on torch's stream) are complete
        for l in range(L - 1, -1, -1):
            dh[l] = d.clone()
            d = self.bwd(l, d, got["saved"])
            for p in ql.PROJ:
                assert torch.equal(self.dA[0][p], got["dA"][l][p]), f"chain L{l}:{p}:dA"
                assert torch.equal(self.dB[0][p], got["dB"][l][p]), f"chain L{l}:{p}:dB"
        assert torch.equal(d.view(torch.int16), got["dx"].view(torch.int16)), "chain dx0"
        return dh


LIVE = ("v", "o", "gate", "up", "down")
ACTS = ("n1", "q", "k", "v", "h_mid", "n2", "gate", "up", "act") + tuple("U_" + p for p in ql.PROJ)


def teacher_forced_layer(s, got, dh, layer, l, full_saved=True):
    """Oracle layer l on the GPU's input to l, compared element-wise with the GPU.

    Forward: every saved activation of l (when the run keeps them) and l's
    output (h_in of l + 1, or y). Backward: the gradient at l's input (the
    upstream of l - 1, or dx0), and dA, dB of the live projections; q and k
    must be exactly zero.
    """
    from gpu_util import close
    L = s.cfg.n_layers
    h_in = f64(s.saved_tensor(l, "h_in", got["saved"]))
    h_out, sv = layer.fwd(h_in)
    if full_saved:
        for name in ACTS:
            close(f64(s.saved_tensor(l, name, got["saved"])), sv[name], what=f"L{l}:{name}")
    # the two residual sums are compared with their stored first term's
    # magnitude in the bound (h_out = h_mid + down(...), dh_in = dh_mid + ...)
    out = got["y"] if l == L - 1 else s.saved_tensor(l + 1, "h_in", got["saved"])
    close(f64(out), h_out, what=f"L{l}:h_out", summand=sv["h_mid"])
    keep = {}
    dh_in, g = layer.bwd(f64(dh[l]), sv, keep=keep)
    close(f64(got["dx"] if l == 0 else dh[l - 1]), dh_in, what=f"L{l}:dh_in", summand=keep["dh_mid"])
    for p in LIVE:
        close(f64(got["dA"][l][p]), g[p][0], what=f"L{l}:{p}:dA")
        close(f64(got["dB"][l][p]), g[p][1], what=f"L{l}:{p}:dB")
    for p in ("q", "k"):
        assert torch.count_nonzero(got["dA"][l][p]) == 0 and torch.count_nonzero(got["dB"][l][p]) == 0
    layer.drop_cache()


def teacher_forced(s, got, layers=None, full_saved=True, dh=None):
    """Teacher-forced check of every layer in `layers` (default: all) of a run's results."""
    if dh is None:
        dh = LayerChain(s).upstream(got)
    for l in (range(s.cfg.n_layers) if layers is None else layers):
        teacher_forced_layer(s, got, dh, s.oracle_layer(l), l, full_saved)
    return dh
