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

    def saved_tensor(self, layer, name):
        offs, per = ql.stream_layer_stack_saved_layout(self.cfg, self.M)
        H, I, KV, r = self.w["H"], self.w["I"], self.w["KV"], self.w["r"]
        cols = dict(h_in=H, n1=H, q=H, k=KV, v=KV, h_mid=H, n2=H, gate=I, up=I, act=I)
        c = cols.get(name, r)
        o = layer * per + offs[name]
        return self.saved[o: o + self.M * c * 2].view(torch.bfloat16).view(self.M, c)

    def oracle_layers(self):
        from oracle import stack as ostack
        w = self.w
        layers = []
        for d in self.inp["layers"]:
            weights = {p: (d[p]["packed"].cpu().numpy(), d[p]["absmax"].cpu().numpy()) for p in ql.PROJ}
            lora = {p: (f64(d[p]["A"]), f64(d[p]["B"])) for p in ql.PROJ}
            layers.append(ostack.Layer(w["H"], w["I"], w["KV"], w["head_dim"], w["alpha"], weights, lora))
        return layers


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
