"""Python binding of libnf4qlora.so, the MI355X (gfx950) NF4 + LoRA layer-streaming library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch supplies device memory and streams. The functions carry the
names of the C ABI in include/nf4qlora.h and raise QlError on a negative
status. If the library is not built, importing works but every call raises.
"""

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnf4qlora.so")

QL_OK = 0
QL_WARN_PAGEABLE_HOST = 1
QL_ERR_ARG, QL_ERR_SHAPE, QL_ERR_ALIGN, QL_ERR_RANK = -1, -2, -3, -4
QL_ERR_NONFINITE, QL_ERR_WORKSPACE, QL_ERR_HIP, QL_ERR_UNSUPPORTED = -5, -6, -7, -8
QL_BF16, QL_F32 = 0, 1
PROJ = ("q", "k", "v", "o", "gate", "up", "down")
NPROJ = 7
SAVED = ("h_in", "n1", "q", "k", "v", "h_mid", "n2", "gate", "up", "act") + tuple("U_" + p for p in PROJ)

EXPORTS = (
    "ql_last_error", "ql_abi_version", "nf4_codebook", "nf4_quantize", "nf4_dequant",
    "nf4_dq_layout", "nf4_double_quant", "nf4_dq_expand",
    "qlora_linear_workspace", "qlora_linear_fwd", "qlora_linear_bwd",
    "stream_layer_stack_layout", "stream_layer_stack_workspace", "stream_layer_stack_saved_layout",
    "stream_layer_stack_fwd", "stream_layer_stack_fwd_ref", "stream_layer_stack_bwd", "ql_profile_enable",
    "ql_profile_read", "stream_layer_stack_step_capture", "ql_step_graph_launch", "ql_step_graph_destroy",
    "ql_debug_poison_slots", "qlora_linear_bwd_noalloc", "ql_step_graph_info",
)
QL_NOALLOC_SCRATCH_BYTES = 128 << 20
QL_KERNEL_GEMM_FWD, QL_KERNEL_GEMM_BWD, QL_KERNEL_GEMM_FWD_NARROW, QL_KERNEL_GEMM_BWD_NARROW = 0, 1, 2, 3
QL_KERNEL_LORA_ROW, QL_KERNEL_LORA_COL, QL_KERNEL_DEQUANT = 4, 5, 6
# kernel symbol of each profiling id (the names rocprofv3 reports): the fused
# GEMMs (work in FLOPs) and the HBM-bound kernels (work in bytes)
KERNEL_SYMBOLS = {0: "k_gemm_fwd<64>", 1: "k_gemm_bwd<128, 8>", 2: "k_gemm_fwd<32>", 3: "k_gemm_bwd<64, 4>"}
HBM_KERNEL_SYMBOLS = {4: "k_rowc", 5: "k_colc", 6: "k_nf4_dequant"}


class QlError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class ql_nf4_weight(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class ql_lora(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("r", ctypes.c_int32), ("alpha", ctypes.c_float)]


class ql_stack_cfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("kv_dim", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("r", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("n_buffers", ctypes.c_int32), ("resident", ctypes.c_int32), ("recompute", ctypes.c_int32),
                ("absmax_dq", ctypes.c_int32)]


_lib = None


def load(path=LIB_PATH):
    """Loads the library (once); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise QlError(QL_ERR_UNSUPPORTED, f"{path} is not built: run nf4_layer_streamed_amd.build.build()")
    lib = ctypes.CDLL(path)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sigs = {
        "ql_last_error": (ctypes.c_char_p, []),
        "ql_abi_version": (I32, []),
        "nf4_codebook": (I32, [P]),
        "nf4_quantize": (I32, [P, I64, P, P, P]),
        "nf4_dequant": (I32, [P, P, I64, I32, P, P]),
        "nf4_dq_layout": (I32, [I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "nf4_double_quant": (I32, [P, I64, P, SZ, P]),
        "nf4_dq_expand": (I32, [P, I64, P, P]),
        "qlora_linear_workspace": (I32, [I64, I64, I64, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "qlora_linear_fwd": (I32, [P, I64, ql_nf4_weight, ql_lora, P, P, P, SZ, P]),
        "qlora_linear_bwd": (I32, [P, P, P, I64, ql_nf4_weight, ql_lora, P, P, P, I32, P, SZ, P]),
        "qlora_linear_bwd_noalloc": (I32, [P, P, P, I64, ql_nf4_weight, ql_lora, P, P, P, I32, P]),
        "stream_layer_stack_layout": (I32, [ctypes.POINTER(ql_stack_cfg), P, P, ctypes.POINTER(SZ)]),
        "stream_layer_stack_workspace": (I32, [ctypes.POINTER(ql_stack_cfg), I64, ctypes.POINTER(SZ),
                                               ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "stream_layer_stack_saved_layout": (I32, [ctypes.POINTER(ql_stack_cfg), I64, P, ctypes.POINTER(SZ)]),
        "stream_layer_stack_fwd": (I32, [ctypes.POINTER(ql_stack_cfg), P, SZ, P, P, I64, P, P, SZ, I32, P, SZ,
                                         P, SZ, P, P]),
        "stream_layer_stack_fwd_ref": (I32, [ctypes.POINTER(ql_stack_cfg), P, SZ, P, P, I64, P, P, SZ, P, P, SZ,
                                             I32, P, SZ, P, SZ, P, P]),
        "stream_layer_stack_step_capture": (I32, [ctypes.POINTER(ql_stack_cfg), P, SZ, P, P, P, I64, P, P, SZ, P,
                                                  P, P, I32, I32, P, SZ, P, SZ, P, P,
                                                  ctypes.POINTER(ctypes.c_void_p)]),
        "ql_step_graph_launch": (I32, [P, P]),
        "ql_step_graph_destroy": (I32, [P]),
        "ql_step_graph_info": (I32, [P, ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(I64)]),
        "stream_layer_stack_bwd": (I32, [ctypes.POINTER(ql_stack_cfg), P, SZ, P, P, I64, P, SZ, P, P, P,
                                         I32, I32, P, SZ, P, SZ, P, P]),
        "ql_profile_enable": (I32, [I32]),
        "ql_debug_poison_slots": (I32, [I32]),
        "ql_profile_read": (I32, [I32, ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(st):
    if st < 0:
        raise QlError(st, load().ql_last_error().decode(errors="replace"))
    return st


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s):
    if s is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, torch.cuda.Stream):
        return ctypes.c_void_p(s.cuda_stream)
    return ctypes.c_void_p(int(s))


def ql_last_error():
    return load().ql_last_error().decode(errors="replace")


def ql_abi_version():
    return load().ql_abi_version()


def nf4_codebook():
    """The 16 float32 NF4 levels used by the library (host tensor)."""
    out = torch.empty(16, dtype=torch.float32)
    _check(load().nf4_codebook(_ptr(out)))
    return out


def nf4_quantize(w, packed, absmax, stream=None):
    """w float32 [n] (device) -> packed uint8 [n/2], absmax float32 [n/64]. Synchronous."""
    return _check(load().nf4_quantize(_ptr(w), w.numel(), _ptr(packed), _ptr(absmax), _stream(stream)))


def nf4_dequant(packed, absmax, n, out, stream=None):
    """Decodes n weights into out (bf16 or float32 tensor with n elements)."""
    dt = QL_F32 if out.dtype == torch.float32 else QL_BF16
    return _check(load().nf4_dequant(_ptr(packed), _ptr(absmax), n, dt, _ptr(out), _stream(stream)))


def nf4_dq_layout(nblocks):
    """-> (scale offset, mean offset, bytes) of the double-quantised block of nblocks scales."""
    so, mo, nb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().nf4_dq_layout(nblocks, ctypes.byref(so), ctypes.byref(mo), ctypes.byref(nb)))
    return so.value, mo.value, nb.value


def nf4_double_quant(absmax, dq, stream=None):
    """absmax (float32 device tensor of n scales) -> the block in dq (uint8 device tensor)."""
    return _check(load().nf4_double_quant(_ptr(absmax), absmax.numel(), _ptr(dq), _nbytes(dq), _stream(stream)))


def nf4_dq_expand(dq, nblocks, out, stream=None):
    """The block in dq -> float32 scales in out (nblocks elements)."""
    return _check(load().nf4_dq_expand(_ptr(dq), nblocks, _ptr(out), _stream(stream)))


@dataclass
class NF4Weight:
    packed: torch.Tensor
    absmax: torch.Tensor
    N: int
    K: int

    def c(self):
        return ql_nf4_weight(self.packed.data_ptr(), self.absmax.data_ptr(), self.N, self.K)


@dataclass
class Lora:
    A: torch.Tensor
    B: torch.Tensor
    r: int
    alpha: float

    def c(self):
        return ql_lora(self.A.data_ptr(), self.B.data_ptr(), self.r, self.alpha)


def qlora_linear_workspace(M, N, K, r):
    f, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().qlora_linear_workspace(M, N, K, r, ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def qlora_linear_fwd(x, M, W, L, y, u_save, ws, stream=None):
    return _check(load().qlora_linear_fwd(_ptr(x), M, W.c(), L.c(), _ptr(y), _ptr(u_save), _ptr(ws),
                                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def qlora_linear_bwd(dy, x, u_saved, M, W, L, dx, dA, dB, accumulate, ws, stream=None):
    return _check(load().qlora_linear_bwd(_ptr(dy), _ptr(x), _ptr(u_saved), M, W.c(), L.c(), _ptr(dx), _ptr(dA),
                                          _ptr(dB), int(accumulate), _ptr(ws),
                                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def qlora_linear_bwd_noalloc(dy, x, u_saved, M, W, L, dx, dA, dB, accumulate, stream=None):
    """qlora_linear_bwd with its temporaries in the library's fixed per-device scratch."""
    return _check(load().qlora_linear_bwd_noalloc(_ptr(dy), _ptr(x), _ptr(u_saved), M, W.c(), L.c(), _ptr(dx),
                                                  _ptr(dA), _ptr(dB), int(accumulate), _stream(stream)))


@dataclass
class StackCfg:
    n_layers: int
    hidden: int
    inter: int
    kv_dim: int
    head_dim: int
    r: int
    alpha: float
    rms_eps: float = 1e-5
    n_buffers: int = 2
    resident: int = 0
    recompute: int = 0
    absmax_dq: int = 0

    def c(self):
        return ql_stack_cfg(self.n_layers, self.hidden, self.inter, self.kv_dim, self.head_dim, self.r,
                            self.alpha, self.rms_eps, self.n_buffers, self.resident, self.recompute,
                            self.absmax_dq)

    def proj_shape(self, p):
        H, I, KV = self.hidden, self.inter, self.kv_dim
        return {"q": (H, H), "k": (KV, H), "v": (KV, H), "o": (H, H),
                "gate": (I, H), "up": (I, H), "down": (H, I)}[p]


def stream_layer_stack_layout(cfg):
    """-> (layer_offsets [L+1], proj_offsets {p: (packed_off, absmax_off)}, store_bytes)."""
    c = cfg.c()
    lo = (ctypes.c_int64 * (cfg.n_layers + 1))()
    po = (ctypes.c_int64 * (2 * NPROJ))()
    sb = ctypes.c_size_t()
    _check(load().stream_layer_stack_layout(ctypes.byref(c), lo, po, ctypes.byref(sb)))
    return list(lo), {p: (po[2 * i], po[2 * i + 1]) for i, p in enumerate(PROJ)}, sb.value


def stream_layer_stack_workspace(cfg, M):
    """-> (slots_bytes, saved_bytes, ws_bytes)."""
    c = cfg.c()
    a, b, w = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().stream_layer_stack_workspace(ctypes.byref(c), M, ctypes.byref(a), ctypes.byref(b),
                                               ctypes.byref(w)))
    return a.value, b.value, w.value


def stream_layer_stack_saved_layout(cfg, M):
    """-> ({name: byte offset within a layer}, per_layer_bytes)."""
    c = cfg.c()
    offs = (ctypes.c_int64 * len(SAVED))()
    per = ctypes.c_size_t()
    _check(load().stream_layer_stack_saved_layout(ctypes.byref(c), M, offs, ctypes.byref(per)))
    return dict(zip(SAVED, list(offs))), per.value


def _lora_array(cfg, lora):
    arr = (ql_lora * (cfg.n_layers * NPROJ))()
    for l in range(cfg.n_layers):
        for i, p in enumerate(PROJ):
            A, B = lora[l][p]
            arr[l * NPROJ + i] = ql_lora(A.data_ptr(), B.data_ptr(), cfg.r, cfg.alpha)
    return arr


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def stream_layer_stack_fwd(cfg, store, lora, x0, M, y, saved, slots, ws, compute=None, copy=None,
                           reuse_bwd_slots=0):
    """lora: list over layers of {proj: (A, B)} device bf16 tensors."""
    c = cfg.c()
    arr = _lora_array(cfg, lora)
    return _check(load().stream_layer_stack_fwd(
        ctypes.byref(c), _ptr(store), _nbytes(store), arr, _ptr(x0), M, _ptr(y), _ptr(saved), _nbytes(saved),
        int(reuse_bwd_slots), _ptr(slots), _nbytes(slots), _ptr(ws), _nbytes(ws), _stream(compute), _stream(copy)))


def stream_layer_stack_fwd_ref(cfg, store, lora, x0, M, y, saved, ref_y, ref_scratch, slots, ws, compute=None,
                               copy=None, reuse_bwd_slots=0):
    """Policy forward (lora: as stream_layer_stack_fwd, or None for the
    reference alone) and the adapter-off reference forward into ref_y, sharing
    each layer's copy."""
    c = cfg.c()
    arr = _lora_array(cfg, lora) if lora is not None else None
    return _check(load().stream_layer_stack_fwd_ref(
        ctypes.byref(c), _ptr(store), _nbytes(store), arr, _ptr(x0), M, _ptr(y), _ptr(saved), _nbytes(saved),
        _ptr(ref_y), _ptr(ref_scratch), _nbytes(ref_scratch), int(reuse_bwd_slots), _ptr(slots), _nbytes(slots),
        _ptr(ws), _nbytes(ws), _stream(compute), _stream(copy)))


def stream_layer_stack_bwd(cfg, store, lora, dy, M, saved, dx0, dA, dB, accumulate, reuse_fwd_slots, slots, ws,
                           compute=None, copy=None):
    """dA, dB: list over layers of {proj: float32 device tensor}."""
    c = cfg.c()
    arr = _lora_array(cfg, lora)
    n = cfg.n_layers * NPROJ
    pa = (ctypes.c_void_p * n)(*[dA[l][p].data_ptr() for l in range(cfg.n_layers) for p in PROJ])
    pb = (ctypes.c_void_p * n)(*[dB[l][p].data_ptr() for l in range(cfg.n_layers) for p in PROJ])
    return _check(load().stream_layer_stack_bwd(
        ctypes.byref(c), _ptr(store), _nbytes(store), arr, _ptr(dy), M, _ptr(saved), _nbytes(saved), _ptr(dx0),
        pa, pb, int(accumulate), int(reuse_fwd_slots), _ptr(slots), _nbytes(slots), _ptr(ws), _nbytes(ws),
        _stream(compute), _stream(copy)))


class StepGraph:
    """A captured training step (stream_layer_stack_step_capture); launch() replays it."""

    def __init__(self, handle, keep):
        self._h = handle
        self._keep = keep   # the tensors whose addresses the graph holds

    def launch(self, stream=None):
        return _check(load().ql_step_graph_launch(self._h, _stream(stream)))

    def info(self):
        """-> (kernel launches, copies, all nodes) of one replay."""
        k, c, n = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(load().ql_step_graph_info(self._h, ctypes.byref(k), ctypes.byref(c), ctypes.byref(n)))
        return k.value, c.value, n.value

    def destroy(self):
        if self._h:
            load().ql_step_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def stream_layer_stack_step_capture(cfg, store, lora, x0, dy, M, y, saved, dx0, dA, dB, accumulate, turnaround,
                                    slots, ws, compute, copy=None):
    """Captures fwd + bwd (reuse_fwd_slots = 1) into a graph; see the header for the rules."""
    c = cfg.c()
    arr = _lora_array(cfg, lora)
    n = cfg.n_layers * NPROJ
    pa = (ctypes.c_void_p * n)(*[dA[l][p].data_ptr() for l in range(cfg.n_layers) for p in PROJ])
    pb = (ctypes.c_void_p * n)(*[dB[l][p].data_ptr() for l in range(cfg.n_layers) for p in PROJ])
    h = ctypes.c_void_p()
    _check(load().stream_layer_stack_step_capture(
        ctypes.byref(c), _ptr(store), _nbytes(store), arr, _ptr(x0), _ptr(dy), M, _ptr(y), _ptr(saved),
        _nbytes(saved), _ptr(dx0), pa, pb, int(accumulate), int(turnaround), _ptr(slots), _nbytes(slots), _ptr(ws),
        _nbytes(ws), _stream(compute), _stream(copy), ctypes.byref(h)))
    return StepGraph(h, (store, x0, dy, y, saved, dx0, dA, dB, slots, ws, lora))


def build_store(cfg, layers, pinned=True, device=None):
    """Assembles the layer records from per-layer {proj: (packed, absmax)} tensors.

    Byte placement only (offsets from stream_layer_stack_layout). Returns a host
    uint8 tensor (page-locked when pinned) or, with device set, a device tensor.
    """
    offs, proj, total = stream_layer_stack_layout(cfg)
    if device is not None:
        store = torch.empty(total, dtype=torch.uint8, device=device)
    else:
        store = torch.empty(total, dtype=torch.uint8, pin_memory=pinned)
    for l, d in enumerate(layers):
        base = offs[l]
        for p in PROJ:
            packed, absmax = d[p]
            po, ao = proj[p]
            store[base + po: base + po + packed.numel()].copy_(packed.reshape(-1).view(torch.uint8))
            if cfg.absmax_dq:
                # the scale block is made on the GPU (nf4_double_quant)
                dev = device if device is not None else "cuda"
                a = absmax.reshape(-1).to(dev, torch.float32)
                ab = torch.empty(nf4_dq_layout(a.numel())[2], dtype=torch.uint8, device=dev)
                nf4_double_quant(a, ab)
                torch.cuda.synchronize()
            else:
                ab = absmax.reshape(-1).view(torch.uint8)
            store[base + ao: base + ao + ab.numel()].copy_(ab)
    return store


def ql_debug_poison_slots(on):
    return _check(load().ql_debug_poison_slots(int(on)))


def ql_profile_enable(on):
    return _check(load().ql_profile_enable(int(on)))


def ql_profile_read(kernel):
    """-> (launches, total ms, total algorithmic work) of one kernel id: FLOPs
    for the fused GEMMs, bytes for the HBM-bound kernels."""
    n, ms, fl = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
    _check(load().ql_profile_read(kernel, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl)))
    return n.value, ms.value, fl.value
