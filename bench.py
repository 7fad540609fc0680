"""Benchmark: fwd+bwd tok/s of the Llama-3.1-8B-shaped NF4 layer-streamed QLoRA stack on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: 32 layers, hidden 4096, intermediate 14336, kv 1024, head_dim 128,
LoRA r=16, alpha=32, M = 2048 tokens (batch 4 x seq 512). Frozen weights are
drawn N(0, 0.02) float32 on the GPU and NF4-quantised by the library into a
page-locked host store (3.93 GB); activations and upstream gradients N(0, 1)
bf16; LoRA factors N(0, 0.01) bf16; all seeded, synthetic.

One step = stream_layer_stack_fwd + stream_layer_stack_bwd (layers streamed
from pinned host memory into two device slots; at each turnaround the two
layers already in the slots are reused, so a steady-state step makes 2L - 4
layer copies). `value` is tokens per second of
the whole step (M tokens per step). The JSON line also carries:

* roofline - the dominant kernel (the fused NF4-dequant MFMA GEMM build, by
  kernel symbol, with the largest summed time), its algorithmic FLOPs over its
  launch durations, measured with HIP events stamped on its dispatches on its
  own stream during a second timed pass of the same steps (the first pass,
  which gives `value`, runs untimed kernels), against the bf16 dense MFMA peak
  (2.5166 PFLOP/s); `traffic` is its
  HBM bytes per launch from the committed counter summary (null if the kernel
  sources changed since). gemm_all: all fused-GEMM launches together.
* hbm_kernels - the HBM-bound kernels against the 8 TB/s HBM peak: the LoRA
  side products of the step (k_rowc: U, G, with the fused SwiGLU; k_colc: dA,
  dB), timed in the same pass as the GEMMs, with the bytes each launch must
  move once; and the standalone nf4_dequant of one gate projection.
* dense_bf16_gemm - same-session practical ceiling: torch's dense bf16 GEMM
  (hipBLASLt) on pre-dequantised weights at the stack's forward and dX
  shapes; gemm_all.vs_dense_bf16 is the fused NF4 GEMMs' rate over it.
* pcie - H2D bytes per step over the step time, against 64 GB/s (PCIe Gen5
  x16 per direction) and a same-session pinned-copy ceiling.
* ring8 - the same streamed step with 8 device slots instead of 2 (each
  turnaround then reuses 8 layers: 2 (L - 8) copies per step).
* with_reference - a preference-training step: the policy forward and the
  adapter-off reference forward in one pass over the streamed layers, then
  the backward (no extra copies for the reference).
* recompute - the same streamed step with per-layer activation recomputation
  (only layer inputs saved; the backward recomputes each layer from its slot).
* double_quant - the same streamed step from a store whose block scales are
  double-quantised (nf4_double_quant; the pages' 3.60 GB form of this store).
* small_stack_graph - the launch-bound SmolLM2-shaped stack: eager steps
  against the same step captured once into a HIP graph and replayed.
* qwen3b_stack - the Qwen2.5-3B-shaped streamed stack at M = 512 (PCIe-bound
  like the 8B stack): tok/s, its H2D rate and the tok/s 64 GB/s would allow.
* llama8b_layer_m512 - one 8B-shaped layer's seven projections, resident, at
  M = 512 through the single-linear calls: layer time and TFLOP/s, and the
  fused GEMMs' FLOP-weighted rate against the bf16 peak and against torch's
  dense bf16 GEMM at the same shapes.
* linear_pr1 - the smallest configuration's single linear (M = 64, K = 256,
  N = 512, r = 8): microseconds per forward and per backward call.
* hbm_copy_ceiling - a same-session device-to-device copy (2 GiB, 4 GiB
  moved): the practical HBM rate next to the 8 TB/s the HBM kernels are
  measured against.
* resident - the same step with the store resident in HBM (no copies).
* step_ms - median / min / max of the timed steps (events on the compute
  stream between steps); clocks_after - SCLK / MCLK from rocm-smi.
* cpu_baseline - the CPU oracle timed on a bounded sample.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6
HBM_PEAK_GBS = 8000.0
PCIE_PEAK_GBS = 64.0


CALIB_COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_llama8b_stack_m2048.json")
KERNEL_SOURCES = ("nf4_layer_streamed_amd/csrc/nf4_gemm.hip", "nf4_layer_streamed_amd/csrc/ql_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def hbm_entry(n, ms, nbytes, steps):
    """Rate of an HBM-bound kernel id from its timed launches (bytes = the
    algorithmic bytes the library records for each launch)."""
    gbs = nbytes / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
    e = dict(bound="hbm", launches=n, avg_us=round(1000.0 * ms / n, 2), bytes_per_launch=round(nbytes / n),
             achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4))
    if steps:
        e["ms_per_step"] = round(ms / steps, 3)
    return e


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a
    plain device copy of known size), or None when there is no summary for it
    or the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def build_inputs(ql, synth, torch, w, dev):
    L, M, H, I, KV, d, r, alpha = (w[k] for k in ("L", "M", "H", "I", "KV", "head_dim", "r", "alpha"))
    cfg = ql.StackCfg(L, H, I, KV, d, r, alpha)
    offs, proj, total = ql.stream_layer_stack_layout(cfg)
    store = torch.empty(total, dtype=torch.uint8, pin_memory=True)
    lora = []
    maxn = max(n * k for n, k in (cfg.proj_shape(p) for p in ql.PROJ))
    packed = torch.empty(maxn // 2, dtype=torch.uint8, device=dev)
    absmax = torch.empty(maxn // 64, dtype=torch.float32, device=dev)
    for layer in range(L):
        lo = {}
        for p in ql.PROJ:
            N, K = cfg.proj_shape(p)
            Wf = synth.normal((N * K,), synth.W_SIGMA, "llama8b_stack", layer, p, "W", device=dev)
            ql.nf4_quantize(Wf, packed[: N * K // 2], absmax[: N * K // 64])
            po, ao = proj[p]
            base = offs[layer]
            store[base + po: base + po + N * K // 2].copy_(packed[: N * K // 2])
            store[base + ao: base + ao + N * K // 16].copy_(absmax[: N * K // 64].view(torch.uint8))
            lo[p] = (synth.normal_bf16((r, K), synth.LORA_SIGMA, "llama8b_stack", layer, p, "A", device=dev),
                     synth.normal_bf16((N, r), synth.LORA_SIGMA, "llama8b_stack", layer, p, "B", device=dev))
            del Wf
        lora.append(lo)
        if layer % 8 == 7:
            log(f"bench: quantised {layer + 1}/{L} layers into the pinned store")
    x = synth.normal_bf16((M, H), 1.0, "llama8b_stack", "x", device=dev)
    dy = synth.normal_bf16((M, H), 1.0, "llama8b_stack", "dy", device=dev)
    return cfg, store, offs, lora, x, dy


def build_dq_store(ql, torch, cfg, store, dev):
    """The same layers with double-quantised scales: each projection's float32
    absmax read back from the fp32 store, double-quantised on the GPU
    (nf4_double_quant) and placed in records of the compact layout."""
    cfg_dq = ql.StackCfg(**{**cfg.__dict__, "absmax_dq": 1})
    offs, proj, _ = ql.stream_layer_stack_layout(cfg)
    offs_dq, proj_dq, total_dq = ql.stream_layer_stack_layout(cfg_dq)
    dq_store = torch.empty(total_dq, dtype=torch.uint8, pin_memory=True)
    for layer in range(cfg.n_layers):
        for p in ql.PROJ:
            N, K = cfg.proj_shape(p)
            nb = N * K // 64
            po, ao = proj[p]
            pq, aq = proj_dq[p]
            src = offs[layer]
            dst = offs_dq[layer]
            dq_store[dst + pq: dst + pq + N * K // 2].copy_(store[src + po: src + po + N * K // 2])
            absmax = store[src + ao: src + ao + nb * 4].to(dev).view(torch.float32)
            blk = torch.empty(ql.nf4_dq_layout(nb)[2], dtype=torch.uint8, device=dev)
            ql.nf4_double_quant(absmax, blk)
            dq_store[dst + aq: dst + aq + blk.numel()].copy_(blk)
    torch.cuda.synchronize()
    return cfg_dq, dq_store


def small_stack_graph(ql, synth, torch, dev, steps=20, warmup=3):
    """The SmolLM2-shaped streamed stack (30 layers, hidden 576, M = 512): a
    step issues about 700 short kernels, so their fixed costs bound it. tok/s
    of eager steps and of the same step captured once and replayed
    (stream_layer_stack_step_capture)."""
    w = synth.WORKLOADS["smollm2_stack"]
    M = w["M"]
    cfg, store, offs, lora, x, dy = build_inputs(ql, synth, torch, w, dev)
    slots_b, saved_b, ws_b = ql.stream_layer_stack_workspace(cfg, M)
    slots = torch.empty(slots_b, dtype=torch.uint8, device=dev)
    saved = torch.empty(saved_b, dtype=torch.uint8, device=dev)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    y = torch.empty(M, w["H"], dtype=torch.bfloat16, device=dev)
    dx = torch.empty_like(y)
    dA = [{p: torch.empty(w["r"], cfg.proj_shape(p)[1], device=dev) for p in ql.PROJ} for _ in range(w["L"])]
    dB = [{p: torch.empty(cfg.proj_shape(p)[0], w["r"], device=dev) for p in ql.PROJ} for _ in range(w["L"])]
    compute, copy = torch.cuda.Stream(dev), torch.cuda.Stream(dev)

    def eager(turnaround):
        ql.stream_layer_stack_fwd(cfg, store, lora, x, M, y, saved, slots, ws, compute, copy,
                                  reuse_bwd_slots=int(turnaround))
        ql.stream_layer_stack_bwd(cfg, store, lora, dy, M, saved, dx, dA, dB, 0, 1, slots, ws, compute, copy)

    for i in range(warmup):
        eager(i > 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        eager(True)
    torch.cuda.synchronize()
    te = (time.perf_counter() - t0) / steps
    g = ql.stream_layer_stack_step_capture(cfg, store, lora, x, dy, M, y, saved, dx, dA, dB, 0, 1, slots, ws,
                                           compute, copy)
    launches, graph_copies, _ = g.info()
    for _ in range(warmup):
        g.launch(compute)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.launch(compute)
    torch.cuda.synchronize()
    tg = (time.perf_counter() - t0) / steps
    g.destroy()
    rec = offs[1]
    copies = 2 * (w["L"] - cfg.n_buffers)
    pcie = copies * rec / tg / 1e9
    return dict(workload="smollm2_stack: 30 layers, hidden 576, intermediate 1536, kv 192, r8, M=512, streamed",
                eager=dict(value=round(M / te, 1), ms_per_step=round(1000 * te, 3)),
                graph=dict(value=round(M / tg, 1), ms_per_step=round(1000 * tg, 3)), unit="tok/s",
                kernel_launches_per_step=launches, us_per_launch=round(1e6 * tg / launches, 2),
                copies_per_step=copies, record_bytes=int(rec),
                pcie=dict(achieved=round(pcie, 2), peak=PCIE_PEAK_GBS, unit="GB/s", frac=round(pcie / PCIE_PEAK_GBS, 4),
                          what="layer copies of the captured step over its time"))


def qwen3b_stack(ql, synth, torch, dev, steps=10, warmup=2):
    """The Qwen2.5-3B-shaped streamed stack (36 layers, hidden 2048,
    intermediate 11008, kv 256, M = 512): tok/s of the streamed step, its H2D
    rate, and the tok/s that 64 GB/s of PCIe would allow for its copies."""
    w = synth.WORKLOADS["qwen3b_stack"]
    M, L = w["M"], w["L"]
    cfg, store, offs, lora, x, dy = build_inputs(ql, synth, torch, w, dev)
    rec = offs[1]
    slots_b, saved_b, ws_b = ql.stream_layer_stack_workspace(cfg, M)
    slots = torch.empty(slots_b, dtype=torch.uint8, device=dev)
    saved = torch.empty(saved_b, dtype=torch.uint8, device=dev)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    y = torch.empty(M, w["H"], dtype=torch.bfloat16, device=dev)
    dx = torch.empty_like(y)
    dA = [{p: torch.empty(w["r"], cfg.proj_shape(p)[1], device=dev) for p in ql.PROJ} for _ in range(L)]
    dB = [{p: torch.empty(cfg.proj_shape(p)[0], w["r"], device=dev) for p in ql.PROJ} for _ in range(L)]
    compute, copy = torch.cuda.Stream(dev), torch.cuda.Stream(dev)

    def step(turnaround):
        ql.stream_layer_stack_fwd(cfg, store, lora, x, M, y, saved, slots, ws, compute, copy,
                                  reuse_bwd_slots=int(turnaround))
        ql.stream_layer_stack_bwd(cfg, store, lora, dy, M, saved, dx, dA, dB, 0, 1, slots, ws, compute, copy)

    for i in range(warmup):
        step(i > 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    copies = 2 * (L - cfg.n_buffers)
    return dict(workload="qwen3b_stack: 36 layers, hidden 2048, intermediate 11008, kv 256, r16, M=512, streamed",
                value=round(M / t, 1), unit="tok/s", ms_per_step=round(1000 * t, 3), copies_per_step=copies,
                record_bytes=int(rec), pcie_GBs=round(copies * rec / t / 1e9, 2),
                pcie_bound_tok_s=round(M / (copies * rec / (PCIE_PEAK_GBS * 1e9)), 1))


def llama8b_layer_m512(ql, synth, torch, dev, reps=10):
    """One Llama-3.1-8B-shaped layer's seven projections, resident, at M = 512
    (batch 1, seq 512): each projection's forward and backward through
    qlora_linear_fwd / qlora_linear_bwd on its own seeded x and dY. The whole
    layer's time and FLOP rate, and the fused GEMMs' FLOP-weighted rate from
    the library's kernel timing, against the bf16 peak."""
    w = synth.WORKLOADS["llama8b_layer"]
    M, H, I, KV, r, alpha = (w[k] for k in ("M", "H", "I", "KV", "r", "alpha"))
    projs, flop, wsb = [], 0, 0
    for p in synth.PROJ:
        N, K = synth.proj_shape(p, H, I, KV)
        packed, absmax = synth.nf4_store(N * K, "llama8b_layer", p, device=dev)
        inp = synth.linear_inputs(M, K, N, r, ("llama8b_layer", p), device=dev)
        del inp["W"]
        W = ql.NF4Weight(packed, absmax, N, K)
        Lr = ql.Lora(inp["A"], inp["B"], r, alpha)
        fw, bw = ql.qlora_linear_workspace(M, N, K, r)
        wsb = max(wsb, fw, bw)
        bufs = dict(y=torch.empty(M, N, dtype=torch.bfloat16, device=dev),
                    U=torch.empty(M, r, dtype=torch.bfloat16, device=dev),
                    dx=torch.empty(M, K, dtype=torch.bfloat16, device=dev),
                    dA=torch.empty(r, K, device=dev), dB=torch.empty(N, r, device=dev))
        projs.append((W, Lr, inp, bufs))
        # fwd: x W^T, U = x A^T, U B^T; bwd: dX = dY W, G = dY B, G A; dA = G^T x, dB = dY^T U
        flop += 2 * M * N * K + 2 * M * K * r + 2 * M * r * N
        flop += 2 * M * N * K + 2 * M * N * r + 2 * M * r * K + 2 * r * M * K + 2 * N * M * r
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def layer():
        for W, Lr, inp, b in projs:
            ql.qlora_linear_fwd(inp["x"], M, W, Lr, b["y"], b["U"], ws)
            ql.qlora_linear_bwd(inp["dy"], inp["x"], b["U"], M, W, Lr, b["dx"], b["dA"], b["dB"], 0, ws)

    for _ in range(2):
        layer()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        layer()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    ql.ql_profile_enable(1)
    layer()
    torch.cuda.synchronize()
    ql.ql_profile_enable(0)
    gms, gfl = 0.0, 0.0
    for k in (ql.QL_KERNEL_GEMM_FWD, ql.QL_KERNEL_GEMM_BWD, ql.QL_KERNEL_GEMM_FWD_NARROW, ql.QL_KERNEL_GEMM_BWD_NARROW):
        _, kms, kfl = ql.ql_profile_read(k)
        gms += kms
        gfl += kfl
    g_tf = gfl / (gms * 1e-3) / 1e12
    del projs, ws
    shapes = [synth.proj_shape(p, H, I, KV) for p in synth.PROJ]
    dense = dense_gemm_ceiling(torch, dev, M, w, fwd=shapes, bwd=shapes,
                               what="torch.mm bf16 (hipBLASLt), weights pre-dequantised in HBM, the seven "
                                    "projections' fwd and dX shapes at M=512")
    return dict(workload="llama8b_layer: q, k, v, o, gate, up, down of one 8B-shaped layer, r16 alpha32, M=512, "
                         "resident, each on its own x and dY",
                ms_per_layer=round(1000 * t, 3), layer_flop=int(flop), tflops=round(flop / t / 1e12, 1),
                gemm=dict(tflops=round(g_tf, 1), frac=round(g_tf / MFMA_BF16_PEAK_TFLOPS, 4), ms=round(gms, 3),
                          vs_dense_bf16=round(g_tf / dense["tflops"], 4)),
                dense_bf16_gemm=dense, unit="TFLOP/s")


def linear_pr1(ql, synth, torch, dev, reps=200):
    """The single NF4 + LoRA linear of the smallest configuration (M = 64
    tokens, K = 256, N = 512, r = 8, alpha = 16): microseconds per forward and
    per backward call, back to back on one stream. Launch latency bounds it."""
    M, K, N, r, alpha = 64, 256, 512, 8, 16.0
    packed, absmax = synth.nf4_store(N * K, "linear_pr1", device=dev)
    inp = synth.linear_inputs(M, K, N, r, ("linear_pr1",), device=dev)
    W = ql.NF4Weight(packed, absmax, N, K)
    L = ql.Lora(inp["A"], inp["B"], r, alpha)
    fw, bw = ql.qlora_linear_workspace(M, N, K, r)
    ws = torch.empty(max(fw, bw, 256), dtype=torch.uint8, device=dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    U = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(r, K, device=dev)
    dB = torch.empty(N, r, device=dev)
    out = {}
    for name, fn in (("fwd", lambda: ql.qlora_linear_fwd(inp["x"], M, W, L, y, U, ws)),
                     ("bwd", lambda: ql.qlora_linear_bwd(inp["dy"], inp["x"], U, M, W, L, dx, dA, dB, 0, ws))):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_us"] = round(1000.0 * e0.elapsed_time(e1) / reps, 2)
    return dict(workload="linear_pr1: M=64, K=256, N=512, r8 alpha16, one NF4 + LoRA linear", **out)


def dense_gemm_ceiling(torch, dev, M, w, reps=10, fwd=None, bwd=None, what=None):
    """Same-session practical ceiling for the fused NF4 GEMMs: torch's dense
    bf16 GEMM (hipBLASLt) on weights that are already bf16 in HBM, over the
    stack's forward shapes (y = x W^T: q|k|v, o, gate|up, down) and dX shapes
    (dX = dY W: v, o, gate|up, down), FLOP-weighted like one step's mix (or
    over the given (N, K) lists)."""
    H, I, KV = w["H"], w["I"], w["KV"]
    if fwd is None:
        fwd = [(H + 2 * KV, H), (H, H), (2 * I, H), (H, I)]     # (N, K)
        bwd = [(KV, H), (H, H), (2 * I, H), (H, I)]
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    ops = []
    for N, K in fwd:
        x = torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16)
        wt = torch.randn(K, N, device=dev, generator=g).to(torch.bfloat16)   # W^T, contiguous
        ops.append((x, wt, 2.0 * M * N * K))
    for N, K in bwd:
        dy = torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16)
        wn = torch.randn(N, K, device=dev, generator=g).to(torch.bfloat16)   # W, contiguous
        ops.append((dy, wn, 2.0 * M * N * K))
    for a_, b_, _ in ops:
        torch.mm(a_, b_)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for a_, b_, _ in ops:
            torch.mm(a_, b_)
    e1.record()
    torch.cuda.synchronize()
    flop = reps * sum(f for _, _, f in ops)
    tf = flop / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del ops
    return dict(tflops=round(tf, 1), frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                what=what or "torch.mm bf16 (hipBLASLt), weights pre-dequantised in HBM, stack fwd+dX shapes at M=%d" % M)


def hbm_copy_ceiling(torch, dev, gib=2, reps=5):
    """Same-session practical HBM ceiling: a device-to-device copy of a 2 GiB
    buffer (4 GiB moved: read once, written once), GB/s of bytes moved."""
    n = gib << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = reps * 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return dict(GBs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4),
                what="device-to-device copy of 2 GiB (4 GiB moved), torch copy_")


def gpu_clocks():
    """Current SCLK / MCLK of GPU 0 as rocm-smi reports them (None when it is
    unavailable)."""
    import os
    import subprocess
    # Under rocprofv3 a child inherits the profiler's preloaded library, which
    # starts the GPU before rocm-smi's interpreter takes over the process.
    if any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    try:
        out = subprocess.run(["rocm-smi", "-d", "0", "--showclocks", "--json"], capture_output=True, text=True,
                             timeout=20).stdout
        card = next(iter(json.loads(out).values()))
        return {k: v for k, v in card.items() if "sclk" in k.lower() or "mclk" in k.lower()} or None
    except Exception:
        return None


def cpu_baseline(rows=2048, layers=3):
    """The oracle on a bounded sample: the first `layers` layers of the 8B
    stack with all 2048 tokens (or `rows` of them), forward + backward in
    bf16-faithful mode, one layer at a time; tok/s for the whole 32-layer step
    extrapolated as rows / (32 t / layers), since every layer has the same
    shapes and work."""
    import numpy as np
    import synth
    from oracle import stack as ostack
    w = synth.WORKLOADS["llama8b_stack"]
    H, I, KV, d, r, alpha = w["H"], w["I"], w["KV"], w["head_dim"], w["r"], w["alpha"]
    inp = synth.stack_inputs(layers, rows, H, I, KV, r, ("llama8b_stack_cpu",))
    x, dy = synth.as_f64(inp["x"]), synth.as_f64(inp["dy"])
    t = 0.0
    for li in range(layers):
        ld = inp["layers"][li]
        weights = {p: (ld[p]["packed"].numpy(), ld[p]["absmax"].numpy()) for p in ostack.PROJ}
        lora = {p: (synth.as_f64(ld[p]["A"]), synth.as_f64(ld[p]["B"])) for p in ostack.PROJ}
        layer = ostack.Layer(H, I, KV, d, alpha, weights, lora)
        t0 = time.perf_counter()
        h, sv = layer.fwd(x)
        layer.bwd(dy, sv)
        t += time.perf_counter() - t0
        layer.drop_cache()
        del layer, sv
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = _blas_threads(cores)
    return dict(value=rows * layers / (w["L"] * t), unit="tok/s", cores=threads, kind="oracle",
                sample=f"layers 0..{layers - 1} of {w['L']}, {rows} of {w['M']} tokens, fwd+bwd bf16-faithful "
                       f"NumPy float64, {t:.1f} s; tok/s = {rows} / ({w['L']} x t / {layers})",
                seconds=round(t, 2), host_cores=cores)


def _blas_threads(default):
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            return max(i.get("num_threads", 0) for i in info) or default
    except Exception:
        pass
    return default


def cpu_baseline_configs(runs=3):
    """The oracle, as it stands, on each smaller configuration in full (not a
    sample), median of `runs` runs: wall seconds of one forward + backward and
    the token rate. Inputs are the same seeded synthetic recipe as the GPU
    runs; weight quantisation (offline on the pages) is outside the timing.

    linear_pr1     one NF4 + LoRA linear, M=64, K=256, N=512, r=8
    llama8b_layer  the seven projections of one 8B-shaped layer at M=512, each
                   on its own x and dY (oracle.linear fwd + bwd per projection)
    smollm2_stack  30 layers, hidden 576, M=512 (oracle.stack fwd + bwd)
    qwen3b_stack   36 layers, hidden 2048, intermediate 11008, M=512
    """
    import numpy as np
    import synth
    from oracle import linear as olin
    from oracle import nf4 as onf4
    from oracle import stack as ostack

    def med(fn):
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2], ts

    out = {}
    # linear_pr1
    M, K, N, r, alpha = 64, 256, 512, 8, 16.0
    inp = synth.linear_inputs(M, K, N, r, ("linear_pr1",))
    pk, am = onf4.quantize(inp["W"].numpy().reshape(-1))
    x, A, B, dy = (synth.as_f64(inp[k]) for k in ("x", "A", "B", "dy"))

    def pr1():
        y, U = olin.fwd(x, pk, am, N, K, A, B, alpha)
        olin.bwd(dy, x, U, pk, am, N, K, A, B, alpha)
    t, ts = med(pr1)
    out["linear_pr1"] = dict(seconds=round(t, 4), runs=[round(v, 4) for v in ts], value=round(M / t, 1), unit="tok/s")
    # llama8b_layer
    w = synth.WORKLOADS["llama8b_layer"]
    M, H, I, KV, r, alpha = (w[k] for k in ("M", "H", "I", "KV", "r", "alpha"))
    projs = []
    for p in synth.PROJ:
        N, K = synth.proj_shape(p, H, I, KV)
        pk, am = synth.nf4_store(N * K, "llama8b_layer", p)
        li = synth.linear_inputs(M, K, N, r, ("llama8b_layer", p))
        projs.append((N, K, pk.numpy(), am.numpy(), *(synth.as_f64(li[k]) for k in ("x", "A", "B", "dy"))))

    def layer8b():
        for N, K, pk, am, x, A, B, dy in projs:
            y, U = olin.fwd(x, pk, am, N, K, A, B, alpha)
            olin.bwd(dy, x, U, pk, am, N, K, A, B, alpha)
    t, ts = med(layer8b)
    out["llama8b_layer"] = dict(seconds=round(t, 3), runs=[round(v, 3) for v in ts], value=round(M / t, 2),
                                unit="tok/s")
    del projs
    # the two streamed stacks
    for name in ("smollm2_stack", "qwen3b_stack"):
        w = synth.WORKLOADS[name]
        L, M, H, I, KV, d, r, alpha = (w[k] for k in ("L", "M", "H", "I", "KV", "head_dim", "r", "alpha"))
        inp = synth.stack_inputs(L, M, H, I, KV, r, (name, "cpu"))
        x, dy = synth.as_f64(inp["x"]), synth.as_f64(inp["dy"])
        layers = []
        for ld in inp["layers"]:
            weights = {p: (ld[p]["packed"].numpy(), ld[p]["absmax"].numpy()) for p in ostack.PROJ}
            lora = {p: (synth.as_f64(ld[p]["A"]), synth.as_f64(ld[p]["B"])) for p in ostack.PROJ}
            layers.append(ostack.Layer(H, I, KV, d, alpha, weights, lora))
        del inp

        def stack():
            h, saved = ostack.stack_fwd(layers, x)
            ostack.stack_bwd(layers, saved, dy)
            for lay in layers:
                lay.drop_cache()
        t, ts = med(stack)
        out[name] = dict(seconds=round(t, 2), runs=[round(v, 2) for v in ts], value=round(M / t, 2), unit="tok/s")
        del layers
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return dict(configs=out, kind="oracle", runs=runs, cores=_blas_threads(cores), host_cores=cores,
                what="bf16-faithful NumPy float64 oracle, each configuration in full, fwd + bwd, median of %d runs"
                     % runs)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-resident", action="store_true")
    ap.add_argument("--main-only", action="store_true",
                    help="time only the headline step (no ring8 / reference / recompute / double-quant / "
                         "small-stack / dense-GEMM lines), e.g. for counter runs")
    ap.add_argument("--section", choices=("llama8b_layer_m512", "small_stack_graph", "qwen3b_stack", "linear_pr1"),
                    help="run only this one extra line and print it as JSON (e.g. to profile one configuration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)

    import torch
    import nf4_layer_streamed_amd as ql
    import synth

    ql.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.section:
        fn = {"llama8b_layer_m512": llama8b_layer_m512, "small_stack_graph": small_stack_graph,
              "qwen3b_stack": qwen3b_stack, "linear_pr1": linear_pr1}[args.section]
        print(json.dumps({args.section: fn(ql, synth, torch, dev)}), flush=True)
        return
    w = synth.WORKLOADS["llama8b_stack"]
    M = w["M"]
    log("bench: building the 8B-shaped store")
    cfg, store, offs, lora, x, dy = build_inputs(ql, synth, torch, w, dev)
    rec = offs[1]
    slots_b, saved_b, ws_b = ql.stream_layer_stack_workspace(cfg, M)
    slots = torch.empty(slots_b, dtype=torch.uint8, device=dev)
    saved = torch.empty(saved_b, dtype=torch.uint8, device=dev)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    y = torch.empty(M, w["H"], dtype=torch.bfloat16, device=dev)
    dx = torch.empty(M, w["H"], dtype=torch.bfloat16, device=dev)
    dA = [{p: torch.empty(w["r"], cfg.proj_shape(p)[1], device=dev) for p in ql.PROJ} for _ in range(w["L"])]
    dB = [{p: torch.empty(cfg.proj_shape(p)[0], w["r"], device=dev) for p in ql.PROJ} for _ in range(w["L"])]
    compute = torch.cuda.Stream(dev)
    copy = torch.cuda.Stream(dev)

    def step(c, st, turnaround):
        # a training step: the forward reuses the layers the previous step's
        # backward left in the slots (turnaround), the backward those the
        # forward left
        streamed = not c.resident
        s1 = ql.stream_layer_stack_fwd(c, st, lora, x, M, y, saved, slots if streamed else None, ws,
                                       compute, copy, reuse_bwd_slots=int(streamed and turnaround))
        s2 = ql.stream_layer_stack_bwd(c, st, lora, dy, M, saved, dx, dA, dB, 0, int(streamed),
                                       slots if streamed else None, ws, compute, copy)
        return max(s1, s2)

    step_ms = []

    def timed(c, st, steps, warmup, profile, per_step=False):
        for i in range(warmup):
            step(c, st, i > 0)
        torch.cuda.synchronize()
        if profile:
            ql.ql_profile_enable(1)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)] if per_step else None
        t0 = time.perf_counter()
        status = 0
        if per_step:
            marks[0].record(compute)
        for i in range(steps):
            status = max(status, step(c, st, warmup > 0 or i > 0))
            if per_step:
                marks[i + 1].record(compute)
        torch.cuda.synchronize()
        t = time.perf_counter() - t0
        if per_step:
            step_ms[:] = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
        prof = None
        if profile:
            ql.ql_profile_enable(0)
            prof = {k: ql.ql_profile_read(k) for k in list(ql.KERNEL_SYMBOLS) + list(ql.HBM_KERNEL_SYMBOLS)}
        return t, status, prof

    log(f"bench: warmup {args.warmup}, timing {args.steps} streamed steps")
    t, status, _ = timed(cfg, store, args.steps, args.warmup, False, per_step=True)
    ms = 1000.0 * t / args.steps
    value = M * args.steps / t
    # kernel durations come from a second pass of the same steps with the
    # GEMM launches timed, so that the timing cannot perturb `value`
    log(f"bench: kernel timing pass, {args.steps} streamed steps")
    _, _, prof = timed(cfg, store, args.steps, 1, True)
    # algorithmic work per step
    L, H, I, KV, r = w["L"], w["H"], w["I"], w["KV"], w["r"]
    flop_fwd = 0.0
    for p in ql.PROJ:
        N, K = cfg.proj_shape(p)
        flop_fwd += 2.0 * M * N * K + 2.0 * M * N * r + 2.0 * M * K * r
    flop_bwd = 0.0
    for p in ("v", "o", "gate", "up", "down"):   # q and k feed nothing: no upstream gradient
        N, K = cfg.proj_shape(p)
        flop_bwd += 2.0 * M * K * (N + r) + 2.0 * M * N * r + 2.0 * M * N * r + 2.0 * M * K * r
    step_flop = L * (flop_fwd + flop_bwd)
    copies = 2 * L - 4  # per step in the steady state: both turnarounds reuse two slots
    h2d_bytes = copies * rec
    kern = {}
    for k, name in ql.KERNEL_SYMBOLS.items():
        n, kms, kfl = prof[k]
        if n == 0:
            continue
        kern[name] = dict(launches=n, total_ms=kms, avg_us=1000.0 * kms / n,
                          tflops=kfl / (kms * 1e-3) / 1e12 if kms > 0 else 0.0, flop=kfl)
    dom = max(kern, key=lambda k: kern[k]["total_ms"])
    dk = kern[dom]
    traffic = measured_traffic(dom)
    roofline = dict(bound="mfma", kernel=dom, achieved=round(dk["tflops"], 1), peak=MFMA_BF16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(dk["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                    traffic=traffic, flop_per_launch=dk["flop"] / dk["launches"],
                    avg_launch_us=round(dk["avg_us"], 2), launches=dk["launches"])
    # HBM-bound kernels of the step (LoRA side products), timed in the same pass
    hbm = {}
    for k in (ql.QL_KERNEL_LORA_ROW, ql.QL_KERNEL_LORA_COL):
        n, kms, kb = prof[k]
        if n:
            hbm[ql.HBM_KERNEL_SYMBOLS[k]] = hbm_entry(n, kms, kb, args.steps)
    gemm_ms_per_step = sum(v["total_ms"] for v in kern.values()) / args.steps
    gemm_flop = sum(v["flop"] for v in kern.values())
    gemm_all = dict(tflops=round(gemm_flop / (sum(v["total_ms"] for v in kern.values()) * 1e-3) / 1e12, 1))
    gemm_all["frac"] = round(gemm_all["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)

    # a plain device copy of known size, outside the timed region: the
    # reference point that scales the HBM byte counters of a counter run
    calib = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib)
    calib_dst.copy_(calib)
    torch.cuda.synchronize()
    del calib, calib_dst

    # standalone nf4_dequant, cold: one whole 8B-shaped layer per launch
    # (218 M weights: 122.7 MB of codes and scales in, 436 MB of bf16 out),
    # alternating between two layers' buffers, so every launch starts with its
    # 559 MB outside the 256 MB Infinity Cache; and warm: one gate projection
    # (150 MB in + out) back to back on the same buffers
    nl = sum(n_ * k_ for n_, k_ in (cfg.proj_shape(p) for p in ql.PROJ))
    dq_sets = []
    for i in range(2):
        pk_ = synth.nf4_store(nl, "dequant_cold", i, device=dev)
        dq_sets.append((pk_[0], pk_[1], torch.empty(nl, dtype=torch.bfloat16, device=dev)))
    for i in range(4):
        pk_, am_, o_ = dq_sets[i % 2]
        ql.nf4_dequant(pk_, am_, nl, o_)
    torch.cuda.synchronize()
    ql.ql_profile_enable(1)
    for i in range(10):
        pk_, am_, o_ = dq_sets[i % 2]
        ql.nf4_dequant(pk_, am_, nl, o_)
    torch.cuda.synchronize()
    ql.ql_profile_enable(0)
    n, kms, kb = ql.ql_profile_read(ql.QL_KERNEL_DEQUANT)
    dequant_s_per_weight = kms * 1e-3 / (n * nl)
    hbm["k_nf4_dequant"] = dict(hbm_entry(n, kms, kb, None),
                                what="nf4_dequant of a whole 8B-shaped layer (%d weights) to bf16 per launch, "
                                     "alternating between two layers' buffers (cold: 559 MB per launch)" % nl)
    del dq_sets
    Ng, Kg = cfg.proj_shape("gate")
    gpk, gam = synth.nf4_store(Ng * Kg, "dequant_warm", device=dev)
    gout = torch.empty(Ng * Kg, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        ql.nf4_dequant(gpk, gam, Ng * Kg, gout)
    torch.cuda.synchronize()
    ql.ql_profile_enable(1)
    for _ in range(20):
        ql.nf4_dequant(gpk, gam, Ng * Kg, gout)
    torch.cuda.synchronize()
    ql.ql_profile_enable(0)
    n, kms, kb = ql.ql_profile_read(ql.QL_KERNEL_DEQUANT)
    hbm["k_nf4_dequant_warm"] = dict(hbm_entry(n, kms, kb, None),
                                     what="nf4_dequant of a %d x %d projection to bf16, 20 launches back to back on "
                                          "the same buffers (150 MB, inside the Infinity Cache)" % (Ng, Kg))
    del gpk, gam, gout

    # same-session PCIe ceiling: one 1 GiB pinned host-to-device copy
    nb = 1 << 30
    src = store[:nb] if store.numel() >= nb else store
    dst = torch.empty(src.numel(), dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d_ceiling = 3 * src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del dst
    pcie = dict(achieved=round(h2d_bytes / (ms * 1e-3) / 1e9, 2), peak=PCIE_PEAK_GBS, unit="GB/s",
                frac=round(h2d_bytes / (ms * 1e-3) / 1e9 / PCIE_PEAK_GBS, 4),
                same_session_h2d_GBs=round(h2d_ceiling, 2), bytes_per_step=h2d_bytes,
                copies_per_step=copies, record_bytes=rec)

    ring8 = with_ref = recompute = double_quant = small = qwen = layer512 = pr1 = dense = hbm_copy = None
    fused_vs_unfused = None
    if not args.main_only:
        # the same step with a deeper slot ring (the docs' stream_buffers up to 8):
        # each turnaround reuses 8 layers, so 2 (L - 8) copies per step
        log(f"bench: 8-slot ring, {args.steps} streamed steps")
        cfg8 = ql.StackCfg(**{**cfg.__dict__, "n_buffers": 8})
        slots8 = torch.empty(ql.stream_layer_stack_workspace(cfg8, M)[0], dtype=torch.uint8, device=dev)
        slots_main = slots
        slots = slots8
        t8, _, _ = timed(cfg8, store, args.steps, args.warmup, False)
        slots = slots_main
        del slots8
        ms8 = 1000.0 * t8 / args.steps
        ring8 = dict(n_buffers=8, value=round(M * args.steps / t8, 1), unit="tok/s", ms_per_step=round(ms8, 3),
                     copies_per_step=2 * (w["L"] - 8), pcie_GBs=round(2 * (w["L"] - 8) * rec / (ms8 * 1e-3) / 1e9, 2))

        # preference-training step: policy + adapter-off reference forward in one
        # pass over the streamed layers, then the backward (same copies per step)
        log(f"bench: step with the reference forward, {args.steps} streamed steps")
        _, per_layer = ql.stream_layer_stack_saved_layout(cfg, M)
        ref_scratch = torch.empty(per_layer, dtype=torch.uint8, device=dev)
        ref_y = torch.empty(M, w["H"], dtype=torch.bfloat16, device=dev)

        def pref_step(turnaround):
            s1 = ql.stream_layer_stack_fwd_ref(cfg, store, lora, x, M, y, saved, ref_y, ref_scratch, slots, ws,
                                               compute, copy, reuse_bwd_slots=int(turnaround))
            s2 = ql.stream_layer_stack_bwd(cfg, store, lora, dy, M, saved, dx, dA, dB, 0, 1, slots, ws, compute, copy)
            return max(s1, s2)

        for i in range(args.warmup):
            pref_step(i > 0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            pref_step(True)
        torch.cuda.synchronize()
        tr = time.perf_counter() - t0
        with_ref = dict(value=round(M * args.steps / tr, 1), unit="tok/s", ms_per_step=round(1000 * tr / args.steps, 3),
                        copies_per_step=copies, note="policy + adapter-off reference forward share each layer copy")
        del ref_scratch, ref_y

        # the same streamed step with per-layer recomputation (gradient
        # checkpointing): the forward keeps only layer inputs, the backward
        # recomputes each layer from its slot
        log(f"bench: recompute mode, {args.steps} streamed steps")
        cfg_rc = ql.StackCfg(**{**cfg.__dict__, "recompute": 1})
        _, saved_rc_b, ws_rc_b = ql.stream_layer_stack_workspace(cfg_rc, M)
        saved_main, ws_main = saved, ws
        saved = torch.empty(saved_rc_b, dtype=torch.uint8, device=dev)
        ws = torch.empty(ws_rc_b, dtype=torch.uint8, device=dev)
        trc, _, _ = timed(cfg_rc, store, args.steps, args.warmup, False)
        saved, ws = saved_main, ws_main
        recompute = dict(value=round(M * args.steps / trc, 1), unit="tok/s", ms_per_step=round(1000 * trc / args.steps, 3),
                         saved_bytes=int(saved_rc_b), saved_bytes_without=int(saved.numel()),
                         ws_bytes=int(ws_rc_b), ws_bytes_without=int(ws.numel()))

        # the same streamed step from a store with double-quantised scales (the
        # pages' 3.60 GB form): 8% fewer bytes per layer copy
        log("bench: double-quantised store")
        cfg_dq, dq_store = build_dq_store(ql, torch, cfg, store, dev)
        rec_dq = ql.stream_layer_stack_layout(cfg_dq)[0][1]
        slots_dq_b, _, ws_dq_b = ql.stream_layer_stack_workspace(cfg_dq, M)
        slots_main, ws_main = slots, ws
        slots = torch.empty(slots_dq_b, dtype=torch.uint8, device=dev)
        ws = torch.empty(ws_dq_b, dtype=torch.uint8, device=dev)
        log(f"bench: double-quantised store, {args.steps} streamed steps")
        tdq, status_dq, _ = timed(cfg_dq, dq_store, args.steps, args.warmup, False)
        slots, ws = slots_main, ws_main
        msdq = 1000.0 * tdq / args.steps
        double_quant = dict(value=round(M * args.steps / tdq, 1), unit="tok/s", ms_per_step=round(msdq, 3),
                            store_bytes=int(dq_store.numel()), record_bytes=int(rec_dq), copies_per_step=copies,
                            pcie_GBs=round(copies * rec_dq / (msdq * 1e-3) / 1e9, 2), status=int(status_dq))
        del dq_store

        log("bench: SmolLM2-shaped stack, eager and captured steps")
        small = small_stack_graph(ql, synth, torch, dev)
        log("bench: Qwen2.5-3B-shaped stack")
        qwen = qwen3b_stack(ql, synth, torch, dev)
        log("bench: one 8B-shaped layer's projections at M=512")
        layer512 = llama8b_layer_m512(ql, synth, torch, dev)
        pr1 = linear_pr1(ql, synth, torch, dev)

        dense = dense_gemm_ceiling(torch, dev, M, w)
        hbm_copy = hbm_copy_ceiling(torch, dev)
        gemm_all["vs_dense_bf16"] = round(gemm_all["tflops"] / dense["tflops"], 4)
        # the unfused alternative: each layer's weights dequantised to bf16 in
        # HBM by nf4_dequant (cold rate above) before its forward GEMMs and
        # again before its dX GEMMs (q and k have none), then dense bf16 GEMMs
        # at the same-session hipBLASLt rate over the same FLOPs
        w_fwd = sum(n_ * k_ for n_, k_ in (cfg.proj_shape(p) for p in ql.PROJ))
        w_bwd = sum(n_ * k_ for n_, k_ in (cfg.proj_shape(p) for p in ("v", "o", "gate", "up", "down")))
        deq_ms = 1000.0 * dequant_s_per_weight * L * (w_fwd + w_bwd)
        dense_ms = 1000.0 * (gemm_flop / args.steps) / (dense["tflops"] * 1e12)
        fused_vs_unfused = dict(
            fused_gemm_ms_per_step_streamed=round(gemm_ms_per_step, 3),
            unfused_ms_per_step=round(deq_ms + dense_ms, 3), unfused_dequant_ms=round(deq_ms, 3),
            unfused_dense_gemm_ms=round(dense_ms, 3),
            unfused_over_fused_streamed=round((deq_ms + dense_ms) / gemm_ms_per_step, 4),
            what="per step at M=2048: the fused NF4 GEMMs (kernel timing, in the streamed step, where the layer "
                 "copies share the CUs, and in the resident step) against nf4_dequant of every layer before its "
                 "forward and again before its dX GEMMs (%d + %d weights per layer, cold dequant rate) plus dense bf16 "
                 "GEMMs of the same FLOPs at the same-session hipBLASLt rate, both timed alone" % (w_fwd, w_bwd))

    resident = None
    if not args.no_resident:
        log("bench: resident ablation (store in HBM, no copies)")
        store_dev = store.to(dev)
        rcfg = ql.StackCfg(**{**cfg.__dict__, "resident": 1})
        rt, _, _ = timed(rcfg, store_dev, args.steps, 1, False)
        # the fused GEMMs once more, in this copy-free step (kernel timing pass)
        _, _, rprof = timed(rcfg, store_dev, args.steps, 1, True)
        r_ms = sum(rprof[k][1] for k in ql.KERNEL_SYMBOLS) / args.steps
        r_fl = sum(rprof[k][2] for k in ql.KERNEL_SYMBOLS) / args.steps
        resident = dict(value=round(M * args.steps / rt, 1), unit="tok/s", ms_per_step=round(1000 * rt / args.steps, 3),
                        tflops=round(step_flop / (rt / args.steps) / 1e12, 1),
                        gemm_ms_per_step=round(r_ms, 3),
                        gemm_all=dict(tflops=round(r_fl / (r_ms * 1e-3) / 1e12, 1),
                                      frac=round(r_fl / (r_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)))
        if dense is not None:
            resident["gemm_all"]["vs_dense_bf16"] = round(resident["gemm_all"]["tflops"] / dense["tflops"], 4)
        if fused_vs_unfused is not None:
            # the copy-free comparison: fused GEMMs of the resident step
            fused_vs_unfused["fused_gemm_ms_per_step_resident"] = round(r_ms, 3)
            fused_vs_unfused["unfused_over_fused_resident"] = round(fused_vs_unfused["unfused_ms_per_step"] / r_ms, 4)
        del store_dev

    cpu = cpu_configs = None
    if not args.no_cpu_baseline:
        log("bench: cpu_baseline (oracle on a bounded sample)")
        cpu = cpu_baseline()
        if not args.main_only:
            log("bench: oracle timings of the smaller configurations (in full, median of 3)")
            cpu_configs = cpu_baseline_configs()

    out = {
        "metric": "tok/s fwd+bwd, 8B-shape NF4 streamed QLoRA stack; NF4 GEMM % MFMA peak",
        "value": round(value, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "step_ms": dict(median=round(sorted(step_ms)[len(step_ms) // 2], 3), min=round(min(step_ms), 3),
                        max=round(max(step_ms), 3), what="GPU time between events on the compute stream") if step_ms else None,
        "clocks_after": gpu_clocks(),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama8b_stack: 32 layers, hidden 4096, intermediate 14336, kv 1024, "
                               "NF4 block 64 fp32 absmax, LoRA r16 alpha32, M=2048 (4 x 512), "
                               "pinned-host store streamed through 2 device slots",
                   "global_batch": 4, "seq_len": 512, "parallelism": "none (1 GPU)",
                   "store_bytes": int(store.numel()), "status": int(status)},
        "tflops_step": round(step_flop / (ms * 1e-3) / 1e12, 1),
        "step_flop": step_flop,
        "gemm_ms_per_step": round(gemm_ms_per_step, 3),
        "gemm_all": gemm_all,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kern.items()},
        "roofline": roofline,
        "hbm_kernels": hbm,
        "dense_bf16_gemm": dense,
        "fused_vs_unfused": fused_vs_unfused,
        "hbm_copy_ceiling": hbm_copy,
        "pcie": pcie,
        "ring8": ring8,
        "with_reference": with_ref,
        "recompute": recompute,
        "double_quant": double_quant,
        "small_stack_graph": small,
        "qwen3b_stack": qwen,
        "llama8b_layer_m512": layer512,
        "linear_pr1": pr1,
        "resident": resident,
        "cpu_baseline": cpu,
        "cpu_baseline_configs": cpu_configs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
