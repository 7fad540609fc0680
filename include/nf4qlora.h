/*
 * nf4qlora.h - C ABI of the MI355X (gfx950) NF4 + LoRA layer-streaming library.
 *
 * The library computes the hot path of layer-streamed QLoRA training: a frozen
 * linear layer stored as 4-bit NormalFloat (NF4) codes with one float32 absmax
 * per 64 weights, a trainable rank-r LoRA adapter beside it, forward and
 * backward, and a decoder stack fed one layer at a time from pinned host
 * memory through two device buffers.
 *
 * Sources (the Soup pages): the frozen base is held in host memory and fed to
 * the GPU layer by layer, and the adapter is the only trained part (Soup README intro,
 * "Citing Soup"; blog "The trick: layer streaming"); it is stored as NF4,
 * quantised once offline, and dequantised on the fly per layer (soup-cli
 * 0.72.2 docs "NF4 streaming (quantization: 4bit)"); copies come from
 * page-locked memory into two pre-allocated device buffers so they overlap
 * compute, and a pageable store falls back with its cost reported (CHANGELOG
 * [0.72.0]; docs "Layer Streaming", "Honest scope" and "Troubleshooting");
 * streaming changes only when the bytes arrive, so a streamed run is bit-identical to
 * a resident one (blog "Why the evidence is better than usual"; CHANGELOG
 * [0.72.2] "Correctness"). The NF4 codebook, block size, scale format and
 * rounding are not on the pages; the library follows the QLoRA paper
 * (Dettmers et al. 2023, section 3), with block 64 and a float32 absmax.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless the argument says "host".
 *  - Matrices are row-major. x is [M x K], the frozen weight W is [N x K]
 *    (K contiguous), LoRA A is [r x K], B is [N x r], s = alpha / r.
 *  - bf16 tensors are IEEE bfloat16 (uint16 storage), float32 is IEEE binary32.
 *  - Every call validates all of its arguments before it enqueues anything; on
 *    an error (status < 0) nothing has been enqueued and the outputs are
 *    untouched. ql_last_error() then names the offending argument and rule.
 *  - Calls are asynchronous on the given stream(s) unless stated otherwise.
 *    Buffers must stay alive until the stream has passed the call.
 *  - The library never mutates its inputs and keeps no state between calls.
 *    It allocates no device memory: nf4_quantize's finiteness flag is one
 *    word in the library's code object on each device.
 *  - Matrix dimensions (N, K; hidden, inter) are at most QL_MAX_DIM, so that
 *    every per-row byte offset the kernels form fits in 32 bits; element
 *    counts and the products N * K are unrestricted (64-bit).
 *  - The caller allocates every buffer (device memory, pinned host store,
 *    workspaces); the *_workspace / *_layout calls give the sizes.
 *  - Results are deterministic: no atomics take part in any reduction, and
 *    kernel selection does not depend on pointer values.
 */
#ifndef NF4QLORA_H
#define NF4QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ql_status;

enum {
  QL_OK = 0,
  /* Success, but the host store is pageable: copies could not overlap compute
     (docs "Layer Streaming": the pageable fallback runs and reports its cost). */
  QL_WARN_PAGEABLE_HOST = 1,
  QL_ERR_ARG = -1,         /* null pointer, bad enum, bad flag */
  QL_ERR_SHAPE = -2,       /* K % 64, N % 16, negative sizes, a dimension above QL_MAX_DIM */
  QL_ERR_ALIGN = -3,       /* pointer not aligned as the call requires */
  QL_ERR_RANK = -4,        /* LoRA rank outside 1..64 (the pages refuse r < 1) */
  QL_ERR_NONFINITE = -5,   /* nf4_quantize met NaN or Inf */
  QL_ERR_WORKSPACE = -6,   /* a workspace or buffer is smaller than required */
  QL_ERR_HIP = -7,         /* a HIP runtime call failed */
  QL_ERR_UNSUPPORTED = -8  /* a valid request this library does not implement */
};

enum { QL_BF16 = 0, QL_F32 = 1 };

/* Largest matrix dimension (rows or columns of a weight, hidden and
 * intermediate widths of a stack). */
#define QL_MAX_DIM (1 << 21)

/* A hipStream_t passed as an opaque pointer; NULL means the null stream. */
typedef void* ql_stream;

/* Thread-local message for the last failing call on this thread ("" if none). */
const char* ql_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int32_t ql_abi_version(void);

/* The 16 float32 NF4 levels the library uses, copied to host memory `out`. */
ql_status nf4_codebook(float* out /* host [16] */);

/* ---------------------------------------------------------------- NF4 codec
 * nf4_quantize: block-wise NF4 quantisation of w (float32, n elements,
 * row-major flattened; n % 64 == 0). For each block of 64 consecutive
 * elements: absmax = max |w|; each element's code is the index of the nearest
 * NF4 level to fl32(w / absmax) (ties to the lower index); an all-zero block
 * gets code 7 (the zero level) and absmax 0. Codes are packed 8 to a 32-bit
 * little-endian word (elements 8w..8w+7 in bytes 4w..4w+3): byte j of word w
 * holds element 8w+j in its low nibble and element 8w+j+4 in its high nibble.
 * Quantisation is offline, done once per tensor (docs "Layer Streaming",
 * "NF4 streaming": the base is quantised a tensor at a time, once, before
 * training).
 *   packed: uint8 [n/2], absmax: float32 [n/64]; all 16-byte aligned.
 * Non-finite input is refused with QL_ERR_NONFINITE, and then nothing is
 * written. To refuse it before any output is written, the call first scans w
 * on the stream and waits for that scan (the one synchronous step of the
 * library; host threads calling it concurrently take turns); the
 * quantisation itself is then enqueued asynchronously like every other call.
 */
ql_status nf4_quantize(const float* w, int64_t n, uint8_t* packed, float* absmax, ql_stream s);

/* nf4_dequant: out[i] = fl32(level[code_i] * absmax[i / 64]); with
 * out_dtype == QL_BF16 that float32 value rounded to nearest even bfloat16.
 * This is the standalone form of the per-layer dequantisation the Soup README
 * ("Citing Soup", v3 retraction) names as streaming's largest own cost; the
 * GEMMs below fuse it instead. n % 64 == 0; pointers 16-byte aligned.
 */
ql_status nf4_dequant(const uint8_t* packed, const float* absmax, int64_t n,
                      int32_t out_dtype, void* out, ql_stream s);

/* ------------------------------------------- double-quantised block scales
 * The pages' NF4 stores (3.60 GB for Llama-3.1-8B with 113 MB layer buffers:
 * Soup README, header figure caption; 1.43 GB for Qwen2.5-3B: CHANGELOG
 * [0.72.2]) are about 0.516 bytes per weight, which is NF4 codes plus 8-bit
 * block scales: the second-level quantisation of QLoRA section 3 ("Double
 * Quantization"). Reading taken here:
 *   mu = fl32(S / n), S the float64 sum of the n float32 absmax values taken
 *     in a fixed order (runs of 256 left to right, then the run sums left to
 *     right);
 *   per run of 256: d = fl32(c - mu), s = fl32(max |d| / 448),
 *     code = OCP FP8 E4M3 of fl32(d / s), round-to-nearest-even, saturated to
 *     +-448 (s = 0: code 0);
 *   expansion: c' = fl32(fl32(e4m3(code) * s) + mu).
 * The NF4 codes are those of the float32 absmax; only the scale storage
 * changes (c' replaces absmax in every use).
 *
 * nf4_dq_layout: the block for nblocks scales: codes (nblocks bytes) at 0, the
 * run scales (float32, ceil(nblocks / 256)) at *scale_off, mu (float32) at
 * *mean_off, *bytes in all (multiples of 256).
 * nf4_double_quant: absmax (float32 [nblocks], finite, as nf4_quantize makes
 * it) -> the block at dq (256-byte aligned, dq_bytes >= the block size).
 * nf4_dq_expand: the block -> c' (float32 [nblocks]).
 */
ql_status nf4_dq_layout(int64_t nblocks, size_t* scale_off, size_t* mean_off, size_t* bytes);
ql_status nf4_double_quant(const float* absmax, int64_t nblocks, void* dq, size_t dq_bytes, ql_stream s);
ql_status nf4_dq_expand(const void* dq, int64_t nblocks, float* absmax, ql_stream s);

/* ------------------------------------------------------- NF4 + LoRA linear */
typedef struct {
  const uint8_t* packed; /* uint8 [N*K/2] as written by nf4_quantize */
  const float* absmax;   /* float32 [N*K/64] */
  int64_t N, K;          /* out-features, in-features; K % 64 == 0, N % 16 == 0,
                            both <= QL_MAX_DIM */
} ql_nf4_weight;

typedef struct {
  const void* A;  /* bf16 [r x K] */
  const void* B;  /* bf16 [N x r] */
  int32_t r;      /* 1..64 */
  float alpha;    /* scale s = alpha / r */
} ql_lora;

/* Workspace sizes (bytes) of qlora_linear_fwd and qlora_linear_bwd for a shape. */
ql_status qlora_linear_workspace(int64_t M, int64_t N, int64_t K, int32_t r,
                                 size_t* fwd_bytes, size_t* bwd_bytes);

/* qlora_linear_fwd: the frozen NF4 linear with its LoRA adapter,
 *   U = bf16(x A^T)                    -> u_save, bf16 [M x r] (kept for the backward)
 *   y = bf16(x W^T + s U B^T)          -> y, bf16 [M x N]
 * with W = bf16(fl32(level * absmax)) dequantised inside the GEMM's tile
 * loader (never materialised) and float32 accumulation. s B is rounded to
 * bf16 as an MFMA operand (exact when s is a power of two).
 * Forward of the LoRA linear on the pages: the quantised base is frozen and
 * the adapter is the trained part (blog, "The trick: layer streaming"); the
 * NF4 weights are decoded on the fly (docs "NF4 streaming").
 *   x: bf16 [M x K]; M >= 0 (M == 0 is a no-op); 16-byte aligned pointers.
 *   ws: device workspace of at least fwd_bytes from qlora_linear_workspace.
 */
ql_status qlora_linear_fwd(const void* x, int64_t M, ql_nf4_weight W, ql_lora L,
                           void* y, void* u_save, void* ws, size_t ws_bytes, ql_stream s);

/* qlora_linear_bwd: gradients of the linear above for upstream dY (bf16 [M x N]):
 *   G  = bf16(dY B)                    (internal, [M x r])
 *   dX = bf16(dY W + s G A)            -> dx, bf16 [M x K]; skipped if dx == NULL
 *   dB = s dY^T U                      -> dB, float32 [N x r]
 *   dA = s G^T x                       -> dA, float32 [r x K]
 * There is no gradient for the frozen W: only the adapter trains (blog, "The
 * trick: layer streaming"). With accumulate != 0, dA and dB are added to
 * their current values (float32), else overwritten. Reductions over M use a fixed order.
 *   u_saved: the U written by qlora_linear_fwd for the same x.
 *   ws: device workspace of at least bwd_bytes from qlora_linear_workspace.
 */
ql_status qlora_linear_bwd(const void* dy, const void* x, const void* u_saved, int64_t M,
                           ql_nf4_weight W, ql_lora L, void* dx, float* dA, float* dB,
                           int32_t accumulate, void* ws, size_t ws_bytes, ql_stream s);

/* qlora_linear_bwd_noalloc: exactly qlora_linear_bwd (same kernels, same
 * bits) without a workspace argument, for callers that cannot allocate device
 * memory: code recorded under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc. Its temporaries live in a fixed array of
 * QL_NOALLOC_SCRATCH_BYTES in the library's code object on each device, held
 * until the process ends; the call itself allocates nothing. A shape whose
 * workspace (bwd_bytes of qlora_linear_workspace) exceeds that size is
 * refused with QL_ERR_WORKSPACE before anything is enqueued. The scratch
 * needs no clearing (every temporary is written before it is read) and keeps
 * nothing between calls, but all calls on one device share it: calls that
 * overlap on one device (concurrent streams, or host threads) race, so order
 * them on one stream. The wide dX kernel keeps a few values in per-lane
 * private memory (register spills, 44 bytes per lane), which the HIP runtime
 * backs from its own scratch pool when such a kernel first runs on a queue. */
#define QL_NOALLOC_SCRATCH_BYTES (128u << 20)
ql_status qlora_linear_bwd_noalloc(const void* dy, const void* x, const void* u_saved, int64_t M,
                                   ql_nf4_weight W, ql_lora L, void* dx, float* dA, float* dB,
                                   int32_t accumulate, ql_stream s);

/* ----------------------------------------------------- layer-streamed stack
 * A stack of n_layers decoder-layer stand-ins, each
 *   n1 = RMSNorm(h); q,k,v = P_q,P_k,P_v(n1); a = repeat_kv(v);
 *   h = h + P_o(a); n2 = RMSNorm(h); g,u = P_gate,P_up(n2);
 *   h = h + P_down(silu(g) * u)
 * with every P an NF4 + LoRA linear (shapes: q,o [H x H]; k,v [kv x H];
 * gate,up [I x H]; down [H x I]). RMSNorm has unit gain; repeat_kv gives head
 * j of `a` the kv head j / (H / kv_dim). q and k feed nothing in this
 * attention-free stand-in: they are computed and saved, their gradients are 0.
 *
 * The frozen NF4 weights live in one "store" of n_layers records (layout from
 * stream_layer_stack_layout). Streamed mode (resident == 0): the store is HOST
 * memory, ideally page-locked; each layer's record is copied asynchronously
 * host-to-device on the `copy` stream into one of n_buffers device slots,
 * while the `compute` stream works on another; events order the two (docs
 * "Layer Streaming": pre-allocated device buffers, two by default). A record
 * goes as one copy, except each pass's last one (records of 8 MiB or more),
 * which goes weight group by weight group so that its layer starts each GEMM
 * as soon as that GEMM's group has landed. With two slots, part of each
 * pass's first refill (the groups its slot's layer has finished with) runs
 * on a side copy stream that the library creates on first use, one per
 * device with default priority, and keeps for the process; calls recorded
 * into a graph do not use it.
 * Peak device memory for weights is the n_buffers slots.
 * Resident mode (resident == 1): the store is a DEVICE buffer, nothing is
 * copied and the same kernels run in the same order on the same bytes, so the
 * results are bit-identical to streamed mode (blog "Why the evidence is better
 * than usual": streaming reorders copies, not arithmetic).
 * A pageable host store still works, but its copies cannot overlap compute;
 * the call then returns QL_WARN_PAGEABLE_HOST (docs "Layer Streaming":
 * pageable fallback with its cost reported).
 * Slots: n_buffers device records (2..QL_MAX_BUFFERS; the docs' buffer count
 * for layer streaming, "Layer Streaming" section of performance-and-
 * quantization, whose default is double buffering). Layer l always uses slot
 * l % n_buffers; after computing layer l the forward refills its slot with
 * layer l + n_buffers and the backward with layer l - n_buffers, so up to
 * n_buffers - 1 copies run ahead of the compute stream. Reusing the slots at
 * a turnaround (reuse_bwd_slots / reuse_fwd_slots) skips n_buffers copies, so
 * a steady-state fwd + bwd step makes 2 (n_layers - n_buffers) copies.
 * Slot ordering: a streamed call's first copy
 * waits for all work enqueued before the call on the compute stream (which
 * may still read the slots), so successive calls may share the slots when
 * they use the same compute stream; with different compute streams the
 * caller orders the streams.
 * Host wait (streamed mode with layer records of 8 MiB or more, not while
 * the compute stream is capturing):
 * before it enqueues anything, a forward call (stream_layer_stack_fwd or
 * _fwd_ref) blocks the host until the previous streamed forward call on the
 * same device has finished on the GPU, and a backward call likewise for the
 * previous backward. So at most one of each is queued, and the call's own
 * work stays asynchronous. Deeper device queues slow the hand-off between
 * the copy and compute streams. With n_buffers == 2 the call also blocks
 * the host, before it enqueues each layer, until the layer two back has
 * finished on the GPU: the host stays at most two layers ahead.
 */
#define QL_MAX_BUFFERS 8

typedef struct {
  int32_t n_layers, hidden, inter, kv_dim, head_dim, r;
  float alpha, rms_eps;
  int32_t n_buffers;  /* device slots, 2..QL_MAX_BUFFERS (2: double buffering) */
  int32_t resident;   /* 0: host store, streamed; 1: device store, no copies */
  int32_t recompute;  /* 1: per-layer activation recomputation (gradient checkpointing) */
  int32_t absmax_dq;  /* 1: each projection's absmax in the record is its nf4_double_quant
                       * block; the layer's scales are expanded on the device before
                       * its GEMMs (8% fewer bytes per copy) */
} ql_stack_cfg;

enum { QL_PROJ_Q = 0, QL_PROJ_K, QL_PROJ_V, QL_PROJ_O, QL_PROJ_GATE, QL_PROJ_UP, QL_PROJ_DOWN,
       QL_NPROJ };

/* Store layout. layer_offsets (host int64 [n_layers + 1]) gets each record's
 * byte offset and the total; proj_offsets (host int64 [2 * QL_NPROJ], may be
 * NULL) gets, within a record, the byte offset of projection p's packed codes
 * at [2p] and of its absmax at [2p+1]. Every offset is a multiple of 256.
 * A record holds four contiguous weight groups, q|k|v, o, gate|up, down, each
 * its projections' codes then their absmax; the streamer may copy a record
 * group by group. */
ql_status stream_layer_stack_layout(const ql_stack_cfg* cfg, int64_t* layer_offsets,
                                    int64_t* proj_offsets, size_t* store_bytes);

/* Buffer sizes for M tokens: slots (n_buffers device layer records; none in
 * resident mode), saved activations (written by the forward, read by the
 * backward), and workspace. */
ql_status stream_layer_stack_workspace(const ql_stack_cfg* cfg, int64_t M, size_t* slots_bytes,
                                       size_t* saved_bytes, size_t* ws_bytes);

enum { QL_SAVED_H_IN = 0, QL_SAVED_N1, QL_SAVED_Q, QL_SAVED_K, QL_SAVED_V, QL_SAVED_H_MID,
       QL_SAVED_N2, QL_SAVED_GATE, QL_SAVED_UP, QL_SAVED_ACT, QL_SAVED_U0 /* + QL_PROJ_* */,
       QL_SAVED_COUNT = QL_SAVED_U0 + QL_NPROJ };

/* Byte offsets (host int64 [QL_SAVED_COUNT]) of each saved tensor within one
 * layer's part of `saved`, and that part's size; layer l starts at
 * l * per_layer_bytes. All saved tensors are bf16, row-major with M rows.
 * recompute = 1 (gradient checkpointing, handled per layer by the streamer as
 * in the docs' "Layer Streaming" configuration): the forward keeps only each
 * layer's input h_in (every other offset is -1) and the backward recomputes
 * the layer's activations from it, with the weights already in the layer's
 * slot, into a one-layer area of the workspace. No extra copies; the
 * recomputed values are those the forward produced, so y, dx0, dA and dB are
 * bitwise those of recompute = 0. */
ql_status stream_layer_stack_saved_layout(const ql_stack_cfg* cfg, int64_t M, int64_t* offsets,
                                          size_t* per_layer_bytes);

/* Forward over all layers: y (bf16 [M x H]) = stack(x0). lora is a HOST array
 * of n_layers * QL_NPROJ adapters (device A, B; r and alpha must equal cfg's),
 * indexed [layer * QL_NPROJ + proj].
 * reuse_bwd_slots != 0 skips the copies of layers 0 .. n_buffers - 1, which
 * a stream_layer_stack_bwd call with the same cfg, store and slots left in
 * the slots (the training loop's turnaround from one step's backward to the
 * next step's forward); it requires that nothing wrote the slots since and
 * that the same compute stream is used (2 (L - n_buffers) copies per training
 * step with both reuse flags). Ignored in resident mode. */
ql_status stream_layer_stack_fwd(const ql_stack_cfg* cfg, const void* store, size_t store_bytes,
                                 const ql_lora* lora, const void* x0, int64_t M, void* y,
                                 void* saved, size_t saved_bytes, int32_t reuse_bwd_slots,
                                 void* slots, size_t slots_bytes, void* ws, size_t ws_bytes,
                                 ql_stream compute, ql_stream copy);

/* Policy forward plus the adapter-off reference forward, in one pass over the
 * layers. For preference losses the reference model is the same streamed
 * frozen base with the adapters switched off, which on the pages costs extra
 * layer reads (the aiany.app entry "Soup", section "How It Works"). Here each
 * streamed layer, once in its slot, serves both forwards before the slot is
 * refilled, so the reference adds compute but no host-to-device copies.
 * y, saved: exactly those of stream_layer_stack_fwd with the same arguments
 * (bitwise). ref_y (bf16 [M x H]): the stack's output with every LoRA term
 * removed (y = x W^T per projection), on the same x0. ref_scratch: one
 * layer's activations (per_layer_bytes of stream_layer_stack_saved_layout
 * for the same cfg with recompute = 0), overwritten; its contents afterwards
 * are unspecified. lora == NULL: the reference alone (y and saved are then not
 * used and may be NULL). reuse_bwd_slots and the slot ordering are as in
 * stream_layer_stack_fwd, so a following stream_layer_stack_bwd may reuse the
 * slots this call leaves. */
ql_status stream_layer_stack_fwd_ref(const ql_stack_cfg* cfg, const void* store, size_t store_bytes,
                                     const ql_lora* lora, const void* x0, int64_t M, void* y,
                                     void* saved, size_t saved_bytes, void* ref_y, void* ref_scratch,
                                     size_t ref_scratch_bytes, int32_t reuse_bwd_slots, void* slots,
                                     size_t slots_bytes, void* ws, size_t ws_bytes,
                                     ql_stream compute, ql_stream copy);

/* Backward over all layers, last to first, from dy (bf16 [M x H]) at the
 * output: dx0 (bf16 [M x H], may be NULL) and dA / dB (HOST arrays of
 * n_layers * QL_NPROJ device float32 pointers, [r x K] and [N x r]).
 * reuse_fwd_slots != 0 skips the copies of the last n_buffers layers, which
 * a stream_layer_stack_fwd call with the same cfg, store and slots left in
 * the slots; it requires that nothing wrote the slots since and that the same
 * compute stream is used. Ignored in resident mode. */
ql_status stream_layer_stack_bwd(const ql_stack_cfg* cfg, const void* store, size_t store_bytes,
                                 const ql_lora* lora, const void* dy, int64_t M,
                                 const void* saved, size_t saved_bytes, void* dx0,
                                 float* const* dA, float* const* dB, int32_t accumulate,
                                 int32_t reuse_fwd_slots, void* slots, size_t slots_bytes,
                                 void* ws, size_t ws_bytes, ql_stream compute, ql_stream copy);

/* --------------------------------------------------------------- step graphs
 * A whole training step (stream_layer_stack_fwd then stream_layer_stack_bwd
 * with reuse_fwd_slots = 1) captured once into a HIP graph and replayed with
 * one launch. A small model's layer loop is bound by per-launch cost, not by
 * the GPU (the SmolLM2 shape issues about 1,400 kernels per step); the pages
 * meet the same kind of limit when an H100 runs no faster than a laptop GPU
 * at batch 1 (Soup README, "Citing Soup", v3 notes). All pointers are baked into the
 * graph: between replays the caller rewrites the contents of x0 and dy (and
 * of lora's factors), never their addresses. turnaround = 1: the forward
 * reuses the layers the previous step's backward left in the slots (the
 * first replay must then follow a step of this cfg on the same slots);
 * turnaround = 0: every replay copies its first layers itself. The store must
 * be page-locked host memory (or a device store in resident mode) and kernel
 * timing must be off. The capture enqueues nothing that runs; a replay runs
 * on `stream` like the two calls would on `compute` (the copies keep their own
 * engine), and results are bitwise those of the uncaptured calls.
 * Capturing code must not create hipMemsetAsync nodes; none is used here.
 */
typedef struct ql_step_graph_s* ql_step_graph;
ql_status stream_layer_stack_step_capture(const ql_stack_cfg* cfg, const void* store, size_t store_bytes,
                                          const ql_lora* lora, const void* x0, const void* dy, int64_t M,
                                          void* y, void* saved, size_t saved_bytes, void* dx0,
                                          float* const* dA, float* const* dB, int32_t accumulate,
                                          int32_t turnaround, void* slots, size_t slots_bytes, void* ws,
                                          size_t ws_bytes, ql_stream compute, ql_stream copy,
                                          ql_step_graph* out);
ql_status ql_step_graph_launch(ql_step_graph g, ql_stream stream);
ql_status ql_step_graph_destroy(ql_step_graph g);
/* What one replay of a captured step runs (host counts, may be NULL): kernel
 * launches, copy nodes (the layer copies among them) and all graph nodes.
 * The launch count is what bounds a small model's step (the v3 notes of
 * "Citing Soup" above). */
ql_status ql_step_graph_info(ql_step_graph g, int64_t* kernels, int64_t* copies, int64_t* nodes);

/* ----------------------------------------------------------- measurement
 * Kernel timing for roofline measurement. While enabled, every launch of the
 * timed kernels is bracketed by two hipEvents recorded on the stream it runs
 * on, together with its algorithmic work:
 *  - fused NF4 GEMMs (MFMA-bound): FLOPs, 2 M N (K + r) for the forward and
 *    2 M K (N + r) per reduction segment for dX, over the columns the launch
 *    covers. Each comes in a wide-tile (256 x 256 outputs per workgroup) and a
 *    narrow-tile (256 x 128) build, timed separately;
 *  - the LoRA side products and the standalone dequantisation (HBM-bound):
 *    bytes each must move once (operands read, outputs written; for a split
 *    launch the float32 partials written and read back are counted too, and
 *    the time spans both of its kernels).
 * ql_profile_enable(1) starts a fresh record and reserves a pool of events
 * (reused across records, so timed launches create none), ql_profile_enable(0)
 * stops recording. ql_profile_read waits for the recorded events and returns,
 * for one kernel id, the number of launches, their summed duration (ms) and
 * summed work. Results are unaffected by profiling. The events belong to the
 * device current at ql_profile_enable(1). Not thread-safe against concurrent
 * calls on other threads. */
enum {
  QL_KERNEL_GEMM_FWD = 0,        /* forward, wide tiles (FLOP) */
  QL_KERNEL_GEMM_BWD = 1,        /* dX, wide tiles (FLOP) */
  QL_KERNEL_GEMM_FWD_NARROW = 2, /* forward, narrow tiles (FLOP) */
  QL_KERNEL_GEMM_BWD_NARROW = 3, /* dX, narrow tiles (FLOP) */
  QL_KERNEL_LORA_ROW = 4,        /* U = x A^T, G = dY B, with a fused SwiGLU when asked (bytes) */
  QL_KERNEL_LORA_COL = 5,        /* dA = s G^T x, dB = s dY^T U (bytes) */
  QL_KERNEL_DEQUANT = 6,         /* nf4_dequant (bytes) */
  QL_KERNEL_COUNT = 7
};
ql_status ql_profile_enable(int32_t on);
ql_status ql_profile_read(int32_t kernel, int64_t* launches, double* ms, double* work);

/* Race check for the streamer (test use). The pages' evidence for streaming
 * is that a streamed run equals a normal one bit for bit, checked in a
 * notebook that caps the process's memory (Soup README intro). A read of a
 * slot before its copy has landed would usually see the previous layer's
 * bytes: wrong, but finite and easy to miss. With on = 1, every streamed call
 * fills a slot with 0xFF bytes on the copy stream right before each copy
 * into it (NaN scales, code 15), so such a read turns the outputs into NaN.
 * Results of correct runs are unchanged. Refused (QL_ERR_UNSUPPORTED) by
 * stream_layer_stack_step_capture while on. Process-wide; not thread-safe
 * against concurrent streamed calls. */
ql_status ql_debug_poison_slots(int32_t on);

#ifdef __cplusplus
}
#endif

#endif /* NF4QLORA_H */
