// C ABI: argument validation, the NF4 + LoRA linear, and the layer streamer.
// Every entry point validates all arguments before it enqueues anything.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "ql_internal.h"

namespace ql {

static thread_local char g_err[512];

ql_status set_error(ql_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

static void clear_error() { g_err[0] = 0; }

static inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ------------------------------------------------------------ small helpers
static ql_status check_ptr(const char* fn, const char* name, const void* p, size_t align) {
  if (!p) return set_error(QL_ERR_ARG, "%s: %s is NULL", fn, name);
  if (!aligned(p, align))
    return set_error(QL_ERR_ALIGN, "%s: %s (%p) must be %zu-byte aligned", fn, name, p, align);
  return QL_OK;
}

static ql_status check_weight(const char* fn, const ql_nf4_weight& W) {
  if (W.N <= 0 || W.K <= 0) return set_error(QL_ERR_SHAPE, "%s: W.N (%lld) and W.K (%lld) must be > 0", fn,
                                             (long long)W.N, (long long)W.K);
  if (W.K % 64) return set_error(QL_ERR_SHAPE, "%s: W.K (%lld) must be a multiple of 64 (NF4 block)", fn,
                                 (long long)W.K);
  if (W.N % 16) return set_error(QL_ERR_SHAPE, "%s: W.N (%lld) must be a multiple of 16", fn, (long long)W.N);
  if (W.N > QL_MAX_DIM || W.K > QL_MAX_DIM)
    return set_error(QL_ERR_SHAPE, "%s: W.N (%lld) and W.K (%lld) must be <= QL_MAX_DIM (%d)", fn, (long long)W.N,
                     (long long)W.K, QL_MAX_DIM);
  QL_TRY(check_ptr(fn, "W.packed", W.packed, 16));
  QL_TRY(check_ptr(fn, "W.absmax", W.absmax, 16));
  return QL_OK;
}

static ql_status check_lora(const char* fn, const ql_lora& L) {
  if (L.r < 1 || L.r > 64)
    return set_error(QL_ERR_RANK, "%s: LoRA rank r (%d) must be in 1..64", fn, (int)L.r);
  if (!(L.alpha == L.alpha) || L.alpha == __builtin_inff() || L.alpha == -__builtin_inff())
    return set_error(QL_ERR_ARG, "%s: LoRA alpha must be finite", fn);
  QL_TRY(check_ptr(fn, "L.A", L.A, 16));
  QL_TRY(check_ptr(fn, "L.B", L.B, 16));
  return QL_OK;
}

// nf4_quantize's finiteness check runs on the device's flag word one call at
// a time (host threads take turns), so concurrent calls never share it
static std::mutex g_quant_mu;

// --------------------------------------------------------- linear helpers
struct LinearWs {
  size_t fwd, bwd;
  size_t fpartial_off, bt_off, g_off, scratch_off, partial_off;
};

static LinearWs linear_ws(int64_t M, int64_t N, int64_t K, int32_t r) {
  LinearWs w;
  w.fpartial_off = align256(rowc_ws_bytes(M, K, r));
  w.fwd = w.fpartial_off + align256(bwd_partial_bytes(M, N));
  w.bt_off = 0;
  w.g_off = align256((size_t)r * N * 2);
  w.scratch_off = w.g_off + align256((size_t)M * r * 2);
  size_t scratch = rowc_ws_bytes(M, N, r);
  const size_t c = colc_ws_bytes(M, N, r) + colc_ws_bytes(M, K, r);  // dB and dA in one launch
  if (c > scratch) scratch = c;
  w.partial_off = w.scratch_off + align256(scratch);
  w.bwd = w.partial_off + align256(bwd_partial_bytes(M, K));
  return w;
}

// ---------------------------------------------------------- stack layout
// A layer record holds four weight groups, in the order the forward reads
// them: q|k|v, o, gate|up, down; each group's codes, then its scales. A group
// is one contiguous range, so it can be copied on its own.
constexpr int kGroups = 4;
constexpr int kGroupOf[QL_NPROJ] = {0, 0, 0, 1, 2, 2, 3};
struct StackLayout {
  int64_t N[QL_NPROJ], K[QL_NPROJ];
  int64_t packed_off[QL_NPROJ], absmax_off[QL_NPROJ];
  int64_t grp_off[kGroups + 1];  // group g spans [grp_off[g], grp_off[g + 1])
  int64_t rec;                   // bytes per layer record (multiple of 256)
};

static ql_status check_cfg(const char* fn, const ql_stack_cfg* c) {
  if (!c) return set_error(QL_ERR_ARG, "%s: cfg is NULL", fn);
  if (c->n_layers < 1) return set_error(QL_ERR_SHAPE, "%s: n_layers (%d) must be >= 1", fn, c->n_layers);
  if (c->hidden < 64 || c->hidden % 64 || c->hidden > QL_MAX_DIM)
    return set_error(QL_ERR_SHAPE, "%s: hidden (%d) must be a positive multiple of 64, at most QL_MAX_DIM (%d)", fn,
                     c->hidden, QL_MAX_DIM);
  if (c->inter < 64 || c->inter % 64 || c->inter > QL_MAX_DIM)
    return set_error(QL_ERR_SHAPE, "%s: inter (%d) must be a positive multiple of 64, at most QL_MAX_DIM (%d)", fn,
                     c->inter, QL_MAX_DIM);
  if (c->head_dim < 64 || c->head_dim % 64)
    return set_error(QL_ERR_SHAPE, "%s: head_dim (%d) must be a positive multiple of 64", fn, c->head_dim);
  if (c->kv_dim < c->head_dim || c->kv_dim % c->head_dim || c->hidden % c->kv_dim)
    return set_error(QL_ERR_SHAPE,
                     "%s: kv_dim (%d) must be a multiple of head_dim (%d) that divides hidden (%d)", fn,
                     c->kv_dim, c->head_dim, c->hidden);
  if (c->r < 1 || c->r > 64) return set_error(QL_ERR_RANK, "%s: r (%d) must be in 1..64", fn, c->r);
  if (c->n_buffers < 2 || c->n_buffers > QL_MAX_BUFFERS)
    return set_error(QL_ERR_UNSUPPORTED, "%s: n_buffers (%d) must be in 2..%d", fn, c->n_buffers, QL_MAX_BUFFERS);
  if (c->resident != 0 && c->resident != 1)
    return set_error(QL_ERR_ARG, "%s: resident (%d) must be 0 or 1", fn, c->resident);
  if (c->recompute != 0 && c->recompute != 1)
    return set_error(QL_ERR_ARG, "%s: recompute (%d) must be 0 or 1", fn, c->recompute);
  if (c->absmax_dq != 0 && c->absmax_dq != 1)
    return set_error(QL_ERR_ARG, "%s: absmax_dq (%d) must be 0 or 1", fn, c->absmax_dq);
  if (!(c->rms_eps > 0.f) || !(c->alpha == c->alpha))
    return set_error(QL_ERR_ARG, "%s: rms_eps must be > 0 and alpha finite", fn);
  return QL_OK;
}

static StackLayout stack_layout(const ql_stack_cfg* c) {
  StackLayout s;
  const int64_t H = c->hidden, I = c->inter, KV = c->kv_dim;
  const int64_t n[QL_NPROJ] = {H, KV, KV, H, I, I, H};
  const int64_t k[QL_NPROJ] = {H, H, H, H, H, H, I};
  size_t off = 0;
  for (int g = 0; g < kGroups; ++g) {
    s.grp_off[g] = (int64_t)off;
    for (int p = 0; p < QL_NPROJ; ++p) {
      if (kGroupOf[p] != g) continue;
      s.N[p] = n[p];
      s.K[p] = k[p];
      s.packed_off[p] = (int64_t)off;
      off += align256((size_t)(n[p] * k[p] / 2));
    }
    // float32 absmax per 64 weights, or its double-quantised block
    for (int p = 0; p < QL_NPROJ; ++p) {
      if (kGroupOf[p] != g) continue;
      s.absmax_off[p] = (int64_t)off;
      const int64_t nb = n[p] * (k[p] / 64);
      off += c->absmax_dq ? dq_layout(nb).bytes : align256((size_t)(nb * 4));
    }
  }
  s.grp_off[kGroups] = (int64_t)off;
  s.rec = (int64_t)align256(off);
  return s;
}

struct SavedLayout {
  int64_t off[QL_SAVED_COUNT];
  size_t per_layer;
};

// Every activation of one layer (what the backward reads).
static SavedLayout full_layout(const ql_stack_cfg* c, int64_t M) {
  SavedLayout s;
  const int64_t H = c->hidden, I = c->inter, KV = c->kv_dim, r = c->r;
  const int64_t cols[QL_SAVED_COUNT] = {H, H, H, KV, KV, H, H, I, I, I, r, r, r, r, r, r, r};
  size_t off = 0;
  for (int i = 0; i < QL_SAVED_COUNT; ++i) {
    s.off[i] = (int64_t)off;
    off += align256((size_t)(M * cols[i] * 2));
  }
  s.per_layer = off;
  return s;
}

// What the forward keeps per layer: every activation, or with recompute only
// the layer input h_in (the other offsets are -1).
static SavedLayout saved_layout(const ql_stack_cfg* c, int64_t M) {
  if (!c->recompute) return full_layout(c, M);
  SavedLayout s;
  for (int i = 0; i < QL_SAVED_COUNT; ++i) s.off[i] = -1;
  s.off[QL_SAVED_H_IN] = 0;
  s.per_layer = align256((size_t)(M * c->hidden * 2));
  return s;
}

// internal temporaries of the stack (offsets into ws); with recompute also one
// layer of activations (ck, full layout) and the recomputed layer output
struct StackWs {
  size_t dhA, dhB, dhmid, dact, dg, du, dn, da32, dv, bt, G[5], scratch, scratch_bytes, ck, ck_out, partial,
      partial_bytes;
  size_t absx[QL_NPROJ];  // absmax_dq: the layer's expanded float32 scales
  size_t total;
};

static StackWs stack_ws(const ql_stack_cfg* c, int64_t M) {
  const int64_t H = c->hidden, I = c->inter, KV = c->kv_dim, r = c->r;
  StackWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  w.dhA = take(M * H * 2);
  w.dhB = take(M * H * 2);
  w.dhmid = take(M * H * 2);
  w.dact = take(M * I * 2);
  w.dg = take(M * I * 2);
  w.du = take(M * I * 2);
  w.dn = take(M * H * 2);
  w.da32 = take(M * H * 4);
  w.dv = take(M * KV * 2);
  // transposed B of down, gate, up, o, v (in that order)
  w.bt = take((size_t)r * (H + I + I + H + KV) * 2 + 5 * 256);
  for (int i = 0; i < 5; ++i) w.G[i] = take((size_t)M * r * 2);
  size_t sc = 0;
  auto mx = [&](size_t v) { if (v > sc) sc = v; };
  mx(rowc_ws_bytes(M, H, 3 * r));                            // U of q | k | v
  mx(rowc_ws_bytes(M, H, 2 * r));                            // U of gate | up
  mx(rowc_ws_bytes(M, I, r));                                // U of down
  mx(rowc_ws_bytes(M, H, r));                                // U of o; G of down, o
  mx(2 * rowc_ws_bytes(M, I, r));                            // G of gate and up
  mx(rowc_ws_bytes(M, KV, r));                               // G of v
  mx(colc_ws_bytes(M, H, r) * 5 + colc_ws_bytes(M, I, r) * 3 + colc_ws_bytes(M, H, 2 * r) +
     colc_ws_bytes(M, KV, r));                               // all adapter gradients of a layer
  w.scratch = take(sc);
  w.scratch_bytes = sc;
  // float32 partials of the split dX GEMMs (outputs of I or H columns)
  w.partial_bytes = bwd_partial_bytes(M, I) > bwd_partial_bytes(M, H) ? bwd_partial_bytes(M, I)
                                                                      : bwd_partial_bytes(M, H);
  w.partial = take(w.partial_bytes);
  for (int p = 0; p < QL_NPROJ; ++p) w.absx[p] = 0;
  if (c->absmax_dq) {
    const int64_t n[QL_NPROJ] = {H, KV, KV, H, I, I, H};
    const int64_t k[QL_NPROJ] = {H, H, H, H, H, H, I};
    for (int p = 0; p < QL_NPROJ; ++p) w.absx[p] = take((size_t)(n[p] * (k[p] / 64) * 4));
  }
  w.ck = w.ck_out = 0;
  if (c->recompute) {
    w.ck = take(full_layout(c, M).per_layer);
    w.ck_out = take((size_t)(M * H * 2));
  }
  w.total = off;
  return w;
}

// -------------------------------------------------------------- one layer
struct LayerW {
  const uint8_t* packed[QL_NPROJ];
  const float* absmax[QL_NPROJ];
};

static LayerW layer_weights(const StackLayout& L, const uint8_t* base) {
  LayerW w;
  for (int p = 0; p < QL_NPROJ; ++p) {
    w.packed[p] = base + L.packed_off[p];
    w.absmax[p] = (const float*)(base + L.absmax_off[p]);
  }
  return w;
}

// Expansion of double-quantised scales into the workspace's float32 area for
// the projections p with group_of[p] == g (g < 0: all seven).
static DqExpandArgs dq_expand_args(const StackLayout& L, const StackWs& WS, const uint8_t* base, uint8_t* ws,
                                   int g) {
  DqExpandArgs a{};
  int64_t cum = 0;
  for (int p = 0; p < QL_NPROJ; ++p) {
    if (g >= 0 && kGroupOf[p] != g) continue;
    const int64_t nb = L.N[p] * (L.K[p] / 64);
    const DqLayout dl = dq_layout(nb);
    const int i = a.nblk++;
    a.src[i] = base + L.absmax_off[p];
    a.scale_off[i] = dl.scale_off;
    a.mean_off[i] = dl.mean_off;
    a.dst[i] = (float*)(ws + WS.absx[p]);
    cum += nb;
    a.end[i] = cum;
  }
  return a;
}

// The layer's weights in a slot (or the resident store). With double-quantised
// scales the GEMMs read float32 scales from the workspace: all seven blocks
// are expanded there in one launch once the layer's record has landed, or,
// with by_group, group by group as each group lands (group_wait).
static ql_status layer_weights_ready(const ql_stack_cfg* c, const StackLayout& L, const StackWs& WS,
                                     const uint8_t* base, uint8_t* ws, hipStream_t st, LayerW& W,
                                     bool by_group = false) {
  W = layer_weights(L, base);
  if (!c->absmax_dq) return QL_OK;
  for (int p = 0; p < QL_NPROJ; ++p) W.absmax[p] = (const float*)(ws + WS.absx[p]);
  return by_group ? QL_OK : launch_dq_expand(dq_expand_args(L, WS, base, ws, -1), st);
}

// Hand-offs with the copy streams inside a layer (only the GEMMs read the
// slot). With wait, the record lands one weight group at a time: before the
// GEMM that reads group g the compute stream waits for ready[g], then
// expands the group's double-quantised scales (dq[g].nblk > 0). With early,
// the event is recorded after the GEMM of group early_after, the layer's last
// reader of that group, so that a refill can start on it before the layer
// ends. Null: the caller handles the whole record.
struct GroupReady {
  bool wait = false;
  hipEvent_t ready[kGroups] = {};
  DqExpandArgs dq[kGroups] = {};
  hipEvent_t early = nullptr;
  int early_after = -1;
};
static ql_status group_wait(const GroupReady* gr, int g, hipStream_t C) {
  if (!gr || !gr->wait) return QL_OK;
  QL_HIP_CHECK(hipStreamWaitEvent(C, gr->ready[g], 0));
  if (gr->dq[g].nblk > 0) QL_TRY(launch_dq_expand(gr->dq[g], C));
  return QL_OK;
}
static ql_status group_done(const GroupReady* gr, int g, hipStream_t C) {
  if (gr && gr->early && gr->early_after == g) QL_HIP_CHECK(hipEventRecord(gr->early, C));
  return QL_OK;
}

static inline const uint16_t* u16(const void* p) { return (const uint16_t*)p; }
static inline uint16_t* u16w(void* p) { return (uint16_t*)p; }

// One layer's forward. lo == nullptr: the adapters are off (the base model,
// x W^T only): no LoRA-down launches and no LoRA step in the GEMMs; the U
// entries of sv are left untouched.
static ql_status layer_fwd(const ql_stack_cfg* c, const StackLayout& SL, const LayerW& W,
                           const ql_lora* lo, int64_t M, const SavedLayout& SV, uint8_t* sv,
                           uint16_t* h_out, uint8_t* ws, const StackWs& WS, hipStream_t st,
                           const GroupReady* gr = nullptr) {
  const int64_t H = c->hidden, I = c->inter, KV = c->kv_dim;
  const bool on = lo != nullptr;
  const int r = on ? c->r : 0;
  const float s = on ? c->alpha / (float)c->r : 0.f;
  auto S = [&](int i) { return (uint16_t*)(sv + SV.off[i]); };
  void* scratch = ws + WS.scratch;
  const uint16_t* h_in = S(QL_SAVED_H_IN);
  // n = RMSNorm(h) and the LoRA down of the nseg projections that read n
  // (first at p0): one launch that makes n as it contracts it when their
  // columns fit one, else the standalone RMSNorm and a plain row launch
  auto norm_down = [&](const uint16_t* h, int n_slot, int p0, int nseg) -> ql_status {
    if (!on) return launch_rmsnorm_fwd(h, M, H, c->rms_eps, S(n_slot), st);
    const bool fuse = r * nseg <= 64 && rowc_ws_bytes(M, H, r * nseg) == 0;
    if (!fuse) QL_TRY(launch_rmsnorm_fwd(h, M, H, c->rms_eps, S(n_slot), st));
    RowArgs ra{};
    ra.nprob = 1;
    ra.mode = fuse ? 3 : 0;
    RowProb& a = ra.p[0];
    a.X = fuse ? h : S(n_slot); a.M = M; a.K = H; a.ldx = H; a.r = r; a.nseg = nseg;
    a.Xout[0] = fuse ? S(n_slot) : nullptr; a.eps = c->rms_eps;
    for (int p = 0; p < nseg; ++p) { a.Bt[p] = u16(lo[p0 + p].A); a.out[p] = S(QL_SAVED_U0 + p0 + p); }
    return launch_rowc(ra, scratch, WS.scratch_bytes, st);
  };

  QL_TRY(norm_down(h_in, QL_SAVED_N1, QL_PROJ_Q, 3));  // q, k, v share n1
  {  // q | k | v in one launch
    FwdArgs a{};
    a.X = S(QL_SAVED_N1); a.M = M; a.K = H; a.ldx = H; a.r = r; a.s = s; a.nseg = 3;
    a.partial = (float*)(ws + WS.partial);
    a.partial_bytes = WS.partial_bytes;
    const int outs[3] = {QL_SAVED_Q, QL_SAVED_K, QL_SAVED_V};
    for (int p = 0; p < 3; ++p) {
      FwdSeg& g = a.seg[p];
      g.packed = W.packed[p]; g.absmax = W.absmax[p];
      g.U = on ? S(QL_SAVED_U0 + p) : nullptr; g.B = on ? u16(lo[p].B) : nullptr;
      g.out = S(outs[p]); g.N = SL.N[p]; g.ldo = SL.N[p]; g.col0 = 0; g.resid = nullptr;
    }
    QL_TRY(group_wait(gr, 0, st));
    QL_TRY(launch_gemm_fwd(a, st));
    QL_TRY(group_done(gr, 0, st));
  }
  const int n_rep = (int)(H / KV);
  {  // o: input a = repeat_kv(v) read through the column remap; residual h_in
    if (on) {
      RowArgs ra{};
      ra.nprob = 1;
      RowProb& u = ra.p[0];
      u.X = S(QL_SAVED_V); u.M = M; u.K = H; u.ldx = KV; u.head_dim = c->head_dim; u.n_rep = n_rep;
      u.r = r; u.nseg = 1; u.Bt[0] = u16(lo[QL_PROJ_O].A); u.out[0] = S(QL_SAVED_U0 + QL_PROJ_O);
      QL_TRY(launch_rowc(ra, scratch, WS.scratch_bytes, st));
    }
    FwdArgs a{};
    a.X = S(QL_SAVED_V); a.M = M; a.K = H; a.ldx = KV; a.head_dim = c->head_dim; a.n_rep = n_rep;
    a.r = r; a.s = s; a.nseg = 1;
    a.partial = (float*)(ws + WS.partial);
    a.partial_bytes = WS.partial_bytes;
    FwdSeg& g = a.seg[0];
    g.packed = W.packed[QL_PROJ_O]; g.absmax = W.absmax[QL_PROJ_O];
    g.U = on ? S(QL_SAVED_U0 + QL_PROJ_O) : nullptr; g.B = on ? u16(lo[QL_PROJ_O].B) : nullptr;
    g.out = S(QL_SAVED_H_MID); g.N = H; g.ldo = H; g.resid = h_in;
    QL_TRY(group_wait(gr, 1, st));
    QL_TRY(launch_gemm_fwd(a, st));
    QL_TRY(group_done(gr, 1, st));
  }
  QL_TRY(norm_down(S(QL_SAVED_H_MID), QL_SAVED_N2, QL_PROJ_GATE, 2));  // gate, up share n2
  {  // gate | up
    FwdArgs a{};
    a.X = S(QL_SAVED_N2); a.M = M; a.K = H; a.ldx = H; a.r = r; a.s = s; a.nseg = 2;
    const int outs[2] = {QL_SAVED_GATE, QL_SAVED_UP};
    for (int q = 0; q < 2; ++q) {
      const int p = QL_PROJ_GATE + q;
      FwdSeg& g = a.seg[q];
      g.packed = W.packed[p]; g.absmax = W.absmax[p];
      g.U = on ? S(QL_SAVED_U0 + p) : nullptr; g.B = on ? u16(lo[p].B) : nullptr;
      g.out = S(outs[q]); g.N = I; g.ldo = I; g.resid = nullptr;
    }
    QL_TRY(group_wait(gr, 2, st));
    QL_TRY(launch_gemm_fwd(a, st));
    QL_TRY(group_done(gr, 2, st));
  }
  {  // down, residual h_mid
    if (on) {  // act = SwiGLU(gate, up) and U of down in one pass
      RowArgs ra{};
      ra.nprob = 1;
      ra.mode = 1;
      RowProb& u = ra.p[0];
      u.Xin[0] = S(QL_SAVED_GATE); u.Xin[1] = S(QL_SAVED_UP); u.Xout[0] = S(QL_SAVED_ACT);
      u.M = M; u.K = I; u.ldx = I; u.r = r; u.nseg = 1;
      u.Bt[0] = u16(lo[QL_PROJ_DOWN].A); u.out[0] = S(QL_SAVED_U0 + QL_PROJ_DOWN);
      QL_TRY(launch_rowc(ra, scratch, WS.scratch_bytes, st));
    } else {
      QL_TRY(launch_swiglu_fwd(S(QL_SAVED_GATE), S(QL_SAVED_UP), M * I, S(QL_SAVED_ACT), st));
    }
    FwdArgs a{};
    a.X = S(QL_SAVED_ACT); a.M = M; a.K = I; a.ldx = I; a.r = r; a.s = s; a.nseg = 1;
    FwdSeg& g = a.seg[0];
    g.packed = W.packed[QL_PROJ_DOWN]; g.absmax = W.absmax[QL_PROJ_DOWN];
    g.U = on ? S(QL_SAVED_U0 + QL_PROJ_DOWN) : nullptr; g.B = on ? u16(lo[QL_PROJ_DOWN].B) : nullptr;
    g.out = h_out; g.N = H; g.ldo = H; g.resid = S(QL_SAVED_H_MID);
    a.partial = (float*)(ws + WS.partial);
    a.partial_bytes = WS.partial_bytes;
    QL_TRY(group_wait(gr, 3, st));
    QL_TRY(launch_gemm_fwd(a, st));
    QL_TRY(group_done(gr, 3, st));
  }
  return QL_OK;
}

// One row-contraction problem: G = bf16(dY Bt^T) (Bt: B transposed, [r x N])
static RowProb g_prob(const uint16_t* dy, int64_t M, int64_t N, int r, const uint16_t* bt, uint16_t* G) {
  RowProb a{};
  a.X = dy; a.M = M; a.K = N; a.ldx = N; a.r = r; a.nseg = 1; a.Bt[0] = bt; a.out[0] = G;
  return a;
}

// Column-contraction problems of one projection: dB = s dY^T U, stored
// transposed into [N x r], and dA = s G^T X (X columns remapped by repeat_kv
// when n_rep > 0)
static ColProb db_prob(const uint16_t* dy, int64_t M, int64_t N, const uint16_t* U, int r, float s, float* dB,
                       int accumulate) {
  ColProb b{};
  b.Z = dy; b.M = M; b.C = N; b.ldz = N; b.r = r; b.nseg = 1; b.V[0] = U; b.out[0] = dB; b.s = s;
  b.transpose_out = 1; b.accumulate = accumulate;
  return b;
}
static ColProb da_prob(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, int head_dim, int n_rep,
                       const uint16_t* G, int r, float s, float* dA, int accumulate) {
  ColProb a{};
  a.Z = X; a.M = M; a.C = K; a.ldz = ldx; a.head_dim = head_dim; a.n_rep = n_rep; a.r = r; a.nseg = 1;
  a.V[0] = G; a.out[0] = dA; a.s = s; a.transpose_out = 0; a.accumulate = accumulate;
  return a;
}
// zero output of a gradient that is exactly zero ([rows x cols] float32)
static ColProb zero_prob(float* out, int64_t n, int r) {
  ColProb z{};
  z.M = 0; z.C = n / r; z.r = r; z.nseg = 1; z.out[0] = out; z.accumulate = 0;
  return z;
}

static ql_status layer_bwd(const ql_stack_cfg* c, const StackLayout& SL, const LayerW& W,
                           const ql_lora* lo, int64_t M, const SavedLayout& SV, const uint8_t* sv,
                           const uint16_t* dh, uint16_t* dh_out, float* const* dA, float* const* dB,
                           int accumulate, uint8_t* ws, const StackWs& WS, hipStream_t st,
                           const GroupReady* gr = nullptr) {
  const int64_t H = c->hidden, I = c->inter, KV = c->kv_dim;
  const int r = c->r;
  const float s = c->alpha / (float)r;
  auto S = [&](int i) { return (const uint16_t*)(sv + SV.off[i]); };
  auto T = [&](size_t off) { return (uint16_t*)(ws + off); };
  void* scratch = ws + WS.scratch;
  const int n_rep = (int)(H / KV);

  // B of down, gate, up, o, v transposed to [r x N] in one launch
  const int tp[5] = {QL_PROJ_DOWN, QL_PROJ_GATE, QL_PROJ_UP, QL_PROJ_O, QL_PROJ_V};
  uint16_t* bt[5];
  {
    TransArgs ta{};
    ta.n = 5;
    size_t off = WS.bt;
    for (int i = 0; i < 5; ++i) {
      const int64_t N = SL.N[tp[i]];
      bt[i] = T(off);
      off += align256((size_t)r * N * 2);
      ta.in[i] = u16(lo[tp[i]].B); ta.out[i] = bt[i]; ta.rows[i] = N; ta.cols[i] = r;
    }
    QL_TRY(launch_transpose_bf16(ta, st));
  }
  auto row1 = [&](const RowProb& p) {
    RowArgs ra{};
    ra.nprob = 1;
    ra.p[0] = p;
    return launch_rowc(ra, scratch, WS.scratch_bytes, st);
  };
  // the adapter gradients of the layer, one launch at the end
  ColArgs grads{};
  auto add = [&](const ColProb& p) { grads.p[grads.nprob++] = p; };

  // down: dact = dh W_d + s G_d A_d
  uint16_t* Gd = T(WS.G[0]);
  QL_TRY(row1(g_prob(dh, M, H, r, bt[0], Gd)));
  {
    BwdArgs a{};
    a.M = M; a.K = I; a.r = r; a.s = s; a.out = T(WS.dact); a.nseg = 1;
    a.seg[0] = BwdSeg{dh, W.packed[QL_PROJ_DOWN], W.absmax[QL_PROJ_DOWN], Gd, u16(lo[QL_PROJ_DOWN].A), H};
    a.partial = (float*)(ws + WS.partial); a.partial_bytes = WS.partial_bytes;
    QL_TRY(group_wait(gr, 3, st));
    QL_TRY(launch_gemm_bwd(a, st));
    QL_TRY(group_done(gr, 3, st));
  }
  add(db_prob(dh, M, H, S(QL_SAVED_U0 + QL_PROJ_DOWN), r, s, dB[QL_PROJ_DOWN], accumulate));
  add(da_prob(S(QL_SAVED_ACT), M, I, I, 0, 0, Gd, r, s, dA[QL_PROJ_DOWN], accumulate));
  // SwiGLU backward and G of gate and up: one pass when the rank allows
  uint16_t* Gg = T(WS.G[1]);
  uint16_t* Gu = T(WS.G[2]);
  if (r <= kSwigluBwdMaxR) {
    RowArgs ra{};
    ra.nprob = 1;
    ra.mode = 2;
    RowProb& q = ra.p[0];
    q.Xin[0] = S(QL_SAVED_GATE); q.Xin[1] = S(QL_SAVED_UP); q.Xin[2] = T(WS.dact);
    q.Xout[0] = T(WS.dg); q.Xout[1] = T(WS.du);
    q.M = M; q.K = I; q.ldx = I; q.r = r; q.nseg = 2;
    q.Bt[0] = bt[1]; q.Bt[1] = bt[2]; q.out[0] = Gg; q.out[1] = Gu;
    QL_TRY(launch_rowc(ra, scratch, WS.scratch_bytes, st));
  } else {
    QL_TRY(launch_swiglu_bwd(S(QL_SAVED_GATE), S(QL_SAVED_UP), T(WS.dact), M * I, T(WS.dg), T(WS.du), st));
    RowArgs ra{};
    ra.nprob = 2;
    ra.p[0] = g_prob(T(WS.dg), M, I, r, bt[1], Gg);
    ra.p[1] = g_prob(T(WS.du), M, I, r, bt[2], Gu);
    QL_TRY(launch_rowc(ra, scratch, WS.scratch_bytes, st));
  }
  {
    BwdArgs a{};
    a.M = M; a.K = H; a.r = r; a.s = s; a.out = T(WS.dn); a.nseg = 2;
    a.seg[0] = BwdSeg{T(WS.dg), W.packed[QL_PROJ_GATE], W.absmax[QL_PROJ_GATE], Gg, u16(lo[QL_PROJ_GATE].A), I};
    a.seg[1] = BwdSeg{T(WS.du), W.packed[QL_PROJ_UP], W.absmax[QL_PROJ_UP], Gu, u16(lo[QL_PROJ_UP].A), I};
    a.partial = (float*)(ws + WS.partial); a.partial_bytes = WS.partial_bytes;
    QL_TRY(group_wait(gr, 2, st));
    QL_TRY(launch_gemm_bwd(a, st));
    QL_TRY(group_done(gr, 2, st));
  }
  add(db_prob(T(WS.dg), M, I, S(QL_SAVED_U0 + QL_PROJ_GATE), r, s, dB[QL_PROJ_GATE], accumulate));
  add(db_prob(T(WS.du), M, I, S(QL_SAVED_U0 + QL_PROJ_UP), r, s, dB[QL_PROJ_UP], accumulate));
  {  // dA of gate and up share n2: one pass over it
    ColProb a = da_prob(S(QL_SAVED_N2), M, H, H, 0, 0, Gg, r, s, dA[QL_PROJ_GATE], accumulate);
    a.nseg = 2; a.V[1] = Gu; a.out[1] = dA[QL_PROJ_UP];
    add(a);
  }
  // RMSNorm 2 + residual
  QL_TRY(launch_rmsnorm_bwd(S(QL_SAVED_H_MID), T(WS.dn), dh, M, H, c->rms_eps, T(WS.dhmid), st));
  const uint16_t* dhm = T(WS.dhmid);
  // o: da = dh_mid W_o + s G_o A_o (float32), dv = head-group sum
  uint16_t* Go = T(WS.G[3]);
  QL_TRY(row1(g_prob(dhm, M, H, r, bt[3], Go)));
  {
    BwdArgs a{};
    a.M = M; a.K = H; a.r = r; a.s = s; a.out = ws + WS.da32; a.out_f32 = 1; a.nseg = 1;
    a.seg[0] = BwdSeg{dhm, W.packed[QL_PROJ_O], W.absmax[QL_PROJ_O], Go, u16(lo[QL_PROJ_O].A), H};
    a.partial = (float*)(ws + WS.partial); a.partial_bytes = WS.partial_bytes;
    QL_TRY(group_wait(gr, 1, st));
    QL_TRY(launch_gemm_bwd(a, st));
    QL_TRY(group_done(gr, 1, st));
  }
  add(db_prob(dhm, M, H, S(QL_SAVED_U0 + QL_PROJ_O), r, s, dB[QL_PROJ_O], accumulate));
  add(da_prob(S(QL_SAVED_V), M, H, KV, c->head_dim, n_rep, Go, r, s, dA[QL_PROJ_O], accumulate));
  QL_TRY(launch_repeat_kv_bwd((const float*)(ws + WS.da32), M, H, KV, c->head_dim, T(WS.dv), st));
  // v: dn1 = dv W_v + s G_v A_v
  uint16_t* Gv = T(WS.G[4]);
  QL_TRY(row1(g_prob(T(WS.dv), M, KV, r, bt[4], Gv)));
  {
    BwdArgs a{};
    a.M = M; a.K = H; a.r = r; a.s = s; a.out = T(WS.dn); a.nseg = 1;
    a.seg[0] = BwdSeg{T(WS.dv), W.packed[QL_PROJ_V], W.absmax[QL_PROJ_V], Gv, u16(lo[QL_PROJ_V].A), KV};
    a.partial = (float*)(ws + WS.partial); a.partial_bytes = WS.partial_bytes;
    QL_TRY(group_wait(gr, 0, st));  // of q|k|v only v is read here
    QL_TRY(launch_gemm_bwd(a, st));
    QL_TRY(group_done(gr, 0, st));
  }
  add(db_prob(T(WS.dv), M, KV, S(QL_SAVED_U0 + QL_PROJ_V), r, s, dB[QL_PROJ_V], accumulate));
  add(da_prob(S(QL_SAVED_N1), M, H, H, 0, 0, Gv, r, s, dA[QL_PROJ_V], accumulate));
  // q, k feed nothing: their adapter gradients are exactly zero
  if (!accumulate) {
    for (int p = 0; p < 2; ++p) {
      add(zero_prob(dA[p], (int64_t)r * H, r));
      add(zero_prob(dB[p], SL.N[p] * r, r));
    }
  }
  QL_TRY(launch_colc(grads, scratch, WS.scratch_bytes, st));
  // RMSNorm 1 + residual
  QL_TRY(launch_rmsnorm_bwd(S(QL_SAVED_H_IN), T(WS.dn), dhm, M, H, c->rms_eps, dh_out, st));
  return QL_OK;
}

// ------------------------------------------------------------- the streamer
enum PtrKind { PK_DEVICE, PK_PINNED, PK_PAGEABLE };

static PtrKind pointer_kind(const void* p) {
  hipPointerAttribute_t at;
  memset(&at, 0, sizeof(at));
  hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return PK_PAGEABLE;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) return PK_DEVICE;
  if (at.type == hipMemoryTypeHost) return PK_PINNED;
  return PK_PAGEABLE;
}

// Race check (ql_debug_poison_slots): every slot is filled with 0xFF bytes
// on the copy stream right before a record is copied into it, after the
// slot's previous readers are done. A kernel that read a slot before its
// `ready` event would then meet NaN scales and codes 15 instead of a stale
// but plausible layer, and the outputs would show it.
static std::atomic<bool> g_poison{false};

// Host-to-device copy of a small page-locked record by the library's own
// kernel. The runtime's copy of a pinned buffer is itself a kernel whose grid
// grows with the bytes: a 2 MB record takes about 490 workgroups that hold
// every CU while their loads cross PCIe, so the compute kernels that start
// beside it (the next layer's first kernels) wait for it (SmolLM2-shaped
// stack: its first RMSNorm of each layer took 47 us instead of 4). This
// kernel keeps a fixed grid of 8 workgroups, each thread with 8 16-byte loads
// in flight, which keeps the link busy for such records. A large record's
// copy lasts milliseconds, and 8 workgroups held that long would keep 8 CUs
// from every GEMM launched meanwhile (8B-shaped stack: 136 -> 155 ms per
// step), so records of kSmallCopy bytes or more take the runtime's copy,
// whose many short workgroups interleave with the GEMMs. Records are
// multiples of 256 bytes.
constexpr int kCopyWGs = 8, kCopyInflight = 8;
constexpr size_t kSmallCopy = 8u << 20;
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_h2d(const u32x4v* __restrict__ src, u32x4v* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (kCopyInflight - 1) * stride < n; i += kCopyInflight * stride) {
    u32x4v v[kCopyInflight];
#pragma unroll
    for (int k = 0; k < kCopyInflight; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kCopyInflight; ++k) dst[i + k * stride] = v[k];
  }
  for (; i < n; i += stride) dst[i] = __builtin_nontemporal_load(src + i);
}

// One layer record host -> device on the copy stream (a pageable store always
// goes through the runtime's copy, which stages it).
static ql_status copy_record(void* dst, const void* src, size_t bytes, hipStream_t P, bool pinned) {
  if (g_poison.load()) QL_HIP_CHECK(hipMemsetAsync(dst, 0xFF, bytes, P));
  if (pinned && bytes < kSmallCopy) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    QL_HIP_CHECK(hipStreamIsCapturing(P, &cap));
    if (cap == hipStreamCaptureStatusActive) {
      // In a captured step the record becomes a copy node that the DMA
      // engines run without compute units (the page-locked store is mapped
      // into the device's address space). The SmolLM2-shaped step replays in
      // 9.1 ms against 10.2 with the copy kernel; issued eagerly, such copies
      // cost more than the kernel (10.7 against 10.2 ms per step).
      QL_HIP_CHECK(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDeviceNoCU, P));
    } else {
      hipLaunchKernelGGL(k_h2d, dim3(kCopyWGs), dim3(256), 0, P, (const u32x4v*)src, (u32x4v*)dst,
                         (int64_t)(bytes / 16));
      QL_HIP_CHECK(hipGetLastError());
    }
  } else {
    QL_HIP_CHECK(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, P));
  }
  return QL_OK;
}

// A layer record into a slot one weight group at a time, groups in the order
// ord, each followed by its ready event.
static ql_status copy_groups(const StackLayout& SL, uint8_t* dst, const uint8_t* src, hipStream_t P, bool pinned,
                             const int (&ord)[kGroups], const hipEvent_t* ready_g) {
  for (int i = 0; i < kGroups; ++i) {
    const int g = ord[i];
    const size_t o = (size_t)SL.grp_off[g], n = (size_t)(SL.grp_off[g + 1] - SL.grp_off[g]);
    QL_TRY(copy_record(dst + o, src + o, n, P, pinned));
    QL_HIP_CHECK(hipEventRecord(ready_g[g], P));
  }
  return QL_OK;
}
constexpr int kFwdOrder[kGroups] = {0, 1, 2, 3}, kBwdOrder[kGroups] = {3, 2, 1, 0};

// The library's side copy stream on the current device (default priority,
// created on first use, kept for the process). It carries the part of a
// pass's first refill that starts before the slot's layer has finished, so
// that the copy stream itself never waits between copies on an event
// recorded in the middle of a layer: with such waits on the copy stream the
// 8B-shaped step took 139-150 ms instead of 133; with the side stream it
// takes 132.2 against 133.2 ms (Qwen2.5-3B-shaped: 53.75 against 54.0 ms).
// Only two-slot rings take it: with 3 or 8 slots it measured 2-2.5 ms slower.
static ql_status side_stream(hipStream_t* out) {
  static std::mutex mu;
  static hipStream_t streams[64] = {};
  int dev = 0;
  QL_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return set_error(QL_ERR_UNSUPPORTED, "device ordinal %d", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!streams[dev]) QL_HIP_CHECK(hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking));
  *out = streams[dev];
  return QL_OK;
}

struct Events {
  hipEvent_t ready[QL_MAX_BUFFERS] = {}, free_[QL_MAX_BUFFERS] = {}, entry = nullptr;
  hipEvent_t gready[QL_MAX_BUFFERS][kGroups] = {};  // per weight group
  hipEvent_t early = nullptr, side = nullptr;        // a pass's early refill part
  int n = 0;
  ~Events() {
    for (int i = 0; i < n; ++i) {
      if (ready[i]) (void)hipEventDestroy(ready[i]);
      if (free_[i]) (void)hipEventDestroy(free_[i]);
      for (int g = 0; g < kGroups; ++g)
        if (gready[i][g]) (void)hipEventDestroy(gready[i][g]);
    }
    if (entry) (void)hipEventDestroy(entry);
    if (early) (void)hipEventDestroy(early);
    if (side) (void)hipEventDestroy(side);
  }
  // `ready` (copy -> compute) keeps the default system-scope fence: the
  // compute stream must observe bytes the copy engine wrote. `free_` and
  // `entry` (compute -> copy) only order the copy engine's writes after the
  // kernels' reads of a slot, so they skip it; with the fence, every layer
  // boundary would also write back the L2's dirty lines.
  ql_status create(int nbuf, bool groups) {
    n = nbuf;
    for (int i = 0; i < n; ++i) {
      QL_HIP_CHECK(hipEventCreateWithFlags(&ready[i], hipEventDisableTiming));
      QL_HIP_CHECK(hipEventCreateWithFlags(&free_[i], hipEventDisableTiming | hipEventDisableSystemFence));
      for (int g = 0; g < kGroups && groups; ++g)
        QL_HIP_CHECK(hipEventCreateWithFlags(&gready[i][g], hipEventDisableTiming));
    }
    QL_HIP_CHECK(hipEventCreateWithFlags(&entry, hipEventDisableTiming | hipEventDisableSystemFence));
    if (groups) {
      QL_HIP_CHECK(hipEventCreateWithFlags(&early, hipEventDisableTiming | hipEventDisableSystemFence));
      QL_HIP_CHECK(hipEventCreateWithFlags(&side, hipEventDisableTiming));
    }
    return QL_OK;
  }
  // The slots may still be read by work enqueued earlier on the compute
  // stream (the previous streamed call): the copy stream waits for all of it
  // before this call's first copy.
  ql_status after_compute(hipStream_t C, hipStream_t P) {
    QL_HIP_CHECK(hipEventRecord(entry, C));
    QL_HIP_CHECK(hipStreamWaitEvent(P, entry, 0));
    return QL_OK;
  }
};

// Streamed calls in flight. Before it enqueues anything, an eager streamed
// call waits on the host until the previous streamed call of the same
// direction (forward or backward) has finished on the GPU, so at most one of
// each is queued on the device. With more queued, the copy engine's handoffs
// slow down (8B stack at M=2048, 10 steps queued back to back: 142-146 ms per
// step; one step in flight: 135 ms). A full queue also stalls the host in
// mid-call, between a layer's kernels and the copy enqueued after them. Calls
// recorded into a graph skip this, and so do stacks whose layer records are
// below kThrottleRecord: their copies are short, and keeping more calls queued
// hides the host's enqueue time of their launch-bound steps (SmolLM2-shaped
// stack, 2 MB records: 12.9 ms eager steps unthrottled, 13.3 throttled).
constexpr size_t kThrottleRecord = 8u << 20;

// Within such a call with two slots, the host also stays at most
// kLayersAhead layers ahead of the GPU: before it enqueues a layer it waits
// for the layer kLayersAhead back to finish. The Qwen2.5-3B-shaped stack (43
// MB records, short layers) steps in 54.0 ms against 58-59 unlimited; the
// 8B-shaped step is unchanged (133.1 against 133.2-133.8 ms). With deeper
// rings every limit measured slower (8 slots: 112-115 against 107 ms; 3
// slots: 131-133 against 129-130 ms), so they keep only the call-level wait.
constexpr int kLayersAhead = 2;
struct LayerAhead {
  bool on = false;
  hipEvent_t done[kLayersAhead] = {};
  ql_status init(bool enable) {
    on = enable;
    for (int i = 0; i < kLayersAhead && on; ++i)
      QL_HIP_CHECK(hipEventCreateWithFlags(&done[i], hipEventDisableTiming));
    return QL_OK;
  }
  // before enqueueing the pass's layer number idx (0, 1, ... in pass order)
  ql_status before(int idx) {
    if (on && idx >= kLayersAhead) QL_HIP_CHECK(hipEventSynchronize(done[idx % kLayersAhead]));
    return QL_OK;
  }
  // after enqueueing it (and its refill)
  ql_status after(int idx, hipStream_t C) {
    if (on) QL_HIP_CHECK(hipEventRecord(done[idx % kLayersAhead], C));
    return QL_OK;
  }
  ~LayerAhead() {
    for (int i = 0; i < kLayersAhead; ++i)
      if (done[i]) (void)hipEventDestroy(done[i]);
  }
};
struct InFlight {
  std::mutex mu;
  hipEvent_t done[64][2] = {};
};
static InFlight g_inflight;

static bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

// dir 0: forward, 1: backward
static ql_status inflight_wait(int dir) {
  int dev = 0;
  QL_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return QL_OK;
  hipEvent_t e;
  {
    std::lock_guard<std::mutex> lk(g_inflight.mu);
    e = g_inflight.done[dev][dir];
  }
  if (e) QL_HIP_CHECK(hipEventSynchronize(e));
  return QL_OK;
}

static ql_status inflight_mark(int dir, hipStream_t C) {
  int dev = 0;
  QL_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return QL_OK;
  std::lock_guard<std::mutex> lk(g_inflight.mu);
  hipEvent_t& e = g_inflight.done[dev][dir];
  if (!e) QL_HIP_CHECK(hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventBlockingSync));
  QL_HIP_CHECK(hipEventRecord(e, C));
  return QL_OK;
}

struct StackCall {
  StackLayout SL;
  SavedLayout SV, SVF;  // caller's saved layout; every activation of one layer
  StackWs WS;
  size_t store_need, slots_need, saved_need;
  bool pageable = false;
};

// policy == false: no adapters and no saved activations are used (the
// adapter-off forward alone); lora and saved are then not checked.
static ql_status validate_stack(const char* fn, const ql_stack_cfg* cfg, const void* store, size_t store_bytes,
                                const ql_lora* lora, int64_t M, const void* saved, size_t saved_bytes,
                                const void* slots, size_t slots_bytes, const void* ws, size_t ws_bytes,
                                StackCall& sc, bool policy = true) {
  QL_TRY(check_cfg(fn, cfg));
  if (M < 0) return set_error(QL_ERR_SHAPE, "%s: M (%lld) must be >= 0", fn, (long long)M);
  sc.SL = stack_layout(cfg);
  sc.SV = saved_layout(cfg, M);
  sc.SVF = full_layout(cfg, M);
  sc.WS = stack_ws(cfg, M);
  sc.store_need = (size_t)sc.SL.rec * cfg->n_layers;
  sc.slots_need = cfg->resident ? 0 : (size_t)sc.SL.rec * cfg->n_buffers;
  sc.saved_need = sc.SV.per_layer * cfg->n_layers;
  if (!store) return set_error(QL_ERR_ARG, "%s: store is NULL", fn);
  if (!aligned(store, 256)) return set_error(QL_ERR_ALIGN, "%s: store must be 256-byte aligned", fn);
  if (store_bytes < sc.store_need)
    return set_error(QL_ERR_WORKSPACE, "%s: store_bytes (%zu) < layout size (%zu)", fn, store_bytes,
                     sc.store_need);
  const PtrKind pk = pointer_kind(store);
  if (cfg->resident) {
    if (pk != PK_DEVICE) return set_error(QL_ERR_ARG, "%s: resident mode needs a device store", fn);
  } else {
    if (pk == PK_DEVICE) return set_error(QL_ERR_ARG, "%s: streamed mode needs a host store", fn);
    sc.pageable = pk == PK_PAGEABLE;
    if (!slots) return set_error(QL_ERR_ARG, "%s: slots is NULL", fn);
    if (!aligned(slots, 256)) return set_error(QL_ERR_ALIGN, "%s: slots must be 256-byte aligned", fn);
    if (slots_bytes < sc.slots_need)
      return set_error(QL_ERR_WORKSPACE, "%s: slots_bytes (%zu) < n_buffers (%d) layer records (%zu)", fn,
                       slots_bytes, cfg->n_buffers, sc.slots_need);
  }
  if (M > 0) {
    if (policy) {
      if (!saved) return set_error(QL_ERR_ARG, "%s: saved is NULL", fn);
      if (!aligned(saved, 256)) return set_error(QL_ERR_ALIGN, "%s: saved must be 256-byte aligned", fn);
      if (saved_bytes < sc.saved_need)
        return set_error(QL_ERR_WORKSPACE, "%s: saved_bytes (%zu) < required (%zu)", fn, saved_bytes,
                         sc.saved_need);
    }
    if (!ws) return set_error(QL_ERR_ARG, "%s: ws is NULL", fn);
    if (!aligned(ws, 256)) return set_error(QL_ERR_ALIGN, "%s: ws must be 256-byte aligned", fn);
    if (ws_bytes < sc.WS.total)
      return set_error(QL_ERR_WORKSPACE, "%s: ws_bytes (%zu) < required (%zu)", fn, ws_bytes, sc.WS.total);
  }
  if (!policy) return QL_OK;
  if (!lora) return set_error(QL_ERR_ARG, "%s: lora is NULL", fn);
  for (int l = 0; l < cfg->n_layers; ++l)
    for (int p = 0; p < QL_NPROJ; ++p) {
      const ql_lora& L = lora[l * QL_NPROJ + p];
      if (L.r != cfg->r || L.alpha != cfg->alpha)
        return set_error(QL_ERR_RANK, "%s: lora[%d] r/alpha (%d, %g) differ from cfg (%d, %g)", fn,
                         l * QL_NPROJ + p, L.r, (double)L.alpha, cfg->r, (double)cfg->alpha);
      if (!L.A || !L.B) return set_error(QL_ERR_ARG, "%s: lora[%d] has a NULL factor", fn, l * QL_NPROJ + p);
      if (!aligned(L.A, 16) || !aligned(L.B, 16))
        return set_error(QL_ERR_ALIGN, "%s: lora[%d] factors must be 16-byte aligned", fn, l * QL_NPROJ + p);
    }
  return QL_OK;
}

// ------------------------------------------------------- kernel timing
struct ProfRec {
  hipEvent_t a, b;
  int kernel;
  double work;  // FLOPs or bytes, by kernel id
};
static std::mutex g_prof_mu;
static bool g_prof_on = false;
static std::vector<ProfRec> g_prof;
// Events are pooled and reused across recordings, and the pool is filled when
// recording is switched on, so a timed launch creates nothing (creating events
// inside a timed region perturbs the concurrent layer copies).
static std::vector<hipEvent_t> g_pool;
static size_t g_pool_next = 0;
constexpr size_t kPoolReserve = 4096;

static ql_status pool_grow(size_t n) {
  while (g_pool.size() < n) {
    hipEvent_t e;
    QL_HIP_CHECK(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
    g_pool.push_back(e);
  }
  return QL_OK;
}

bool profiling_on() { return g_prof_on; }

// The two events are handed to hipExtLaunchKernelGGL, which stamps them at
// the start and end of the kernel's own dispatch (no separate stream markers).
// They skip the system-scope fence a default event performs when it
// completes, which would write back the L2 after every timed kernel.
ql_status profile_begin(hipEvent_t* start, hipEvent_t* stop) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  QL_TRY(pool_grow(g_pool_next + 2));
  *start = g_pool[g_pool_next++];
  *stop = g_pool[g_pool_next++];
  return QL_OK;
}

ql_status profile_end(hipEvent_t start, hipEvent_t stop, int kernel, double work) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back(ProfRec{start, stop, kernel, work});
  return QL_OK;
}

static void profile_clear() {
  for (auto& r : g_prof) (void)hipEventSynchronize(r.b);
  g_prof.clear();
  g_pool_next = 0;
}

// ------------------------------------------------------- linear backward
// Argument checks of the linear backward other than its workspace.
static ql_status check_linear_bwd(const char* fn, const void* dy, const void* x, const void* u_saved, int64_t M,
                                  const ql_nf4_weight& W, const ql_lora& L, const void* dx, const float* dA,
                                  const float* dB, int32_t accumulate) {
  if (M < 0) return set_error(QL_ERR_SHAPE, "%s: M (%lld) must be >= 0", fn, (long long)M);
  if (accumulate != 0 && accumulate != 1) return set_error(QL_ERR_ARG, "%s: accumulate must be 0 or 1", fn);
  QL_TRY(check_weight(fn, W));
  QL_TRY(check_lora(fn, L));
  QL_TRY(check_ptr(fn, "dA", dA, 16));
  QL_TRY(check_ptr(fn, "dB", dB, 16));
  if (M > 0) {
    QL_TRY(check_ptr(fn, "dy", dy, 16));
    QL_TRY(check_ptr(fn, "x", x, 16));
    QL_TRY(check_ptr(fn, "u_saved", u_saved, 16));
    if (dx) QL_TRY(check_ptr(fn, "dx", dx, 16));
  }
  return QL_OK;
}

// The linear backward with its temporaries in ws (lw.bwd bytes, 256-byte
// aligned; unused when M == 0). Every temporary is written before it is
// read, so ws needs no clearing and keeps nothing between calls.
static ql_status run_linear_bwd(const void* dy, const void* x, const void* u_saved, int64_t M,
                                const ql_nf4_weight& W, const ql_lora& L, void* dx, float* dA, float* dB,
                                int32_t accumulate, uint8_t* w8, const LinearWs& lw, hipStream_t st) {
  const float sc = L.alpha / (float)L.r;
  if (M == 0) {
    if (!accumulate) {
      QL_TRY(launch_zero_f32(dA, (int64_t)L.r * W.K, st));
      QL_TRY(launch_zero_f32(dB, W.N * L.r, st));
    }
    return QL_OK;
  }
  uint16_t* bt = (uint16_t*)(w8 + lw.bt_off);
  uint16_t* G = (uint16_t*)(w8 + lw.g_off);
  void* scratch = w8 + lw.scratch_off;
  const size_t scratch_bytes = lw.partial_off - lw.scratch_off;
  {
    TransArgs ta{};
    ta.n = 1; ta.in[0] = (const uint16_t*)L.B; ta.out[0] = bt; ta.rows[0] = W.N; ta.cols[0] = L.r;
    QL_TRY(launch_transpose_bf16(ta, st));
    RowArgs ra{};
    ra.nprob = 1;
    ra.p[0] = g_prob((const uint16_t*)dy, M, W.N, L.r, bt, G);
    QL_TRY(launch_rowc(ra, scratch, scratch_bytes, st));
  }
  if (dx) {
    BwdArgs a{};
    a.M = M; a.K = W.K; a.r = L.r; a.s = sc; a.out = dx; a.nseg = 1;
    a.seg[0] = BwdSeg{(const uint16_t*)dy, W.packed, W.absmax, G, (const uint16_t*)L.A, W.N};
    a.partial = (float*)(w8 + lw.partial_off);
    a.partial_bytes = bwd_partial_bytes(M, W.K);
    QL_TRY(launch_gemm_bwd(a, st));
  }
  ColArgs grads{};
  grads.nprob = 2;
  grads.p[0] = db_prob((const uint16_t*)dy, M, W.N, (const uint16_t*)u_saved, L.r, sc, dB, accumulate);
  grads.p[1] = da_prob((const uint16_t*)x, M, W.K, W.K, 0, 0, G, L.r, sc, dA, accumulate);
  return launch_colc(grads, scratch, scratch_bytes, st);
}

// The workspace of qlora_linear_bwd_noalloc: a fixed array in the library's
// code object, one per device, held until the process ends. In host code the
// array's name stands for a host-side shadow, not device memory, so it is
// used only to ask the runtime for the device address (on each device, on the
// first call there, with that device current); kernels get that address.
static __device__ __align__(256) uint8_t scratch[QL_NOALLOC_SCRATCH_BYTES];
static std::mutex g_scratch_mu;
static uint8_t* g_scratch_dev[64] = {};

static ql_status noalloc_scratch(uint8_t** out) {
  int dev = 0;
  QL_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return set_error(QL_ERR_UNSUPPORTED, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    QL_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || (uintptr_t)p % 256)
      return set_error(QL_ERR_HIP, "qlora_linear_bwd_noalloc: scratch address %p is not 256-byte aligned", p);
    g_scratch_dev[dev] = (uint8_t*)p;
  }
  *out = g_scratch_dev[dev];
  return QL_OK;
}

}  // namespace ql

using namespace ql;

extern "C" {

const char* ql_last_error(void) { return g_err; }

ql_status ql_profile_enable(int32_t on) {
  clear_error();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on) {
    profile_clear();
    QL_TRY(pool_grow(kPoolReserve));
  }
  g_prof_on = on != 0;
  return QL_OK;
}

ql_status ql_profile_read(int32_t kernel, int64_t* launches, double* ms, double* work) {
  clear_error();
  if (kernel < 0 || kernel >= QL_KERNEL_COUNT)
    return set_error(QL_ERR_ARG, "ql_profile_read: kernel (%d) out of range", kernel);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int64_t n = 0;
  double t = 0, f = 0;
  for (auto& r : g_prof) {
    if (r.kernel != kernel) continue;
    QL_HIP_CHECK(hipEventSynchronize(r.b));
    float e = 0;
    QL_HIP_CHECK(hipEventElapsedTime(&e, r.a, r.b));
    ++n;
    t += e;
    f += r.work;
  }
  if (launches) *launches = n;
  if (ms) *ms = t;
  if (work) *work = f;
  return QL_OK;
}

int32_t ql_abi_version(void) { return 101; }

ql_status ql_debug_poison_slots(int32_t on) {
  clear_error();
  if (on != 0 && on != 1) return set_error(QL_ERR_ARG, "ql_debug_poison_slots: on must be 0 or 1");
  g_poison.store(on != 0);
  return QL_OK;
}

ql_status nf4_codebook(float* out) {
  clear_error();
  if (!out) return set_error(QL_ERR_ARG, "nf4_codebook: out is NULL");
  memcpy(out, kNF4LevelBitsHost, sizeof(kNF4LevelBitsHost));
  return QL_OK;
}

ql_status nf4_quantize(const float* w, int64_t n, uint8_t* packed, float* absmax, ql_stream s) {
  clear_error();
  const char* fn = "nf4_quantize";
  if (n < 0 || n % 64) return set_error(QL_ERR_SHAPE, "%s: n (%lld) must be a non-negative multiple of 64", fn,
                                        (long long)n);
  if (n == 0) return QL_OK;
  QL_TRY(check_ptr(fn, "w", w, 16));
  QL_TRY(check_ptr(fn, "packed", packed, 16));
  QL_TRY(check_ptr(fn, "absmax", absmax, 16));
  hipStream_t st = (hipStream_t)s;
  {  // refuse non-finite input before anything is written
    std::lock_guard<std::mutex> lk(g_quant_mu);
    int nonfinite = 0;
    QL_TRY(scan_nonfinite(w, n, &nonfinite, st));
    if (nonfinite) return set_error(QL_ERR_NONFINITE, "%s: w holds NaN or Inf", fn);
  }
  return launch_nf4_quantize(w, n, packed, absmax, st);
}

ql_status nf4_dq_layout(int64_t nblocks, size_t* scale_off, size_t* mean_off, size_t* bytes) {
  clear_error();
  if (nblocks < 0) return set_error(QL_ERR_SHAPE, "nf4_dq_layout: nblocks (%lld) must be >= 0", (long long)nblocks);
  const DqLayout l = dq_layout(nblocks);
  if (scale_off) *scale_off = l.scale_off;
  if (mean_off) *mean_off = l.mean_off;
  if (bytes) *bytes = l.bytes;
  return QL_OK;
}

ql_status nf4_double_quant(const float* absmax, int64_t nblocks, void* dq, size_t dq_bytes, ql_stream s) {
  clear_error();
  const char* fn = "nf4_double_quant";
  if (nblocks < 0) return set_error(QL_ERR_SHAPE, "%s: nblocks (%lld) must be >= 0", fn, (long long)nblocks);
  if (nblocks == 0) return QL_OK;
  QL_TRY(check_ptr(fn, "absmax", absmax, 4));
  QL_TRY(check_ptr(fn, "dq", dq, 256));
  const DqLayout l = dq_layout(nblocks);
  if (dq_bytes < l.bytes)
    return set_error(QL_ERR_WORKSPACE, "%s: dq_bytes (%zu) < block size (%zu)", fn, dq_bytes, l.bytes);
  return launch_dq_quant(absmax, nblocks, (uint8_t*)dq, (hipStream_t)s);
}

ql_status nf4_dq_expand(const void* dq, int64_t nblocks, float* absmax, ql_stream s) {
  clear_error();
  const char* fn = "nf4_dq_expand";
  if (nblocks < 0) return set_error(QL_ERR_SHAPE, "%s: nblocks (%lld) must be >= 0", fn, (long long)nblocks);
  if (nblocks == 0) return QL_OK;
  QL_TRY(check_ptr(fn, "dq", dq, 256));
  QL_TRY(check_ptr(fn, "absmax", absmax, 4));
  const DqLayout l = dq_layout(nblocks);
  DqExpandArgs a{};
  a.nblk = 1;
  a.src[0] = (const uint8_t*)dq;
  a.scale_off[0] = l.scale_off;
  a.mean_off[0] = l.mean_off;
  a.dst[0] = absmax;
  a.end[0] = nblocks;
  return launch_dq_expand(a, (hipStream_t)s);
}

ql_status nf4_dequant(const uint8_t* packed, const float* absmax, int64_t n, int32_t out_dtype, void* out,
                      ql_stream s) {
  clear_error();
  const char* fn = "nf4_dequant";
  if (n < 0 || n % 64) return set_error(QL_ERR_SHAPE, "%s: n (%lld) must be a non-negative multiple of 64", fn,
                                        (long long)n);
  if (out_dtype != QL_BF16 && out_dtype != QL_F32)
    return set_error(QL_ERR_ARG, "%s: out_dtype (%d) must be QL_BF16 or QL_F32", fn, out_dtype);
  if (n == 0) return QL_OK;
  QL_TRY(check_ptr(fn, "packed", packed, 16));
  QL_TRY(check_ptr(fn, "absmax", absmax, 16));
  QL_TRY(check_ptr(fn, "out", out, 16));
  return launch_nf4_dequant(packed, absmax, n, out_dtype == QL_F32, out, (hipStream_t)s);
}

ql_status qlora_linear_workspace(int64_t M, int64_t N, int64_t K, int32_t r, size_t* fwd_bytes,
                                 size_t* bwd_bytes) {
  clear_error();
  if (M < 0 || N <= 0 || K <= 0 || K % 64 || N % 16 || N > QL_MAX_DIM || K > QL_MAX_DIM)
    return set_error(QL_ERR_SHAPE, "qlora_linear_workspace: need M >= 0, N % 16 == 0, K % 64 == 0, "
                     "N and K <= QL_MAX_DIM");
  if (r < 1 || r > 64) return set_error(QL_ERR_RANK, "qlora_linear_workspace: r (%d) must be in 1..64", r);
  LinearWs w = linear_ws(M, N, K, r);
  if (fwd_bytes) *fwd_bytes = w.fwd;
  if (bwd_bytes) *bwd_bytes = w.bwd;
  return QL_OK;
}

ql_status qlora_linear_fwd(const void* x, int64_t M, ql_nf4_weight W, ql_lora L, void* y, void* u_save,
                           void* ws, size_t ws_bytes, ql_stream s) {
  clear_error();
  const char* fn = "qlora_linear_fwd";
  if (M < 0) return set_error(QL_ERR_SHAPE, "%s: M (%lld) must be >= 0", fn, (long long)M);
  QL_TRY(check_weight(fn, W));
  QL_TRY(check_lora(fn, L));
  if (M == 0) return QL_OK;
  QL_TRY(check_ptr(fn, "x", x, 16));
  QL_TRY(check_ptr(fn, "y", y, 16));
  QL_TRY(check_ptr(fn, "u_save", u_save, 16));
  LinearWs lw = linear_ws(M, W.N, W.K, L.r);
  if (ws_bytes < lw.fwd) return set_error(QL_ERR_WORKSPACE, "%s: ws_bytes (%zu) < %zu", fn, ws_bytes, lw.fwd);
  if (lw.fwd) QL_TRY(check_ptr(fn, "ws", ws, 16));
  hipStream_t st = (hipStream_t)s;
  RowArgs ra{};
  ra.nprob = 1;
  RowProb& u = ra.p[0];
  u.X = u16(x); u.M = M; u.K = W.K; u.ldx = W.K; u.r = L.r; u.nseg = 1; u.Bt[0] = u16(L.A);
  u.out[0] = u16w(u_save);
  QL_TRY(launch_rowc(ra, ws, lw.fpartial_off, st));
  FwdArgs a{};
  a.X = u16(x); a.M = M; a.K = W.K; a.ldx = W.K; a.r = L.r; a.s = L.alpha / (float)L.r; a.nseg = 1;
  FwdSeg& g = a.seg[0];
  g.packed = W.packed; g.absmax = W.absmax; g.U = u16(u_save); g.B = u16(L.B); g.out = y; g.N = W.N;
  g.ldo = W.N; g.col0 = 0; g.resid = nullptr;
  a.partial = (float*)((uint8_t*)ws + lw.fpartial_off);
  a.partial_bytes = bwd_partial_bytes(M, W.N);
  return launch_gemm_fwd(a, st);
}

ql_status qlora_linear_bwd(const void* dy, const void* x, const void* u_saved, int64_t M, ql_nf4_weight W,
                           ql_lora L, void* dx, float* dA, float* dB, int32_t accumulate, void* ws,
                           size_t ws_bytes, ql_stream s) {
  clear_error();
  const char* fn = "qlora_linear_bwd";
  QL_TRY(check_linear_bwd(fn, dy, x, u_saved, M, W, L, dx, dA, dB, accumulate));
  LinearWs lw = linear_ws(M, W.N, W.K, L.r);
  if (M > 0) {
    if (ws_bytes < lw.bwd) return set_error(QL_ERR_WORKSPACE, "%s: ws_bytes (%zu) < %zu", fn, ws_bytes, lw.bwd);
    QL_TRY(check_ptr(fn, "ws", ws, 256));
  }
  return run_linear_bwd(dy, x, u_saved, M, W, L, dx, dA, dB, accumulate, (uint8_t*)ws, lw, (hipStream_t)s);
}

ql_status qlora_linear_bwd_noalloc(const void* dy, const void* x, const void* u_saved, int64_t M,
                                   ql_nf4_weight W, ql_lora L, void* dx, float* dA, float* dB,
                                   int32_t accumulate, ql_stream s) {
  clear_error();
  const char* fn = "qlora_linear_bwd_noalloc";
  QL_TRY(check_linear_bwd(fn, dy, x, u_saved, M, W, L, dx, dA, dB, accumulate));
  LinearWs lw = linear_ws(M, W.N, W.K, L.r);
  uint8_t* ws = nullptr;
  if (M > 0) {
    if (lw.bwd > (size_t)QL_NOALLOC_SCRATCH_BYTES)
      return set_error(QL_ERR_WORKSPACE,
                       "%s: M %lld, N %lld, K %lld, r %d needs %zu bytes of scratch, more than the fixed %zu "
                       "(qlora_linear_bwd takes a workspace of any size)",
                       fn, (long long)M, (long long)W.N, (long long)W.K, (int)L.r, lw.bwd,
                       (size_t)QL_NOALLOC_SCRATCH_BYTES);
    QL_TRY(noalloc_scratch(&ws));
  }
  return run_linear_bwd(dy, x, u_saved, M, W, L, dx, dA, dB, accumulate, ws, lw, (hipStream_t)s);
}

ql_status stream_layer_stack_layout(const ql_stack_cfg* cfg, int64_t* layer_offsets, int64_t* proj_offsets,
                                    size_t* store_bytes) {
  clear_error();
  QL_TRY(check_cfg("stream_layer_stack_layout", cfg));
  StackLayout SL = stack_layout(cfg);
  if (layer_offsets)
    for (int l = 0; l <= cfg->n_layers; ++l) layer_offsets[l] = SL.rec * l;
  if (proj_offsets)
    for (int p = 0; p < QL_NPROJ; ++p) {
      proj_offsets[2 * p] = SL.packed_off[p];
      proj_offsets[2 * p + 1] = SL.absmax_off[p];
    }
  if (store_bytes) *store_bytes = (size_t)SL.rec * cfg->n_layers;
  return QL_OK;
}

ql_status stream_layer_stack_workspace(const ql_stack_cfg* cfg, int64_t M, size_t* slots_bytes,
                                       size_t* saved_bytes, size_t* ws_bytes) {
  clear_error();
  QL_TRY(check_cfg("stream_layer_stack_workspace", cfg));
  if (M < 0) return set_error(QL_ERR_SHAPE, "stream_layer_stack_workspace: M must be >= 0");
  StackLayout SL = stack_layout(cfg);
  if (slots_bytes) *slots_bytes = cfg->resident ? 0 : (size_t)SL.rec * cfg->n_buffers;
  if (saved_bytes) *saved_bytes = saved_layout(cfg, M).per_layer * cfg->n_layers;
  if (ws_bytes) *ws_bytes = stack_ws(cfg, M).total;
  return QL_OK;
}

ql_status stream_layer_stack_saved_layout(const ql_stack_cfg* cfg, int64_t M, int64_t* offsets,
                                          size_t* per_layer_bytes) {
  clear_error();
  QL_TRY(check_cfg("stream_layer_stack_saved_layout", cfg));
  if (M < 0) return set_error(QL_ERR_SHAPE, "stream_layer_stack_saved_layout: M must be >= 0");
  SavedLayout SV = saved_layout(cfg, M);
  if (offsets)
    for (int i = 0; i < QL_SAVED_COUNT; ++i) offsets[i] = SV.off[i];
  if (per_layer_bytes) *per_layer_bytes = SV.per_layer;
  return QL_OK;
}

}  // extern "C"

// Forward pass over the layers shared by the public entry points. Policy
// (lora != nullptr): the adapted stack, activations saved for the backward,
// output y. Reference (ref_y != nullptr): the adapter-off stack on the same
// x0, activations of one layer at a time in ref_sv (the saved layout of one
// layer; its h_in entry carries the running hidden state), output ref_y. With
// both, each layer's slot serves the two passes before it is refilled, so the
// reference adds no copies.
static ql_status stack_fwd(const ql_stack_cfg* cfg, const StackCall& sc, const void* store, const ql_lora* lora,
                           const void* x0, int64_t M, void* y, void* saved, void* ref_y, void* ref_sv,
                           int32_t reuse_bwd_slots, void* slots, void* ws, hipStream_t C, hipStream_t P) {
  const int L = cfg->n_layers;
  const int64_t H = cfg->hidden;
  uint8_t* sv = (uint8_t*)saved;
  uint8_t* rv = (uint8_t*)ref_sv;
  uint8_t* w8 = (uint8_t*)ws;
  const uint8_t* st8 = (const uint8_t*)store;
  uint8_t* sl8 = (uint8_t*)slots;
  const size_t rec = (size_t)sc.SL.rec;
  const bool throttle = !cfg->resident && rec >= kThrottleRecord && !capturing(C);
  if (throttle) QL_TRY(inflight_wait(0));
  // layer 0 input into the saved area (the backward reads it)
  if (lora)
    QL_HIP_CHECK(hipMemcpyAsync(sv + sc.SV.off[QL_SAVED_H_IN], x0, (size_t)M * H * 2, hipMemcpyDeviceToDevice, C));
  if (ref_y)
    QL_HIP_CHECK(hipMemcpyAsync(rv + sc.SVF.off[QL_SAVED_H_IN], x0, (size_t)M * H * 2, hipMemcpyDeviceToDevice, C));
  Events ev;
  // layer l uses slot l % nb; with reuse_bwd_slots the preceding backward
  // left layers nb - 1 .. 0 in their slots
  const int nb = cfg->n_buffers;
  bool have_ready[QL_MAX_BUFFERS] = {};
  // The pass's last copy lands one weight group at a time, and the last
  // layer starts each GEMM as soon as its group is in, instead of idling
  // through the whole copy (records of 8 MiB or more; 8B-shaped stack at
  // M = 2048: 133.1 against 134.8 ms per step).
  const bool grouped = !cfg->resident && rec >= kThrottleRecord && L > nb;
  if (!cfg->resident) {
    QL_TRY(ev.create(nb, grouped));
    if (!reuse_bwd_slots) {
      QL_TRY(ev.after_compute(C, P));
      for (int l = 0; l < nb && l < L; ++l) {
        QL_TRY(copy_record(sl8 + l * rec, st8 + l * rec, rec, P, !sc.pageable));
        QL_HIP_CHECK(hipEventRecord(ev.ready[l], P));
        have_ready[l] = true;
      }
    }
  }
  LayerAhead ahead;
  QL_TRY(ahead.init(throttle && nb == 2));
  for (int l = 0; l < L; ++l) {
    QL_TRY(ahead.before(l));
    const int slot = l % nb;
    const uint8_t* base;
    if (cfg->resident) {
      base = st8 + l * rec;
    } else {
      if (have_ready[slot]) QL_HIP_CHECK(hipStreamWaitEvent(C, ev.ready[slot], 0));
      base = sl8 + slot * rec;
    }
    const bool by_group = grouped && l == L - 1;
    LayerW W;
    QL_TRY(layer_weights_ready(cfg, sc.SL, sc.WS, base, w8, C, W, by_group));
    // with two slots the first refill (layer 2 into layer 0's slot) starts
    // on q|k|v and o, on the side stream, once layer 0's o GEMM is done (not
    // in a capture, not when the slot also serves the reference forward)
    const bool early = grouped && nb == 2 && l == 0 && !ref_y && !capturing(C) && l + nb < L - 1;
    GroupReady gr;
    gr.wait = by_group;
    std::copy(ev.gready[slot], ev.gready[slot] + kGroups, gr.ready);
    for (int g = 0; g < kGroups && by_group && cfg->absmax_dq; ++g)
      gr.dq[g] = dq_expand_args(sc.SL, sc.WS, base, w8, g);
    if (early) {
      gr.early = ev.early;
      gr.early_after = 1;
    }
    const GroupReady* grp = (by_group || early) ? &gr : nullptr;
    if (lora) {
      uint8_t* svl = sv + (size_t)l * sc.SV.per_layer;
      uint16_t* h_out = (l + 1 < L) ? (uint16_t*)(sv + (size_t)(l + 1) * sc.SV.per_layer + sc.SV.off[QL_SAVED_H_IN])
                                    : (uint16_t*)y;
      if (cfg->recompute) {
        // the layer runs on the one-layer area ck; only its input is kept
        uint8_t* ck = w8 + sc.WS.ck;
        QL_HIP_CHECK(hipMemcpyAsync(ck + sc.SVF.off[QL_SAVED_H_IN], svl + sc.SV.off[QL_SAVED_H_IN],
                                    (size_t)M * H * 2, hipMemcpyDeviceToDevice, C));
        QL_TRY(layer_fwd(cfg, sc.SL, W, lora + l * QL_NPROJ, M, sc.SVF, ck, h_out, w8, sc.WS, C, grp));
      } else {
        QL_TRY(layer_fwd(cfg, sc.SL, W, lora + l * QL_NPROJ, M, sc.SVF, svl, h_out, w8, sc.WS, C, grp));
      }
    }
    if (ref_y) {
      // the layer's last kernel reads h_in no more, so its output may replace it
      uint16_t* h_out = (l + 1 < L) ? (uint16_t*)(rv + sc.SVF.off[QL_SAVED_H_IN]) : (uint16_t*)ref_y;
      QL_TRY(layer_fwd(cfg, sc.SL, W, nullptr, M, sc.SVF, rv, h_out, w8, sc.WS, C, grp));
    }
    if (!cfg->resident && l + nb < L) {
      uint8_t* dst = sl8 + slot * rec;
      const uint8_t* src = st8 + (size_t)(l + nb) * rec;
      size_t head = 0;  // bytes the side stream copies
      if (early) {
        hipStream_t P2;
        QL_TRY(side_stream(&P2));
        head = (size_t)sc.SL.grp_off[2];
        QL_HIP_CHECK(hipStreamWaitEvent(P2, ev.early, 0));
        QL_TRY(copy_record(dst, src, head, P2, !sc.pageable));
        QL_HIP_CHECK(hipEventRecord(ev.side, P2));
      }
      QL_HIP_CHECK(hipEventRecord(ev.free_[slot], C));
      QL_HIP_CHECK(hipStreamWaitEvent(P, ev.free_[slot], 0));
      if (grouped && l + nb == L - 1) {
        QL_TRY(copy_groups(sc.SL, dst, src, P, !sc.pageable, kFwdOrder, ev.gready[slot]));
        have_ready[slot] = false;
      } else {
        QL_TRY(copy_record(dst + head, src + head, rec - head, P, !sc.pageable));
        if (early) QL_HIP_CHECK(hipStreamWaitEvent(P, ev.side, 0));
        QL_HIP_CHECK(hipEventRecord(ev.ready[slot], P));
        have_ready[slot] = true;
      }
    }
    QL_TRY(ahead.after(l, C));
  }
  if (throttle) QL_TRY(inflight_mark(0, C));
  return sc.pageable ? QL_WARN_PAGEABLE_HOST : QL_OK;
}

extern "C" {

ql_status stream_layer_stack_fwd(const ql_stack_cfg* cfg, const void* store, size_t store_bytes,
                                 const ql_lora* lora, const void* x0, int64_t M, void* y, void* saved,
                                 size_t saved_bytes, int32_t reuse_bwd_slots, void* slots, size_t slots_bytes,
                                 void* ws, size_t ws_bytes, ql_stream compute, ql_stream copy) {
  clear_error();
  const char* fn = "stream_layer_stack_fwd";
  StackCall sc;
  QL_TRY(validate_stack(fn, cfg, store, store_bytes, lora, M, saved, saved_bytes, slots, slots_bytes, ws,
                        ws_bytes, sc));
  if (reuse_bwd_slots != 0 && reuse_bwd_slots != 1)
    return set_error(QL_ERR_ARG, "%s: reuse_bwd_slots must be 0 or 1", fn);
  if (M > 0) {
    QL_TRY(check_ptr(fn, "x0", x0, 16));
    QL_TRY(check_ptr(fn, "y", y, 16));
  }
  if (M == 0) return sc.pageable ? QL_WARN_PAGEABLE_HOST : QL_OK;
  return stack_fwd(cfg, sc, store, lora, x0, M, y, saved, nullptr, nullptr, reuse_bwd_slots, slots, ws,
                   (hipStream_t)compute, (hipStream_t)copy);
}

ql_status stream_layer_stack_fwd_ref(const ql_stack_cfg* cfg, const void* store, size_t store_bytes,
                                     const ql_lora* lora, const void* x0, int64_t M, void* y, void* saved,
                                     size_t saved_bytes, void* ref_y, void* ref_scratch, size_t ref_scratch_bytes,
                                     int32_t reuse_bwd_slots, void* slots, size_t slots_bytes, void* ws,
                                     size_t ws_bytes, ql_stream compute, ql_stream copy) {
  clear_error();
  const char* fn = "stream_layer_stack_fwd_ref";
  StackCall sc;
  QL_TRY(validate_stack(fn, cfg, store, store_bytes, lora, M, saved, saved_bytes, slots, slots_bytes, ws,
                        ws_bytes, sc, lora != nullptr));
  if (reuse_bwd_slots != 0 && reuse_bwd_slots != 1)
    return set_error(QL_ERR_ARG, "%s: reuse_bwd_slots must be 0 or 1", fn);
  if (M > 0) {
    QL_TRY(check_ptr(fn, "x0", x0, 16));
    if (lora) QL_TRY(check_ptr(fn, "y", y, 16));
    QL_TRY(check_ptr(fn, "ref_y", ref_y, 16));
    if (!ref_scratch) return set_error(QL_ERR_ARG, "%s: ref_scratch is NULL", fn);
    if (!aligned(ref_scratch, 256)) return set_error(QL_ERR_ALIGN, "%s: ref_scratch must be 256-byte aligned", fn);
    if (ref_scratch_bytes < sc.SVF.per_layer)
      return set_error(QL_ERR_WORKSPACE, "%s: ref_scratch_bytes (%zu) < one layer of activations (%zu)",
                       fn, ref_scratch_bytes, (size_t)sc.SVF.per_layer);
  }
  if (M == 0) return sc.pageable ? QL_WARN_PAGEABLE_HOST : QL_OK;
  return stack_fwd(cfg, sc, store, lora, x0, M, y, lora ? saved : nullptr, ref_y, ref_scratch, reuse_bwd_slots,
                   slots, ws, (hipStream_t)compute, (hipStream_t)copy);
}

ql_status stream_layer_stack_bwd(const ql_stack_cfg* cfg, const void* store, size_t store_bytes,
                                 const ql_lora* lora, const void* dy, int64_t M, const void* saved,
                                 size_t saved_bytes, void* dx0, float* const* dA, float* const* dB,
                                 int32_t accumulate, int32_t reuse_fwd_slots, void* slots, size_t slots_bytes,
                                 void* ws, size_t ws_bytes, ql_stream compute, ql_stream copy) {
  clear_error();
  const char* fn = "stream_layer_stack_bwd";
  StackCall sc;
  QL_TRY(validate_stack(fn, cfg, store, store_bytes, lora, M, saved, saved_bytes, slots, slots_bytes, ws,
                        ws_bytes, sc));
  if (accumulate != 0 && accumulate != 1) return set_error(QL_ERR_ARG, "%s: accumulate must be 0 or 1", fn);
  if (reuse_fwd_slots != 0 && reuse_fwd_slots != 1)
    return set_error(QL_ERR_ARG, "%s: reuse_fwd_slots must be 0 or 1", fn);
  if (!dA || !dB) return set_error(QL_ERR_ARG, "%s: dA / dB arrays are NULL", fn);
  const int L = cfg->n_layers;
  for (int i = 0; i < L * QL_NPROJ; ++i) {
    if (!dA[i] || !dB[i]) return set_error(QL_ERR_ARG, "%s: dA[%d] or dB[%d] is NULL", fn, i, i);
    if (!aligned(dA[i], 16) || !aligned(dB[i], 16))
      return set_error(QL_ERR_ALIGN, "%s: dA[%d] / dB[%d] must be 16-byte aligned", fn, i, i);
  }
  if (M > 0) {
    QL_TRY(check_ptr(fn, "dy", dy, 16));
    if (dx0) QL_TRY(check_ptr(fn, "dx0", dx0, 16));
  }
  hipStream_t C = (hipStream_t)compute, P = (hipStream_t)copy;
  if (M == 0) {
    if (!accumulate)
      for (int l = 0; l < L; ++l)
        for (int p = 0; p < QL_NPROJ; ++p) {
          QL_TRY(launch_zero_f32(dA[l * QL_NPROJ + p], (int64_t)cfg->r * sc.SL.K[p], C));
          QL_TRY(launch_zero_f32(dB[l * QL_NPROJ + p], sc.SL.N[p] * cfg->r, C));
        }
    return sc.pageable ? QL_WARN_PAGEABLE_HOST : QL_OK;
  }
  const uint8_t* sv = (const uint8_t*)saved;
  uint8_t* w8 = (uint8_t*)ws;
  const uint8_t* st8 = (const uint8_t*)store;
  uint8_t* sl8 = (uint8_t*)slots;
  const size_t rec = (size_t)sc.SL.rec;
  Events ev;
  const bool streamed = !cfg->resident;
  const bool throttle = streamed && rec >= kThrottleRecord && !capturing(C);
  if (throttle) QL_TRY(inflight_wait(1));
  // layers L-1, L-2, ... ; layer l uses slot l % nb (the forward's mapping)
  const int nb = cfg->n_buffers;
  bool have_ready[QL_MAX_BUFFERS] = {};
  // the pass's last copy (layer 0) by weight group, as in the forward, in the
  // order the backward reads them: down, gate|up, o, q|k|v
  const bool grouped = streamed && rec >= kThrottleRecord && L > nb;
  if (streamed) {
    QL_TRY(ev.create(nb, grouped));
    if (!reuse_fwd_slots) QL_TRY(ev.after_compute(C, P));
    for (int i = 0; i < nb && i < L; ++i) {
      const int l = L - 1 - i;
      if (reuse_fwd_slots) continue;  // the forward left layers L-1 .. L-nb in their slots
      QL_TRY(copy_record(sl8 + (l % nb) * rec, st8 + (size_t)l * rec, rec, P, !sc.pageable));
      QL_HIP_CHECK(hipEventRecord(ev.ready[l % nb], P));
      have_ready[l % nb] = true;
    }
  }
  uint16_t* dhA = (uint16_t*)(w8 + sc.WS.dhA);
  uint16_t* dhB = (uint16_t*)(w8 + sc.WS.dhB);
  const uint16_t* dh = (const uint16_t*)dy;
  LayerAhead ahead;
  QL_TRY(ahead.init(throttle && nb == 2));
  for (int l = L - 1; l >= 0; --l) {
    QL_TRY(ahead.before(L - 1 - l));
    const int slot = l % nb;
    const uint8_t* base;
    if (!streamed) {
      base = st8 + (size_t)l * rec;
    } else {
      if (have_ready[slot]) QL_HIP_CHECK(hipStreamWaitEvent(C, ev.ready[slot], 0));
      base = sl8 + slot * rec;
    }
    uint16_t* out = (l == 0 && dx0) ? (uint16_t*)dx0 : (((L - 1 - l) & 1) ? dhB : dhA);
    const bool by_group = grouped && l == 0;
    LayerW W;
    QL_TRY(layer_weights_ready(cfg, sc.SL, sc.WS, base, w8, C, W, by_group));
    // with two slots the first refill (layer L - 3 into layer L - 1's slot)
    // starts on down, on the side stream, once the layer's down dX GEMM is
    // done (a recomputed forward reads down before that GEMM)
    const bool early = grouped && nb == 2 && l == L - 1 && !capturing(C) && l - nb > 0;
    GroupReady gr;
    gr.wait = by_group;
    std::copy(ev.gready[slot], ev.gready[slot] + kGroups, gr.ready);
    for (int g = 0; g < kGroups && by_group && cfg->absmax_dq; ++g)
      gr.dq[g] = dq_expand_args(sc.SL, sc.WS, base, w8, g);
    GroupReady gb = gr;  // the backward's own: only it records the early event
    if (early) {
      gb.early = ev.early;
      gb.early_after = 3;
    }
    const GroupReady* grp = by_group ? &gr : nullptr;
    const GroupReady* gbp = (by_group || early) ? &gb : nullptr;
    const uint8_t* svl = sv + (size_t)l * sc.SV.per_layer;
    if (cfg->recompute) {
      // recompute the layer's activations from its saved input, with the
      // weights already in the slot (same kernels, same bytes: the same values
      // the forward produced)
      uint8_t* ck = w8 + sc.WS.ck;
      QL_HIP_CHECK(hipMemcpyAsync(ck + sc.SVF.off[QL_SAVED_H_IN], svl + sc.SV.off[QL_SAVED_H_IN],
                                  (size_t)M * cfg->hidden * 2, hipMemcpyDeviceToDevice, C));
      QL_TRY(layer_fwd(cfg, sc.SL, W, lora + l * QL_NPROJ, M, sc.SVF, ck, (uint16_t*)(w8 + sc.WS.ck_out), w8,
                       sc.WS, C, grp));
      svl = ck;
    }
    QL_TRY(layer_bwd(cfg, sc.SL, W, lora + l * QL_NPROJ, M, sc.SVF, svl, dh, out, dA + l * QL_NPROJ,
                     dB + l * QL_NPROJ, accumulate, w8, sc.WS, C, gbp));
    dh = out;
    if (streamed && l - nb >= 0) {
      uint8_t* dst = sl8 + slot * rec;
      const uint8_t* src = st8 + (size_t)(l - nb) * rec;
      size_t body = rec;  // bytes the copy stream copies (the rest: the side stream)
      if (early) {
        hipStream_t P2;
        QL_TRY(side_stream(&P2));
        body = (size_t)sc.SL.grp_off[3];
        QL_HIP_CHECK(hipStreamWaitEvent(P2, ev.early, 0));
        QL_TRY(copy_record(dst + body, src + body, rec - body, P2, !sc.pageable));
        QL_HIP_CHECK(hipEventRecord(ev.side, P2));
      }
      QL_HIP_CHECK(hipEventRecord(ev.free_[slot], C));
      QL_HIP_CHECK(hipStreamWaitEvent(P, ev.free_[slot], 0));
      if (grouped && l - nb == 0) {
        QL_TRY(copy_groups(sc.SL, dst, src, P, !sc.pageable, kBwdOrder, ev.gready[slot]));
        have_ready[slot] = false;
      } else {
        QL_TRY(copy_record(dst, src, body, P, !sc.pageable));
        if (early) QL_HIP_CHECK(hipStreamWaitEvent(P, ev.side, 0));
        QL_HIP_CHECK(hipEventRecord(ev.ready[slot], P));
        have_ready[slot] = true;
      }
    }
    QL_TRY(ahead.after(L - 1 - l, C));
  }
  if (throttle) QL_TRY(inflight_mark(1, C));
  return sc.pageable ? QL_WARN_PAGEABLE_HOST : QL_OK;
}


// ------------------------------------------------------------- step graphs
struct ql_step_graph_s {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

ql_status stream_layer_stack_step_capture(const ql_stack_cfg* cfg, const void* store, size_t store_bytes,
                                          const ql_lora* lora, const void* x0, const void* dy, int64_t M, void* y,
                                          void* saved, size_t saved_bytes, void* dx0, float* const* dA,
                                          float* const* dB, int32_t accumulate, int32_t turnaround, void* slots,
                                          size_t slots_bytes, void* ws, size_t ws_bytes, ql_stream compute,
                                          ql_stream copy, ql_step_graph* out) {
  clear_error();
  const char* fn = "stream_layer_stack_step_capture";
  if (!out) return set_error(QL_ERR_ARG, "%s: out is NULL", fn);
  *out = nullptr;
  StackCall sc;
  QL_TRY(validate_stack(fn, cfg, store, store_bytes, lora, M, saved, saved_bytes, slots, slots_bytes, ws,
                        ws_bytes, sc));
  if (sc.pageable)
    return set_error(QL_ERR_UNSUPPORTED, "%s: a pageable host store cannot be captured (copies need page-locked "
                     "memory)", fn);
  if (turnaround != 0 && turnaround != 1) return set_error(QL_ERR_ARG, "%s: turnaround must be 0 or 1", fn);
  if (profiling_on()) return set_error(QL_ERR_UNSUPPORTED, "%s: kernel timing is on (ql_profile_enable)", fn);
  if (!compute) return set_error(QL_ERR_ARG, "%s: capture needs an explicit compute stream", fn);
  if (g_poison.load()) return set_error(QL_ERR_UNSUPPORTED, "%s: slot poisoning is on (ql_debug_poison_slots)", fn);
  if (M == 0) return set_error(QL_ERR_SHAPE, "%s: M must be >= 1", fn);
  hipStream_t C = (hipStream_t)compute;
  QL_HIP_CHECK(hipStreamBeginCapture(C, hipStreamCaptureModeRelaxed));
  ql_status st = stream_layer_stack_fwd(cfg, store, store_bytes, lora, x0, M, y, saved, saved_bytes, turnaround,
                                        slots, slots_bytes, ws, ws_bytes, compute, copy);
  if (st >= 0)
    st = stream_layer_stack_bwd(cfg, store, store_bytes, lora, dy, M, saved, saved_bytes, dx0, dA, dB, accumulate,
                                1, slots, slots_bytes, ws, ws_bytes, compute, copy);
  hipGraph_t g = nullptr;
  const hipError_t ec = hipStreamEndCapture(C, &g);  // always ends the capture
  if (st < 0) {
    if (g) (void)hipGraphDestroy(g);
    return st;
  }
  if (ec != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return set_error(QL_ERR_HIP, "%s: hipStreamEndCapture: %s", fn, hipGetErrorString(ec));
  }
  hipGraphExec_t e = nullptr;
  const hipError_t ei = hipGraphInstantiate(&e, g, nullptr, nullptr, 0);
  if (ei != hipSuccess) {
    (void)hipGraphDestroy(g);
    return set_error(QL_ERR_HIP, "%s: hipGraphInstantiate: %s", fn, hipGetErrorString(ei));
  }
  ql_step_graph_s* h = new ql_step_graph_s;
  h->graph = g;
  h->exec = e;
  *out = h;
  return QL_OK;
}

ql_status ql_step_graph_launch(ql_step_graph g, ql_stream stream) {
  clear_error();
  if (!g) return set_error(QL_ERR_ARG, "ql_step_graph_launch: graph is NULL");
  QL_HIP_CHECK(hipGraphLaunch(g->exec, (hipStream_t)stream));
  return QL_OK;
}

ql_status ql_step_graph_info(ql_step_graph g, int64_t* kernels, int64_t* copies, int64_t* nodes) {
  clear_error();
  if (!g || !g->graph) return set_error(QL_ERR_ARG, "ql_step_graph_info: graph is NULL");
  size_t n = 0;
  QL_HIP_CHECK(hipGraphGetNodes(g->graph, nullptr, &n));
  std::vector<hipGraphNode_t> all(n);
  if (n) QL_HIP_CHECK(hipGraphGetNodes(g->graph, all.data(), &n));
  int64_t k = 0, c = 0;
  for (size_t i = 0; i < n; ++i) {
    hipGraphNodeType t;
    QL_HIP_CHECK(hipGraphNodeGetType(all[i], &t));
    if (t == hipGraphNodeTypeKernel) ++k;
    if (t == hipGraphNodeTypeMemcpy) ++c;
  }
  if (kernels) *kernels = k;
  if (copies) *copies = c;
  if (nodes) *nodes = (int64_t)n;
  return QL_OK;
}

ql_status ql_step_graph_destroy(ql_step_graph g) {
  clear_error();
  if (!g) return QL_OK;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
  return QL_OK;
}

}  // extern "C"
