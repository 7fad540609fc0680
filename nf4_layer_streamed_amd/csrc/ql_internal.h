// Internal declarations of the NF4 + LoRA library (HIP, gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/nf4qlora.h"

namespace ql {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The 16 NF4 levels as float32 bit patterns, ascending. Construction (QLoRA,
// Dettmers et al. 2023, section 3): standard-normal quantiles at evenly spaced
// probabilities from 1 - (1/30 + 1/32)/2 down to 1/2, 8 on the positive side
// and 7 on the negative side, plus an exact zero, divided by the largest level
// in double precision and rounded once to float32. Level 0 is -1, level 7 is
// +0, level 15 is +1.
static __constant__ const uint32_t kNF4LevelBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du,
    0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

static const uint32_t kNF4LevelBitsHost[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du,
    0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Round-to-nearest-even float32 -> bfloat16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two float32 -> one dword of two bfloat16, `lo` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// 8 bf16 <-> 8 float32 (element 0 in the low half of the first dword)
__device__ __forceinline__ void unpack8(const uint4 q, float (&f)[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// RMSNorm statistics, one code path for the standalone kernels and the row
// kernel that fuses them: a lane's sum of squares of its 8-element chunks
// (added in chunk order), the wave's lanes combined by a fixed butterfly, and
// the scale 1 / sqrt(mean + eps).
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ void add_squares8(uint4 q, float& ss) {
  float f[8];
  unpack8(q, f);
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += f[k] * f[k];
}
__device__ __forceinline__ float rms_scale(float ss, int64_t H, float eps) { return 1.0f / sqrtf(ss / (float)H + eps); }
__device__ __forceinline__ uint4 scale8(uint4 q, float rs) {
  float f[8];
  unpack8(q, f);
#pragma unroll
  for (int k = 0; k < 8; ++k) f[k] *= rs;
  return pack8(f);
}

// SwiGLU on 8 bf16 elements (one code path for the elementwise kernels and
// the kernels that fuse it): act = bf16(g sig(g) u);
// dg = bf16(dact u sig(g) (1 + g (1 - sig(g)))), du = bf16(dact g sig(g)).
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ uint4 swiglu_act8(uint4 g, uint4 u) {
  float gf[8], uf[8], o[8];
  unpack8(g, gf);
  unpack8(u, uf);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = gf[i] * sigmoidf_(gf[i]) * uf[i];
  return pack8(o);
}
__device__ __forceinline__ void swiglu_grad8(uint4 g, uint4 u, uint4 da, uint4& dg, uint4& du) {
  float gf[8], uf[8], df[8], og[8], ou[8];
  unpack8(g, gf);
  unpack8(u, uf);
  unpack8(da, df);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float sg = sigmoidf_(gf[i]);
    og[i] = df[i] * uf[i] * (sg * (1.0f + gf[i] * (1.0f - sg)));
    ou[i] = df[i] * (gf[i] * sg);
  }
  dg = pack8(og);
  du = pack8(ou);
}

// Error reporting (thread-local message), defined in capi.hip.
ql_status set_error(ql_status st, const char* fmt, ...);

#define QL_HIP_CHECK(expr)                                                        \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess)                                                         \
      return ::ql::set_error(QL_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define QL_TRY(expr)                 \
  do {                               \
    ql_status rc_ = (expr);          \
    if (rc_ != QL_OK) return rc_;    \
  } while (0)

// ---------------------------------------------------------------- launchers
inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// All launchers enqueue on `st` and report launch errors through the status.

ql_status launch_nf4_quantize(const float* w, int64_t n, uint8_t* packed, float* absmax, hipStream_t st);
// *nonfinite = 1 if w[0 .. n) holds a NaN or an infinity, else 0; waits for
// the stream (the scan's flag is one device word, so callers take turns)
ql_status scan_nonfinite(const float* w, int64_t n, int* nonfinite, hipStream_t st);
ql_status launch_nf4_dequant(const uint8_t* packed, const float* absmax, int64_t n, int out_f32,
                             void* out, hipStream_t st);

// Double-quantised scales (nf4_dq.hip): stored block of n 8-bit scales.
struct DqLayout {
  size_t scale_off, mean_off, bytes;
};
DqLayout dq_layout(int64_t n);
// block <- double quantisation of the n float32 scales c
ql_status launch_dq_quant(const float* c, int64_t n, uint8_t* block, hipStream_t st);
// Expansion of several blocks back to float32 scales, one launch.
constexpr int kMaxDq = 8;
struct DqExpandArgs {
  const uint8_t* src[kMaxDq];
  size_t scale_off[kMaxDq], mean_off[kMaxDq];
  float* dst[kMaxDq];
  int64_t end[kMaxDq];  // cumulative scale counts
  int32_t nblk;
};
ql_status launch_dq_expand(const DqExpandArgs& a, hipStream_t st);

// Segment of a fused NF4 GEMM: one frozen projection with its LoRA factors.
struct FwdSeg {
  const uint8_t* packed;  // [N x K/2]
  const float* absmax;    // [N x K/64]
  const uint16_t* U;      // bf16 [M x r] (row stride r)
  const uint16_t* B;      // bf16 [N x r]
  void* out;              // [M x ldo] at column col0
  const uint16_t* resid;  // optional bf16 residual with the same layout as out
  int64_t N;
  int64_t ldo, col0;
};

constexpr int kMaxSegs = 3;

struct FwdArgs {
  const uint16_t* X;  // bf16 [M x ldx], logical columns 0..K-1 (optionally remapped)
  int64_t M, K, ldx;
  int32_t r;  // 0: adapter off (no LoRA step; U and B unused)
  float s;
  int32_t head_dim, n_rep;  // repeat_kv remap of X's columns (n_rep 0 = none)
  int32_t out_f32;
  int32_t nseg;
  FwdSeg seg[kMaxSegs];
  // Split reduction over K (set by launch_gemm_fwd): nsplit > 1 workgroups
  // per tile write float32 partials, per segment [nsplit][M x N] after the
  // earlier segments' blocks, that a second kernel sums in split order with
  // the residual into out. partial / partial_bytes: the caller's space.
  float* partial;
  size_t partial_bytes;
  int32_t nsplit;
};

// Reduction segment of the dX GEMM: dX += dY_s W_s + s G_s A_s.
struct BwdSeg {
  const uint16_t* dY;     // bf16 [M x N]
  const uint8_t* packed;  // [N x K/2]
  const float* absmax;    // [N x K/64]
  const uint16_t* G;      // bf16 [M x r]
  const uint16_t* A;      // bf16 [r x K]
  int64_t N;
};

struct BwdArgs {
  int64_t M, K;
  int32_t r;
  float s;
  void* out;  // [M x K] bf16 or f32
  int32_t out_f32;
  const uint16_t* resid;
  int32_t nseg;
  BwdSeg seg[kMaxSegs];
  // Split reduction (set by launch_gemm_bwd): nsplit > 1 workgroups share a
  // tile, each over an equal slice of the weight steps (the last also takes
  // the LoRA steps), writing float32 partials [nsplit][M x K] that a second
  // kernel sums in split order. partial / partial_bytes: the caller's space
  // for them (0: no split).
  float* partial;
  size_t partial_bytes;
  int32_t nsplit;
};
// Largest split of a dX GEMM with M rows and K output columns on a chip of at
// most 256 CUs (workspace sizing; 1 = never split): the split fills the chip
// with 256 x 256 tiles when they alone would leave half of it idle.
int bwd_max_split(int64_t M, int64_t K);
inline size_t bwd_partial_bytes(int64_t M, int64_t K) {
  const int s = bwd_max_split(M, K);
  return s > 1 ? (size_t)s * (size_t)M * (size_t)K * 4 : 0;
}

ql_status launch_gemm_fwd(const FwdArgs& a, hipStream_t st);

// Kernel timing (ql_profile_enable): brackets a launch with events when on;
// work is FLOPs or bytes by kernel id.
bool profiling_on();
ql_status profile_begin(hipEvent_t* start, hipEvent_t* stop);
ql_status profile_end(hipEvent_t start, hipEvent_t stop, int kernel, double work);
ql_status launch_gemm_bwd(const BwdArgs& a, hipStream_t st);

// LoRA side products (lora.hip). Both contractions reduce in a fixed order
// (no atomics), so equal inputs give equal bits whatever the stream timing.
//
// Row contraction: out_s[m][j] = bf16(sum_k X[m][k'] Bt_s[j][k]) for the nseg
// projections that share X (k' = k, or its repeat_kv remap). A launch takes up
// to kMaxRowProb problems of the same kind; the launcher fills the fields
// below the line.
struct RowProb {
  const uint16_t* X;  // bf16 [M x ldx]
  int64_t M, K, ldx;
  int32_t head_dim, n_rep;
  int32_t r;  // columns per projection (1..64)
  int32_t nseg;
  const uint16_t* Bt[kMaxSegs];  // bf16 [r x K]
  uint16_t* out[kMaxSegs];       // bf16 [M x r]
  // SwiGLU producer modes (RowArgs::mode, rows of stride ldx, no remap):
  //  1: Xin = gate, up; X := act = swiglu(gate, up), stored to Xout[0]; nseg 1
  //  2: Xin = gate, up, dact; dg, du stored to Xout[0], Xout[1]; projection 0
  //     contracts dg, projection 1 du (nseg 2)
  // RMSNorm producer mode:
  //  3: X = h; X := rmsnorm(h) (unit gain, eps), stored to Xout[0] with the
  //     bits of the standalone RMSNorm; no remap
  const uint16_t* Xin[3];
  uint16_t* Xout[2];
  float eps;
  // ---- launcher
  float* part;  // float32 [nsplit][M][r * nseg] when nsplit > 1
  int32_t nsplit, tile0, rtile0;
};
constexpr int kMaxRowProb = 2;
struct RowArgs {
  int32_t nprob;
  int32_t mode;  // 0: plain X; 1, 2: SwiGLU producers; 3: RMSNorm producer (see RowProb)
  RowProb p[kMaxRowProb];
};
// Largest rank the SwiGLU-backward producer mode takes (two projections'
// accumulators per wave); larger ranks use the elementwise kernel.
constexpr int kSwigluBwdMaxR = 32;
// Workspace of one row problem (float32 split partials; 0 if unsplit).
size_t rowc_ws_bytes(int64_t M, int64_t K, int32_t np);
ql_status launch_rowc(RowArgs a, void* ws, size_t ws_bytes, hipStream_t st);

// Column contraction: out_s[j][c] = s * sum_m Z[m][c'] V_s[m][j] (+ out_s if
// accumulate), c' = c or its repeat_kv remap; transpose_out stores
// out_s[c * r + j] instead. M == 0 writes zeros (keeps out_s if accumulate).
struct ColProb {
  const uint16_t* Z;  // bf16 [M x ldz]
  int64_t M, C, ldz;
  int32_t head_dim, n_rep;
  int32_t r, nseg;
  const uint16_t* V[kMaxSegs];  // bf16 [M x r]
  float* out[kMaxSegs];
  float s;
  int32_t transpose_out, accumulate;
  // ---- launcher
  float* part;  // float32 [nsplit][nseg][C * r] when nsplit > 1
  int64_t rows_per_split;
  int32_t nsplit, tile0, rtile0;
};
constexpr int kMaxColProb = 14;
struct ColArgs {
  int32_t nprob;
  ColProb p[kMaxColProb];
};
size_t colc_ws_bytes(int64_t M, int64_t C, int32_t np);
ql_status launch_colc(ColArgs a, void* ws, size_t ws_bytes, hipStream_t st);

// out_i = in_i^T (bf16 [rows x cols] -> [cols x rows], rows % 8 == 0, outputs
// 16-byte aligned) for up to kMaxTrans matrices.
constexpr int kMaxTrans = 6;
struct TransArgs {
  int32_t n;
  const uint16_t* in[kMaxTrans];
  uint16_t* out[kMaxTrans];
  int64_t rows[kMaxTrans], cols[kMaxTrans];
  int64_t end[kMaxTrans];  // launcher: cumulative counts of 8-element output groups
};
ql_status launch_transpose_bf16(TransArgs a, hipStream_t st);
ql_status launch_zero_f32(float* p, int64_t n, hipStream_t st);

// Glue of the decoder-layer stand-in.
ql_status launch_rmsnorm_fwd(const uint16_t* h, int64_t M, int64_t H, float eps, uint16_t* out,
                             hipStream_t st);
// out = bf16(resid + d/dh RMSNorm(h) applied to dn)
ql_status launch_rmsnorm_bwd(const uint16_t* h, const uint16_t* dn, const uint16_t* resid,
                             int64_t M, int64_t H, float eps, uint16_t* out, hipStream_t st);
ql_status launch_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* act,
                            hipStream_t st);
ql_status launch_swiglu_bwd(const uint16_t* g, const uint16_t* u, const uint16_t* dact, int64_t n,
                            uint16_t* dg, uint16_t* du, hipStream_t st);
// dv[m][g*d + i] = bf16(sum_j da[m][(g*n_rep + j)*d + i]), da float32 [M x H]
ql_status launch_repeat_kv_bwd(const float* da, int64_t M, int64_t H, int64_t kv, int32_t head_dim,
                               uint16_t* dv, hipStream_t st);

}  // namespace ql
