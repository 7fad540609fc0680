// Fused NF4-dequant bf16 MFMA GEMMs for gfx950.
//
// Forward  (NT): Y[M x N]  = X[M x K] W[N x K]^T + U[M x r] (sB)[N x r]^T
// Backward (NN): dX[M x K] = sum_seg dY[M x N] W[N x K] + G[M x r] (sA)[r x K]
//
// W is never materialised: the tile loader reads the packed 4-bit codes and
// the block's float32 absmax from global memory, decodes each element to
// bf16(fl32(level[code] * absmax)) in registers, and writes the bf16 tile to
// LDS, from where the MFMAs read it. This replaces the per-layer dequant pass
// that the Soup README ("Citing Soup", v3 retraction) measures as streaming's
// largest own cost. The LoRA adapter's rank-r product is one more K-step of
// the same loop (K-concatenation [X | U] [W | sB]^T), so y is written once.
//
// Tiles: 128 x 128 outputs per workgroup of 256 threads (4 waves, 2 x 2, each
// 64 x 64 = 4 x 4 MFMA 16x16x32 tiles), K-step 64 = one NF4 block, two LDS
// stages of 32 KB (A and B tiles of 128 rows x 64 bf16). LDS rows are 128 B,
// split in eight 16-B chunks; chunk c of row r is stored at c ^ (r & 7) so the
// 16-B fragment reads of eight consecutive rows hit distinct banks.
// Workgroups are mapped XCD-aware: the hardware deals workgroups round-robin
// to the 8 XCDs, so consecutive logical tiles (the M-tiles of one W tile) are
// made to land on one XCD and share its L2.
#include "ql_internal.h"

namespace ql {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int NT = 256;
constexpr int TILE_BYTES = 128 * 128;          // 128 rows x 64 bf16
constexpr int STAGE_BYTES = 2 * TILE_BYTES;    // A + B
constexpr int LDS_BYTES = 2 * STAGE_BYTES + 64;  // two stages + level table

__device__ __forceinline__ int swz(int row, int chunk) { return (row << 7) + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t n) {
  const uint32_t q = n >> 3, rem = n & 7;
  const uint32_t xcd = bid & 7, local = bid >> 3;
  return xcd * q + (xcd < rem ? xcd : rem) + local;
}

// logical column k of X -> physical column with the repeat_kv head remap
__device__ __forceinline__ int64_t remap_col(int64_t k, int head_dim, int n_rep) {
  if (n_rep <= 0) return k;
  const int64_t head = k / head_dim, i = k - head * head_dim;
  return (head / n_rep) * head_dim + i;
}

// Decode 8 codes of one dword (element 2i in the high nibble of byte i) with a
// float32 scale into 4 dwords of bf16 pairs, element order preserved.
__device__ __forceinline__ uint4 decode8(uint32_t p, float sc, const float* lv) {
  uint4 q;
  q.x = pack_bf16x2(lv[(p >> 4) & 15u] * sc, lv[p & 15u] * sc);
  q.y = pack_bf16x2(lv[(p >> 12) & 15u] * sc, lv[(p >> 8) & 15u] * sc);
  q.z = pack_bf16x2(lv[(p >> 20) & 15u] * sc, lv[(p >> 16) & 15u] * sc);
  q.w = pack_bf16x2(lv[(p >> 28) & 15u] * sc, lv[(p >> 24) & 15u] * sc);
  return q;
}

// The MFMA core: one K-step of 64 from LDS stage `st` into the 4 x 4 accumulators.
__device__ __forceinline__ void mma_step(const uint8_t* st, f32x4_t (&acc)[4][4], int wm, int wn,
                                         int lane) {
  const uint8_t* As = st;
  const uint8_t* Bs = st + TILE_BYTES;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8_t a[4], b[4];
    const int ch = ks * 4 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *(const bf16x8_t*)(As + swz(wm * 64 + i * 16 + (lane & 15), ch));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *(const bf16x8_t*)(Bs + swz(wn * 64 + j * 16 + (lane & 15), ch));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// A operand rows (bf16, reduction-contiguous) of a main K-step: 4 chunks of
// 16 B per thread. Rows at or past M are zero.
__device__ __forceinline__ void load_a_main(uint4 (&ar)[4], const uint16_t* X, int64_t ldx, int64_t M,
                                            int64_t m0, int64_t k0, int head_dim, int n_rep, int t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + NT * i;
    const int row = c >> 3, ch = c & 7;
    const int64_t m = m0 + row;
    if (m < M) {
      const int64_t col = remap_col(k0 + ch * 8, head_dim, n_rep);
      ar[i] = *(const uint4*)(X + m * ldx + col);
    } else {
      ar[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

// Same tile for a reduction-contiguous operand with a column limit (ncols % 16 == 0).
__device__ __forceinline__ void load_a_lim(uint4 (&ar)[4], const uint16_t* X, int64_t ldx, int64_t M,
                                           int64_t m0, int64_t k0, int64_t ncols, int t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + NT * i;
    const int row = c >> 3, ch = c & 7;
    const int64_t m = m0 + row;
    const int64_t k = k0 + ch * 8;
    if (m < M && k < ncols)
      ar[i] = *(const uint4*)(X + m * ldx + k);
    else
      ar[i] = make_uint4(0, 0, 0, 0);
  }
}

// A operand of the LoRA step: rows of a [M x r] bf16 matrix, zero past r.
__device__ __forceinline__ void load_a_rank(uint4 (&ar)[4], const uint16_t* U, int r, int64_t M,
                                            int64_t m0, int t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + NT * i;
    const int row = c >> 3, ch = c & 7;
    const int64_t m = m0 + row;
    uint32_t w[4] = {0, 0, 0, 0};
    if (m < M) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = ch * 8 + e;
        const uint32_t h = j < r ? (uint32_t)U[m * r + j] : 0u;
        w[e >> 1] |= h << ((e & 1) * 16);
      }
    }
    ar[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ void store_a(uint8_t* As, const uint4 (&ar)[4], int t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + NT * i;
    *(uint4*)(As + swz(c >> 3, c & 7)) = ar[i];
  }
}

__device__ __forceinline__ void zero_acc(f32x4_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// Output of a 16x16 MFMA tile: lane l holds rows 4*(l/16)+v, v = 0..3, column l%16.
template <typename F>
__device__ __forceinline__ void for_each_out(const f32x4_t (&acc)[4][4], int wm, int wn, int lane, F f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        f(wm * 64 + i * 16 + 4 * (lane >> 4) + v, wn * 64 + j * 16 + (lane & 15), acc[i][j][v]);
}

// --------------------------------------------------------------- forward
__global__ __launch_bounds__(NT, 2) void k_gemm_fwd(const FwdArgs a, int tiles_m, int tiles_total,
                                                    int seg_tile0_1, int seg_tile0_2) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* lv = (float*)(smem + 2 * STAGE_BYTES);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
  if (t < 16) lv[t] = __builtin_bit_cast(float, kNF4LevelBits[t]);

  const int tile = (int)xcd_remap(blockIdx.x, (uint32_t)tiles_total);
  const int sg = tile >= seg_tile0_2 ? 2 : (tile >= seg_tile0_1 ? 1 : 0);
  const int local = tile - (sg == 2 ? seg_tile0_2 : (sg == 1 ? seg_tile0_1 : 0));
  const FwdSeg& S = a.seg[sg];
  const int64_t m0 = (int64_t)(local % tiles_m) * BM;
  const int64_t n0 = (int64_t)(local / tiles_m) * BN;
  const int64_t K = a.K, KT = K / BK;
  const int64_t kb = K / 64;  // absmax per row
  const int steps = (int)KT + 1;

  // B loader coordinates: one row, 32 codes (16 B) per thread
  const int brow = t >> 1, bhalf = t & 1;
  const int64_t bn = n0 + brow;
  const bool bvalid = bn < S.N;

  uint4 ar[4];
  uint4 bcode;
  float bsc;

  auto load = [&](int step) {
    if (step < KT) {
      const int64_t k0 = (int64_t)step * BK;
      load_a_main(ar, a.X, a.ldx, a.M, m0, k0, a.head_dim, a.n_rep, t);
      if (bvalid) {
        bcode = *(const uint4*)(S.packed + bn * (K / 2) + k0 / 2 + 16 * bhalf);
        bsc = S.absmax[bn * kb + step];
      } else {
        bcode = make_uint4(0, 0, 0, 0);
        bsc = 0.f;
      }
    } else {
      load_a_rank(ar, S.U, a.r, a.M, m0, t);
    }
  };
  auto store = [&](int step, uint8_t* st) {
    store_a(st, ar, t);
    uint8_t* Bs = st + TILE_BYTES;
    if (step < KT) {
      const uint32_t p[4] = {bcode.x, bcode.y, bcode.z, bcode.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) *(uint4*)(Bs + swz(brow, 4 * bhalf + d)) = decode8(p[d], bsc, lv);
    } else {
      // (s B)[n][j] for j < r, zero past r; 32 columns per thread
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j0 = 32 * bhalf + 8 * d + 2 * e;
          float f0 = 0.f, f1 = 0.f;
          if (bvalid && j0 < a.r) f0 = a.s * bf16_to_f32(S.B[bn * a.r + j0]);
          if (bvalid && j0 + 1 < a.r) f1 = a.s * bf16_to_f32(S.B[bn * a.r + j0 + 1]);
          wv[e] = pack_bf16x2(f0, f1);
        }
        *(uint4*)(Bs + swz(brow, 4 * bhalf + d)) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    }
  };

  f32x4_t acc[4][4];
  zero_acc(acc);
  __syncthreads();  // level table visible
  load(0);
  store(0, smem);
  __syncthreads();
  for (int step = 0; step < steps; ++step) {
    uint8_t* cur = smem + (step & 1) * STAGE_BYTES;
    uint8_t* nxt = smem + ((step + 1) & 1) * STAGE_BYTES;
    const bool more = step + 1 < steps;
    if (more) load(step + 1);
    mma_step(cur, acc, wm, wn, lane);
    if (more) store(step + 1, nxt);
    __syncthreads();
  }

  // epilogue
  const int64_t M = a.M, N = S.N;
  for_each_out(acc, wm, wn, lane, [&](int r, int c, float v) {
    const int64_t m = m0 + r, n = n0 + c;
    if (m < M && n < N) {
      const int64_t o = m * S.ldo + S.col0 + n;
      if (S.resid) v += bf16_to_f32(S.resid[o]);
      if (a.out_f32)
        ((float*)S.out)[o] = v;
      else
        ((uint16_t*)S.out)[o] = f32_to_bf16(v);
    }
  });
}

// --------------------------------------------------------------- backward dX
__global__ __launch_bounds__(NT, 2) void k_gemm_bwd(const BwdArgs a, int tiles_m, int tiles_total) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* lv = (float*)(smem + 2 * STAGE_BYTES);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
  if (t < 16) lv[t] = __builtin_bit_cast(float, kNF4LevelBits[t]);

  const int tile = (int)xcd_remap(blockIdx.x, (uint32_t)tiles_total);
  const int64_t m0 = (int64_t)(tile % tiles_m) * BM;
  const int64_t k0 = (int64_t)(tile / tiles_m) * BN;  // output columns (in-features)
  const int64_t K = a.K, kb = K / 64;

  // step enumeration: per segment ceil(N/64) weight steps then one LoRA step
  const int ns0 = (int)((a.seg[0].N + BK - 1) / BK) + 1;
  const int ns1 = a.nseg > 1 ? (int)((a.seg[1].N + BK - 1) / BK) + 1 : 0;
  const int ns2 = a.nseg > 2 ? (int)((a.seg[2].N + BK - 1) / BK) + 1 : 0;
  const int steps = ns0 + ns1 + ns2;

  // transposed-decode coordinates: 4 rows (n) x 8 columns (k) per thread
  const int cg = t & 15, rg = t >> 4;
  const int64_t kcol = k0 + 8 * cg;
  const bool kvalid = kcol < K;
  // LoRA-step B coordinates: one column k, 32 ranks
  const int lk = t & 127, lhalf = t >> 7;

  uint4 ar[4];
  uint32_t bp[4];
  float bs[4];

  // step -> (segment, index within it); the last index of a segment is its LoRA step
  auto locate = [&](int step, int& sg, int& j, int& nst) {
    if (step < ns0) { sg = 0; j = step; nst = ns0; }
    else if (step < ns0 + ns1) { sg = 1; j = step - ns0; nst = ns1; }
    else { sg = 2; j = step - ns0 - ns1; nst = ns2; }
  };
  auto load = [&](int step) {
    int sg, j, nst;
    locate(step, sg, j, nst);
    const BwdSeg& S = a.seg[sg];
    if (j < nst - 1) {
      const int64_t n0 = (int64_t)j * BK;
      load_a_lim(ar, S.dY, S.N, a.M, m0, n0, S.N, t);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + 4 * rg + i;
        if (n < S.N && kvalid) {
          bp[i] = *(const uint32_t*)(S.packed + n * (K / 2) + kcol / 2);
          bs[i] = S.absmax[n * kb + kcol / 64];
        } else {
          bp[i] = 0;
          bs[i] = 0.f;
        }
      }
    } else {
      load_a_rank(ar, S.G, a.r, a.M, m0, t);
    }
  };
  auto store = [&](int step, uint8_t* st) {
    int sg, j, nst;
    locate(step, sg, j, nst);
    const BwdSeg& S = a.seg[sg];
    store_a(st, ar, t);
    uint8_t* Bs = st + TILE_BYTES;
    if (j < nst - 1) {
      // element e of the dword: byte e/2, high nibble when e is even
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 8 * (e >> 1) + ((e & 1) ? 0 : 4);
        const float f0 = lv[(bp[0] >> sh) & 15u] * bs[0];
        const float f1 = lv[(bp[1] >> sh) & 15u] * bs[1];
        const float f2 = lv[(bp[2] >> sh) & 15u] * bs[2];
        const float f3 = lv[(bp[3] >> sh) & 15u] * bs[3];
        const int kr = 8 * cg + e;
        uint2 v;
        v.x = pack_bf16x2(f0, f1);
        v.y = pack_bf16x2(f2, f3);
        *(uint2*)(Bs + (kr << 7) + ((((rg >> 1) ^ (kr & 7))) << 4) + ((rg & 1) << 3)) = v;
      }
    } else {
      // (s A)^T: row k of the tile holds s * A[j][k] for j < r
      const int64_t k = k0 + lk;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = 32 * lhalf + 8 * d + 2 * e;
          float f0 = 0.f, f1 = 0.f;
          if (k < K && jj < a.r) f0 = a.s * bf16_to_f32(S.A[(int64_t)jj * K + k]);
          if (k < K && jj + 1 < a.r) f1 = a.s * bf16_to_f32(S.A[(int64_t)(jj + 1) * K + k]);
          wv[e] = pack_bf16x2(f0, f1);
        }
        *(uint4*)(Bs + swz(lk, 4 * lhalf + d)) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    }
  };

  f32x4_t acc[4][4];
  zero_acc(acc);
  __syncthreads();
  load(0);
  store(0, smem);
  __syncthreads();
  for (int step = 0; step < steps; ++step) {
    uint8_t* cur = smem + (step & 1) * STAGE_BYTES;
    uint8_t* nxt = smem + ((step + 1) & 1) * STAGE_BYTES;
    const bool more = step + 1 < steps;
    if (more) load(step + 1);
    mma_step(cur, acc, wm, wn, lane);
    if (more) store(step + 1, nxt);
    __syncthreads();
  }

  const int64_t M = a.M;
  for_each_out(acc, wm, wn, lane, [&](int r, int c, float v) {
    const int64_t m = m0 + r, k = k0 + c;
    if (m < M && k < K) {
      const int64_t o = m * K + k;
      if (a.resid) v += bf16_to_f32(a.resid[o]);
      if (a.out_f32)
        ((float*)a.out)[o] = v;
      else
        ((uint16_t*)a.out)[o] = f32_to_bf16(v);
    }
  });
}

#define QL_TRY_PROF(expr)        \
  do {                           \
    ql_status rc_ = (expr);      \
    if (rc_ != QL_OK) return rc_; \
  } while (0)

bool g_attr_set[64] = {};

ql_status ensure_attrs() {
  int dev = 0;
  QL_HIP_CHECK(hipGetDevice(&dev));
  if (dev >= 0 && dev < 64 && !g_attr_set[dev]) {
    QL_HIP_CHECK(hipFuncSetAttribute((const void*)k_gemm_fwd,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES));
    QL_HIP_CHECK(hipFuncSetAttribute((const void*)k_gemm_bwd,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES));
    g_attr_set[dev] = true;
  }
  return QL_OK;
}

}  // namespace

ql_status launch_gemm_fwd(const FwdArgs& a, hipStream_t st) {
  if (a.M == 0) return QL_OK;
  ql_status rc = ensure_attrs();
  if (rc != QL_OK) return rc;
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  int start[kMaxSegs + 1] = {0, 0, 0, 0};
  for (int s = 0; s < a.nseg; ++s) start[s + 1] = start[s] + tiles_m * (int)((a.seg[s].N + BN - 1) / BN);
  for (int s = a.nseg; s < kMaxSegs; ++s) start[s + 1] = start[s];
  const int total = start[a.nseg];
  if (total == 0) return QL_OK;
  // unused segment starts point past the end so no tile maps to them
  const int s1 = a.nseg > 1 ? start[1] : total + 1;
  const int s2 = a.nseg > 2 ? start[2] : total + 1;
  void* tok = nullptr;
  const bool prof = profiling_on();
  if (prof) QL_TRY_PROF(profile_begin(st, &tok));
  hipLaunchKernelGGL(k_gemm_fwd, dim3(total), dim3(NT), LDS_BYTES, st, a, tiles_m, total, s1, s2);
  QL_HIP_CHECK(hipGetLastError());
  if (prof) {
    double flop = 0;
    for (int s = 0; s < a.nseg; ++s) flop += 2.0 * (double)a.M * (double)a.seg[s].N * (double)(a.K + a.r);
    QL_TRY_PROF(profile_end(st, tok, QL_KERNEL_GEMM_FWD, flop));
  }
  return QL_OK;
}

ql_status launch_gemm_bwd(const BwdArgs& a, hipStream_t st) {
  if (a.M == 0) return QL_OK;
  ql_status rc = ensure_attrs();
  if (rc != QL_OK) return rc;
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const int total = tiles_m * (int)((a.K + BN - 1) / BN);
  if (total == 0) return QL_OK;
  void* tok = nullptr;
  const bool prof = profiling_on();
  if (prof) QL_TRY_PROF(profile_begin(st, &tok));
  hipLaunchKernelGGL(k_gemm_bwd, dim3(total), dim3(NT), LDS_BYTES, st, a, tiles_m, total);
  QL_HIP_CHECK(hipGetLastError());
  if (prof) {
    double flop = 0;
    for (int s = 0; s < a.nseg; ++s) flop += 2.0 * (double)a.M * (double)a.K * (double)(a.seg[s].N + a.r);
    QL_TRY_PROF(profile_end(st, tok, QL_KERNEL_GEMM_BWD, flop));
  }
  return QL_OK;
}

}  // namespace ql
