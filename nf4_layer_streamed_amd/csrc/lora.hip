// LoRA side products of rank r (r <= 64): the skinny contractions around the
// fused NF4 GEMMs. Only A and B train, and the adapter adds s (x A^T) B^T with
// s = alpha / r (blog "How does Soup train an 8B model on a 4 GB GPU?").
//
//  row:     out[m][j] = bf16( sum_k X[m][k] Bt[j][k] )      U = x A^T, G = dY B
//  column:  out[j][c] = s * sum_m Z[m][c] V[m][j]           dA = s G^T x, dB = s dY^T U
//
// Each reads one large bf16 operand once and does 2 np FLOP per element of it
// (np = r times the projections sharing the operand): bound by HBM. Both run
// on MFMA 16x16x32 bf16, since float32 FMA alone would need np FLOP per byte
// read, more than the vector ALUs sustain at the full HBM rate for np = 16.
//
// Row contraction: a workgroup owns 16 rows and one slice (split) of the
// reduction; its waves interleave over 128-element steps, each lane loading
// 16 bytes of X per MFMA (row = lane % 16) and the next step's operands while
// the current step multiplies. The waves' sums meet in LDS in wave order.
//
// Column contraction: the reduction runs over rows while Z is row-major, so a
// 32-row x 64-column tile goes through a wave-private LDS region and comes
// back transposed with ds_read_b64_tr_b16 (gfx950): within each group of 16
// lanes, lane 4a + b addresses an 8-byte piece (row a, columns 4b..4b+3) and
// lane 4b + e receives element a of it, so every lane holds consecutive rows
// of one column, the MFMA operand layout; V's rows are staged the same way.
// A workgroup owns 64 columns and one slice of the rows; its four waves
// interleave over 32-row steps and add their sums in LDS in wave order.
//
// A split writes float32 partials that a second kernel adds in split order.
// Every sum has a fixed order, so equal inputs give equal bits. One launch can
// carry several independent problems (all LoRA gradients of a layer).
#include <hip/hip_ext.h>

#include "ql_internal.h"

namespace ql {
namespace {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

// floor(x / d) for x < 2^24, d >= 1: a float32 estimate is off by at most one
__device__ __forceinline__ uint32_t udiv24(uint32_t x, uint32_t d, float inv_d) {
  uint32_t q = (uint32_t)((float)x * inv_d);
  const int32_t rem = (int32_t)(x - q * d);
  if (rem < 0) --q;
  else if (rem >= (int32_t)d) ++q;
  return q;
}

// physical column of logical column k of repeat_kv(x): head k / head_dim
// reads kv head (k / head_dim) / n_rep (n_rep 0: identity)
__device__ __forceinline__ int64_t remap_col(int64_t k, int head_dim, int n_rep) {
  if (n_rep <= 0) return k;
  const uint32_t hd = (uint32_t)head_dim;
  const uint32_t head = udiv24((uint32_t)k, hd, 1.f / (float)hd);
  const uint32_t i = (uint32_t)k - head * hd;
  return (int64_t)udiv24(head, (uint32_t)n_rep, 1.f / (float)n_rep) * hd + i;
}

template <typename T>
__device__ __forceinline__ T pick3(int i, T a, T b, T c) {
  return i == 0 ? a : (i == 1 ? b : c);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// v if keep, else zeros, without a branch (a select here tends to become one)
__device__ __forceinline__ uint4 keep_if(uint4 v, bool keep) {
  const uint32_t m = 0u - (uint32_t)keep;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

__device__ __forceinline__ i16x4_t lds_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p);
}

// ------------------------------------------------------- row contraction
constexpr int RC_ROWS = 16;
constexpr int RC_STEP = 128;  // reduction elements per wave step (4 MFMAs)
constexpr int RC_WAVES = 4;
static_assert(RC_ROWS % RC_WAVES == 0, "the RMSNorm statistics give each wave whole rows");

// MODE 0: X is read. MODE 1: X = SwiGLU(gate, up) is made from Xin and
// stored. MODE 2: dg, du are made from gate, up, dact and stored; column
// groups 0 .. NCG/2-1 contract dg with Bt[0], the rest du with Bt[1].
// MODE 3: X = RMSNorm(Xin = h) is made and stored: the workgroup first
// computes its rows' statistics exactly as the standalone RMSNorm does (one
// wave per row, the same sums), then scales each chunk it contracts.
template <int NCG, int MODE>
__global__ __launch_bounds__(64 * RC_WAVES) void k_rowc(const RowArgs a) {
  constexpr int W = RC_WAVES;
  constexpr int NIN = MODE == 1 ? 2 : (MODE == 2 ? 3 : 1);  // operand streams loaded per chunk
  constexpr int NCGS = MODE == 2 ? NCG / 2 : NCG;           // column groups per projection (modes 1, 2)
  __shared__ f32x4_t red[(W - 1) * NCG][64];
  // w is wave-uniform; readfirstlane tells the compiler, so the step loops stay scalar
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int p = 0;
  for (int i = 1; i < a.nprob; ++i)
    if ((int)blockIdx.x >= a.p[i].tile0) p = i;
  const RowProb& P = a.p[p];
  const int64_t M = P.M, K = P.K;
  const int r = P.r, np = r * P.nseg, ns = P.nsplit;
  const int t = (int)blockIdx.x - P.tile0;
  const int tile = t / ns, sp = t - tile * ns;
  const int64_t m0 = (int64_t)tile * RC_ROWS;
  const int64_t nsteps = (K + RC_STEP - 1) / RC_STEP;
  const int64_t s_lo = nsteps * sp / ns, s_hi = nsteps * (sp + 1) / ns;
  const int g = lane >> 4, s16 = lane & 15;
  // rows past M read row 0: MFMA output row i depends on operand row i only,
  // and those rows are never stored
  const int64_t m = m0 + s16;
  const bool mrow = m < M;
  const int64_t roff = (mrow ? m : 0) * P.ldx;
  const uint16_t* xin[NIN];
#pragma unroll
  for (int i = 0; i < NIN; ++i) xin[i] = (MODE == 0 || MODE == 3 ? P.X : P.Xin[i]) + roff;
  // output column of group c for this lane: projection sg, column j
  auto colmap = [&](int c, int& sg, int& j) -> bool {
    if (MODE == 0 || MODE == 3) {
      const int jt = 16 * c + s16;
      sg = jt < np ? jt / r : 0;
      j = jt < np ? jt - sg * r : 0;
      return jt < np;
    }
    sg = c / NCGS;
    j = 16 * (c - sg * NCGS) + s16;
    const bool ok = j < r;
    if (!ok) j = 0;
    return ok;
  };
  const uint16_t* bcol[NCG];
#pragma unroll
  for (int c = 0; c < NCG; ++c) {  // columns past r read row 0 (never stored)
    int sg, j;
    colmap(c, sg, j);
    bcol[c] = pick3(sg, P.Bt[0], P.Bt[1], P.Bt[2]) + (int64_t)j * K;
  }
  float rs = 0.f;  // MODE 3: the RMSNorm scale of this lane's row, m0 + lane % 16
  // Loads have no branches (a branch around them would make the compiler
  // wait for the prefetch too): reduction elements past K load element 0 and
  // are zeroed in both operands before use.
  auto load = [&](int64_t st, uint4 (&xa)[NIN][4], uint4 (&xb)[NCG][4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t k = st * RC_STEP + 32 * q + 8 * g;
      const int64_t kc = k < K ? k : 0;
      const int64_t kx = MODE == 0 ? remap_col(kc, P.head_dim, P.n_rep) : kc;
#pragma unroll
      for (int i = 0; i < NIN; ++i) xa[i][q] = *(const uint4*)(xin[i] + kx);
#pragma unroll
      for (int c = 0; c < NCG; ++c) xb[c][q] = *(const uint4*)(bcol[c] + kc);
    }
  };
  f32x4_t acc[NCG];
#pragma unroll
  for (int c = 0; c < NCG; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](int64_t st, const uint4 (&xa)[NIN][4], const uint4 (&xb)[NCG][4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t k = st * RC_STEP + 32 * q + 8 * g;
      const bool in = k < K;
      uint4 x0 = xa[0][q], x1 = x0;
      if (MODE == 1) {
        x0 = swiglu_act8(xa[0][q], xa[1][q]);
        if (in && mrow) *(uint4*)(P.Xout[0] + roff + k) = x0;
      } else if (MODE == 3) {
        x0 = scale8(xa[0][q], rs);
        if (in && mrow) *(uint4*)(P.Xout[0] + roff + k) = x0;
      } else if (MODE == 2) {
        swiglu_grad8(xa[0][q], xa[1][q], xa[2][q], x0, x1);
        if (in && mrow) {
          *(uint4*)(P.Xout[0] + roff + k) = x0;
          *(uint4*)(P.Xout[1] + roff + k) = x1;
        }
      }
      x0 = keep_if(x0, in);
      x1 = keep_if(x1, in);
#pragma unroll
      for (int c = 0; c < NCG; ++c) {
        const uint4 xc = (MODE == 2 && c >= NCGS) ? x1 : x0;
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xc), as_bf16x8(keep_if(xb[c][q], in)), acc[c],
                                                         0, 0, 0);
      }
    }
  };
  // two register sets take turns (no copies, which would wait for the
  // prefetch); a step past the end reloads the current one (cache hits)
  int64_t st = s_lo + w;
  uint4 xa0[NIN][4], xb0[NCG][4], xa1[NIN][4], xb1[NCG][4];
  if constexpr (MODE == 3) {
    // the first chunk is in flight meanwhile (a load of any step stays in
    // bounds); wave w sums rows w, w + W, ... of the tile, each in the order
    // of the standalone kernel; rows past M repeat row M - 1 (never stored)
    load(st, xa0, xb0);
    __shared__ float rsh[RC_ROWS];
    constexpr int RPW = RC_ROWS / W;
    const uint4* hr[RPW];
    float ss[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int64_t mr = m0 + w + W * j;
      hr[j] = (const uint4*)(P.X + (mr < M ? mr : M - 1) * P.ldx);
      ss[j] = 0.f;
    }
    for (int64_t q = lane; q < K / 8; q += 64) {
      uint4 v[RPW];
#pragma unroll
      for (int j = 0; j < RPW; ++j) v[j] = hr[j][q];
#pragma unroll
      for (int j = 0; j < RPW; ++j) add_squares8(v[j], ss[j]);
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const float v = rms_scale(wave_sum(ss[j]), K, P.eps);
      if (lane == 0) rsh[w + W * j] = v;
    }
    __syncthreads();
    rs = rsh[s16];
  }
  if (st < s_hi) {
    if constexpr (MODE != 3) load(st, xa0, xb0);
    while (true) {
      load(st + W < s_hi ? st + W : st, xa1, xb1);
      mma(st, xa0, xb0);
      if (st + W >= s_hi) break;
      st += W;
      load(st + W < s_hi ? st + W : st, xa0, xb0);
      mma(st, xa1, xb1);
      if (st + W >= s_hi) break;
      st += W;
    }
  }
  if (w > 0) {
#pragma unroll
    for (int c = 0; c < NCG; ++c) red[(w - 1) * NCG + c][lane] = acc[c];
  }
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int q = 0; q < W - 1; ++q)
#pragma unroll
    for (int c = 0; c < NCG; ++c) acc[c] += red[q * NCG + c][lane];
  // lane holds rows 4 (lane / 16) + v, column lane % 16 of each 16 x 16 tile
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    int sg, j;
    if (!colmap(c, sg, j)) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = m0 + 4 * g + v;
      if (mm >= M) continue;
      if (ns == 1) {
        uint16_t* o = pick3(sg, P.out[0], P.out[1], P.out[2]);
        o[mm * r + j] = f32_to_bf16(acc[c][v]);
      } else {
        P.part[((int64_t)sp * M + mm) * np + sg * r + j] = acc[c][v];
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_rowc_reduce(const RowArgs a) {
  int p = 0;
  for (int i = 1; i < a.nprob; ++i)
    if ((int)blockIdx.x >= a.p[i].rtile0) p = i;
  const RowProb& P = a.p[p];
  const int r = P.r, np = r * P.nseg;
  const int64_t idx = (int64_t)((int)blockIdx.x - P.rtile0) * 256 + threadIdx.x;
  if (idx >= P.M * np) return;
  const int64_t m = idx / np;
  const int jt = (int)(idx - m * np);
  float s = 0.f;
  for (int sp = 0; sp < P.nsplit; ++sp) s += P.part[((int64_t)sp * P.M + m) * np + jt];
  const int sg = jt / r, j = jt - sg * r;
  uint16_t* o = pick3(sg, P.out[0], P.out[1], P.out[2]);
  o[m * r + j] = f32_to_bf16(s);
}

// ---------------------------------------------------- column contraction
constexpr int CC_COLS = 64;
constexpr int CC_ROWS = 32;
constexpr int CC_ZERO = 4096;  // outputs zeroed per workgroup for a problem without rows

// NJ: 16-column groups of V (np <= 16 NJ); VEC: r % 8 == 0, so 8 consecutive
// columns of V lie in one projection and load as 16 bytes.
template <int NJ, bool VEC>
__global__ __launch_bounds__(256) void k_colc(const ColArgs a) {
  // V rows are padded to an odd multiple of 32 bytes: the four rows one
  // transposed read touches per 16 lanes then fall on distinct banks
  constexpr int PV = 32 * (NJ | 1);
  constexpr int ZB = CC_ROWS * 128;     // Z tile: 32 rows x 64 bf16
  constexpr int WB = ZB + CC_ROWS * PV;  // one wave's region
  constexpr int RB = 3 * 4 * NJ * 64 * 16;
  constexpr int LB = 4 * WB > RB ? 4 * WB : RB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LB];
  // w is wave-uniform; readfirstlane tells the compiler, so the step loops stay scalar
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int p = 0;
  for (int i = 1; i < a.nprob; ++i)
    if ((int)blockIdx.x >= a.p[i].tile0) p = i;
  const ColProb& P = a.p[p];
  const int64_t C = P.C;
  const int r = P.r, np = r * P.nseg, ns = P.nsplit;
  const int t = (int)blockIdx.x - P.tile0;
  if (P.M == 0) {  // a gradient that is exactly zero: CC_ZERO outputs per workgroup
    const int64_t n = C * r;
#pragma unroll
    for (int k = 0; k < CC_ZERO / 256; ++k) {
      const int64_t e = (int64_t)t * CC_ZERO + k * 256 + threadIdx.x;
      if (e < n * P.nseg) {
        const int sg = (int)(e / n);
        pick3(sg, P.out[0], P.out[1], P.out[2])[e - sg * n] = 0.f;
      }
    }
    return;
  }
  const int cb = t / ns, sp = t - cb * ns;
  const int64_t c0 = (int64_t)cb * CC_COLS;
  const int64_t r_lo = (int64_t)sp * P.rows_per_split;
  const int64_t r_hi = r_lo + P.rows_per_split < P.M ? r_lo + P.rows_per_split : P.M;
  const int64_t nsteps = (r_hi - r_lo + CC_ROWS - 1) / CC_ROWS;
  uint8_t* zt = smem + w * WB;
  uint8_t* vt = zt + ZB;

  // Z: lane loads rows zr + 8u (u < 4), 16-byte chunk zc of the 64 columns.
  // Columns past C read column 0 (MFMA output row c depends on column c
  // only). Loads have no branches (a branch around them would make the
  // compiler wait for the prefetch too): rows past the slice load row r_lo and
  // are zeroed, with their V rows, when the tile is stored to LDS.
  const int zr = lane >> 3, zc = lane & 7;
  const int64_t zcol = c0 + 8 * zc;
  const uint16_t* zbase = P.Z + remap_col(zcol < C ? zcol : 0, P.head_dim, P.n_rep);
  const int64_t ldz8 = 8 * P.ldz;
  const uint16_t* zlo = zbase + r_lo * P.ldz;
  auto loadZ = [&](int64_t mb, uint4 (&z)[4]) {
    const uint16_t* p0 = zbase + (mb + zr) * P.ldz;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint16_t* pu = mb + zr + 8 * u < r_hi ? p0 + u * ldz8 : zlo;
      z[u] = *(const uint4*)pu;
    }
  };
  // V: chunk q = lane + 64 i is row q / (2 NJ), columns 8 (q % (2 NJ)) .. + 7
  constexpr int VE = VEC ? 4 : 8;  // registers per chunk: 16 bytes, or one element each
  auto loadV = [&](int64_t mb, uint32_t (&v)[NJ][VE]) {
#pragma unroll
    for (int i = 0; i < NJ; ++i) {
      const int q = lane + 64 * i;
      const int row = q / (2 * NJ), jt0 = 8 * (q - row * 2 * NJ);
      const int64_t mm = mb + row < r_hi ? mb + row : r_lo;
      if (VEC) {
        const int jc = jt0 < np ? jt0 : 0;
        const int sg = jc / r, j = jc - sg * r;
        const uint4 x = *(const uint4*)(pick3(sg, P.V[0], P.V[1], P.V[2]) + mm * r + j);
        v[i][0] = x.x; v[i][1] = x.y; v[i][2] = x.z; v[i][3] = x.w;
      } else {
#pragma unroll
        for (int k = 0; k < VE; ++k) {
          const int jc = jt0 + k < np ? jt0 + k : 0;
          const int sg = jc / r, j = jc - sg * r;
          v[i][k] = pick3(sg, P.V[0], P.V[1], P.V[2])[mm * r + j];
        }
      }
    }
  };
  // Z rows are 128 B; chunk zc of row R sits at chunk zc ^ 2 (R & 3), so the
  // four rows of one transposed read cover all banks
  auto stash = [&](int64_t mb, const uint4 (&z)[4], const uint32_t (&v)[NJ][VE]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int R = zr + 8 * u;
      *(uint4*)(zt + R * 128 + ((zc ^ (2 * (R & 3))) << 4)) = keep_if(z[u], mb + R < r_hi);
    }
#pragma unroll
    for (int i = 0; i < NJ; ++i) {
      const int q = lane + 64 * i;
      const int row = q / (2 * NJ), ch = q - row * 2 * NJ, jt0 = 8 * ch;
      const bool rok = mb + row < r_hi;
      uint4 x;
      if (VEC) {
        x = keep_if(make_uint4(v[i][0], v[i][1], v[i][2], v[i][3]), rok && jt0 < np);
      } else {
        uint32_t e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = v[i][k] & (0u - (uint32_t)(rok && jt0 + k < np)) & 0xffffu;
        x = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
      }
      *(uint4*)(vt + row * PV + ch * 16) = x;
    }
  };
  // transposed reads: lane 16 g + 4 ra + cbq addresses rows 8 g + ra (+4),
  // the 4-column piece cbq of a 16-column group
  const int g = lane >> 4, s16 = lane & 15, ra = s16 >> 2, cbq = s16 & 3;
  auto frag_z = [&](int tt) {
    const int ch = 2 * tt + (cbq >> 1);
    const int off = (8 * g + ra) * 128 + ((ch ^ (2 * ra)) << 4) + (cbq & 1) * 8;
    const i16x4_t lo = lds_tr(zt + off), hi = lds_tr(zt + off + 4 * 128);
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  };
  auto frag_v = [&](int jj) {
    const int off = (8 * g + ra) * PV + jj * 32 + cbq * 8;
    const i16x4_t lo = lds_tr(vt + off), hi = lds_tr(vt + off + 4 * PV);
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  };

  f32x4_t acc[4][NJ];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) acc[tt][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](int64_t mb, const uint4 (&z)[4], const uint32_t (&v)[NJ][VE]) {
    // LDS runs one wave's operations in order: these writes land after the
    // previous step's transposed reads
    stash(mb, z, v);
    bf16x8_t bv[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) bv[jj] = frag_v(jj);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const bf16x8_t av = frag_z(tt);
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
        acc[tt][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[jj], acc[tt][jj], 0, 0, 0);
    }
  };
  // two register sets take turns (no copies, which would wait for the
  // prefetch); a step past the end reloads the current one (cache hits)
  int64_t st = w;
  if (st < nsteps) {
    uint4 z0[4], z1[4];
    uint32_t v0[NJ][VE], v1[NJ][VE];
    loadZ(r_lo + st * CC_ROWS, z0);
    loadV(r_lo + st * CC_ROWS, v0);
    while (true) {
      int64_t nx = st + 4 < nsteps ? st + 4 : st;
      loadZ(r_lo + nx * CC_ROWS, z1);
      loadV(r_lo + nx * CC_ROWS, v1);
      mma(r_lo + st * CC_ROWS, z0, v0);
      if (st + 4 >= nsteps) break;
      st += 4;
      nx = st + 4 < nsteps ? st + 4 : st;
      loadZ(r_lo + nx * CC_ROWS, z0);
      loadV(r_lo + nx * CC_ROWS, v0);
      mma(r_lo + st * CC_ROWS, z1, v1);
      if (st + 4 >= nsteps) break;
      st += 4;
    }
  }
  // waves 1..3 hand their sums to wave 0 through LDS (over the tiles)
  __syncthreads();
  f32x4_t* red = (f32x4_t*)smem;
  if (w > 0) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) red[(((w - 1) * 4 + tt) * NJ + jj) * 64 + lane] = acc[tt][jj];
  }
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) acc[tt][jj] += red[((q * 4 + tt) * NJ + jj) * 64 + lane];
  // lane holds columns c0 + 16 tt + 4 g + v, V column 16 jj + lane % 16
  const int64_t CR = C * r;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t c = c0 + 16 * tt + 4 * g + v;
        const int jt = 16 * jj + s16;
        if (c >= C || jt >= np) continue;
        const int sg = jt / r, j = jt - sg * r;
        const int64_t o = P.transpose_out ? c * r + j : j * C + c;
        const float x = acc[tt][jj][v];
        if (ns == 1) {
          float* out = pick3(sg, P.out[0], P.out[1], P.out[2]);
          const float y = P.s * x;
          out[o] = P.accumulate ? out[o] + y : y;
        } else {
          P.part[((int64_t)sp * P.nseg + sg) * CR + o] = x;
        }
      }
}

// Split sums, in split order.
__global__ __launch_bounds__(256) void k_colc_reduce(const ColArgs a) {
  int p = 0;
  for (int i = 1; i < a.nprob; ++i)
    if ((int)blockIdx.x >= a.p[i].rtile0) p = i;
  const ColProb& P = a.p[p];
  const int64_t n = P.C * P.r;
  const int64_t idx = (int64_t)((int)blockIdx.x - P.rtile0) * 256 + threadIdx.x;
  if (idx >= n * P.nseg) return;
  const int sg = (int)(idx / n);
  const int64_t o = idx - sg * n;
  float* out = pick3(sg, P.out[0], P.out[1], P.out[2]);
  float x = 0.f;
  for (int sp = 0; sp < P.nsplit; ++sp) x += P.part[((int64_t)sp * P.nseg + sg) * n + o];
  const float y = P.s * x;
  out[o] = P.accumulate ? out[o] + y : y;
}

// ------------------------------------------------------------- misc
// A thread writes 8 consecutive elements of one output row (16 bytes) and
// gathers them from 8 input rows: rows % 8 == 0. Consecutive threads take
// consecutive 8-element groups of the same output row, so the stores are
// contiguous; the small input stays in cache across the gathers.
__global__ __launch_bounds__(256) void k_transpose_bf16(const TransArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.end[a.n - 1]) return;
  int b = 0;
#pragma unroll
  for (int i = 0; i < kMaxTrans - 1; ++i) b += (i < a.n - 1 && idx >= a.end[i]) ? 1 : 0;
  const int64_t local = idx - (b ? a.end[b - 1] : 0);  // unit: 8 output elements
  const int64_t rows = a.rows[b], cols = a.cols[b], g8 = rows / 8;
  const int64_t c = local / g8, r0 = 8 * (local - c * g8);
  const uint16_t* in = a.in[b] + r0 * cols + c;
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = (uint32_t)in[(2 * e) * cols] | ((uint32_t)in[(2 * e + 1) * cols] << 16);
  *(uint4*)(a.out[b] + c * rows + r0) = make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ void k_zero_f32(float* p, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < n) p[idx] = 0.f;
}

// Row splits: enough workgroups of 16 rows for one per CU, each split at
// least 1024 reduction elements (measured: more splits cost more in partials
// and the second pass than they gain in parallelism).
int rowc_split(int64_t M, int64_t K) {
  const int64_t tiles = (M + RC_ROWS - 1) / RC_ROWS;
  int64_t s = (256 + tiles - 1) / (tiles > 0 ? tiles : 1);
  const int64_t maxs = K / 1024 > 1 ? K / 1024 : 1;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

// Column splits, at most one per 512 rows and at most 8 (workspace sizing).
int colc_max_split(int64_t M) {
  int64_t s = (M + 511) / 512;
  if (s > 8) s = 8;
  if (s < 1) s = 1;
  return (int)s;
}

// Split of a launch with `tiles` 64-column tiles in all: none once the tiles
// alone give about one workgroup per CU (a wave then streams its rows with no
// second pass, measured fastest), else enough to fill the chip.
int colc_split(int64_t tiles, int64_t M) {
  int64_t s = tiles > 0 ? 256 / tiles : 1;
  const int64_t mx = colc_max_split(M);
  if (s > mx) s = mx;
  if (s < 1) s = 1;
  return (int)s;
}

ql_status check_row(const RowProb& P) {
  if (P.r < 1 || P.r > 64 || P.nseg < 1 || P.nseg > kMaxSegs)
    return set_error(QL_ERR_UNSUPPORTED, "row contraction: r %d, nseg %d", P.r, P.nseg);
  if (P.K % 8 || P.ldx % 8 || (P.n_rep > 0 && P.head_dim % 8))
    return set_error(QL_ERR_SHAPE, "row contraction: K, row stride and head size must be multiples of 8");
  if (P.n_rep > 0 && P.K >= (1 << 24)) return set_error(QL_ERR_SHAPE, "row contraction: remapped K >= 2^24");
  return QL_OK;
}

template <int NCG, int MODE>
void launch_rowc_t(const RowArgs& a, unsigned grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  hipExtLaunchKernelGGL((k_rowc<NCG, MODE>), dim3(grid), dim3(64 * RC_WAVES), 0, st, e0, e1, 0, a);
}

// Bytes a row launch must move once: its operand streams, the SwiGLU values
// it stores, Bt, the outputs, and the float32 partials of a split (written
// and read back).
double rowc_bytes(const RowArgs& a) {
  double b = 0;
  for (int i = 0; i < a.nprob; ++i) {
    const RowProb& P = a.p[i];
    if (P.M <= 0) continue;
    const double M = (double)P.M, K = (double)P.K, np = (double)(P.r * P.nseg);
    const double xcols = P.n_rep > 0 ? K / P.n_rep : K;
    const int nin = a.mode == 1 ? 2 : (a.mode == 2 ? 3 : 1), nout = a.mode == 3 ? 1 : a.mode;
    b += 2.0 * M * xcols * nin + 2.0 * M * K * nout + 2.0 * np * K + 2.0 * M * np;
    if (P.nsplit > 1) b += 8.0 * P.nsplit * M * np;
  }
  return b;
}

// The same for a column launch: Z, V, the outputs (read too when
// accumulating), split partials; zero outputs of problems without rows.
double colc_bytes(const ColArgs& a) {
  double b = 0;
  for (int i = 0; i < a.nprob; ++i) {
    const ColProb& P = a.p[i];
    const double nout = (double)P.C * P.r * P.nseg;
    if (P.M <= 0) {
      if (!P.accumulate) b += 4.0 * nout;
      continue;
    }
    const double M = (double)P.M, C = (double)P.C;
    const double zcols = P.n_rep > 0 ? C / P.n_rep : C;
    b += 2.0 * M * zcols + 2.0 * M * P.r * P.nseg + 4.0 * nout * (P.accumulate ? 2 : 1);
    if (P.nsplit > 1) b += 8.0 * P.nsplit * nout;
  }
  return b;
}

}  // namespace

size_t rowc_ws_bytes(int64_t M, int64_t K, int32_t np) {
  const int s = rowc_split(M, K);
  return s > 1 ? align256((size_t)s * (size_t)M * (size_t)np * 4) : 0;
}

ql_status launch_rowc(RowArgs a, void* ws, size_t ws_bytes, hipStream_t st) {
  if (a.nprob < 1 || a.nprob > kMaxRowProb) return set_error(QL_ERR_ARG, "row contraction: %d problems", a.nprob);
  if (a.mode < 0 || a.mode > 3) return set_error(QL_ERR_ARG, "row contraction: mode %d", a.mode);
  for (int i = 0; i < a.nprob; ++i) {
    const RowProb& P = a.p[i];
    QL_TRY(check_row(P));
    if (a.mode == 1 && (P.nseg != 1 || P.n_rep > 0))
      return set_error(QL_ERR_ARG, "row contraction: the SwiGLU forward mode takes one projection, no remap");
    if (a.mode == 2 && (P.nseg != 2 || P.n_rep > 0 || P.r > kSwigluBwdMaxR))
      return set_error(QL_ERR_ARG, "row contraction: the SwiGLU backward mode takes two projections of r <= %d",
                       kSwigluBwdMaxR);
    if (a.mode == 3 && (P.n_rep > 0 || P.ldx != P.K || P.r * P.nseg > 64 || !P.Xout[0]))
      return set_error(QL_ERR_ARG, "row contraction: the RMSNorm mode takes contiguous rows, no remap, at most 64 "
                       "columns and an output");
  }
  // more than 64 columns: one launch per projection (keeps the operand
  // registers of a wave in bounds)
  for (int i = 0; i < a.nprob && a.mode == 0; ++i) {
    if (a.p[i].r * a.p[i].nseg > 64 && a.p[i].nseg > 1) {
      for (int i2 = 0; i2 < a.nprob; ++i2) {
        const RowProb& P = a.p[i2];
        for (int sgi = 0; sgi < P.nseg; ++sgi) {
          RowArgs b{};
          b.nprob = 1;
          b.mode = 0;
          b.p[0] = P;
          b.p[0].nseg = 1;
          b.p[0].Bt[0] = P.Bt[sgi];
          b.p[0].out[0] = P.out[sgi];
          QL_TRY(launch_rowc(b, ws, ws_bytes, st));
        }
      }
      return QL_OK;
    }
  }
  int ncg = 1, tiles = 0, rtiles = 0;
  size_t off = 0;
  for (int i = 0; i < a.nprob; ++i) {
    RowProb& P = a.p[i];
    const int np = P.r * P.nseg;
    const int c = a.mode == 2 ? 2 * ((P.r + 15) / 16) : (np + 15) / 16;
    if (c > ncg) ncg = c;
    P.tile0 = tiles;
    P.rtile0 = rtiles;
    P.nsplit = 1;
    P.part = nullptr;
    if (P.M <= 0) continue;
    // the RMSNorm producer runs unsplit: its workgroups read whole rows for
    // the statistics, which a split would repeat per slice
    P.nsplit = a.mode == 3 ? 1 : rowc_split(P.M, P.K);
    tiles += (int)((P.M + RC_ROWS - 1) / RC_ROWS) * P.nsplit;
    if (P.nsplit > 1) {
      P.part = (float*)((uint8_t*)ws + off);
      off += rowc_ws_bytes(P.M, P.K, np);
      rtiles += (int)((P.M * np + 255) / 256);
    }
  }
  if (off > ws_bytes) return set_error(QL_ERR_WORKSPACE, "row contraction: workspace %zu < %zu", ws_bytes, off);
  if (tiles == 0) return QL_OK;
  const unsigned grid = (unsigned)tiles;
  // timing events span the launch and its second pass
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool prof = profiling_on();
  if (prof) QL_TRY(profile_begin(&e0, &e1));
  hipEvent_t e1m = rtiles > 0 ? nullptr : e1;
  if (a.mode == 0) {
    switch (ncg) {
      case 1: launch_rowc_t<1, 0>(a, grid, st, e0, e1m); break;
      case 2: launch_rowc_t<2, 0>(a, grid, st, e0, e1m); break;
      case 3: launch_rowc_t<3, 0>(a, grid, st, e0, e1m); break;
      case 4: launch_rowc_t<4, 0>(a, grid, st, e0, e1m); break;
      default: return set_error(QL_ERR_UNSUPPORTED, "row contraction: %d column groups", ncg);
    }
  } else if (a.mode == 1) {
    switch (ncg) {
      case 1: launch_rowc_t<1, 1>(a, grid, st, e0, e1m); break;
      case 2: launch_rowc_t<2, 1>(a, grid, st, e0, e1m); break;
      case 3: launch_rowc_t<3, 1>(a, grid, st, e0, e1m); break;
      case 4: launch_rowc_t<4, 1>(a, grid, st, e0, e1m); break;
      default: return set_error(QL_ERR_UNSUPPORTED, "row contraction: %d column groups", ncg);
    }
  } else if (a.mode == 3) {
    switch (ncg) {
      case 1: launch_rowc_t<1, 3>(a, grid, st, e0, e1m); break;
      case 2: launch_rowc_t<2, 3>(a, grid, st, e0, e1m); break;
      case 3: launch_rowc_t<3, 3>(a, grid, st, e0, e1m); break;
      case 4: launch_rowc_t<4, 3>(a, grid, st, e0, e1m); break;
      default: return set_error(QL_ERR_UNSUPPORTED, "row contraction: %d column groups", ncg);
    }
  } else {
    switch (ncg) {
      case 2: launch_rowc_t<2, 2>(a, grid, st, e0, e1m); break;
      case 4: launch_rowc_t<4, 2>(a, grid, st, e0, e1m); break;
      default: return set_error(QL_ERR_UNSUPPORTED, "row contraction: %d column groups", ncg);
    }
  }
  QL_HIP_CHECK(hipGetLastError());
  if (rtiles > 0) {
    hipExtLaunchKernelGGL(k_rowc_reduce, dim3((unsigned)rtiles), dim3(256), 0, st, nullptr, e1, 0, a);
    QL_HIP_CHECK(hipGetLastError());
  }
  if (prof) QL_TRY(profile_end(e0, e1, QL_KERNEL_LORA_ROW, rowc_bytes(a)));
  return QL_OK;
}

size_t colc_ws_bytes(int64_t M, int64_t C, int32_t np) {
  const int s = colc_max_split(M);
  return s > 1 ? align256((size_t)s * (size_t)np * (size_t)C * 4) : 0;
}

ql_status launch_colc(ColArgs a, void* ws, size_t ws_bytes, hipStream_t st) {
  if (a.nprob < 1 || a.nprob > kMaxColProb) return set_error(QL_ERR_ARG, "column contraction: %d problems", a.nprob);
  for (int i = 0; i < a.nprob; ++i) {
    const ColProb& P = a.p[i];
    if (P.r < 1 || P.r > 64 || P.nseg < 1 || P.nseg > kMaxSegs)
      return set_error(QL_ERR_UNSUPPORTED, "column contraction: r %d, nseg %d", P.r, P.nseg);
  }
  // more than 64 columns: one launch per projection (keeps the accumulators
  // of a wave in registers); partials are reused launch after launch
  for (int i = 0; i < a.nprob; ++i) {
    if (a.p[i].r * a.p[i].nseg <= 64) continue;
    for (int i2 = 0; i2 < a.nprob; ++i2) {
      const ColProb& P = a.p[i2];
      for (int sgi = 0; sgi < P.nseg; ++sgi) {
        ColArgs b{};
        b.nprob = 1;
        b.p[0] = P;
        b.p[0].nseg = 1;
        b.p[0].V[0] = P.V[sgi];
        b.p[0].out[0] = P.out[sgi];
        QL_TRY(launch_colc(b, ws, ws_bytes, st));
      }
    }
    return QL_OK;
  }
  int64_t tiles1 = 0;  // column tiles of the launch before splitting
  for (int i = 0; i < a.nprob; ++i)
    if (a.p[i].M > 0) tiles1 += (a.p[i].C + CC_COLS - 1) / CC_COLS;
  int nj = 1, tiles = 0, rtiles = 0;
  bool vec = true;
  size_t off = 0;
  for (int i = 0; i < a.nprob; ++i) {
    ColProb& P = a.p[i];
    const int np = P.r * P.nseg;
    if (P.C % 8 || (P.M > 0 && (P.ldz % 8 || (P.n_rep > 0 && P.head_dim % 8))))
      return set_error(QL_ERR_SHAPE, "column contraction: C, row stride and head size must be multiples of 8");
    if (P.n_rep > 0 && P.C >= (1 << 24)) return set_error(QL_ERR_SHAPE, "column contraction: remapped C >= 2^24");
    P.tile0 = tiles;
    P.rtile0 = rtiles;
    P.nsplit = 1;
    P.part = nullptr;
    P.rows_per_split = 0;
    const int64_t nout = P.C * P.r * P.nseg;
    if (P.M > 0) {
      const int s0 = colc_split(tiles1, P.M);
      const int64_t rps = ((P.M + s0 - 1) / s0 + CC_ROWS - 1) / CC_ROWS * CC_ROWS;
      P.rows_per_split = rps;
      P.nsplit = (int)((P.M + rps - 1) / rps);
      tiles += (int)((P.C + CC_COLS - 1) / CC_COLS) * P.nsplit;
      const int c = (np + 15) / 16;
      if (c > nj) nj = c;
      if (P.r % 8) vec = false;
      if (P.nsplit > 1) {
        P.part = (float*)((uint8_t*)ws + off);
        off += align256((size_t)P.nsplit * (size_t)nout * 4);
        rtiles += (int)((nout + 255) / 256);
      }
    } else if (!P.accumulate) {
      tiles += (int)((nout + CC_ZERO - 1) / CC_ZERO);
    }
  }
  if (off > ws_bytes) return set_error(QL_ERR_WORKSPACE, "column contraction: workspace %zu < %zu", ws_bytes, off);
  if (tiles == 0 && rtiles == 0) return QL_OK;
  // timing events span the launch and its second pass
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool prof = profiling_on();
  if (prof) QL_TRY(profile_begin(&e0, &e1));
  hipEvent_t e1m = rtiles > 0 ? nullptr : e1;
  if (tiles > 0) {
#define QL_CC(n)                                                                                           \
  case n:                                                                                                  \
    if (vec) hipExtLaunchKernelGGL((k_colc<n, true>), dim3((unsigned)tiles), dim3(256), 0, st, e0, e1m, 0, a); \
    else hipExtLaunchKernelGGL((k_colc<n, false>), dim3((unsigned)tiles), dim3(256), 0, st, e0, e1m, 0, a);    \
    break;
    switch (nj) {
      QL_CC(1) QL_CC(2) QL_CC(3) QL_CC(4)
      default: return set_error(QL_ERR_UNSUPPORTED, "column contraction: %d column groups", nj);
    }
#undef QL_CC
    QL_HIP_CHECK(hipGetLastError());
  }
  if (rtiles > 0) {
    hipExtLaunchKernelGGL(k_colc_reduce, dim3((unsigned)rtiles), dim3(256), 0, st, tiles > 0 ? nullptr : e0, e1, 0,
                          a);
    QL_HIP_CHECK(hipGetLastError());
  }
  if (prof) QL_TRY(profile_end(e0, e1, QL_KERNEL_LORA_COL, colc_bytes(a)));
  return QL_OK;
}

ql_status launch_transpose_bf16(TransArgs a, hipStream_t st) {
  if (a.n < 1 || a.n > kMaxTrans) return set_error(QL_ERR_ARG, "transpose: %d matrices", a.n);
  int64_t tot = 0;  // in units of 8 output elements
  for (int i = 0; i < a.n; ++i) {
    if (a.rows[i] % 8) return set_error(QL_ERR_SHAPE, "transpose: rows (%lld) must be a multiple of 8", (long long)a.rows[i]);
    tot += a.rows[i] / 8 * a.cols[i];
    a.end[i] = tot;
  }
  if (tot == 0) return QL_OK;
  hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, a);
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

ql_status launch_zero_f32(float* p, int64_t n, hipStream_t st) {
  if (n == 0) return QL_OK;
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

}  // namespace ql
