// LoRA side products of rank r (r <= 64): the skinny contractions around the
// fused NF4 GEMMs. They are memory-bound (about r FLOP per byte read), so the
// design goal is one coalesced pass over the large operand with a fixed
// reduction order (no atomics): split the long dimension into chunks, write
// float32 partial sums to a workspace, and sum the chunks in index order.
//
//  skinny:  out[m][j] = bf16( sum_k X[m][k] Bt[j][k] )      U = x A^T, G = dY B
//  colred:  out[j][c] = s * sum_m Z[m][c] V[m][j]           dA = s G^T x, dB = s dY^T U
//
// The adapter formula is the LoRA one (y = x W^T + s (x A^T) B^T, s = alpha/r);
// only A and B train (blog "How does Soup train an 8B model on a 4 GB GPU?").
#include "ql_internal.h"

namespace ql {
namespace {

constexpr int SK_ROWS = 64;    // rows of X per workgroup (16 per wave)
constexpr int SK_SPLIT = 256;  // reduction length per split

__device__ __forceinline__ int64_t remap_col(int64_t k, int head_dim, int n_rep) {
  if (n_rep <= 0) return k;
  const int64_t head = k / head_dim, i = k - head * head_dim;
  return (head / n_rep) * head_dim + i;
}

// MFMA 16x16x32: A fragment = 16 rows of X, 8 reduction elements per lane;
// B fragment = 16 columns (j) of Bt with the same 8 reduction elements.
template <int NCG>
__global__ __launch_bounds__(256) void k_skinny_partial(const SkinnyArgs a, float* __restrict__ part) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * SK_ROWS + w * 16;
  const int64_t kbeg = (int64_t)blockIdx.y * SK_SPLIT;
  const int64_t kend = kbeg + SK_SPLIT < a.K ? kbeg + SK_SPLIT : a.K;
  const int np = a.r * a.nseg;
  f32x4_t acc[NCG];
#pragma unroll
  for (int c = 0; c < NCG; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t m = m0 + (lane & 15);
  for (int64_t k = kbeg; k < kend; k += 32) {
    const int64_t kk = k + 8 * (lane >> 4);
    uint4 av = make_uint4(0, 0, 0, 0);
    if (m < a.M && kk < a.K) av = *(const uint4*)(a.X + m * a.ldx + remap_col(kk, a.head_dim, a.n_rep));
    const bf16x8_t af = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      const int jt = 16 * c + (lane & 15);
      uint4 bv = make_uint4(0, 0, 0, 0);
      if (jt < np && kk < a.K) {
        const int sg = jt / a.r, j = jt - sg * a.r;
        const uint16_t* bt = sg == 0 ? a.Bt[0] : (sg == 1 ? a.Bt[1] : a.Bt[2]);
        bv = *(const uint4*)(bt + (int64_t)j * a.K + kk);
      }
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8_t, bv), acc[c], 0, 0, 0);
    }
  }
  // lane holds rows 4*(lane/16)+v, column lane%16 of each 16x16 tile
#pragma unroll
  for (int c = 0; c < NCG; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = m0 + 4 * (lane >> 4) + v;
      const int jt = 16 * c + (lane & 15);
      if (mm < a.M && jt < np) part[((int64_t)blockIdx.y * a.M + mm) * np + jt] = acc[c][v];
    }
}

__global__ void k_skinny_reduce(const SkinnyArgs a, const float* __restrict__ part, int nsplit) {
  const int np = a.r * a.nseg;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.M * np) return;
  const int64_t m = idx / np;
  const int jt = (int)(idx - m * np);
  float s = 0.f;
  for (int p = 0; p < nsplit; ++p) s += part[((int64_t)p * a.M + m) * np + jt];
  const int sg = jt / a.r, j = jt - sg * a.r;
  uint16_t* o = sg == 0 ? a.out[0] : (sg == 1 ? a.out[1] : a.out[2]);
  o[m * a.r + j] = f32_to_bf16(s);
}

int64_t skinny_nsplit(int64_t K) { return (K + SK_SPLIT - 1) / SK_SPLIT; }

// Column reduction out[j][c] = s * sum_m Z[m][c] V[m][j]. A workgroup owns
// CR_COLS columns (two per lane: one 4-byte load per row) and one block of
// rows, 16 ranks per pass (blockIdx.z). Its four waves take interleaved rows;
// the block's V rows are staged in LDS as float32 (read by broadcast). The
// waves' sums are combined in LDS in wave order. With one row block the
// workgroup writes the result; with several, float32 partials go to the
// workspace and a second pass adds them in block order.
constexpr int CR_COLS = 128;
constexpr int CR_SUB = 256;  // V rows staged per LDS round

__global__ __launch_bounds__(256) void k_colred_partial(const ColRedArgs a, int64_t rows_per_block, int nblk,
                                                        float* __restrict__ part) {
  __shared__ float vs[CR_SUB][16];
  __shared__ float red[3][CR_COLS][17];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t c = (int64_t)blockIdx.x * CR_COLS + 2 * lane;
  const int64_t mb = (int64_t)blockIdx.y * rows_per_block;
  const int64_t me = mb + rows_per_block < a.M ? mb + rows_per_block : a.M;
  const int j0 = blockIdx.z * 16;
  const bool live = c < a.C;
  // columns c, c + 1 stay inside one head under the repeat_kv remap (C, head_dim even)
  const int64_t pc = live ? remap_col(c, a.head_dim, a.n_rep) : 0;
  const uint32_t* zp = (const uint32_t*)(a.Z + pc);
  const int64_t ldw = a.ldz / 2;
  float acc0[16], acc1[16];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) acc0[jj] = acc1[jj] = 0.f;
  for (int64_t sb = mb; sb < me; sb += CR_SUB) {
    const int64_t se = sb + CR_SUB < me ? sb + CR_SUB : me;
    __syncthreads();
    for (int64_t i = t; i < (se - sb) * 16; i += 256) {
      const int64_t mi = i >> 4;
      const int jj = (int)(i & 15);
      vs[mi][jj] = (j0 + jj < a.r) ? bf16_to_f32(a.V[(sb + mi) * a.r + j0 + jj]) : 0.f;
    }
    __syncthreads();
    if (live) {
      int64_t m = sb + w;
      for (; m + 12 < se; m += 16) {  // four rows of this wave in flight
        uint32_t zz[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) zz[u] = zp[(m + 4 * u) * ldw];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float z0 = __builtin_bit_cast(float, zz[u] << 16);
          const float z1 = __builtin_bit_cast(float, zz[u] & 0xffff0000u);
          const float* vr = vs[m + 4 * u - sb];
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            acc0[jj] += z0 * vr[jj];
            acc1[jj] += z1 * vr[jj];
          }
        }
      }
      for (; m < se; m += 4) {
        const uint32_t zz = zp[m * ldw];
        const float z0 = __builtin_bit_cast(float, zz << 16);
        const float z1 = __builtin_bit_cast(float, zz & 0xffff0000u);
        const float* vr = vs[m - sb];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          acc0[jj] += z0 * vr[jj];
          acc1[jj] += z1 * vr[jj];
        }
      }
    }
  }
  // waves 1..3 hand their sums to wave 0, which adds them in wave order
  if (w > 0) {
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      red[w - 1][2 * lane][jj] = acc0[jj];
      red[w - 1][2 * lane + 1][jj] = acc1[jj];
    }
  }
  __syncthreads();
  if (w > 0 || !live) return;
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      acc0[jj] += red[q][2 * lane][jj];
      acc1[jj] += red[q][2 * lane + 1][jj];
    }
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int j = j0 + jj;
    if (j >= a.r) break;
    if (nblk == 1) {
      const float v0 = a.s * acc0[jj], v1 = a.s * acc1[jj];
      const int64_t o0 = a.transpose_out ? c * a.r + j : j * a.C + c;
      const int64_t o1 = a.transpose_out ? (c + 1) * a.r + j : j * a.C + c + 1;
      a.out[o0] = a.accumulate ? a.out[o0] + v0 : v0;
      a.out[o1] = a.accumulate ? a.out[o1] + v1 : v1;
    } else {
      float* pp = part + ((int64_t)blockIdx.y * a.r + j) * a.C + c;
      pp[0] = acc0[jj];
      pp[1] = acc1[jj];
    }
  }
}

__global__ void k_colred_reduce(const ColRedArgs a, const float* __restrict__ part, int nchunk) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.C * a.r) return;
  const int64_t j = idx / a.C, c = idx - j * a.C;
  float s = 0.f;
  for (int p = 0; p < nchunk; ++p) s += part[((int64_t)p * a.r + j) * a.C + c];
  s *= a.s;
  const int64_t o = a.transpose_out ? c * a.r + j : j * a.C + c;
  a.out[o] = a.accumulate ? a.out[o] + s : s;
}

// Row blocks of a column reduction: enough for about 512 workgroups, at
// least 64 rows each.
int colred_blocks(int64_t M, int64_t C, int32_t r) {
  const int64_t tiles = ((C + CR_COLS - 1) / CR_COLS) * ((r + 15) / 16);
  int64_t nb = 512 / (tiles > 0 ? tiles : 1);
  const int64_t maxb = M / 64 > 1 ? M / 64 : 1;
  if (nb > maxb) nb = maxb;
  if (nb < 1) nb = 1;
  return (int)nb;
}

__global__ void k_transpose_bf16(const uint16_t* __restrict__ in, int64_t rows, int64_t cols,
                                 uint16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * cols) return;
  const int64_t r = idx / cols, c = idx - r * cols;
  out[c * rows + r] = in[idx];
}

__global__ void k_zero_f32(float* p, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < n) p[idx] = 0.f;
}

}  // namespace

size_t skinny_ws_bytes(int64_t M, int64_t K, int32_t r, int32_t nseg) {
  return (size_t)skinny_nsplit(K) * (size_t)M * (size_t)(r * nseg) * sizeof(float);
}

ql_status launch_skinny(const SkinnyArgs& a, void* ws, hipStream_t st) {
  if (a.M == 0) return QL_OK;
  const int np = a.r * a.nseg;
  const int ncg = (np + 15) / 16;
  const int64_t nsplit = skinny_nsplit(a.K);
  dim3 grid((unsigned)((a.M + SK_ROWS - 1) / SK_ROWS), (unsigned)nsplit);
  float* part = (float*)ws;
  switch (ncg) {
#define QL_SK(n) case n: hipLaunchKernelGGL(k_skinny_partial<n>, grid, dim3(256), 0, st, a, part); break;
    QL_SK(1) QL_SK(2) QL_SK(3) QL_SK(4) QL_SK(5) QL_SK(6) QL_SK(7) QL_SK(8) QL_SK(9) QL_SK(10)
    QL_SK(11) QL_SK(12)
#undef QL_SK
    default: return set_error(QL_ERR_UNSUPPORTED, "skinny: %d columns exceed 192", np);
  }
  QL_HIP_CHECK(hipGetLastError());
  const int64_t n = a.M * np;
  hipLaunchKernelGGL(k_skinny_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, part,
                     (int)nsplit);
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

size_t colred_ws_bytes(int64_t M, int64_t C, int32_t r) {
  const int nb = colred_blocks(M, C, r);
  return nb > 1 ? (size_t)nb * (size_t)r * (size_t)C * sizeof(float) : 0;
}

ql_status launch_colred(const ColRedArgs& a, void* ws, hipStream_t st) {
  const int64_t n = a.C * a.r;
  if (a.M == 0) {
    if (!a.accumulate && n > 0) return launch_zero_f32(a.out, n, st);
    return QL_OK;
  }
  if ((a.C & 1) || (a.ldz & 1) || (a.n_rep > 0 && (a.head_dim & 1)))
    return set_error(QL_ERR_SHAPE, "colred: column count and row stride must be even");
  const int nb = colred_blocks(a.M, a.C, a.r);
  const int64_t rows = (a.M + nb - 1) / nb;
  dim3 grid((unsigned)((a.C + CR_COLS - 1) / CR_COLS), (unsigned)nb, (unsigned)((a.r + 15) / 16));
  float* part = (float*)ws;
  hipLaunchKernelGGL(k_colred_partial, grid, dim3(256), 0, st, a, rows, nb, part);
  QL_HIP_CHECK(hipGetLastError());
  if (nb > 1) {
    hipLaunchKernelGGL(k_colred_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, part, nb);
    QL_HIP_CHECK(hipGetLastError());
  }
  return QL_OK;
}

ql_status launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                hipStream_t st) {
  const int64_t n = rows * cols;
  if (n == 0) return QL_OK;
  hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, in, rows,
                     cols, out);
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
