// Glue of the attention-free decoder-layer stand-in: RMSNorm (unit gain,
// float32 statistics), SwiGLU silu(g) * u, and the head-group sum that is the
// backward of repeat_kv. All are memory-bound row or elementwise kernels;
// reductions run in a fixed lane order, so results are deterministic.
#include "ql_internal.h"

namespace ql {
namespace {

// One wave per row, 8 elements per lane per chunk (H % 8 == 0): lane l
// takes chunks l, l + 64, ... (NQL of them, the last ones masked when H is
// not a multiple of 512). All of a lane's chunks are loaded before the first
// is used, so the row streams in one round trip and is read once. Each lane
// sums its chunks in order; lanes are combined by a fixed butterfly.
template <int NQL>
__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const uint16_t* __restrict__ h, int64_t M, int64_t H,
                                                     float eps, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint4* hr = (const uint4*)(h + row * H);
  const int nq = (int)(H / 8);
  uint4 v[NQL];
#pragma unroll
  for (int i = 0; i < NQL; ++i) {
    const int q = lane + 64 * i;
    v[i] = hr[q < nq ? q : 0];
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NQL; ++i) {
    if (lane + 64 * i >= nq) continue;
    add_squares8(v[i], ss);
  }
  const float rs = rms_scale(wave_sum(ss), H, eps);
  uint4* orow = (uint4*)(out + row * H);
#pragma unroll
  for (int i = 0; i < NQL; ++i) {
    const int q = lane + 64 * i;
    if (q >= nq) continue;
    orow[q] = scale8(v[i], rs);
  }
}

// out = bf16(resid + rs * dn - (rs^3 / H) * h * sum(dn * h)), rs = 1/sqrt(mean(h^2) + eps);
// the same row layout and order as the forward
template <int NQL>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const uint16_t* __restrict__ h,
                                                     const uint16_t* __restrict__ dn,
                                                     const uint16_t* __restrict__ resid, int64_t M,
                                                     int64_t H, float eps, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint4* hr = (const uint4*)(h + row * H);
  const uint4* dr = (const uint4*)(dn + row * H);
  const uint4* rr = (const uint4*)(resid + row * H);
  const int nq = (int)(H / 8);
  uint4 va[NQL], vb[NQL], vr[NQL];
#pragma unroll
  for (int i = 0; i < NQL; ++i) {
    const int q = lane + 64 * i < nq ? lane + 64 * i : 0;
    va[i] = hr[q];
    vb[i] = dr[q];
  }
#pragma unroll
  for (int i = 0; i < NQL; ++i) vr[i] = rr[lane + 64 * i < nq ? lane + 64 * i : 0];
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int i = 0; i < NQL; ++i) {
    if (lane + 64 * i >= nq) continue;
    float a[8], b[8];
    unpack8(va[i], a);
    unpack8(vb[i], b);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ss += a[k] * a[k];
      dot += a[k] * b[k];
    }
  }
  ss = wave_sum(ss);
  dot = wave_sum(dot);
  const float rs = 1.0f / sqrtf(ss / (float)H + eps);
  const float c = rs * rs * rs / (float)H * dot;
  uint4* orow = (uint4*)(out + row * H);
#pragma unroll
  for (int i = 0; i < NQL; ++i) {
    const int q = lane + 64 * i;
    if (q >= nq) continue;
    float a[8], b[8], r[8];
    unpack8(va[i], a);
    unpack8(vb[i], b);
    unpack8(vr[i], r);
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = r[k] + (rs * b[k] - c * a[k]);
    orow[q] = pack8(r);
  }
}

// Rows too long for registers: the same sums, read in two passes.
__global__ __launch_bounds__(256) void k_rmsnorm_fwd_long(const uint16_t* __restrict__ h, int64_t M, int64_t H,
                                                          float eps, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint4* hr = (const uint4*)(h + row * H);
  const int64_t nq = H / 8;
  float ss = 0.f;
  for (int64_t q = lane; q < nq; q += 64) add_squares8(hr[q], ss);
  const float rs = rms_scale(wave_sum(ss), H, eps);
  uint4* orow = (uint4*)(out + row * H);
  for (int64_t q = lane; q < nq; q += 64) orow[q] = scale8(hr[q], rs);
}

__global__ __launch_bounds__(256) void k_rmsnorm_bwd_long(const uint16_t* __restrict__ h,
                                                          const uint16_t* __restrict__ dn,
                                                          const uint16_t* __restrict__ resid, int64_t M,
                                                          int64_t H, float eps, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint4* hr = (const uint4*)(h + row * H);
  const uint4* dr = (const uint4*)(dn + row * H);
  const uint4* rr = (const uint4*)(resid + row * H);
  const int64_t nq = H / 8;
  float ss = 0.f, dot = 0.f;
  for (int64_t q = lane; q < nq; q += 64) {
    float a[8], b[8];
    unpack8(hr[q], a);
    unpack8(dr[q], b);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ss += a[k] * a[k];
      dot += a[k] * b[k];
    }
  }
  ss = wave_sum(ss);
  dot = wave_sum(dot);
  const float rs = 1.0f / sqrtf(ss / (float)H + eps);
  const float c = rs * rs * rs / (float)H * dot;
  uint4* orow = (uint4*)(out + row * H);
  for (int64_t q = lane; q < nq; q += 64) {
    float a[8], b[8], r[8];
    unpack8(hr[q], a);
    unpack8(dr[q], b);
    unpack8(rr[q], r);
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = r[k] + (rs * b[k] - c * a[k]);
    orow[q] = pack8(r);
  }
}

__global__ __launch_bounds__(256) void k_swiglu_fwd(const uint4* __restrict__ g, const uint4* __restrict__ u,
                                                    int64_t nq, uint4* __restrict__ act) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nq; q += stride)
    act[q] = swiglu_act8(g[q], u[q]);
}

__global__ __launch_bounds__(256) void k_swiglu_bwd(const uint4* __restrict__ g, const uint4* __restrict__ u,
                                                    const uint4* __restrict__ da, int64_t nq,
                                                    uint4* __restrict__ dg, uint4* __restrict__ du) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nq; q += stride)
    swiglu_grad8(g[q], u[q], da[q], dg[q], du[q]);
}

__global__ void k_repeat_kv_bwd(const float* __restrict__ da, int64_t M, int64_t H, int64_t kv, int d,
                                uint16_t* __restrict__ dv) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * kv) return;
  const int64_t m = idx / kv, c = idx - m * kv;
  const int64_t g = c / d, i = c - g * d;
  const int64_t n_rep = H / kv;
  float s = 0.f;
  for (int64_t j = 0; j < n_rep; ++j) s += da[m * H + (g * n_rep + j) * d + i];
  dv[idx] = f32_to_bf16(s);
}

unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 256 * 32) g = 256 * 32;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

// rows of up to 16 x 512 elements (forward) or 8 x 512 (backward, three
// operands) stay in registers
ql_status launch_rmsnorm_fwd(const uint16_t* h, int64_t M, int64_t H, float eps, uint16_t* out,
                             hipStream_t st) {
  if (M == 0) return QL_OK;
  const int nql = (int)((H / 8 + 63) / 64);
  const dim3 grid((unsigned)((M + 3) / 4));
  switch (nql) {
#define QL_RF(n) case n: hipLaunchKernelGGL(k_rmsnorm_fwd<n>, grid, dim3(256), 0, st, h, M, H, eps, out); break;
    QL_RF(1) QL_RF(2) QL_RF(3) QL_RF(4) QL_RF(5) QL_RF(6) QL_RF(7) QL_RF(8)
    QL_RF(9) QL_RF(10) QL_RF(11) QL_RF(12) QL_RF(13) QL_RF(14) QL_RF(15) QL_RF(16)
#undef QL_RF
    default: hipLaunchKernelGGL(k_rmsnorm_fwd_long, grid, dim3(256), 0, st, h, M, H, eps, out); break;
  }
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

ql_status launch_rmsnorm_bwd(const uint16_t* h, const uint16_t* dn, const uint16_t* resid, int64_t M,
                             int64_t H, float eps, uint16_t* out, hipStream_t st) {
  if (M == 0) return QL_OK;
  const int nql = (int)((H / 8 + 63) / 64);
  const dim3 grid((unsigned)((M + 3) / 4));
  switch (nql) {
#define QL_RB(n)                                                                                       \
  case n: hipLaunchKernelGGL(k_rmsnorm_bwd<n>, grid, dim3(256), 0, st, h, dn, resid, M, H, eps, out); break;
    QL_RB(1) QL_RB(2) QL_RB(3) QL_RB(4) QL_RB(5) QL_RB(6) QL_RB(7) QL_RB(8)
#undef QL_RB
    default: hipLaunchKernelGGL(k_rmsnorm_bwd_long, grid, dim3(256), 0, st, h, dn, resid, M, H, eps, out); break;
  }
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

ql_status launch_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* act,
                            hipStream_t st) {
  const int64_t nq = n / 8;
  if (nq == 0) return QL_OK;
  hipLaunchKernelGGL(k_swiglu_fwd, dim3(grid_for(nq)), dim3(256), 0, st, (const uint4*)g, (const uint4*)u,
                     nq, (uint4*)act);
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

ql_status launch_swiglu_bwd(const uint16_t* g, const uint16_t* u, const uint16_t* dact, int64_t n,
                            uint16_t* dg, uint16_t* du, hipStream_t st) {
  const int64_t nq = n / 8;
  if (nq == 0) return QL_OK;
  hipLaunchKernelGGL(k_swiglu_bwd, dim3(grid_for(nq)), dim3(256), 0, st, (const uint4*)g, (const uint4*)u,
                     (const uint4*)dact, nq, (uint4*)dg, (uint4*)du);
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

ql_status launch_repeat_kv_bwd(const float* da, int64_t M, int64_t H, int64_t kv, int32_t head_dim,
                               uint16_t* dv, hipStream_t st) {
  const int64_t n = M * kv;
  if (n == 0) return QL_OK;
  hipLaunchKernelGGL(k_repeat_kv_bwd, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, da, M, H, kv,
                     head_dim, dv);
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

}  // namespace ql
