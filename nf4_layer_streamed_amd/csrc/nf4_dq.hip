// Double-quantised NF4 block scales (QLoRA, section 3, "Double Quantization").
//
// The float32 absmax c of every 64-weight block is stored as one byte: the
// tensor's scales are centred by their mean mu and quantised to OCP FP8 E4M3
// (bias 7, 3 mantissa bits, largest finite 448, no infinities) in runs of 256,
// each run with one float32 scale s = max |c - mu| / 448. With the NF4 codes
// this is about 0.516 bytes per weight: the pages' 3.60 GB Llama-3.1-8B store
// with 113 MB layer buffers (Soup README, header figure caption).
//
// Stored block of n scales (byte offsets): codes [0, n); run scales (float32,
// ceil(n / 256)) at align256(n); mu (float32) at that plus
// align256(4 ceil(n / 256)); total padded to a multiple of 256.
//
// mu = fl32(S / n), S the float64 sum taken in a fixed order: each run of 256
// consecutive scales summed left to right, then the run sums left to right;
// any implementation following that order gets the same bits. Per run:
// d = fl32(c - mu), s = fl32(max |d| / 448), code = E4M3(fl32(d / s)) rounded
// to nearest even and saturated to +-448 (s = 0: code 0). Expansion:
// c' = fl32(fl32(e4m3(code) * s) + mu), two roundings (no fused multiply-add).

#include "ql_internal.h"

namespace ql {

namespace {

constexpr int RUN = 256;

// E4M3 code of a finite float, round-to-nearest-even, saturating to +-448.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (m = 8 is 2^-6, code 0x08)
    const float m = rintf(a * 512.f);  // exact scaling by a power of two, then ties to even
    return sign | (uint32_t)m;
  }
  // 3 of float32's 23 fraction bits survive: round the 20 below them to
  // nearest even; a carry rolls into the exponent
  const uint32_t ab = bits & 0x7fffffffu;
  const uint32_t r = ab + 0x7ffffu + ((ab >> 20) & 1u);
  const uint32_t e8 = (r >> 23) - 127 + 7;  // E4M3 biased exponent (>= 1 here)
  const uint32_t code = (e8 << 3) | ((r >> 20) & 7u);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// Exact float value of an E4M3 code (never a NaN code here).
__device__ __forceinline__ float e4m3_decode(uint32_t k) {
  const uint32_t e = (k >> 3) & 15u, m = k & 7u;
  const float v = e ? ldexpf((float)(8u + m), (int)e - 10) : ldexpf((float)m, -9);
  return (k & 0x80u) ? -v : v;
}

// mu: one workgroup. For each chunk of 256 runs, thread t sums run t of the
// chunk left to right in float64; thread 0 then adds the chunk's run sums in
// order to the running total.
__global__ __launch_bounds__(256) void k_dq_mean(const float* __restrict__ c, int64_t n, float* __restrict__ mu) {
  __shared__ double part[RUN];
  const int t = threadIdx.x;
  const int64_t nruns = (n + RUN - 1) / RUN;
  double total = 0.0;
  for (int64_t r0 = 0; r0 < nruns; r0 += RUN) {
    const int64_t run = r0 + t;
    double s = 0.0;
    if (run < nruns) {
      const int64_t b = run * RUN, e = b + RUN < n ? b + RUN : n;
      for (int64_t i = b; i < e; ++i) s = s + (double)c[i];
    }
    part[t] = s;
    __syncthreads();
    if (t == 0) {
      const int64_t cnt = nruns - r0 < RUN ? nruns - r0 : RUN;
      for (int64_t j = 0; j < cnt; ++j) total = total + part[j];
    }
    __syncthreads();
  }
  if (t == 0) mu[0] = (float)(total / (double)n);  // float64 division, one rounding to float32
}

// One workgroup per run of 256 scales.
__global__ __launch_bounds__(256) void k_dq_quant(const float* __restrict__ c, int64_t n,
                                                  const float* __restrict__ mu_p, uint8_t* __restrict__ codes,
                                                  float* __restrict__ scales) {
  __shared__ float red[RUN];
  const int t = threadIdx.x;
  const int64_t i = (int64_t)blockIdx.x * RUN + t;
  const float mu = mu_p[0];
  const float d = i < n ? __fsub_rn(c[i], mu) : 0.f;
  red[t] = fabsf(d);
  __syncthreads();
  for (int w = RUN / 2; w > 0; w >>= 1) {  // max is exact in any order
    if (t < w) red[t] = fmaxf(red[t], red[t + w]);
    __syncthreads();
  }
  const float s = red[0] / 448.f;  // IEEE float32 division
  if (t == 0) scales[blockIdx.x] = s;
  if (i < n) codes[i] = (uint8_t)(s > 0.f ? e4m3_encode(d / s) : 0u);
}

// Expansion of up to kMaxDq blocks in one launch: element g of the
// concatenated index space belongs to the block whose range holds it.
__global__ __launch_bounds__(256) void k_dq_expand(DqExpandArgs a) {
  // two roundings (product, then sum): HIP contracts a * b + c into one fma
  // by default, so contraction is switched off here
#pragma clang fp contract(off)
  const int64_t total = a.end[a.nblk - 1];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += stride) {
    int b = 0;
#pragma unroll
    for (int j = 0; j < kMaxDq - 1; ++j) b += (j < a.nblk - 1 && g >= a.end[j]) ? 1 : 0;
    const int64_t i = g - (b ? a.end[b - 1] : 0);
    const uint8_t* blk = a.src[b];
    const float s = ((const float*)(blk + a.scale_off[b]))[i >> 8];
    const float mu = *(const float*)(blk + a.mean_off[b]);
    const float prod = e4m3_decode(blk[i]) * s;  // rounded product
    a.dst[b][i] = prod + mu;                      // rounded sum
  }
}

}  // namespace

DqLayout dq_layout(int64_t n) {
  DqLayout l;
  const int64_t runs = (n + RUN - 1) / RUN;
  l.scale_off = align256((size_t)n);
  l.mean_off = l.scale_off + align256((size_t)(4 * runs));
  l.bytes = l.mean_off + 256;
  return l;
}

ql_status launch_dq_quant(const float* c, int64_t n, uint8_t* block, hipStream_t st) {
  if (n <= 0) return QL_OK;
  const DqLayout l = dq_layout(n);
  float* mu = (float*)(block + l.mean_off);
  hipLaunchKernelGGL(k_dq_mean, dim3(1), dim3(256), 0, st, c, n, mu);
  QL_HIP_CHECK(hipGetLastError());
  const int64_t runs = (n + RUN - 1) / RUN;
  if (runs > 0x7fffffff) return set_error(QL_ERR_SHAPE, "double quantisation: too many scales");
  hipLaunchKernelGGL(k_dq_quant, dim3((unsigned)runs), dim3(256), 0, st, c, n, (const float*)mu, block,
                     (float*)(block + l.scale_off));
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

ql_status launch_dq_expand(const DqExpandArgs& a, hipStream_t st) {
  if (a.nblk <= 0 || a.end[a.nblk - 1] == 0) return QL_OK;
  int64_t grid = (a.end[a.nblk - 1] + 255) / 256;
  if (grid > 2048) grid = 2048;
  hipLaunchKernelGGL(k_dq_expand, dim3((unsigned)grid), dim3(256), 0, st, a);
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

}  // namespace ql
