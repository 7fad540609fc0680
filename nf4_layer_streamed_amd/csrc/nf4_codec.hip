// NF4 codec kernels: block-wise quantisation and standalone dequantisation.
//
// Format (the pages leave it open; QLoRA section 3 with a float32 scale):
// blocks of 64 consecutive elements of the row-major weight, one float32
// absmax per block, one 4-bit code per element. Codes are packed 8 to a 32-bit
// little-endian word: byte j of the word holds code j in its low nibble and
// code j + 4 in its high nibble. (This order lets a decoder split a word into
// two byte-lane index vectors with one mask and one shift each.)
#include <hip/hip_ext.h>

#include "ql_internal.h"

namespace ql {

// One block of 64 weights per 16 lanes, 4 elements per lane (one float4).
// Code of a normalised value n = number of level midpoints strictly below n;
// the midpoints (c_j + c_{j+1}) / 2 are exact in double precision and the
// comparison of a float32 with them is exact, so this is the nearest level
// with ties going to the lower index.
__global__ __launch_bounds__(256) void k_nf4_quantize(const float4* __restrict__ w, int64_t nblocks,
                                                      uint8_t* __restrict__ packed,
                                                      float* __restrict__ absmax) {
  __shared__ double mid[15];
  if (threadIdx.x < 15) {
    double a = (double)__builtin_bit_cast(float, kNF4LevelBits[threadIdx.x]);
    double b = (double)__builtin_bit_cast(float, kNF4LevelBits[threadIdx.x + 1]);
    mid[threadIdx.x] = 0.5 * (a + b);
  }
  __syncthreads();
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gid >> 4;
  const int lane16 = threadIdx.x & 15;
  const bool active = blk < nblocks;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (active) v = w[blk * 16 + lane16];
  float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  // max over the 16 lanes of this block (xor offsets stay inside aligned groups of 16)
  for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 16));
  if (active && lane16 == 0) absmax[blk] = m;
  uint32_t c[4];
  const float e[4] = {v.x, v.y, v.z, v.w};
  for (int i = 0; i < 4; ++i) {
    if (m == 0.f) {
      c[i] = 7;
    } else {
      const double n = (double)(e[i] / m);  // IEEE float32 division, then exact widening
      uint32_t k = 0;
      for (int j = 0; j < 15; ++j) k += (n > mid[j]) ? 1u : 0u;
      c[i] = k;
    }
  }
  // Lane pair (2w, 2w+1) holds the 8 codes of word w; the even lane's codes are
  // the low nibbles, the odd lane's the high nibbles.
  const uint32_t mine = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
  const uint32_t other = (uint32_t)__shfl_xor((int)mine, 1, 16);
  if (active && (lane16 & 1) == 0) ((uint32_t*)packed)[blk * 8 + (lane16 >> 1)] = mine | (other << 4);
}

// The finiteness flag of nf4_quantize: one word per device, in the code
// object, so the library keeps no allocation of its own. Host code reaches it
// only through the address hipGetSymbolAddress gives for the current device.
static __device__ int g_nonfinite;
static int* g_nonfinite_dev[64] = {};

// flag = 1 if any element is NaN or infinite (every writer stores the same
// value, so plain stores suffice); grid-stride over float4 groups
__global__ __launch_bounds__(256) void k_scan_nonfinite(const float4* __restrict__ w, int64_t n4, int* flag) {
  bool bad = false;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 v = w[i];
    bad |= !(__builtin_isfinite(v.x) && __builtin_isfinite(v.y) && __builtin_isfinite(v.z) &&
             __builtin_isfinite(v.w));
  }
  if (bad) *flag = 1;
}

__global__ void k_set_i32(int* p, int v) { *p = v; }

ql_status scan_nonfinite(const float* w, int64_t n, int* nonfinite, hipStream_t st) {
  int dev = 0;
  QL_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return set_error(QL_ERR_UNSUPPORTED, "device id %d out of range", dev);
  if (!g_nonfinite_dev[dev]) QL_HIP_CHECK(hipGetSymbolAddress((void**)&g_nonfinite_dev[dev], HIP_SYMBOL(g_nonfinite)));
  int* flag = g_nonfinite_dev[dev];
  hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, st, flag, 0);
  QL_HIP_CHECK(hipGetLastError());
  int64_t grid = (n / 4 + 255) / 256;
  if (grid > 256 * 16) grid = 256 * 16;
  if (grid > 0) {
    hipLaunchKernelGGL(k_scan_nonfinite, dim3((unsigned)grid), dim3(256), 0, st, (const float4*)w, n / 4, flag);
    QL_HIP_CHECK(hipGetLastError());
  }
  int host = 0;
  QL_HIP_CHECK(hipMemcpyAsync(&host, flag, sizeof(int), hipMemcpyDeviceToHost, st));
  QL_HIP_CHECK(hipStreamSynchronize(st));
  *nonfinite = host != 0;
  return QL_OK;
}

ql_status launch_nf4_quantize(const float* w, int64_t n, uint8_t* packed, float* absmax, hipStream_t st) {
  const int64_t nblocks = n / 64;
  const int64_t threads = nblocks * 16;
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7fffffff) return set_error(QL_ERR_SHAPE, "nf4_quantize: n too large for one launch");
  if (grid == 0) return QL_OK;
  hipLaunchKernelGGL(k_nf4_quantize, dim3((unsigned)grid), dim3(256), 0, st,
                     (const float4*)w, nblocks, packed, absmax);
  QL_HIP_CHECK(hipGetLastError());
  return QL_OK;
}

// Standalone dequant: each thread decodes 8 consecutive elements (one dword of
// codes) with the level table in LDS, multiplies by the block's absmax in
// float32, and stores 8 bf16 (16 B) or 8 float32 (32 B). Grid-stride loop.
template <bool F32>
__global__ __launch_bounds__(256) void k_nf4_dequant(const uint32_t* __restrict__ packed,
                                                     const float* __restrict__ absmax, int64_t ngroups,
                                                     void* __restrict__ out) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = __builtin_bit_cast(float, kNF4LevelBits[threadIdx.x]);
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < ngroups; g += stride) {
    const uint32_t p = packed[g];
    const float a = absmax[g >> 3];
    float f[8];
    // byte j holds element j (low nibble) and element j + 4 (high nibble)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] = lv[(p >> (8 * j)) & 15u] * a;
      f[j + 4] = lv[(p >> (8 * j + 4)) & 15u] * a;
    }
    if (F32) {
      float4* o = (float4*)out + g * 2;
      o[0] = make_float4(f[0], f[1], f[2], f[3]);
      o[1] = make_float4(f[4], f[5], f[6], f[7]);
    } else {
      uint4 q;
      q.x = pack_bf16x2(f[0], f[1]);
      q.y = pack_bf16x2(f[2], f[3]);
      q.z = pack_bf16x2(f[4], f[5]);
      q.w = pack_bf16x2(f[6], f[7]);
      ((uint4*)out)[g] = q;
    }
  }
}

ql_status launch_nf4_dequant(const uint8_t* packed, const float* absmax, int64_t n, int out_f32,
                             void* out, hipStream_t st) {
  const int64_t ngroups = n / 8;
  if (ngroups == 0) return QL_OK;
  int64_t grid = (ngroups + 255) / 256;
  if (grid > 256 * 64) grid = 256 * 64;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool prof = profiling_on();
  if (prof) QL_TRY(profile_begin(&e0, &e1));
  if (out_f32)
    hipExtLaunchKernelGGL(k_nf4_dequant<true>, dim3((unsigned)grid), dim3(256), 0, st, e0, e1, 0,
                          (const uint32_t*)packed, absmax, ngroups, out);
  else
    hipExtLaunchKernelGGL(k_nf4_dequant<false>, dim3((unsigned)grid), dim3(256), 0, st, e0, e1, 0,
                          (const uint32_t*)packed, absmax, ngroups, out);
  QL_HIP_CHECK(hipGetLastError());
  // codes and scales read once (0.5625 B per weight), the output written once
  if (prof) QL_TRY(profile_end(e0, e1, QL_KERNEL_DEQUANT, (double)n * (0.5625 + (out_f32 ? 4.0 : 2.0))));
  return QL_OK;
}

}  // namespace ql
