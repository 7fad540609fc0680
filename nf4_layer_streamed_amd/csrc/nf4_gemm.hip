// Fused NF4-dequant bf16 MFMA GEMMs for gfx950.
//
// Forward  (NT): Y[M x N]  = X[M x K] W[N x K]^T + U[M x r] (sB)[N x r]^T
// Backward (NN): dX[M x K] = sum_seg dY[M x N] W[N x K] + G[M x r] (sA)[r x K]
//
// W is never materialised in memory. Its packed 4-bit codes and per-block
// float32 absmax are read from global memory and decoded on chip to
// bf16(fl32(level[code] * absmax)); this replaces the separate per-layer
// dequantisation pass that the Soup README ("Citing Soup", v3 retraction)
// measures as streaming's largest own cost. The LoRA adapter's rank-r product
// is one extra K-step of the same loop (K-concatenation [X | U] [W | sB]^T),
// so each output is written once.
//
// Decode. Within one NF4 block (64 weights of a row) there are only 16
// distinct values, bf16(level[j] * absmax). A lane computes these 16 values
// once per row and block (16 multiplies, 8 packed conversions), keeps them as
// two 16-byte tables (low bytes and high bytes of the bf16 values), and looks
// codes up four at a time with v_perm_b32 byte selects: two 8-entry selects and
// a third select on bit 3 of the code, per byte plane.
//
// MFMA: v_mfma_f32_32x32x16_bf16. A lane of a 32x32x16 product holds row or
// column (lane % 32) and 8 consecutive values of the reduction; here lane
// group g = lane / 32 takes reduction elements [32 g + 8 q, 32 g + 8 q + 8)
// in sub-step q of a 64-wide K-step (the A and B operands use the same split,
// so the product sums over all 64). Output: lane holds column lane % 32 and
// rows 8 i + 4 g + j for accumulator 4 i + j.
//
// Forward layout: 256 x BN outputs per workgroup of 4 waves side by side along
// N (each wave 256 x BN/4). X tiles (256 rows x 64) go through LDS (rows of
// 128 B with the 16-B chunks XOR-swizzled by row); each wave decodes
// its own W rows straight into MFMA B registers, so W never touches LDS and
// each weight is decoded once per workgroup.
//
// dX layout: 256 x BN outputs per workgroup, 8 waves (2 x 4, two per SIMD) on
// 256 x 256 tiles and 4 waves (2 x 2) on 256 x 128 tiles. The reduction
// runs over N, while the codes are K-contiguous, so each thread decodes one
// row-block (64 weights) into an LDS tile [n][k], and the MFMA B operand is
// read from it transposed with ds_read_b64_tr_b16 (gfx950): within a group of
// 16 lanes, lane 4b + e receives element a of the 8-byte piece addressed by
// lane 4a + b, which turns four 4-wide row pieces into four 4-tall columns.
//
// Workgroups are mapped XCD-aware: the hardware deals workgroups round-robin
// to the 8 XCDs, so consecutive logical tiles (the M-tiles of one W tile) are
// made to land on one XCD and share its L2.
#include <hip/hip_ext.h>

#include <atomic>
#include <type_traits>

#include "ql_internal.h"

namespace ql {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr int NT = 256;
constexpr int BM = 256;
constexpr int BK = 64;
constexpr int A_TILE = BM * BK * 2;  // 32 KB: 256 rows x 128 B

// A tile rows are 128 B (8 chunks of 16 B); chunk c of row r is stored at
// chunk c ^ f(r). The forward GEMM uses f(r) = (r ^ (r >> 3)) mod 8: its
// fragment reads (32 consecutive rows, one chunk per lane half) then run at
// about twice the LDS throughput of f(r) = r mod 8 in isolation, and the
// kernel gains a few percent. The backward GEMM keeps f(r) = r mod 8, which
// times a few percent faster there (its reads interleave with the decode's
// LDS traffic differently).
template <bool XS>
__device__ __forceinline__ int swz_row(int row) { return (XS ? row ^ (row >> 3) : row) & 7; }
template <bool XS>
__device__ __forceinline__ int swz_a(int row, int chunk) { return (row << 7) + ((chunk ^ swz_row<XS>(row)) << 4); }

__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t n) {
  const uint32_t q = n >> 3, rem = n & 7;
  const uint32_t xcd = bid & 7, local = bid >> 3;
  return xcd * q + (xcd < rem ? xcd : rem) + local;
}

// Coordinates of tile t of a tiles_m x tiles_n grid (dX). Consecutive tiles
// (one XCD's share after xcd_remap) cover blocks of 4 M-tiles across several
// column tiles, so each XCD's L2 fetches fewer distinct dY rows and weight rows
// than with all M-tiles of one column block first (4-5% faster at the 8B
// shapes; the forward keeps M-tiles first, which measured faster there).
// tiles_m not a multiple of 4: M-tiles first.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& mt, int& nt) {
  const int gm = tiles_m % 4 == 0 ? 4 : tiles_m;
  const int rb = t / (gm * tiles_n), u = t - rb * gm * tiles_n;
  mt = rb * gm + u % gm;
  nt = u / gm;
}

__device__ __forceinline__ int64_t remap_col(int64_t k, int head_dim, int n_rep) {
  if (n_rep <= 0) return k;
  const int64_t head = k / head_dim, i = k - head * head_dim;
  return (head / n_rep) * head_dim + i;
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 16-entry bf16 table of one row-block as two byte planes:
// lo[q] = low bytes of entries 4q..4q+3, hi[q] = high bytes.
struct Lut {
  uint32_t lo[4], hi[4];
};

__device__ __forceinline__ Lut make_lut(float a) {
  uint32_t d[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    d[i] = pack_bf16x2(__builtin_bit_cast(float, kNF4LevelBits[2 * i]) * a,
                       __builtin_bit_cast(float, kNF4LevelBits[2 * i + 1]) * a);
  Lut t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t.lo[q] = perm(d[2 * q + 1], d[2 * q], 0x06040200u);
    t.hi[q] = perm(d[2 * q + 1], d[2 * q], 0x07050301u);
  }
  return t;
}

// Four codes (one per byte, values 0..15, given as their low 3 bits `s3` and a
// byte-select vector `blend` = 0x03020100 + 4 * bit3) -> byte plane of 4 values.
__device__ __forceinline__ uint32_t plane4(const uint32_t (&tab)[4], uint32_t s3, uint32_t blend) {
  const uint32_t r0 = perm(tab[1], tab[0], s3);  // entries 0..7
  const uint32_t r1 = perm(tab[3], tab[2], s3);  // entries 8..15
  return perm(r1, r0, blend);
}

// One word of 8 codes (byte j: code j low nibble, code j+4 high nibble) ->
// 8 bf16 in element order, as 4 dwords.
__device__ __forceinline__ uint4 decode8(uint32_t p, const Lut& t) {
  const uint32_t s3l = p & 0x07070707u;
  const uint32_t bl = ((p >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t s3h = (p >> 4) & 0x07070707u;
  const uint32_t bh = ((p >> 5) & 0x04040404u) | 0x03020100u;
  const uint32_t lo_l = plane4(t.lo, s3l, bl), hi_l = plane4(t.hi, s3l, bl);  // codes 0..3
  const uint32_t lo_h = plane4(t.lo, s3h, bh), hi_h = plane4(t.hi, s3h, bh);  // codes 4..7
  uint4 r;
  r.x = perm(hi_l, lo_l, 0x05010400u);
  r.y = perm(hi_l, lo_l, 0x07030602u);
  r.z = perm(hi_h, lo_h, 0x05010400u);
  r.w = perm(hi_h, lo_h, 0x07030602u);
  return r;
}

// Eight consecutive bf16 s * B[j] (j < r, zero past r) as 4 dwords.
__device__ __forceinline__ uint4 lora_row8(const uint16_t* row, int j0, int r, float s) {
  float f[8];
  if ((r & 7) == 0) {  // 16-byte aligned groups of 8
    uint4 v = j0 < r ? *(const uint4*)(row + j0) : make_uint4(0, 0, 0, 0);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = s * __builtin_bit_cast(float, wv[e] << 16);
      f[2 * e + 1] = s * __builtin_bit_cast(float, wv[e] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (j0 + e < r) ? s * bf16_to_f32(row[j0 + e]) : 0.f;
  }
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// Buffer resources: loads through a base in SGPRs and a 32-bit lane offset;
// a raw buffer load at or past num_records returns zero, which masks the rows
// past the end of a tile without branches. The range is clamped to 2^31 - 1
// bytes: every descriptor here is based at the block it serves (at most 256
// rows of activations, or 64 rows of codes in a dX reduction step), and with
// dimensions of at most QL_MAX_DIM every offset into such a block stays below
// 2^31 whatever the size of the whole tensor.
// Base and size are made provably wave-uniform so the descriptor lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  const uint64_t p = (uint64_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)n), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// A lane offset past every descriptor's range (buffer loads return zeros,
// stores are dropped).
constexpr uint32_t kPastRange = 0x80000000u;

// s * v for 8 bf16 values, rounded back to bf16.
__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float s) {
  const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = pack_bf16x2(s * __builtin_bit_cast(float, wv[e] << 16), s * __builtin_bit_cast(float, wv[e] & 0xffff0000u));
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Buffer-to-LDS DMA (gfx950): each lane's 16 bytes land at lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// A tile (256 rows x 64 bf16) by DMA: wave w moves 1-KB blocks b = 4 i + w
// (rows 8 b .. 8 b + 7); lane l fills row 8 b + l / 8 at physical chunk l % 8,
// which holds logical chunk (l % 8) ^ swz_row(8 b + l / 8): (l % 8) ^ (l / 8)
// for f(r) = r mod 8; with the XOR of r >> 3 also ^ (b mod 8), where b mod 8
// is w for even i and w + 4 for odd i.
template <bool XS>
__device__ __forceinline__ int dma_chunk(int lane, int w, int odd) {
  return (lane & 7) ^ (lane >> 3) ^ (XS ? w + 4 * odd : 0);
}

// A tile of the LoRA step: rows of a [M x r] bf16 matrix, zero past r (outside the main loop).
__device__ __forceinline__ void load_a_rank(uint4 (&ar)[8], const uint16_t* U, int r, int64_t M, int64_t m0,
                                            int t) {
  if ((r & 7) == 0) {  // whole 16-byte groups: buffer loads, zero past M and past r, no branches
    const __amdgpu_buffer_rsrc_t ur = rsrc(U + m0 * r, (M - m0) * r * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = t + NT * i;
      const int row = c >> 3, ch = c & 7;
      ar[i] = bload16(ur, ch * 8 < r ? (row * r + ch * 8) * 2 : (int)kPastRange, 0);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = t + NT * i;
    const int row = c >> 3, ch = c & 7;
    const int64_t m = m0 + row;
    uint32_t w[4] = {0, 0, 0, 0};
    if (m < M && ch * 8 < r) {
      if ((r & 7) == 0) {  // 16-byte aligned groups of 8
        const uint4 v = *(const uint4*)(U + m * r + ch * 8);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = ch * 8 + e;
          const uint32_t h = j < r ? (uint32_t)U[m * r + j] : 0u;
          w[e >> 1] |= h << ((e & 1) * 16);
        }
      }
    }
    ar[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Thread t moves chunks c = t + 256 i (i < 8) of a 256 x 64 A tile: row
// (t >> 3) + 32 i, 16-byte chunk t & 7.
template <bool XS>
__device__ __forceinline__ void store_a(uint8_t* As, const uint4 (&ar)[8], int t) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = t + NT * i;
    *(uint4*)(As + swz_a<XS>(c >> 3, c & 7)) = ar[i];
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t word(const uint4& v, int q) {
  return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
}

// Epilogue stores of one 32-row block: lane value v[it] holds row it * RPI + rr
// (of the block) and columns col .. col + 3 (float32). MODE 0 stores float32
// partials, 1 bf16, 2 float32; with hres the bf16 residual (row stride ldr
// elements) is added first. Output row stride ld elements. Offsets of lanes
// with !col_ok lie past every descriptor's range (stores dropped, loads zero).
// Branch-free, so the loads and stores issue back to back.
template <int MODE, int NIT, int RPI>
__device__ __forceinline__ void epilogue_rows(const f32x4_t (&v)[NIT], __amdgpu_buffer_rsrc_t orr,
                                              __amdgpu_buffer_rsrc_t rrr, int rr, int col, bool col_ok, int ld,
                                              bool hres, int ldr) {
  constexpr uint32_t kPast = 0x80000000u;
  constexpr int ESZ = MODE == 1 ? 2 : 4;
  if constexpr (MODE == 0) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const uint32_t off = col_ok ? (uint32_t)(((it * RPI + rr) * ld + col) * 4) : kPast;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v[it]), orr, off, 0, 0);
    }
  } else {
    uint2 rv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const uint32_t off = col_ok ? (uint32_t)(((it * RPI + rr) * ldr + col) * 2) : kPast;
      rv[it] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rrr, off, 0, 0));
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float f[4] = {v[it][0], v[it][1], v[it][2], v[it][3]};
      const float r[4] = {__builtin_bit_cast(float, rv[it].x << 16), __builtin_bit_cast(float, rv[it].x & 0xffff0000u),
                          __builtin_bit_cast(float, rv[it].y << 16), __builtin_bit_cast(float, rv[it].y & 0xffff0000u)};
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = hres ? f[e] + r[e] : f[e];
      const uint32_t off = col_ok ? (uint32_t)(((it * RPI + rr) * ld + col) * ESZ) : kPast;
      if constexpr (MODE == 2)
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4_t{__builtin_bit_cast(uint32_t, f[0]), __builtin_bit_cast(uint32_t, f[1]),
                    __builtin_bit_cast(uint32_t, f[2]), __builtin_bit_cast(uint32_t, f[3])},
            orr, off, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])}, orr, off, 0, 0);
    }
  }
}

// =============================================================== forward
// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]); only vmcnt is limited here.
// vmcnt(n) together with lgkmcnt(0). The K-loop's barriers use explicit waits
// rather than __syncthreads, whose release fence would also wait for the
// A-tile DMA issued two steps ahead (DMA writes to LDS count in vmcnt).
constexpr int vm_lgkm_wait(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }

constexpr int FWD_STAGES = 3;
// One forward LDS stage: the X tile (256 rows x 128 B, swizzled), the codes of
// the workgroup's BN weight rows for one K-step (BN rows x 32 B) and their
// absmax (256 floats; rows past BN are loaded as zeros and never read). The
// three X tiles come first, then the three code + scale blocks, so that the
// fragment reads of stages 0 and 1 fit the 16-bit LDS offset field.
template <int BN>
constexpr int fwd_cs_bytes() { return BN * 32 + 1024; }
template <int BN>
constexpr int fwd_stage_bytes() { return A_TILE + fwd_cs_bytes<BN>(); }

// DMA of 4-byte elements: lane l's word lands at lds + 4 * l.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

// WN: columns per wave (64 or 32); workgroup tile 256 x (4 WN).
// Every global read of the K-loop is a buffer-to-LDS DMA issued two K-steps
// ahead into a three-stage ring: while step s computes from stage
// (s - r) mod 3, step s + 2's X tile, codes and scales stream into the stage
// after the next. A barrier between sub-steps 2 and 3 of step s certifies step
// s + 1's data (each wave first waits for its own DMAs of it) and that no wave
// still reads the stage that is refilled next. The offset r = (KT - 2) mod 3
// aligns the stages so that the K-loop unrolls by three with every stage
// offset a compile-time constant and the last two steps use stages 0 and 1.
template <int WN>
__global__ __launch_bounds__(NT, 1) void k_gemm_fwd(const FwdArgs a, int tiles_m, int tiles_total,
                                                    int seg_tile0_1, int seg_tile0_2) {
  constexpr int NTW = WN / 32;
  constexpr int BN = 4 * WN;
  constexpr int CSB = fwd_cs_bytes<BN>();
  constexpr int SCALES = BN * 32;  // within a code + scale block
  // DMA instructions per wave per K-step: 8 for X, BN / 128 for codes, 1 for scales
  constexpr int NDMA = 8 + BN / 128 + 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int t = threadIdx.x, lane = t & 63, g = lane >> 5, li = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);

  // grid = tiles x nsplit; split sp of a tile takes K-steps [KT_all sp / S, KT_all (sp + 1) / S)
  const int gt = (int)xcd_remap(blockIdx.x, (uint32_t)(tiles_total * a.nsplit));
  const int sp = gt / tiles_total, tile = gt % tiles_total;
  const int sg = tile >= seg_tile0_2 ? 2 : (tile >= seg_tile0_1 ? 1 : 0);
  const int local = tile - (sg == 2 ? seg_tile0_2 : (sg == 1 ? seg_tile0_1 : 0));
  const FwdSeg& S = a.seg[sg];
  const int64_t m0 = (int64_t)(local % tiles_m) * BM;
  const int64_t n0 = (int64_t)(local / tiles_m) * BN;
  const int64_t K = a.K, kb = K / 64, M = a.M, N = S.N;
  const int KT_all = (int)(K / BK);
  const int ks0 = (int)((int64_t)KT_all * sp / a.nsplit);
  const int KT = (int)((int64_t)KT_all * (sp + 1) / a.nsplit) - ks0;

  // X tile rows m0.. (zero past M), W rows n0.. (zero past N)
  const int64_t xrows = M - m0 < BM ? M - m0 : BM;
  const int64_t wrows = N - n0 < BN ? N - n0 : BN;
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.X + m0 * a.ldx, xrows * a.ldx * 2);
  const __amdgpu_buffer_rsrc_t cr = rsrc(S.packed + n0 * (K / 2), wrows * (K / 2));
  const __amdgpu_buffer_rsrc_t sr = rsrc(S.absmax + n0 * kb, wrows * kb * 4);
  const int ldx = __builtin_amdgcn_readfirstlane((int)a.ldx);
  // lane's source offset for even / odd DMA blocks (the logical chunk differs)
  const int xrow = 8 * w + (lane >> 3);
  const int xvoff0 = xrow * ldx * 2 + dma_chunk<true>(lane, w, 0) * 16;
  const int xvoff1 = xrow * ldx * 2 + dma_chunk<true>(lane, w, 1) * 16;
  // codes: DMA instruction c moves rows 32 c .. 32 c + 31 (lane l: row 32 c + l / 2,
  // bytes 16 (l % 2) ..), landing contiguously at 1024 c of the code block
  const int cvoff = (lane >> 1) * (int)(K / 2) + 16 * (lane & 1);
  // scales: wave w moves rows 64 w + lane, landing at SCALES + 256 w
  const int svoff = (64 * w + lane) * (int)kb * 4;

  // Byte column of X for the K-step whose A tile is DMAed next (uniform). The
  // repeat_kv remap keeps a 64-wide step inside one head: step k0 = 64 t reads
  // column (head / n_rep) * head_dim + (k0 mod head_dim), head = k0 / head_dim.
  // Kept as running counters (ci: column in head, hr: head mod n_rep, hq:
  // head / n_rep) so the loop has no divisions or branches.
  const int hd = a.n_rep > 0 ? a.head_dim : (1 << 30);
  const int nrep = a.n_rep > 0 ? a.n_rep : 1;
  int ci, hr, hq;  // of the slice's first step, K-step ks0
  {
    const int k0 = ks0 * BK, head = k0 / hd;
    ci = k0 - head * hd;
    hr = head % nrep;
    hq = head / nrep;
  }
  auto xcol_next = [&]() -> int {
    const int c = 2 * (hq * hd + ci);
    ci += BK;
    const bool wrap = ci >= hd;
    ci = wrap ? 0 : ci;
    hr += wrap ? 1 : 0;
    const bool wrap2 = hr >= nrep;
    hr = wrap2 ? 0 : hr;
    hq += wrap2 ? 1 : 0;
    return c;
  };
  // stage si: X tile at A_of(si), codes and scales at CS_of(si)
  auto A_of = [&](int si) -> uint8_t* { return smem + si * A_TILE; };
  auto CS_of = [&](int si) -> uint8_t* { return smem + FWD_STAGES * A_TILE + si * CSB; };
  const int KT2 = KT - 2;
  const int roff = (KT2 % 3 + 3) % 3;
  auto stage_of = [&](int s) { return (s - roff + 3) % 3; };

  // DMA part h (0 or 1) of K-step `step` into stage si: half of the X tile
  // (1-KB blocks 4 i + w, i in [4 h, 4 h + 4)); part 0 also moves the codes
  // and scales. Steps are DMAed in order.
  int sc = 0;
  auto dma_part = [&](int step, int h, int si) {
    uint8_t* st = A_of(si);
    uint8_t* cs = CS_of(si);
    if (h == 0) sc = __builtin_amdgcn_readfirstlane(xcol_next());
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i)
      dma16(xr, st + (4 * i + w) * 1024, ((i & 1) ? xvoff1 : xvoff0) + i * 32 * ldx * 2, sc);
    if (h == 0) {
#pragma unroll
      for (int cc = 0; cc < BN / 128; ++cc) {
        const int c = w + 4 * cc;
        dma16(cr, cs + 1024 * c, cvoff + 32 * c * (int)(K / 2), (ks0 + step) * 32);
      }
      dma4(sr, cs + SCALES + 256 * w, svoff, (ks0 + step) * 4);
    }
  };

  f32x16_t acc[8][NTW];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x16_t{};

  uint4 bcur[NTW];
  Lut lut[NTW];
  const int code_lane = (w * WN + li) * 32 + 16 * g;
  auto decoded = [&](int j, int q) { return decode8(word(bcur[j], q), lut[j]); };
  // Codes and block tables of the K-step whose code block is cs. (All LDS reads of the
  // K-loop are typed loads; ordering against the DMAs is carried by the
  // explicit waits before each barrier.) Lane (li, g) takes the
  // 16 code bytes 16 g.. of rows w WN + 32 j + li. With two row groups the
  // lanes g = 0 and 1 hold the same rows, so each builds the table of one
  // (row group g) and the halves swap them (v_permlane32_swap: lanes 32..63 of
  // the first operand trade places with lanes 0..31 of the second).
  auto tables = [&](const uint8_t* cs) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const u32x4_t v = *(const u32x4_t*)(cs + code_lane + 1024 * j);
      bcur[j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    if constexpr (NTW == 2) {
      const float sc_own = *(const float*)(cs + SCALES + 4 * (w * WN + 32 * g + li));
      const Lut own = make_lut(sc_own);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto xl = __builtin_amdgcn_permlane32_swap(own.lo[e], own.lo[e], false, false);
        const auto xh = __builtin_amdgcn_permlane32_swap(own.hi[e], own.hi[e], false, false);
        lut[0].lo[e] = xl[0];
        lut[1].lo[e] = xl[1];
        lut[0].hi[e] = xh[0];
        lut[1].hi[e] = xh[1];
      }
    } else {
      lut[0] = make_lut(*(const float*)(cs + SCALES + 4 * (w * WN + li)));
    }
  };

  // One K-step of MFMAs on stage SI (a compile-time constant). Sub-step q's
  // MFMAs overlap the LDS reads and B decode of sub-step q + 1. HAS_NEXT:
  // between sub-steps 2 and 3 the workgroup meets at a barrier (every wave's
  // reads of this stage done, its DMAs of step + 1 landed), after which
  // sub-step 3 prefetches step + 1's first A fragments, codes and tables from
  // stage SI + 1, so the next step starts without waiting. DMA: step + 2's
  // data is issued in sub-steps 0 and 1 into stage SI + 2, read last in step
  // - 1. Scheduling groups pin the interleaving (LDS reads first, then MFMA /
  // VMEM / VALU alternating).
  bf16x8_t af[8], an[8];
  uint4 bq[NTW], bn[NTW];
  auto read_a = [&](bf16x8_t (&dst)[8], const uint8_t* As, int q) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = *(const bf16x8_t*)(As + swz_a<true>(i * 32 + li, 4 * g + q));
  };
  auto mma_step = [&](int step, auto si_c, auto has_next_c, auto dma_c) {
    constexpr int SI = decltype(si_c)::value;
    constexpr bool has_next = decltype(has_next_c)::value;
    constexpr bool dma = decltype(dma_c)::value;
    const uint8_t* As = A_of(SI);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int nvm = 0;
      if (dma && q < 2) {
        dma_part(step + 2, q, (SI + 2) % 3);
        nvm = q == 0 ? NDMA - 4 : 4;
      }
      if (q < 3) {
        read_a(an, As, q + 1);
#pragma unroll
        for (int j = 0; j < NTW; ++j) bn[j] = decoded(j, q + 1);
      } else if constexpr (has_next) {
        read_a(an, A_of((SI + 1) % 3), 0);
        tables(CS_of((SI + 1) % 3));
#pragma unroll
        for (int j = 0; j < NTW; ++j) bn[j] = decoded(j, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(bq[j]), af[i], acc[i][j], 0, 0, 0);
      if (q < 3) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      else if (has_next) __builtin_amdgcn_sched_group_barrier(0x100, 8 + NTW + 1, 0);
#pragma unroll
      for (int k = 0; k < 8 * NTW; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k < nvm) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (q < 3 || has_next) {
#pragma unroll
        for (int i = 0; i < 8; ++i) af[i] = an[i];
#pragma unroll
        for (int j = 0; j < NTW; ++j) bq[j] = bn[j];
      }
      if (q == 2 && has_next) {
        // only step + 2's DMAs (the last NDMA issued) may still be in flight
        __builtin_amdgcn_s_waitcnt(dma ? vm_lgkm_wait(NDMA) : vm_lgkm_wait(0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // prologue: steps 0 and 1 in flight; step 0's operands ready
  dma_part(0, 0, stage_of(0));
  dma_part(0, 1, stage_of(0));
  if (KT > 1) {
    dma_part(1, 0, stage_of(1));
    dma_part(1, 1, stage_of(1));
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(NDMA));
  } else {
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  read_a(af, A_of(stage_of(0)), 0);
  tables(CS_of(stage_of(0)));
#pragma unroll
  for (int j = 0; j < NTW; ++j) bq[j] = decoded(j, 0);
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  // steps 0 .. KT - 3 issue DMAs; the first roff of them bring the rest to a
  // multiple of three
  int step = 0;
  if (roff == 1 && KT2 >= 1) {
    mma_step(0, S2{}, T_{}, T_{});
    step = 1;
  } else if (roff == 2 && KT2 >= 2) {
    mma_step(0, S1{}, T_{}, T_{});
    mma_step(1, S2{}, T_{}, T_{});
    step = 2;
  }
  for (; step < KT2; step += 3) {
    mma_step(step, S0{}, T_{}, T_{});
    mma_step(step + 1, S1{}, T_{}, T_{});
    mma_step(step + 2, S2{}, T_{}, T_{});
  }
  if (KT > 1) {  // step KT - 2, stage 0
    mma_step(step, S0{}, T_{}, F_{});
    ++step;
  }
  {  // last weight step (stage 1); the LoRA step's A tile (U) goes to stage 2,
     // last read two steps ago (before the barrier of the previous step)
    mma_step(step, S1{}, F_{}, F_{});
    if (a.r > 0 && sp == a.nsplit - 1) {
      uint4 ar[8];
      load_a_rank(ar, S.U, a.r, M, m0, t);
      store_a<true>(A_of(2), ar, t);
      __syncthreads();
    }
  }
  // LoRA step: [U | 0] [s B | 0]^T (none with r = 0: the adapter is off;
  // with a split reduction, in the last split only)
  if (a.r > 0 && sp == a.nsplit - 1) {
    uint4 lb[NTW][4];
    if ((a.r & 7) == 0) {  // buffer loads, zero past N and past r, no branches
      const __amdgpu_buffer_rsrc_t br = rsrc(S.B + n0 * a.r, (N - n0) * a.r * 2);
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int nl = w * WN + 32 * j + li;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j0 = 32 * g + 8 * q;
          lb[j][q] = scale_bf16x8(bload16(br, j0 < a.r ? (nl * a.r + j0) * 2 : (int)kPastRange, 0), a.s);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int64_t n = n0 + w * WN + 32 * j + li;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          lb[j][q] = n < N ? lora_row8(S.B + n * a.r, 32 * g + 8 * q, a.r, a.s) : make_uint4(0, 0, 0, 0);
      }
    }
    const uint8_t* As = A_of(2);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x8_t a8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a8[i] = *(const bf16x8_t*)(As + swz_a<true>(i * 32 + li, 4 * g + q));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lb[j][q]), a8[i], acc[i][j], 0, 0, 0);
    }
  }

  // Partials of a split reduction: per segment, nsplit blocks of [M x N]
  // float32 after those of the earlier segments.
  const int64_t ppart = (int64_t)a.nsplit * M * ((sg >= 1 ? a.seg[0].N : 0) + (sg >= 2 ? a.seg[1].N : 0));
  // Epilogue. The products above are C = W X^T (the weight operand first), so
  // lane (li, g) of accumulator [i][j] holds output row m = m0 + 32 i + li and,
  // in entries 4 v .. 4 v + 3, the four consecutive columns
  // n0 + w WN + 32 j + 8 v + 4 g + (0..3). Stored as they are, one store
  // instruction would touch 32 rows with 16 or 32 bytes each. Instead each
  // 32-row block of a wave's columns goes through LDS (stage 0's X tile, whose
  // last reads precede the barrier of step KT - 2 and which no DMA targets
  // after it) and comes back as whole row segments: lanes 16 r' + c read
  // 16-byte chunk c of row r', so each store covers WN / 16 rows with
  // WN * 4 (float32) or WN * 2 (bf16) contiguous bytes per row. Chunks are
  // XOR-swizzled by row so the writes, 32 rows of one chunk, spread over the
  // banks. N % 16 == 0, so a 4-column group is wholly inside or outside.
  constexpr int CPRW = WN / 4;       // 16-byte chunks per staged row
  constexpr int RPI = 64 / CPRW;     // rows per read instruction
  uint8_t* E = A_of(0) + w * (32 * WN * 4);
  const int rc = lane % CPRW, rr = lane / CPRW;
  const int64_t n = n0 + w * WN + 4 * rc;
  // Stores go through buffer descriptors based at each 32-row block, whose
  // ranges end at the last valid element: rows past M are dropped by the
  // hardware, lanes past column N get an offset beyond every range, and no
  // store or residual load sits behind a branch, so they issue back to back
  // with no per-row wait. Offsets stay below 32 rows of at most QL_MAX_DIM
  // float32 columns.
  const int mode = a.nsplit > 1 ? 0 : (a.out_f32 ? 2 : 1);  // partial, float32, bf16 (uniform)
  const bool hres = mode != 0 && S.resid != nullptr;
  const int esz = mode == 1 ? 2 : 4;
  const int64_t ldo = mode == 0 ? N : S.ldo;  // elements per output row
  const uint8_t* obase = mode == 0 ? (const uint8_t*)(a.partial + ppart + ((int64_t)sp * M + m0) * N)
                                   : (const uint8_t*)S.out + (m0 * S.ldo + S.col0) * esz;
  const uint8_t* rbase = hres ? (const uint8_t*)(S.resid + m0 * S.ldo + S.col0) : nullptr;
  const bool n_ok = n < N;
  auto epilogue = [&](auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    f32x4_t fv[32 / RPI];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int c = 8 * j + 2 * v + g;
          *(f32x4_t*)(E + li * (WN * 4) + ((c ^ (li & (CPRW - 1))) << 4)) =
              f32x4_t{acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2], acc[i][j][4 * v + 3]};
        }
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int row = it * RPI + rr;
        fv[it] = *(const f32x4_t*)(E + row * (WN * 4) + ((rc ^ (row & (CPRW - 1))) << 4));
      }
      const int64_t rows = M - m0 - 32 * i < 32 ? M - m0 - 32 * i : 32;
      const int64_t span = rows > 0 ? (rows - 1) * ldo + N : 0;  // elements
      const __amdgpu_buffer_rsrc_t orr = rsrc(obase + 32 * i * ldo * esz, span * esz);
      const __amdgpu_buffer_rsrc_t rrr = rsrc(hres ? rbase + 32 * i * ldo * 2 : nullptr, hres ? span * 2 : 0);
      epilogue_rows<MODE, 32 / RPI, RPI>(fv, orr, rrr, rr, (int)n, n_ok, (int)ldo, hres, (int)ldo);
    }
  };
  if (mode == 0) epilogue(std::integral_constant<int, 0>{});
  else if (mode == 1) epilogue(std::integral_constant<int, 1>{});
  else epilogue(std::integral_constant<int, 2>{});
}

// =============================================================== backward dX
// LDS B tile: [64 reduction rows n][BN output columns k] bf16, rows of 2 BN
// bytes (a multiple of 256, so every row starts at bank 0). The LDS serves
// 256 B (64 banks) per clock, so conflict-free means 16 distinct 16-B chunk
// slots mod 16 among the lanes served together:
// - a 16-B row-chunk write (16 lanes: 16 consecutive rows, one chunk) gets
//   slot bits 0-2 from n mod 8 and bit 3 from n bit 3;
// - a transposed 8-B read (32 lanes: rows 4a..4a+3, chunks 4b..4b+3) gets
//   bits 1-2 from n mod 4, bit 0 from the chunk, and bit 3 from chunk bit 1.
// The XOR term depends on the chunk only through bit 1, which it leaves
// unchanged, so each row's chunks stay a permutation.
__device__ __forceinline__ int swz_f(int n) { return ((n & 3) << 1) | ((n >> 2) & 1) | (((n >> 3) & 1) << 3); }

template <int BN>
__device__ __forceinline__ int bt_off(int n, int k) {
  const int chunk = k >> 3;
  return n * (BN * 2) + ((chunk ^ swz_f(n) ^ (((chunk >> 1) & 1) << 3)) << 4) + ((k & 4) << 1);
}

// Raw weight data of one reduction step in LDS: the codes of 64 rows x BN
// columns (BN / 2 bytes per row in 16-byte chunks; chunk c of row n sits in
// slot n CPR + (c ^ ((n >> SH) mod CPR)), so 16 lanes reading one chunk of 16
// consecutive rows hit distinct banks), then the absmax of 64 rows x 4 blocks.
template <int BN>
constexpr int bwd_raw_bytes() { return 64 * (BN / 2) + 1024; }
// By-value select among three uniform values (a ternary on lvalues would
// select an address and keep the values in private memory).
template <typename T>
__device__ __forceinline__ T sel3(int s, T v0, T v1, T v2) {
  T r = v2;
  r = s == 1 ? v1 : r;
  r = s == 0 ? v0 : r;
  return r;
}

template <int BN>
__device__ __forceinline__ int raw_slot(int n, int c) {
  constexpr int CPR = BN / 32;
  constexpr int SH = CPR == 8 ? 1 : 2;
  return n * CPR + (c ^ ((n >> SH) & (CPR - 1)));
}

// Workgroup tile 256 x BN (BN = 2 WNB) at columns k_base + (tile / tiles_m) BN.
// NWV = 4: waves 2 x 2, each 128 rows x WNB columns (2 WNB accumulator
// registers per lane), one wave per SIMD. NWV = 8: waves 2 x 4, each 128 rows x BN / 4
// columns with 128 accumulators, two waves per SIMD, so that one wave's VALU
// and LDS work issues while the other's MFMAs run. The workgroup decodes each
// weight step once either way; with 8 waves each thread decodes half a block
// row (32 weights) and every dY fragment feeds half as many MFMAs. Reduction
// order: for each segment its 64-row weight steps, then the LoRA steps of all
// segments.
//
// LDS: two dY stages and two raw-code stages (the DMA targets) and two decoded
// weight tiles, in separate arrays. The transposing reads of the weight tiles
// then provably touch no DMA target, so the compiler does not wait for the
// DMAs in flight before them, and each sub-step can read the next sub-step's
// operands while its MFMAs run.
//
// Pipeline. Reduction step t's codes arrive by DMA during step t - 2, are
// loaded into registers at the end of step t - 2, and are decoded during
// sub-steps 0-2 of step t - 1 into the decoded tile of t; its dY tile is
// DMAed from sub-step 3 of step t - 2. In step s, sub-step q reads the
// operands of q + 1. One barrier per step, between sub-steps 2 and 3, where
// each wave has first waited for its own DMAs and LDS operations: after it,
// step s + 1's decoded tile and dY tile are complete, and no wave reads step
// s's stages again, so sub-step 3 prefetches step s + 1's first operands and
// DMAs step s + 2's dY tile into step s's stage.
// The dY tile's 16-byte chunks are swizzled by f(r) = (r ^ (r >> 3)) mod 8,
// as in the forward: a fragment read (16 lanes, 16 consecutive rows, one
// chunk) then meets 16 distinct bank groups, where f(r) = r mod 8 would put
// rows r and r + 8 on the same ones.
constexpr bool BXS = true;

template <int WNB, int NWV>
__global__ __launch_bounds__(64 * NWV, 1) void k_gemm_bwd(const BwdArgs a, int tiles_m, int tiles_total, int k_base) {
  constexpr int BN = 2 * WNB;
  // NWV = 4: waves 2 x 2 of 128 x WNB; NWV = 8: waves 2 x 4 of 128 x BN / 4 (two per SIMD)
  constexpr int WAVES_K = NWV / 2;
  constexpr int WC = BN / WAVES_K;
  constexpr int NTH = 64 * NWV;
  constexpr int NTW = WC / 32;
  constexpr int CPR = BN / 32;
  constexpr int SH = CPR == 8 ? 1 : 2;
  constexpr int RAW = bwd_raw_bytes<BN>();
  constexpr int DEC_BYTES = 64 * BN * 2;
  constexpr int ABS = 64 * (BN / 2);
  // one array per stage: with compile-time stages, a read of one stage
  // provably misses a DMA in flight into the other
  __shared__ __attribute__((aligned(16))) uint8_t lds_a0[A_TILE], lds_a1[A_TILE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_r0[RAW], lds_r1[RAW];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b0[DEC_BYTES], lds_b1[DEC_BYTES];
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto stage_a = [&](auto si) -> uint8_t* { return decltype(si)::value ? lds_a1 : lds_a0; };
  auto stage_r = [&](auto si) -> uint8_t* { return decltype(si)::value ? lds_r1 : lds_r0; };
  auto stage_b = [&](auto si) -> uint8_t* { return decltype(si)::value ? lds_b1 : lds_b0; };
  const int t = threadIdx.x, lane = t & 63, g = lane >> 5, li = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), wm = w / WAVES_K, wn = w % WAVES_K;

  // grid = tiles x nsplit; split sp of a tile takes weight steps [WS sp / S, WS (sp + 1) / S)
  const int gt = (int)xcd_remap(blockIdx.x, (uint32_t)(tiles_total * a.nsplit));
  const int sp = gt / tiles_total, tile = gt % tiles_total;
  int mt, nt;
  tile_coords(tile, tiles_m, tiles_total / tiles_m, mt, nt);
  const int64_t m0 = (int64_t)mt * BM;
  const int64_t k0 = (int64_t)k_base + (int64_t)nt * BN;
  const int64_t K = a.K, kbn = K / 64, M = a.M;
  const int64_t xrows = M - m0 < BM ? M - m0 : BM;
  const int nseg = a.nseg;

  // per-segment descriptors (uniform; selected, never indexed)
  auto seg_n = [&](int s) -> int64_t { return s < nseg ? a.seg[s].N : 0; };
  const int64_t N0 = seg_n(0), N1 = seg_n(1), N2 = seg_n(2);
  auto ydesc = [&](int s, int64_t N) {
    return rsrc(s < nseg ? (const void*)(a.seg[s].dY + m0 * N) : nullptr, s < nseg ? xrows * N * 2 : 0);
  };
  const __amdgpu_buffer_rsrc_t yr0 = ydesc(0, N0), yr1 = ydesc(1, N1), yr2 = ydesc(2, N2);
  // codes and scales of each segment from the tile's first output column
  auto seg_codes = [&](int s) { return s < nseg ? a.seg[s].packed + k0 / 2 : (const uint8_t*)nullptr; };
  auto seg_scales = [&](int s) { return s < nseg ? a.seg[s].absmax + k0 / 64 : (const float*)nullptr; };
  const uint8_t *pk0 = seg_codes(0), *pk1 = seg_codes(1), *pk2 = seg_codes(2);
  const float *am0 = seg_scales(0), *am1 = seg_scales(1), *am2 = seg_scales(2);
  const int WS_all = (int)((N0 + BK - 1) / BK + (N1 + BK - 1) / BK + (N2 + BK - 1) / BK);
  const int ws_begin = (int)((int64_t)WS_all * sp / a.nsplit);
  const int WS = (int)((int64_t)WS_all * (sp + 1) / a.nsplit) - ws_begin;

  // DMA cursors (segment, first reduction row) of the next dY tile and the
  // next raw step; both walk the weight steps in order from ws_begin.
  int sgA = 0, nbA = 0;
  {
    int s = ws_begin;
    const int st0 = (int)((N0 + BK - 1) / BK), st1 = (int)((N1 + BK - 1) / BK);
    if (s >= st0) { s -= st0; ++sgA; if (s >= st1) { s -= st1; ++sgA; } }
    nbA = s * BK;
  }
  int sgR = sgA, nbR = nbA;
  auto advance = [&](int& sg, int& nb) {
    const int64_t N = sel3(sg, N0, N1, N2);
    nb += BK;
    const bool wrap = nb >= N;
    nb = wrap ? 0 : nb;
    sg += wrap ? 1 : 0;
  };

  // dY tile (256 rows x 64 columns of segment sgA from nbA) into an A stage;
  // columns past the segment's N read as zeros (offset past the buffer).
  // 1-KB block b = NWV i + w holds rows 8 b .. 8 b + 7 (with 8 waves b mod 8 = w for every i)
  constexpr int DPI = 32 / NWV;  // dY DMAs per wave
  const int arow = 8 * w + (lane >> 3), alc0 = dma_chunk<BXS>(lane, w, 0),
            alc1 = dma_chunk<BXS>(lane, w, NWV == 4 ? 1 : 0);
  auto dma_a = [&](uint8_t* As) {
    const int64_t N = sel3(sgA, N0, N1, N2);
    const __amdgpu_buffer_rsrc_t yr = sel3(sgA, yr0, yr1, yr2);
    const int ldy = __builtin_amdgcn_readfirstlane((int)N);
    const int ylim = __builtin_amdgcn_readfirstlane((int)(xrows * N * 2));
    // all-ones where the lane's 8 columns lie past N (branch-free select)
    const int past0 = -(int)(nbA + 8 * alc0 >= N), past1 = -(int)(nbA + 8 * alc1 >= N);
    const int so = __builtin_amdgcn_readfirstlane(nbA * 2);
#pragma unroll
    for (int i = 0; i < DPI; ++i) {
      const int alc = (i & 1) ? alc1 : alc0, past = (i & 1) ? past1 : past0;
      const int vo = (((arow + 8 * NWV * i) * ldy * 2 + alc * 16) & ~past) | (ylim & past);
      dma16(yr, As + (NWV * i + w) * 1024, vo, so);
    }
    advance(sgA, nbA);
  };
  // Raw codes and scales of the step at (sgR, nbR) into a raw stage. The
  // descriptors are based at the step's first weight row, with the offset
  // formed in 64 bits, so the 32-bit lane offsets stay inside one step (64
  // rows of at most 2^20 bytes) whatever the size of the weight; rows past the
  // segment's end lie past the descriptor's range and read as zeros.
  auto dma_raw = [&](uint8_t* R) {
    const int64_t N = sel3(sgR, N0, N1, N2);
    const int64_t rows_left = N - nbR;
    const __amdgpu_buffer_rsrc_t cr = rsrc(sel3(sgR, pk0, pk1, pk2) + (int64_t)nbR * (K / 2), rows_left * (K / 2) - k0 / 2);
    const __amdgpu_buffer_rsrc_t sr = rsrc(sel3(sgR, am0, am1, am2) + (int64_t)nbR * kbn, (rows_left * kbn - k0 / 64) * 4);
    const int kh = (int)(K / 2);
#pragma unroll
    for (int cc = 0; cc < CPR / NWV; ++cc) {
      const int ci = w + NWV * cc;
      const int slot = ci * 64 + lane;
      const int n = slot / CPR, pc = slot % CPR;
      const int c = pc ^ ((n >> SH) & (CPR - 1));
      dma16(cr, R + ci * 1024, n * kh + c * 16, 0);
    }
    if (NWV == 4 || w < 4) dma4(sr, R + ABS + 256 * w, ((16 * w + (lane >> 2)) * (int)kbn + (lane & 3)) * 4, 0);
    advance(sgR, nbR);
  };

  // decode share of a thread: row dn, 64-column block dc (wide) or half dh of it (narrow)
  constexpr int NCH = 2 * BN / NTH;  // 16-byte code chunks per thread
  constexpr int NW = 4 * NCH;        // code words (8 weights each) per thread per step
  const int dn = t & 63, dc = (t >> 6) & (BN / 64 - 1), dh = NCH == 2 ? 0 : (t >> 6) / (BN / 64);
  uint32_t dcode[NW];
  float dscale;
  Lut dlut;
  // the thread's codes and block scale of one step into registers; the table
  // is built from the scale later (dec_lut), so nothing waits for these reads
  auto dec_load = [&](const uint8_t* R) {
#pragma unroll
    for (int h = 0; h < NCH; ++h) {
      const u32x4_t v = *(const u32x4_t*)(R + raw_slot<BN>(dn, 2 * dc + dh + h) * 16);
      dcode[4 * h] = v[0];
      dcode[4 * h + 1] = v[1];
      dcode[4 * h + 2] = v[2];
      dcode[4 * h + 3] = v[3];
    }
    dscale = *(const float*)(R + ABS + (dn * 4 + dc) * 4);
  };
  auto dec_lut = [&]() { dlut = make_lut(dscale); };
  // word e of the thread's codes -> 8 bf16 at columns 64 dc + 32 dh + 8 e
  auto dec_word = [&](uint8_t* Bd, int e) {
    const uint4 v = decode8(dcode[e], dlut);
    *(u32x4_t*)(Bd + bt_off<BN>(dn, 64 * dc + 32 * dh + 8 * e)) = u32x4_t{v.x, v.y, v.z, v.w};
  };

  f32x16_t acc[4][NTW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x16_t{};

  // transposed-read coordinates: within each group of 16 lanes, lane 4 ra + cbq
  // addresses row ra (of four) and the 4-column piece cbq (of four)
  const int h16 = lane >> 4, s16 = lane & 15, ra = s16 >> 2, cbq = s16 & 3;
  auto read_a = [&](bf16x8_t (&fa)[4], const uint8_t* As, int q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *(const bf16x8_t*)(As + swz_a<BXS>(wm * 128 + i * 32 + li, 2 * q + g));
  };
  // weight fragments of sub-step q, read transposed
  auto read_b = [&](bf16x8_t (&fb)[NTW], const uint8_t* Bs, int q) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      // lanes 32 g + c (c < 32) need column c and reduction rows 16 q + 8 g .. + 8
      const int col = wn * WC + 32 * j + 16 * (h16 & 1) + 4 * cbq;
      const int row = 16 * q + 8 * (h16 >> 1) + ra;
      const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(Bs + bt_off<BN>(row, col)));
      const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(Bs + bt_off<BN>(row + 4, col)));
      const i16x8_t v = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      fb[j] = __builtin_bit_cast(bf16x8_t, v);
    }
  };
  auto mfmas = [&](const bf16x8_t (&fa)[4], const bf16x8_t (&fb)[NTW]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };
  auto barrier_all = [&]() {
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  // Operands of the current sub-step (af, bq) and of the next (an, bn).
  bf16x8_t af[4], an[4], bq[NTW], bn[NTW];
  // Step s on stage SI = s mod 2 (a compile-time constant). Every step runs
  // the whole pipeline: it DMAs step s + 2's codes and dY tile, loads step
  // s + 2's codes, decodes step s + 1 and prefetches its first operands. For
  // the last two steps some of these steps do not exist: their DMAs read
  // in-range bytes (of the last segment, or none at all) and the results go
  // to stages that nothing reads afterwards, so no branch is needed.
  auto step_body = [&](auto si_c) {
    constexpr int SI = decltype(si_c)::value;
    using Cur = std::integral_constant<int, SI>;
    using Oth = std::integral_constant<int, 1 - SI>;
    const uint8_t* As = stage_a(Cur{});
    const uint8_t* Bs = stage_b(Cur{});
    uint8_t* Bd = stage_b(Oth{});
    auto sub = [&](auto q_c) {
      constexpr int q = decltype(q_c)::value;
      // words of step s + 1 decoded in this sub-step: 3, 3, 2 (wide) or 2, 1, 1
      constexpr int e0 = (q * NW + 2) / 3, e1 = q < 3 ? ((q + 1) * NW + 2) / 3 : e0;
      constexpr int nwr = e1 - e0;
      constexpr int nr = 4 + 2 * NTW + (q == 3 ? NCH + 1 : 0);
      constexpr int nd = q == 0 ? CPR / NWV + 1 : (q == 3 ? DPI : 0);
      if (q == 0) {
        dma_raw(stage_r(Cur{}));  // step s + 2's codes (this stage's went to registers at step s - 2)
        dec_lut();                // the table of step s + 1's codes
      }
      if (q < 3) {
        read_a(an, As, q + 1);
        read_b(bn, Bs, q + 1);
      } else {
        read_a(an, stage_a(Oth{}), 0);
        read_b(bn, stage_b(Oth{}), 0);
        dma_a(stage_a(Cur{}));     // step s + 2's dY into this step's stage
        dec_load(stage_r(Cur{}));  // step s + 2's codes, landed at the barrier
      }
#pragma unroll
      for (int e = e0; e < e1; ++e) dec_word(Bd, e);
      mfmas(af, bq);
      // the next operands' LDS reads first, then each MFMA followed by its
      // share of the VALU and the DMAs, with the decoded words' LDS writes last
      __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
#pragma unroll
      for (int k = 0; k < 4 * NTW; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k < nd) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        if (k >= 4 * NTW - nwr) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = an[i];
#pragma unroll
      for (int j = 0; j < NTW; ++j) bq[j] = bn[j];
      if (q == 2) barrier_all();
    };
    sub(std::integral_constant<int, 0>{});
    sub(std::integral_constant<int, 1>{});
    sub(std::integral_constant<int, 2>{});
    sub(std::integral_constant<int, 3>{});
  };

  if (WS > 0) {
    // prologue: dY tiles and codes of steps 0 and 1 in, step 0 decoded, step
    // 1's codes in registers, step 0's first operands read
    dma_a(lds_a0);
    dma_raw(lds_r0);
    dma_a(lds_a1);
    dma_raw(lds_r1);
    barrier_all();
    dec_load(lds_r0);
    dec_lut();
#pragma unroll
    for (int e = 0; e < NW; ++e) dec_word(lds_b0, e);
    dec_load(lds_r1);
    barrier_all();
    read_a(af, lds_a0, 0);
    read_b(bq, lds_b0, 0);
    int st = 0;
    for (; st + 1 < WS; st += 2) {
      step_body(S0{});
      step_body(S1{});
    }
    if (st < WS) step_body(S0{});
  }
  barrier_all();  // every wave done with the stages before the LoRA steps reuse them

  // LoRA steps: A = G_s, B rows j < r = s A_s[j][k0 ..], zero past r
  constexpr int UNITS = 64 * (BN / 64);
  const bool dthread = t < UNITS;
  const int drow = t & 63, dblk = (t >> 6) % (BN / 64);
  const int64_t dk = k0 + 64 * dblk;
  for (int sg = 0; sg < (sp == a.nsplit - 1 ? nseg : 0); ++sg) {
    const BwdSeg& S = a.seg[sg];
    uint8_t* As = (sg & 1) ? lds_a1 : lds_a0;
    uint8_t* Bs = (sg & 1) ? lds_b1 : lds_b0;
    if (NWV == 4 || t < NT) {
      uint4 ar[8];
      load_a_rank(ar, S.G, a.r, M, m0, t);
      store_a<BXS>(As, ar, t);
    }
    if (dthread) {  // buffer loads of A's rows, zero past r and past K, no branches
      const bool live = drow < a.r && dk < K;
      const __amdgpu_buffer_rsrc_t ar_ = rsrc(S.A, (int64_t)a.r * K * 2);
      const int base = live ? (int)((drow * K + dk) * 2) : (int)kPastRange;
      uint4 lv[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) lv[c] = bload16(ar_, live ? base + 16 * c : (int)kPastRange, 0);
#pragma unroll
      for (int c = 0; c < 8; ++c) *(uint4*)(Bs + bt_off<BN>(drow, 64 * dblk + 8 * c)) = scale_bf16x8(lv[c], a.s);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      read_a(af, As, q);
      read_b(bq, Bs, q);
      mfmas(af, bq);
    }
  }

  // Epilogue. The products are C = W^T dY^T (weight operand first), so lane
  // (li, g) of accumulator [i][j] holds output row m = m0 + 128 wm + 32 i + li
  // and, in entries 4 v .. 4 v + 3, the four consecutive columns
  // k0 + WNB wn + 32 j + 8 v + 4 g + (0..3). As in the forward, each 32-row
  // block of a wave's columns is staged through LDS (the dY stages, free after
  // the barrier below; waves 0, 1 in one, 2, 3 in the other) and stored as
  // whole row segments of WNB * 4 (float32) or WNB * 2 (bf16) bytes. K % 64
  // == 0, so a 4-column group is wholly inside or outside.
  __syncthreads();  // every wave done with the LoRA steps' stages
  constexpr int CPRW = WC / 4;  // 16-byte chunks per staged row
  constexpr int RPI = 64 / CPRW;  // rows per read instruction
  uint8_t* E = (wm ? lds_a1 : lds_a0) + wn * (32 * WC * 4);
  const int rc = lane % CPRW, rr = lane / CPRW;
  const int64_t k = k0 + wn * WC + 4 * rc;
  // buffer-descriptor stores per 32-row block, as in the forward
  const int64_t mw = m0 + wm * 128;
  const int mode = a.nsplit > 1 ? 0 : (a.out_f32 ? 2 : 1);  // partial, float32, bf16 (uniform)
  const bool hres = mode != 0 && a.resid != nullptr;
  const int esz = mode == 1 ? 2 : 4;
  const uint8_t* obase = mode == 0 ? (const uint8_t*)(a.partial + ((int64_t)sp * M + mw) * K)
                                   : (const uint8_t*)a.out + mw * K * esz;
  const uint8_t* rbase = hres ? (const uint8_t*)(a.resid + mw * K) : nullptr;
  const bool n_ok = k < K;
  auto epilogue = [&](auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    f32x4_t fv[32 / RPI];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int c = 8 * j + 2 * v + g;
          *(f32x4_t*)(E + li * (WC * 4) + ((c ^ (li & (CPRW - 1))) << 4)) =
              f32x4_t{acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2], acc[i][j][4 * v + 3]};
        }
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int row = it * RPI + rr;
        fv[it] = *(const f32x4_t*)(E + row * (WC * 4) + ((rc ^ (row & (CPRW - 1))) << 4));
      }
      const int64_t rows = M - mw - 32 * i < 32 ? M - mw - 32 * i : 32;
      const int64_t span = rows > 0 ? rows * K : 0;  // elements
      const __amdgpu_buffer_rsrc_t orr = rsrc(obase + 32 * i * K * esz, span * esz);
      const __amdgpu_buffer_rsrc_t rrr = rsrc(hres ? rbase + 32 * i * K * 2 : nullptr, hres ? span * 2 : 0);
      epilogue_rows<MODE, 32 / RPI, RPI>(fv, orr, rrr, rr, (int)k, n_ok, (int)K, hres, (int)K);
    }
  };
  if (mode == 0) epilogue(std::integral_constant<int, 0>{});
  else if (mode == 1) epilogue(std::integral_constant<int, 1>{});
  else epilogue(std::integral_constant<int, 2>{});
}

#define QL_TRY_PROF(expr)         \
  do {                            \
    ql_status rc_ = (expr);       \
    if (rc_ != QL_OK) return rc_; \
  } while (0)

template <int BN>
constexpr int fwd_lds() { return FWD_STAGES * fwd_stage_bytes<BN>(); }

// Per-device caches, filled on a device's first launch. Several host threads
// may launch at once: the flags and counts are atomics, and setting the
// attribute twice is harmless.
constexpr int kMaxDevices = 64;
std::atomic<bool> g_attr_set[kMaxDevices] = {};
std::atomic<int> g_cus[kMaxDevices] = {};

ql_status ensure_attrs() {
  int dev = 0;
  QL_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return set_error(QL_ERR_UNSUPPORTED, "device ordinal %d", dev);
  if (!g_attr_set[dev].load(std::memory_order_acquire)) {
    QL_HIP_CHECK(hipFuncSetAttribute((const void*)k_gemm_fwd<64>, hipFuncAttributeMaxDynamicSharedMemorySize, fwd_lds<256>()));
    QL_HIP_CHECK(hipFuncSetAttribute((const void*)k_gemm_fwd<32>, hipFuncAttributeMaxDynamicSharedMemorySize, fwd_lds<128>()));
    g_attr_set[dev].store(true, std::memory_order_release);
  }
  return QL_OK;
}

// Compute units of the current device (the launch geometry's round size).
// ensure_attrs has checked the device ordinal.
int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int c = g_cus[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  c = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  g_cus[dev].store(c, std::memory_order_relaxed);
  return c;
}

}  // namespace

namespace {

// One launch of the forward kernel over all segments of `a` with one tile width.
ql_status launch_fwd_tiles(const FwdArgs& a, bool wide, hipStream_t st) {
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const int bn = wide ? 256 : 128;
  int start[kMaxSegs + 1];
  start[0] = 0;
  for (int s = 0; s < kMaxSegs; ++s)
    start[s + 1] = start[s] + (s < a.nseg ? tiles_m * (int)((a.seg[s].N + bn - 1) / bn) : 0);
  const int total = start[a.nseg];
  if (total == 0) return QL_OK;
  const int s1 = a.nseg > 1 ? start[1] : total + 1;
  const int s2 = a.nseg > 2 ? start[2] : total + 1;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool prof = profiling_on();
  if (prof) QL_TRY_PROF(profile_begin(&e0, &e1));
  const int grid = total * a.nsplit;
  if (wide)
    hipExtLaunchKernelGGL(k_gemm_fwd<64>, dim3(grid), dim3(NT), fwd_lds<256>(), st, e0, e1, 0, a, tiles_m, total,
                          s1, s2);
  else
    hipExtLaunchKernelGGL(k_gemm_fwd<32>, dim3(grid), dim3(NT), fwd_lds<128>(), st, e0, e1, 0, a, tiles_m, total,
                          s1, s2);
  QL_HIP_CHECK(hipGetLastError());
  if (prof) {
    double flop = 0;
    for (int s = 0; s < a.nseg; ++s) flop += 2.0 * (double)a.M * (double)a.seg[s].N * (double)(a.K + a.r);
    QL_TRY_PROF(profile_end(e0, e1, wide ? QL_KERNEL_GEMM_FWD : QL_KERNEL_GEMM_FWD_NARROW, flop));
  }
  return QL_OK;
}

// Columns [c, N) of segment S as a segment of its own.
FwdSeg seg_from(const FwdSeg& S, int64_t c, int64_t K, int r) {
  FwdSeg o = S;
  o.packed += c * (K / 2);
  o.absmax += c * (K / 64);
  o.B += c * r;
  o.col0 += c;
  o.N -= c;
  return o;
}

}  // namespace

// Sum of the split partials in split order, plus the residual, rounded once
// (the same float32 operations as the unsplit epilogue: acc + resid).
__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ p, int nsplit, int64_t MK,
                                                   const uint16_t* __restrict__ resid, void* __restrict__ out,
                                                   int out_f32) {
  const int64_t n4 = MK / 4, stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n4; g += stride) {
    float4 f = ((const float4*)p)[g];
    for (int s = 1; s < nsplit; ++s) {
      const float4 q = ((const float4*)(p + (int64_t)s * MK))[g];
      f.x += q.x;
      f.y += q.y;
      f.z += q.z;
      f.w += q.w;
    }
    if (resid) {
      const uint2 rv = ((const uint2*)resid)[g];
      f.x += __builtin_bit_cast(float, rv.x << 16);
      f.y += __builtin_bit_cast(float, rv.x & 0xffff0000u);
      f.z += __builtin_bit_cast(float, rv.y << 16);
      f.w += __builtin_bit_cast(float, rv.y & 0xffff0000u);
    }
    if (out_f32)
      ((float4*)out)[g] = f;
    else
      ((uint2*)out)[g] = make_uint2(pack_bf16x2(f.x, f.y), pack_bf16x2(f.z, f.w));
  }
}

// Sum of a forward split reduction, per segment: out[m][col0 + n] = sum over
// splits in order of the float32 partials (+ the bf16 residual, same layout
// as out). grid: x over 4-column groups, y over rows, z over segments.
struct SumSeg {
  const float* p;  // [nsplit][M x N]
  void* out;
  const uint16_t* resid;
  int64_t N, ldo, col0;
};
struct SumArgs {
  SumSeg seg[kMaxSegs];
  int64_t M;
  int32_t nsplit, out_f32;
};
__global__ __launch_bounds__(256) void k_split_sum_segs(const SumArgs a) {
  const int z = blockIdx.z;
  const SumSeg S = z == 0 ? a.seg[0] : (z == 1 ? a.seg[1] : a.seg[2]);
  const int64_t n4 = S.N / 4, MN = a.M * S.N;
  for (int64_t m = blockIdx.y; m < a.M; m += gridDim.y) {
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n4; c += (int64_t)gridDim.x * blockDim.x) {
      const int64_t pi = m * S.N + 4 * c, o = m * S.ldo + S.col0 + 4 * c;
      float4 f = *(const float4*)(S.p + pi);
      for (int sp = 1; sp < a.nsplit; ++sp) {
        const float4 q = *(const float4*)(S.p + sp * MN + pi);
        f.x += q.x;
        f.y += q.y;
        f.z += q.z;
        f.w += q.w;
      }
      if (S.resid) {
        const uint2 rv = *(const uint2*)(S.resid + o);
        f.x += __builtin_bit_cast(float, rv.x << 16);
        f.y += __builtin_bit_cast(float, rv.x & 0xffff0000u);
        f.z += __builtin_bit_cast(float, rv.y << 16);
        f.w += __builtin_bit_cast(float, rv.y & 0xffff0000u);
      }
      if (a.out_f32)
        *(float4*)((float*)S.out + o) = f;
      else
        *(uint2*)((uint16_t*)S.out + o) = make_uint2(pack_bf16x2(f.x, f.y), pack_bf16x2(f.z, f.w));
    }
  }
}

// Launch geometry. Tiles are 256 x 256 (wide) or 256 x 128 (narrow); the chip
// runs cu_count workgroups per round. A narrow tile does half a wide tile's
// work but runs at a lower rate: it takes about kNarrowFwd (kNarrowBwd for dX)
// of a wide tile's time, from the two builds' measured rates. A partial round
// is re-cut into narrow tiles only when that takes fewer wide-tile times
// (8B q|k|v forward at M = 2048: 192 wide tiles in one round beat 384 narrow
// ones in two, 23% faster; 128 wide tiles are better as 256 narrow ones). With
// several rounds the whole rounds take wide tiles and the last partial round
// follows the same rule in a second launch (8B gate|up: 3 wide rounds + 1
// narrow instead of 4 wide). The geometry depends on shapes only, so resident
// and streamed runs pick the same kernels.
constexpr double kNarrowFwd = 0.7, kNarrowBwd = 0.85;
// Minimum K-steps per forward split slice when narrow tiles alone fill at
// least half the chip, from whole calls (the GEMM and the sum of its
// partials): the 4096 x 4096 forward at M=2048 takes 111 us split in two, 32
// steps each, against 99 us on narrow tiles; the M=512 gate forward 97 us
// split in two against 90.
constexpr int kFwdMinSteps = 64;
// A split on wide tiles whose slices are shorter than this many steps is
// re-planned on narrow tiles when those leave at least half the chip idle:
// twice the tiles, so half the split depth for the same workgroups, half the
// float32 partials and twice the steps per slice. Whole calls at M = 512:
// the 4096 x 4096 forward 46 us (narrow, 4 splits) against 56 (wide, 8),
// the 1024 x 4096 forward 35 against 44, the 4096-column dX 62 against 68;
// with 28-step slices (the 14336-row reductions) wide tiles stay ahead.
constexpr int kShortSlice = 16;
// 1 if re-cutting t wide tiles (t <= C) into tn narrow ones takes less time.
int narrow_pays(int t, int tn, int C, double ratio) {
  const int wide_rounds = (t + C - 1) / C, narrow_rounds = (tn + C - 1) / C;
  return ratio * narrow_rounds < (double)wide_rounds ? 1 : 0;
}
ql_status launch_gemm_fwd(const FwdArgs& a_in, hipStream_t st) {
  if (a_in.M == 0) return QL_OK;
  QL_TRY_PROF(ensure_attrs());
  FwdArgs a = a_in;
  a.nsplit = 1;
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const int C = cu_count();
  int t256 = 0, t128 = 0;
  for (int s = 0; s < a.nseg; ++s) {
    t256 += tiles_m * (int)((a.seg[s].N + 255) / 256);
    t128 += tiles_m * (int)((a.seg[s].N + 127) / 128);
  }
  // Split reduction over K when wide tiles would leave at least half the chip
  // idle and the caller gave space for partials: up to 8 workgroups per tile,
  // with at least kFwdMinSteps K-steps per slice when narrow tiles alone fill
  // at least half the chip, else at least 8 (whole calls at M=512: the 8B
  // down forward 95 us split against 141, k 43 against 76); reductions under
  // 24 K-steps are not split (the SmolLM2-shaped down forward, 24 steps on
  // 10 tiles, in three slices: that stack's step 9.67 against 10.03 ms).
  if (a.partial && 2 * t256 <= C) {
    int S = C / t256;
    if (S > 8) S = 8;
    const int kt = (int)(a.K / BK);
    const int min_steps = 2 * t128 >= C ? kFwdMinSteps : 8;
    if (kt < 24) S = 1;
    while (S > 1 && kt < min_steps * S) --S;
    int64_t ntot = 0;
    for (int s = 0; s < a.nseg; ++s) ntot += a.seg[s].N;
    while (S > 1 && (size_t)S * (size_t)a.M * (size_t)ntot * 4 > a.partial_bytes) --S;
    bool wide = true;
    if (S > 1 && kt / S < kShortSlice && 2 * t128 <= C) {
      int Sn = C / t128;
      if (Sn > 8) Sn = 8;
      while (Sn > 1 && kt < min_steps * Sn) --Sn;
      while (Sn > 1 && (size_t)Sn * (size_t)a.M * (size_t)ntot * 4 > a.partial_bytes) --Sn;
      if (Sn > 1) {
        S = Sn;
        wide = false;
      }
    }
    if (S > 1) {
      a.nsplit = S;
      QL_TRY_PROF(launch_fwd_tiles(a, wide, st));
      SumArgs sa{};
      sa.M = a.M;
      sa.nsplit = S;
      sa.out_f32 = a.out_f32;
      int64_t off = 0, nmax = 0;
      for (int s = 0; s < a.nseg; ++s) {
        const FwdSeg& G = a.seg[s];
        sa.seg[s] = SumSeg{a.partial + off, G.out, G.resid, G.N, G.ldo, G.col0};
        off += (int64_t)S * a.M * G.N;
        nmax = G.N > nmax ? G.N : nmax;
      }
      const int gx = (int)((nmax / 4 + 255) / 256);
      const int gy = (int)(a.M < 1024 ? a.M : 1024);
      hipLaunchKernelGGL(k_split_sum_segs, dim3(gx, gy, a.nseg), dim3(256), 0, st, sa);
      QL_HIP_CHECK(hipGetLastError());
      return QL_OK;
    }
  }
  if (t256 <= C) return launch_fwd_tiles(a, narrow_pays(t256, t128, C, kNarrowFwd) == 0, st);
  const int full = (t256 / C) * C;
  if (full == t256 || !narrow_pays(t256 - full, 2 * (t256 - full), C, kNarrowFwd)) return launch_fwd_tiles(a, true, st);
  // split at the column block holding wide tile `full` (enumeration order:
  // segment, column block, row block)
  FwdArgs aw = a, an = a;
  aw.nseg = 0;
  an.nseg = 0;
  int cum = 0;
  for (int s = 0; s < a.nseg; ++s) {
    const FwdSeg& S = a.seg[s];
    const int blocks = (int)((S.N + 255) / 256);
    if (an.nseg == 0 && cum + tiles_m * blocks <= full) {
      aw.seg[aw.nseg++] = S;
      cum += tiles_m * blocks;
      continue;
    }
    if (an.nseg == 0) {
      const int64_t kw = (int64_t)((full - cum) / tiles_m) * 256;  // columns left on wide tiles
      if (kw > 0) {
        aw.seg[aw.nseg] = S;
        aw.seg[aw.nseg].N = kw;
        ++aw.nseg;
      }
      an.seg[an.nseg++] = seg_from(S, kw, a.K, a.r);
    } else {
      an.seg[an.nseg++] = S;
    }
  }
  if (aw.nseg > 0) QL_TRY_PROF(launch_fwd_tiles(aw, true, st));
  return an.nseg > 0 ? launch_fwd_tiles(an, false, st) : QL_OK;
}

namespace {

// One launch of the dX kernel over output columns [k_base, k_base + k_cols).
ql_status launch_bwd_tiles(const BwdArgs& a, bool wide, int64_t k_base, int64_t k_cols, hipStream_t st) {
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const int bn = wide ? 256 : 128;
  const int total = tiles_m * (int)((k_cols + bn - 1) / bn);
  if (total == 0) return QL_OK;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool prof = profiling_on();
  if (prof) QL_TRY_PROF(profile_begin(&e0, &e1));
  const int grid = total * a.nsplit;
  if (wide)
    hipExtLaunchKernelGGL((k_gemm_bwd<128, 8>), dim3(grid), dim3(512), 0, st, e0, e1, 0, a, tiles_m, total,
                          (int)k_base);
  else
    hipExtLaunchKernelGGL((k_gemm_bwd<64, 4>), dim3(grid), dim3(NT), 0, st, e0, e1, 0, a, tiles_m, total,
                          (int)k_base);
  QL_HIP_CHECK(hipGetLastError());
  if (prof) {
    double flop = 0;
    for (int s = 0; s < a.nseg; ++s) flop += 2.0 * (double)a.M * (double)k_cols * (double)(a.seg[s].N + a.r);
    QL_TRY_PROF(profile_end(e0, e1, wide ? QL_KERNEL_GEMM_BWD : QL_KERNEL_GEMM_BWD_NARROW, flop));
  }
  return QL_OK;
}

}  // namespace

int bwd_max_split(int64_t M, int64_t K) {
  const int64_t t256 = ((M + BM - 1) / BM) * ((K + 255) / 256);
  if (t256 <= 0 || 2 * t256 > 256) return 1;
  const int64_t s = 256 / t256;
  return (int)(s > 8 ? 8 : s);
}

// Geometry. When 256 x 256 tiles alone would leave at least half the chip idle
// and the caller gave space for partials, the reduction is split across up to
// 8 workgroups per tile (the minimum slice depth below) and a second kernel
// sums the partials. Otherwise the forward's rule: whole rounds
// on wide tiles, the column blocks of a last partial round on narrow tiles in
// a second launch. Shapes alone decide, so resident and streamed runs match.
ql_status launch_gemm_bwd(const BwdArgs& a_in, hipStream_t st) {
  if (a_in.M == 0) return QL_OK;
  QL_TRY_PROF(ensure_attrs());
  BwdArgs a = a_in;
  a.nsplit = 1;
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const int C = cu_count();
  const int t256 = tiles_m * (int)((a.K + 255) / 256);
  const int t128 = tiles_m * (int)((a.K + 127) / 128);
  if (a.partial && 2 * t256 <= C) {
    int S = C / t256;
    const int cap = bwd_max_split(a.M, a.K);
    if (S > cap) S = cap;
    int ws = 0;
    for (int s = 0; s < a.nseg; ++s) ws += (int)((a.seg[s].N + BK - 1) / BK);
    // Split depth, from whole calls (the GEMM and the sum of its partials).
    // When narrow tiles alone fill at least half the chip, slices keep at
    // least 64 weight steps: split in two, a 4096-column dX at M=2048 (64
    // steps) takes 137-140 us against 132-135 on narrow tiles, and the M=512
    // down dX 116 against 111. Otherwise slices keep at least 8 steps
    // (M=512: the 4096 x 4096 dX 71 us at 8 splits against 103), and a
    // reduction under 32 steps is not split (M=512 k dX: 44 us whole, 52 in
    // four slices).
    const int min_steps = 2 * t128 >= C ? 64 : 8;
    if (ws < 32) S = 1;
    while (S > 1 && ws < min_steps * S) --S;
    while (S > 1 && (size_t)S * (size_t)a.M * (size_t)a.K * 4 > a.partial_bytes) --S;
    bool wide = true;  // short slices: narrow tiles, as in the forward
    if (S > 1 && ws / S < kShortSlice && 2 * t128 <= C) {
      int Sn = C / t128;
      if (Sn > cap) Sn = cap;
      while (Sn > 1 && ws < min_steps * Sn) --Sn;
      while (Sn > 1 && (size_t)Sn * (size_t)a.M * (size_t)a.K * 4 > a.partial_bytes) --Sn;
      if (Sn > 1) {
        S = Sn;
        wide = false;
      }
    }
    if (S > 1) {
      a.nsplit = S;
      QL_TRY_PROF(launch_bwd_tiles(a, wide, 0, a.K, st));
      const int64_t MK = a.M * a.K;
      int64_t grid = (MK / 4 + 255) / 256;
      if (grid > 4096) grid = 4096;
      hipLaunchKernelGGL(k_split_sum, dim3((unsigned)grid), dim3(256), 0, st, (const float*)a.partial, S, MK,
                         a.resid, a.out, a.out_f32);
      QL_HIP_CHECK(hipGetLastError());
      return QL_OK;
    }
  }
  if (t256 <= C) return launch_bwd_tiles(a, narrow_pays(t256, t128, C, kNarrowBwd) == 0, 0, a.K, st);
  const int full = (t256 / C) * C;
  if (full == t256 || !narrow_pays(t256 - full, 2 * (t256 - full), C, kNarrowBwd)) return launch_bwd_tiles(a, true, 0, a.K, st);
  const int64_t kw = (int64_t)(full / tiles_m) * 256;
  if (kw > 0) QL_TRY_PROF(launch_bwd_tiles(a, true, 0, kw, st));
  return launch_bwd_tiles(a, false, kw, a.K - kw, st);
}

}  // namespace ql
