// MXFP8 group quantize, column-wise requantize and grouped bias gradient
// kernels for gfx950.  All of them stream HBM: the design goal is full-width
// coalesced 16-byte accesses and enough bytes in flight per CU, with the
// block maxima reduced inside the wavefront (DPP), the column-wise copies
// transposed through LDS, and the elements encoded and decoded by the chip's
// scaled FP8 conversions (mx_convert.h; an integer path remains for scale
// bytes the fp32 decode cannot represent).
//
// Operations (see mxfp8moe.h for the buffer contracts):
//  * row-wise group quantize: bf16 [T, K] -> E4M3 [T, K] + E8M0 [T, K/32]
//    ("[Pytorch] Add support for row-wise quanted input for grouped gemm",
//    Description: the grouped GEMM takes input quantized row-wise).
//  * fused row-wise + column-wise group quantize from bf16, with the
//    column-wise copy stored transposed ([K, T] + [K, T/32]); used for the
//    grouped weight (forward reads the row-wise copy, dgrad the column-wise
//    one: "[PyTorch] Fix distributed BF16 weights and trim NVFP4 saved state
//    in the fused grouped MLP", last commit message).
//  * column-wise requantize of row-wise MXFP8 (exact dequantize, then the same
//    block rule along tokens), optionally with per-tile bias-gradient partial
//    sums (PR #3244 Description and Greptile Summary flowchart:
//    Dequantize -> Columnwise-only requantize, and -> Bias reductions).
//  * grouped bias gradient from row-wise data alone (PR #3244 Greptile
//    Summary: ordinary dbias reduced directly without a wgrad stage).
#include <algorithm>
#include <mutex>

#include "../../include/mxfp8moe.h"
#include "mx_convert.h"
#include "mx_tile_quant.h"
#include "kernels.h"

namespace mx {

// A launch whose device no-op flag is set writes nothing (outputs keep their
// contents), so that a captured graph can skip re-quantizing unchanged data.
__device__ __forceinline__ bool skip_launch(const int32_t* noop) {
  return noop != nullptr && *noop != 0;
}

constexpr int kRowThreads = 256;
constexpr int kRowUnroll = 4;

// x viewed as a flat array of 16-byte chunks; chunk c holds elements
// [8c, 8c+8) and belongs to block c/4 (blocks are consecutive in the flat
// order because K % 32 == 0).  nchunks is a multiple of 256.
__global__ __launch_bounds__(kRowThreads) void quant_rowwise_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, uint8_t* __restrict__ s,
    int64_t nchunks, const int32_t* __restrict__ noop) {
  if (skip_launch(noop)) return;
  const int64_t stride = (int64_t)gridDim.x * kRowThreads * kRowUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kRowThreads * kRowUnroll + threadIdx.x;
       base < nchunks; base += stride) {
    uint4 w[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t c = base + (int64_t)u * kRowThreads;
      // non-temporal: streamed once (measured 7 % faster for a 16384 x 14336 tensor)
      const u32x4 t = c < nchunks ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + c))
                                  : u32x4{0, 0, 0, 0};
      w[u] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t c = base + (int64_t)u * kRowThreads;
      const uint32_t amax = quad_max(chunk_amax_bits(w[u]));
      const uint32_t byte = scale_byte_from_exp(amax >> 7);
      // 16 lanes hold 16 chunks = 4 blocks: one 32-bit store of their scales
      const uint32_t bytes4 = gather_blocks4(byte);
      if (c < nchunks) {
        q[c] = encode_chunk(w[u], byte);
        if ((threadIdx.x & 15) == 0) *reinterpret_cast<uint32_t*>(s + (c >> 2)) = bytes4;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fused row-wise + column-wise quantize from bf16
// ---------------------------------------------------------------------------

// Tile `tile`: 128 rows x 256 B = 2048 chunks of 16 B, 8 per thread, 16
// chunks per row.
__device__ __forceinline__ void load_bf16_tile(const uint16_t* __restrict__ x, int64_t K,
                                               int tile, int ntk, u32x4 (&w)[8]) {
  int64_t k0, t0;
  tile_origin(tile, ntk, k0, t0);
  // uniform bases (the tile and chunk j: rows 16j..16j+15) plus one 32-bit
  // lane offset
  const uint32_t off = opaque_u32((threadIdx.x >> 4) * (uint32_t)K + (threadIdx.x & 15) * 8);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    w[j] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(x + (t0 * K + k0 + 16 * j * K) + off));
}

// Persistent: workgroup b takes tiles b, b + gridDim.x, ...; the loads of its
// next tile are issued before the column-wise pass of the current one, so
// each workgroup keeps a tile of reads in flight while it computes.
__global__ __launch_bounds__(kColThreads) void quant_rowcol_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t K, uint8_t* __restrict__ q_row,
    uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
    int32_t ntk, int32_t ntiles, const int32_t* __restrict__ noop) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytesBf16];
  if (skip_launch(noop)) return;
  const int tid = threadIdx.x;
  int tile = blockIdx.x;
  u32x4 w[8];
  load_bf16_tile(x, K, tile, ntk, w);
  for (;;) {
    int64_t k0, t0;
    tile_origin(tile, ntk, k0, t0);
    // row-wise stores: chunk jj of this thread is row 16 jj + tid / 16, its
    // 16-byte piece tid % 16; one 32-bit lane offset from uniform bases
    const uint32_t ro = opaque_u32((uint32_t)(tid >> 4) * (uint32_t)K + (tid & 15) * 8);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int idx = tid + kColThreads * jj;
      const int r = idx >> 4, cc = idx & 15;
      *reinterpret_cast<u32x4*>(&lds[lds_off_bf16(r, cc * 16)]) = w[jj];
      if (q_row != nullptr) {
        // row-wise: lanes 4b..4b+3 of a quad hold the 32 values of one block
        const uint4 c = make_uint4(w[jj].x, w[jj].y, w[jj].z, w[jj].w);
        const uint32_t amax = quad_max(chunk_amax_bits(c));
        const uint32_t byte = scale_byte_from_exp(amax >> 7);
        const int64_t rb = t0 * K + k0 + 16 * jj * K;   // uniform
        const uint2 e = encode_chunk(c, byte);
        __builtin_nontemporal_store(u32x2{e.x, e.y}, reinterpret_cast<u32x2*>(q_row + rb + ro));
        // the 16 lanes of a row hold its 4 blocks: one 32-bit scale store
        const uint32_t bytes4 = gather_blocks4(byte);
        if ((tid & 15) == 0)
          *reinterpret_cast<uint32_t*>(s_row + (rb >> 5) + (ro >> 5)) = bytes4;
      }
    }
    __syncthreads();
    const int next = tile + (int)gridDim.x;
    if (next < ntiles) load_bf16_tile(x, K, next, ntk, w);

    colwise_pass_bf16<true>(lds, T, K, k0, t0, q_col, s_col);
    if (next >= ntiles) break;
    __syncthreads();   // every column read of this tile is done before the next LDS write
    tile = next;
  }
}

// ---------------------------------------------------------------------------
// column-wise requantize of row-wise MXFP8 (+ optional dbias partials)
// ---------------------------------------------------------------------------

// Tile `tile`: 128 rows x 128 code bytes (4 chunks of 16 B per thread) and,
// for threads 0..127, the row's four scale bytes of the tile's 32-column blocks.
__device__ __forceinline__ void load_u8_tile(const uint8_t* __restrict__ q_row,
                                             const uint8_t* __restrict__ s_row, int64_t K,
                                             int tile, int ntk, u32x4 (&w)[4], uint32_t& sv) {
  int64_t k0, t0;
  tile_origin(tile, ntk, k0, t0);
  // uniform bases (the tile and chunk j: rows 32j..32j+31) plus one 32-bit
  // lane offset
  const uint32_t off = opaque_u32((threadIdx.x >> 3) * (uint32_t)K + (threadIdx.x & 7) * 16);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(q_row + (t0 * K + k0 + 32 * j * K) + off));
  if (threadIdx.x < kTileT) {
    const uint32_t so = opaque_u32(threadIdx.x * (uint32_t)(K / 32));
    sv = *reinterpret_cast<const uint32_t*>(s_row + (t0 * (K / 32) + (k0 >> 5)) + so);
  }
}

// Requantize one staged tile with the hardware conversions: each code is
// decoded exactly as code * 2^X_row (all row scale bytes of the tile are at
// most kMaxFastScaleByte, so nothing overflows), the column block's maximum
// magnitude gives its scale byte max(E - 8, 0) from the fp32 exponent field E
// (an all-zero or fp32-denormal maximum gives byte 0, the clamp at -127), and
// the values are encoded against it.  The first pass keeps only the raw code
// words and the second decodes them again.
template <bool kDbias>
__device__ __forceinline__ void requant_tile_fast(const uint8_t* lds, const float* lds_sc,
                                                  int64_t T, int64_t K, int64_t k0, int64_t t0,
                                                  uint8_t* __restrict__ q_col,
                                                  uint8_t* __restrict__ s_col,
                                                  float* __restrict__ partial) {
  const int j = threadIdx.x & 7, q = threadIdx.x >> 3;
  const int blk = q >> 3;                  // 32-column scale block of the quad
  uint32_t raw[16];                        // row r: codes of columns 4q..4q+3
  float sc[16];
  uint32_t m[4] = {0, 0, 0, 0};            // max |value| as fp32 bit patterns
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  const uint8_t* src = lds + opaque_off(lds_off_u8(16 * j, 4 * q));   // row 16j + r at r * 128
  const float* scs = lds_sc + opaque_off(lds_sc_idx(16 * j, blk));    // row 16j + r at 4 * r
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    raw[r] = *reinterpret_cast<const uint32_t*>(src + r * 128);
    sc[r] = scs[4 * r];
    const f32x2_t a = cvt2_e4m3_f32(raw[r], sc[r]);
    const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw[r], sc[r], true);
    m[0] = max(m[0], __float_as_uint(a.x) & 0x7FFFFFFFu);
    m[1] = max(m[1], __float_as_uint(a.y) & 0x7FFFFFFFu);
    m[2] = max(m[2], __float_as_uint(b.x) & 0x7FFFFFFFu);
    m[3] = max(m[3], __float_as_uint(b.y) & 0x7FFFFFFFu);
    if (kDbias) {
      s[0] += a.x;
      s[1] += a.y;
      s[2] += b.x;
      s[3] += b.y;
      // pin the running sums here: otherwise the compiler sinks the serial
      // adds below the loop and keeps every decoded value live until then
      if (r % 2 == 1) asm volatile("" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]));
    }
  }
  // the second pass decodes the codes again; hiding the code words from the
  // optimizer stops it from reusing the first pass's 64 decoded values, which
  // would all stay live in between
#pragma unroll
  for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(raw[r]));
  uint32_t xb[4];
  float e[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    m[c] = max(m[c], lane_xor1(m[c]));     // the block's other 16 tokens
    xb[c] = scale_byte_from_exp(m[c] >> 23);
    e[c] = e8m0_operand(xb[c]);
  }
  uint32_t o[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    f32x2_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = cvt2_e4m3_f32(raw[4 * g + i], sc[4 * g + i]);
      b[i] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw[4 * g + i], sc[4 * g + i], true);
    }
    o[0][g] = cvt4_f32_e4m3(a[0].x, a[1].x, a[2].x, a[3].x, e[0]);
    o[1][g] = cvt4_f32_e4m3(a[0].y, a[1].y, a[2].y, a[3].y, e[1]);
    o[2][g] = cvt4_f32_e4m3(b[0].x, b[1].x, b[2].x, b[3].x, e[2]);
    o[3][g] = cvt4_f32_e4m3(b[0].y, b[1].y, b[2].y, b[3].y, e[3]);
  }
  colwise_store<kDbias>(o, xb, s, T, K, k0, t0, q_col, s_col, partial);
}

// Requantize one staged tile with integer arithmetic on the bit fields; exact
// for every scale byte, used for tiles holding a row scale byte above
// kMaxFastScaleByte.  Two passes over LDS: the column blocks' largest
// exponents, then the re-encoding.
template <bool kDbias>
__device__ __forceinline__ void requant_tile_exact(const uint8_t* lds, const uint32_t* lds_s,
                                                   int64_t T, int64_t K, int64_t k0, int64_t t0,
                                                   uint8_t* __restrict__ q_col,
                                                   uint8_t* __restrict__ s_col,
                                                   float* __restrict__ partial) {
  const int j = threadIdx.x & 7, q = threadIdx.x >> 3;
  const int blk = q >> 3;
  constexpr int kNone = -100000;   // no non-zero element seen
  int em[4] = {kNone, kNone, kNone, kNone};
  const uint8_t* src = lds + opaque_off(lds_off_u8(16 * j, 4 * q));   // row 16j + r at r * 128
  const uint32_t* ss = lds_s + opaque_off(16 * j);
#pragma unroll 1
  for (int r = 0; r < 16; ++r) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(src + r * 128);
    const int se = (int)((ss[r] >> (8 * blk)) & 0xFFu) - 127;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t mg = (w >> (8 * c)) & 0x7Fu;
      if (mg) em[c] = max(em[c], e4m3_floor_log2(mg) + se);
    }
  }
  uint32_t xb[4];
  int xs[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    em[c] = max(em[c], __shfl_xor(em[c], 1));   // the block's other 16 tokens
    // X' = floor(log2 amax) - 8, clamped; all-zero column block -> -127
    xs[c] = em[c] == kNone ? -127 : min(max(em[c] - 8, -127), 127);
    xb[c] = (uint32_t)(xs[c] + 127);
  }
  uint32_t o[4][4];
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t acc[4] = {0, 0, 0, 0};
#pragma unroll 1
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(src + r * 128);
      const int se = (int)((ss[r] >> (8 * blk)) & 0xFFu) - 127;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float d = decode_e4m3((w >> (8 * c)) & 0xFFu);
        acc[c] |= encode_e4m3(__builtin_amdgcn_ldexpf(d, se - xs[c])) << (8 * i);
        if (kDbias) s[c] += __builtin_amdgcn_ldexpf(d, se);
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c][g] = acc[c];
  }
  colwise_store<kDbias>(o, xb, s, T, K, k0, t0, q_col, s_col, partial);
}

// Persistent: workgroup b takes tiles b, b + gridDim.x, ...; the loads of its
// next tile are issued right after the current one is staged in LDS.
template <bool kDbias>
__global__ __launch_bounds__(kColThreads, 5) void requant_colwise_kernel(
    const uint8_t* __restrict__ q_row, const uint8_t* __restrict__ s_row, int64_t T, int64_t K,
    uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col, float* __restrict__ partial,
    int32_t ntk, int32_t ntiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytesU8];
  __shared__ uint32_t lds_s[kTileT];                // raw scale bytes per row
  __shared__ float lds_sc[kLdsScWords];             // the same as conversion operands
  __shared__ uint32_t lds_wide[2];      // a row scale byte above kMaxFastScaleByte (per wave)
  const int tid = threadIdx.x;
  int tile = blockIdx.x;
  u32x4 w[4];
  uint32_t sv = 0;
  load_u8_tile(q_row, s_row, K, tile, ntk, w, sv);
  for (;;) {
    int64_t k0, t0;
    tile_origin(tile, ntk, k0, t0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + kColThreads * j;
      const int r = idx >> 3, cc = idx & 7;
      *reinterpret_cast<u32x4*>(&lds[lds_off_u8(r, cc * 16)]) = w[j];
    }
    bool wide = false;
    if (tid < kTileT) {
      const uint32_t e0 = sv & 0xFFu, e1 = (sv >> 8) & 0xFFu, e2 = (sv >> 16) & 0xFFu,
                     e3 = sv >> 24;
      lds_s[tid] = sv;
      lds_sc[lds_sc_idx(tid, 0)] = e8m0_operand(e0);
      lds_sc[lds_sc_idx(tid, 1)] = e8m0_operand(e1);
      lds_sc[lds_sc_idx(tid, 2)] = e8m0_operand(e2);
      lds_sc[lds_sc_idx(tid, 3)] = e8m0_operand(e3);
      wide = max(max(e0, e1), max(e2, e3)) > kMaxFastScaleByte;
    }
    // waves 0 and 1 hold the tile's 128 scale rows: one flag word per wave
    const uint64_t wide_lanes = __ballot(wide);
    if (tid < kTileT && (tid & 63) == 0) lds_wide[tid >> 6] = wide_lanes != 0;
    __syncthreads();
    const bool exact = (lds_wide[0] | lds_wide[1]) != 0;
    const int next = tile + (int)gridDim.x;
    if (next < ntiles) load_u8_tile(q_row, s_row, K, next, ntk, w, sv);
    if (exact)
      requant_tile_exact<kDbias>(lds, lds_s, T, K, k0, t0, q_col, s_col, partial);
    else
      requant_tile_fast<kDbias>(lds, lds_sc, T, K, k0, t0, q_col, s_col, partial);
    if (next >= ntiles) break;
    __syncthreads();   // every LDS read of this tile is done before the next write
    tile = next;
  }
}

// ---------------------------------------------------------------------------
// dbias partials from row-wise data alone: tile 128 rows x 256 cols
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void dbias_partial_kernel(
    const uint8_t* __restrict__ q_row, const uint8_t* __restrict__ s_row, int64_t T, int64_t N,
    float* __restrict__ partial) {
  __shared__ float4 red[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 256 + 4 * lane;
  const int64_t t0 = (int64_t)blockIdx.y * kTileT + wave * 32;
  const int64_t ns = N / 32;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
  for (int r = 0; r < 32; ++r) {
    const int64_t row = t0 + r;
    const uint32_t c = *reinterpret_cast<const uint32_t*>(q_row + row * N + n0);
    const int se = (int)s_row[row * ns + (n0 >> 5)] - 127;
    a0 += __builtin_amdgcn_ldexpf(decode_e4m3(c & 0xFFu), se);
    a1 += __builtin_amdgcn_ldexpf(decode_e4m3((c >> 8) & 0xFFu), se);
    a2 += __builtin_amdgcn_ldexpf(decode_e4m3((c >> 16) & 0xFFu), se);
    a3 += __builtin_amdgcn_ldexpf(decode_e4m3(c >> 24), se);
  }
  red[wave][lane] = make_float4(a0, a1, a2, a3);
  __syncthreads();
  if (wave == 0) {
    float4 s0 = red[0][lane], s1 = red[1][lane], s2 = red[2][lane], s3 = red[3][lane];
    float4 o = make_float4((s0.x + s1.x) + (s2.x + s3.x), (s0.y + s1.y) + (s2.y + s3.y),
                           (s0.z + s1.z) + (s2.z + s3.z), (s0.w + s1.w) + (s2.w + s3.w));
    *reinterpret_cast<float4*>(partial + (int64_t)blockIdx.y * N + n0) = o;
  }
}

// ---------------------------------------------------------------------------
// scaled-bias and routing-scale gradients from row-wise data
// ---------------------------------------------------------------------------
//
// With a bias scaled by each token's routing scale, out_r = x_r W_g^T +
// s_r b_g, the gradients taken from the dequantized output gradient dY are
//   dbias[g, n] = sum over rows r of expert g of s_r dY[r, n]
//   dscale[r]   = sum over n of dY[r, n] b[g, n]
// ("[Pytorch] Add support for row-wise quanted input for grouped gemm",
// Greptile Summary: scaled-bias gradient reductions and the flowchart's
// Dequantize -> bias and routing-scale reductions; the formulas are the
// plain gradients of that scaled bias).

// Expert of every 128-row tile (-1 for a tile no expert covers), from the
// device splits: thread sums over its share of experts, a scan across the
// workgroup, then each thread labels its experts' tiles.  One workgroup;
// any number of experts.  Splits that break the contract are clipped to T.
__global__ __launch_bounds__(256) void tile_expert_kernel(const int64_t* __restrict__ m_splits,
                                                          int32_t G, int64_t T,
                                                          int32_t* __restrict__ tile_expert) {
  __shared__ int64_t pre[256];
  const int tid = threadIdx.x;
  const int per = (G + 255) / 256;
  const int g0 = min(tid * per, G), g1 = min(g0 + per, G);
  const int64_t ntile = T / kTileT;
  for (int64_t i = tid; i < ntile; i += 256) tile_expert[i] = -1;
  int64_t sum = 0;
  for (int g = g0; g < g1; ++g) sum += max(m_splits[g], (int64_t)0);
  pre[tid] = sum;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int64_t v = tid >= d ? pre[tid - d] : 0;
    __syncthreads();
    pre[tid] += v;
    __syncthreads();
  }
  int64_t off = pre[tid] - sum;   // first row of expert g0
  for (int g = g0; g < g1; ++g) {
    const int64_t m = max(m_splits[g], (int64_t)0);
    const int64_t t_lo = min(off, T) / kTileT, t_hi = min(off + m, T) / kTileT;
    for (int64_t i = t_lo; i < t_hi; ++i) tile_expert[i] = g;
    off += m;
  }
}

// Per 128-row tile and 512 columns: lane -> 8 columns (one 8-byte load per
// row), wave -> 32 rows.  dbias_partial[tile, n] = sum over the tile's rows
// of s_r dY[r, n] (rows in order within a wave, then the four waves);
// dscale_partial[r, c] = the dot product of row r with the bias over column
// block c.  Per chunk of 8 rows each lane keeps its partial dot products; a
// reduce-scatter butterfly over the 64 lanes (each exchange halves the rows
// a lane keeps) and a sum over 8 lanes finish them in 10 exchanges instead
// of 6 per row.  Codes are decoded by the hardware conversion
// (scale bytes up to kMaxFastScaleByte) or, above, by integer arithmetic.
// Either output may be absent.
__global__ __launch_bounds__(256) void scaled_bias_partial_kernel(
    const uint8_t* __restrict__ q_row, const uint8_t* __restrict__ s_row, int64_t T, int64_t N,
    const float* __restrict__ scales, const float* __restrict__ bias,
    const int32_t* __restrict__ tile_expert, float* __restrict__ dbias_partial,
    float* __restrict__ dscale_partial) {
  __shared__ float red[4][8][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 512 + 8 * lane;
  const int64_t t0 = (int64_t)blockIdx.y * kTileT + wave * 32;
  const int64_t ns = N / 32, nb = N / 512;
  const int g = tile_expert[blockIdx.y];
  const bool want_db = dbias_partial != nullptr, want_ds = dscale_partial != nullptr;
  float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (want_ds && g >= 0) {
    const float4 b0 = *reinterpret_cast<const float4*>(bias + (int64_t)g * N + n0);
    const float4 b1 = *reinterpret_cast<const float4*>(bias + (int64_t)g * N + n0 + 4);
    bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w;
    bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // rows in chunks of kRows: only one chunk's partial dot products are live
  constexpr int kRows = 8;   // 16 needs 210 registers and ran slower
#pragma unroll 1
  for (int rc = 0; rc < 32; rc += kRows) {
    float pr[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t row = t0 + rc + r;
      const u32x2 c = *reinterpret_cast<const u32x2*>(q_row + row * N + n0);
      const uint32_t byte = s_row[row * ns + (n0 >> 5)];
      float d[8];
      if (byte <= kMaxFastScaleByte) {
        const float sc = e8m0_operand(byte);
        const f32x2_t v0 = cvt2_e4m3_f32(c.x, sc);
        const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.x, sc, true);
        const f32x2_t v2 = cvt2_e4m3_f32(c.y, sc);
        const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.y, sc, true);
        d[0] = v0.x; d[1] = v0.y; d[2] = v1.x; d[3] = v1.y;
        d[4] = v2.x; d[5] = v2.y; d[6] = v3.x; d[7] = v3.y;
      } else {
        const int se = (int)byte - 127;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          d[i] = __builtin_amdgcn_ldexpf(
              decode_e4m3(((i < 4 ? c.x : c.y) >> (8 * (i & 3))) & 0xFFu), se);
      }
      if (want_db) {
        const float sr = scales[row];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += sr * d[i];
      }
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) p += d[i] * bv[i];
      pr[r] = p;
    }
    if (want_ds) {
      // reduce-scatter over the top log2(kRows) lane bits: at the exchange
      // with lane ^ m a lane keeps the lower half of its current rows if
      // (lane & m) == 0, else the upper half, and adds its partner's copy of
      // those rows; then the lanes that share those bits sum their row
      int cnt = kRows;
#pragma unroll
      for (int m = 32; m >= 64 / kRows; m >>= 1) {
        const bool up = (lane & m) != 0;
        cnt >>= 1;
#pragma unroll
        for (int i = 0; i < kRows / 2; ++i) {
          if (i < cnt) {
            const float send = up ? pr[i] : pr[i + cnt];
            const float keep = up ? pr[i + cnt] : pr[i];
            pr[i] = keep + __shfl_xor(send, m);
          }
        }
      }
      float tot = pr[0];
#pragma unroll
      for (int m = 32 / kRows; m >= 1; m >>= 1) tot += __shfl_xor(tot, m);
      int row = 0;   // lane bit 5 selected half of the rows, bit 4 a quarter, ...
#pragma unroll
      for (int m = 32, w = kRows / 2; m >= 64 / kRows; m >>= 1, w >>= 1)
        row += (lane & m) ? w : 0;
      if ((lane & (64 / kRows - 1)) == 0) dscale_partial[(t0 + rc + row) * nb + blockIdx.x] = tot;
    }
  }
  if (!want_db) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0) {
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      o[i] = (red[0][i][lane] + red[1][i][lane]) + (red[2][i][lane] + red[3][i][lane]);
    float* dst = dbias_partial + (int64_t)blockIdx.y * N + n0;
    *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
}

// dscale[r] = sum over the column blocks of dscale_partial[r, c], in order.
__global__ __launch_bounds__(256) void dscale_finalize_kernel(const float* __restrict__ partial,
                                                              int64_t T, int64_t nb,
                                                              float* __restrict__ dscale) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= T) return;
  float s = 0.f;
  for (int64_t c = 0; c < nb; ++c) s += partial[r * nb + c];
  dscale[r] = s;
}

// dbias[g, k] = sum over the 128-row tiles of expert g of partial[tile, k],
// in tile order.  grid = (G, ceil(K / 256)).
// dbias[g, k] = the sum of the expert's tile partials of column k.  A block
// takes 64 columns of one expert; the four waves each sum every fourth tile
// of the expert in tile order, and the four sums are added in wave order: a
// fixed order, so dbias does not depend on timing, with four times the loads
// in flight of one summing thread per column (the Nemotron-proxy dh, whose
// largest expert has 172 tiles, finalized in 65 us with one thread per
// column).
__global__ __launch_bounds__(256) void dbias_finalize_kernel(
    const float* __restrict__ partial, const int64_t* __restrict__ m_splits, int32_t G, int64_t T,
    int64_t K, float* __restrict__ dbias) {
  __shared__ int64_t red[256];
  __shared__ float part[4][64];
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t acc = 0;
  for (int i = tid; i < g; i += 256) acc += max(m_splits[i], (int64_t)0);
  red[tid] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const int64_t off = red[0];
  const int64_t mg = max(m_splits[g], (int64_t)0);
  const int w = tid >> 6, c = tid & 63;
  const int64_t k = (int64_t)blockIdx.y * 64 + c;
  // tiles of the expert, clipped to the token count (splits that break the
  // contract must not make the kernel read out of bounds)
  const int64_t first = min(off, T) / kTileT, last = min(off + mg, T) / kTileT;
  float s = 0.f;
  if (k < K) {
#pragma unroll 4
    for (int64_t tile = first + w; tile < last; tile += 4) s += partial[tile * K + k];
  }
  part[w][c] = s;
  __syncthreads();
  if (w == 0 && k < K)
    dbias[(int64_t)g * K + k] = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
}

// ---------------------------------------------------------------------------
// split validation and SwiGLU
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void validate_splits_kernel(const int64_t* __restrict__ m_splits,
                                                              int32_t G, int64_t T,
                                                              int32_t* __restrict__ flag) {
  __shared__ int64_t red[256];
  __shared__ int32_t bits[256];
  const int tid = threadIdx.x;
  int64_t acc = 0;
  int32_t b = 0;
  for (int i = tid; i < G; i += 256) {
    const int64_t v = m_splits[i];
    if (v < 0) b |= 1;
    if (v % 128 != 0) b |= 2;
    acc += v;
  }
  red[tid] = acc;
  bits[tid] = b;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      red[tid] += red[tid + s];
      bits[tid] |= bits[tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) *flag = bits[0] | (red[0] != T ? 4 : 0);
}


// one thread per 2 output columns; h [T, 2F], a [T, F]
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint32_t* __restrict__ h,
                                                         int64_t T, int64_t F,
                                                         uint32_t* __restrict__ a) {
  const int64_t n = T * F / 2;
  const int64_t f2 = F / 2;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / f2, c = i % f2;
    const uint32_t gw = h[row * F + c];          // gate pair (row stride 2F bf16 = F words)
    const uint32_t uw = h[row * F + f2 + c];     // up pair
    const float g0 = bf16_to_f32(gw & 0xFFFFu), g1 = bf16_to_f32(gw >> 16);
    const float u0 = bf16_to_f32(uw & 0xFFFFu), u1 = bf16_to_f32(uw >> 16);
    a[i] = f32_to_bf16(silu_f(g0) * u0) | (f32_to_bf16(silu_f(g1) * u1) << 16);
  }
}

// SwiGLU backward of one bf16 pair of each of gate, up and da (the same
// arithmetic for swiglu_bwd_kernel and swiglu_bwd_quant_kernel, so that the
// fused kernel's dh equals the written one bit for bit): d gate = da * up * s
// * (1 + gate (1 - s)) and d up = da * gate * s with s = sigmoid(gate), in
// fp32, rounded to bf16 (nearest even).  s from the hardware base-2
// exponential and reciprocal, as silu_f forms it (a few ulp of fp32, far
// inside the half bf16 ulp of the rounding; the library exp and an IEEE
// division cost the fused kernel about a third of its time); for gate below
// about -88 the exponential overflows and s is 0, as with the library form.
__device__ __forceinline__ void swiglu_bwd_pair(uint32_t gw, uint32_t uw, uint32_t dw,
                                                uint32_t& og, uint32_t& ou) {
  og = 0;
  ou = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float g = bf16_to_f32((gw >> (16 * j)) & 0xFFFFu);
    const float u = bf16_to_f32((uw >> (16 * j)) & 0xFFFFu);
    const float d = bf16_to_f32((dw >> (16 * j)) & 0xFFFFu);
    const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
    const float dg = d * u * s * (1.0f + g * (1.0f - s));
    const float du = d * g * s;
    og |= f32_to_bf16(dg) << (16 * j);
    ou |= f32_to_bf16(du) << (16 * j);
  }
}

__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint32_t* __restrict__ h,
                                                         const uint32_t* __restrict__ da,
                                                         int64_t T, int64_t F,
                                                         uint32_t* __restrict__ dh) {
  const int64_t n = T * F / 2;
  const int64_t f2 = F / 2;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / f2, c = i % f2;
    uint32_t og, ou;
    swiglu_bwd_pair(h[row * F + c], h[row * F + f2 + c], da[i], og, ou);
    dh[row * F + c] = og;
    dh[row * F + f2 + c] = ou;
  }
}

// ---------------------------------------------------------------------------
// exhaustive sweep of the conversion helpers (diagnostic)
// ---------------------------------------------------------------------------

// mode 0: entry i = 65536 * s + h: the codes of the bf16 pair (h, h ^ 0x8000)
//         encoded with scale byte s, as a u16 (byte 0 = h, byte 1 = -h).
// mode 1: entry i = 65536 * x + 256 * s + c: code c decoded with scale byte s
//         and encoded again with scale byte x (u8).
// mode 2: entry i = 256 * s + c: codes (c, c ^ 0x80) decoded with scale byte s,
//         as two fp32 bit patterns.
__global__ __launch_bounds__(256) void convert_sweep_kernel(int32_t mode, uint8_t* __restrict__ out,
                                                            uint32_t n) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= n) return;
  if (mode == 0) {
    const uint32_t h = i & 0xFFFFu, sb = i >> 16;
    const uint32_t codes = cvt4_bf16_e4m3(h | ((h ^ 0x8000u) << 16), 0u, e8m0_operand(sb));
    reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)(codes & 0xFFFFu);
  } else if (mode == 1) {
    const uint32_t c = i & 0xFFu, sb = (i >> 8) & 0xFFu, xb = i >> 16;
    const f32x2_t d = cvt2_e4m3_f32(c, e8m0_operand(sb));
    out[i] = (uint8_t)(cvt4_f32_e4m3(d.x, 0.f, 0.f, 0.f, e8m0_operand(xb)) & 0xFFu);
  } else {
    const uint32_t c = i & 0xFFu, sb = i >> 8;
    const f32x2_t d = cvt2_e4m3_f32(c | ((c ^ 0x80u) << 8), e8m0_operand(sb));
    reinterpret_cast<uint32_t*>(out)[2 * i] = __float_as_uint(d.x);
    reinterpret_cast<uint32_t*>(out)[2 * i + 1] = __float_as_uint(d.y);
  }
}

// ---------------------------------------------------------------------------
// SwiGLU fused with the MXFP8 quantize of its output
// ---------------------------------------------------------------------------

// h [T, 2F] bf16 (gate = columns [0, F), up = [F, 2F)) -> a = SwiGLU(h) [T, F]
// quantized row-wise ([T, F] + [T, F/32]) and/or column-wise ([F, T] +
// [F, T/32]) without writing a: the 128 x 128 tile of a is formed in
// registers from the gate and up tiles, quantized row-wise from registers and
// column-wise from LDS, exactly as quant_rowcol_kernel quantizes a bf16 tile.
// The bytes equal swiglu_fwd_kernel followed by the group quantize.
__global__ __launch_bounds__(kColThreads) void swiglu_quant_kernel(
    const uint16_t* __restrict__ h, int64_t T, int64_t F, uint8_t* __restrict__ q_row,
    uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytesBf16];
  const int tid = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * kTileK;
  const int64_t t0 = (int64_t)blockIdx.y * kTileT;
  const int64_t ld = 2 * F;
  const uint32_t off = (uint32_t)(tid >> 4) * (uint32_t)ld + (tid & 15) * 8;
  const uint32_t ro = (uint32_t)(tid >> 4) * (uint32_t)F + (tid & 15) * 8;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int idx = tid + kColThreads * jj;
    const int r = idx >> 4, cc = idx & 15;
    const uint16_t* hb = h + (t0 + 16 * jj) * ld + k0;   // uniform
    const u32x4 g = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(hb + off));
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(hb + F + off));
    const uint4 a = make_uint4(swiglu_pair(g.x, u.x), swiglu_pair(g.y, u.y),
                               swiglu_pair(g.z, u.z), swiglu_pair(g.w, u.w));
    if (q_col != nullptr)
      *reinterpret_cast<u32x4*>(&lds[lds_off_bf16(r, cc * 16)]) = u32x4{a.x, a.y, a.z, a.w};
    if (q_row != nullptr) {
      // lanes 4b..4b+3 of a quad hold the 32 values of one block
      const uint32_t amax = quad_max(chunk_amax_bits(a));
      const uint32_t byte = scale_byte_from_exp(amax >> 7);
      const int64_t rb = t0 * F + k0 + 16 * jj * F;   // uniform
      *reinterpret_cast<uint2*>(q_row + rb + ro) = encode_chunk(a, byte);
      const uint32_t bytes4 = gather_blocks4(byte);
      if ((tid & 15) == 0) *reinterpret_cast<uint32_t*>(s_row + (rb >> 5) + (ro >> 5)) = bytes4;
    }
  }
  if (q_col == nullptr) return;
  __syncthreads();
  colwise_pass_bf16<false>(lds, T, F, k0, t0, q_col, s_col);
}

// ---------------------------------------------------------------------------
// row-wise quantize of bf16 fused with the column-wise requantize of its result
// ---------------------------------------------------------------------------

// One pass over bf16 x that writes what quant_rowwise_kernel followed by
// requant_colwise_kernel writes: the row-wise codes and scales, and the
// column-wise copy requantized from the dequantized row-wise values (+ the
// per-tile dbias partials), reading x once instead of reading the row-wise
// codes back.  The tile's row-wise codes and scale operands are staged in LDS
// in the requantize's layout and requant_tile_fast runs on them unchanged, so
// the bytes and partial sums are those of the two-kernel path.  Row scale
// bytes from bf16 data are at most 246 = kMaxFastScaleByte (the largest bf16
// exponent field, 254, minus 8), so the fast requantize always applies.
// Persistent like quant_rowcol_kernel: the next tile's loads are issued once
// this tile is staged.
template <bool kDbias>
__global__ __launch_bounds__(kColThreads) void quant_row_requant_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t K, uint8_t* __restrict__ q_row,
    uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
    float* __restrict__ partial, int32_t ntk, int32_t ntiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytesU8];
  __shared__ float lds_sc[kLdsScWords];             // row scales as conversion operands
  const int tid = threadIdx.x;
  int tile = blockIdx.x;
  u32x4 w[8];
  load_bf16_tile(x, K, tile, ntk, w);
  for (;;) {
    int64_t k0, t0;
    tile_origin(tile, ntk, k0, t0);
    // chunk jj of this thread: row 16 jj + tid / 16, its 8 elements
    // 8 (tid % 16) .. + 7; the quad of lanes 4b..4b+3 holds block b
    const uint32_t ro = opaque_u32((uint32_t)(tid >> 4) * (uint32_t)K + (tid & 15) * 8);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int idx = tid + kColThreads * jj;
      const int r = idx >> 4, cc = idx & 15;
      const uint4 c = make_uint4(w[jj].x, w[jj].y, w[jj].z, w[jj].w);
      const uint32_t amax = quad_max(chunk_amax_bits(c));
      const uint32_t byte = scale_byte_from_exp(amax >> 7);
      const int64_t rb = t0 * K + k0 + 16 * jj * K;   // uniform
      const uint2 e = encode_chunk(c, byte);
      *reinterpret_cast<uint2*>(q_row + rb + ro) = e;
      *reinterpret_cast<uint2*>(&lds[lds_off_u8(r, cc * 8)]) = e;
      if ((cc & 3) == 0) lds_sc[lds_sc_idx(r, cc >> 2)] = e8m0_operand(byte);
      const uint32_t bytes4 = gather_blocks4(byte);
      if ((tid & 15) == 0)
        *reinterpret_cast<uint32_t*>(s_row + (rb >> 5) + (ro >> 5)) = bytes4;
    }
    __syncthreads();
    const int next = tile + (int)gridDim.x;
    if (next < ntiles) load_bf16_tile(x, K, next, ntk, w);
    requant_tile_fast<kDbias>(lds, lds_sc, T, K, k0, t0, q_col, s_col, partial);
    if (next >= ntiles) break;
    __syncthreads();   // every LDS read of this tile is done before the next write
    tile = next;
  }
}

// ---------------------------------------------------------------------------
// SwiGLU backward fused with the row-wise quantize + column-wise requantize
// of its output
// ---------------------------------------------------------------------------

// h [T, 2F] and da [T, F] bf16 -> what swiglu_bwd_kernel followed by
// quant_row_requant_kernel on dh [T, 2F] writes (row-wise codes and scales,
// the column-wise copy requantized from them, the dbias partials), without
// writing dh.  Tile (t0, c0) of the F columns gives two 128 x 128 tiles of
// dh, the gate part at columns c0.. and the up part at F + c0..: each chunk
// of gate, up and da becomes a chunk of each part, quantized row-wise from
// registers and staged in that part's LDS buffer, and requant_tile_fast then
// runs on both buffers unchanged, so every byte and partial sum is that of
// the two-kernel path (bf16 row scale bytes are at most kMaxFastScaleByte).
// Four resident workgroups per CU keep the reads in flight.
// The tile's loads are issued half at a time (gate, up and da for 4 of the 8
// chunks per thread, then the other 4): 109 VGPRs, so four workgroups fit on
// a CU (the LDS allows four).  All 8 at once took 149 VGPRs and three
// workgroups and was 7 % slower; quarters (86 VGPRs) 1 % slower.
constexpr int kSwigluBwdHalves = 2;
constexpr int kSwigluBwdWgPerCu = 4;
template <bool kDbias>
__global__ __launch_bounds__(kColThreads) void swiglu_bwd_quant_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ da, int64_t T, int64_t F,
    uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_col,
    uint8_t* __restrict__ s_col, float* __restrict__ partial, int32_t ntf, int32_t ntiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kLdsBytesU8];
  __shared__ float lds_sc[2][kLdsScWords];           // row scales as conversion operands
  const int tid = threadIdx.x;
  const int64_t K = 2 * F;                           // dh columns
  for (int tile = blockIdx.x; tile < ntiles; tile += (int)gridDim.x) {
    int64_t c0, t0;
    tile_origin(tile, ntf, c0, t0);
    // chunk jj of this thread: row 16 jj + tid / 16, its 8 elements
    // 8 (tid % 16) .. + 7; the quad of lanes 4b..4b+3 holds block b
    const uint32_t oh = opaque_u32((uint32_t)(tid >> 4) * (uint32_t)K + (tid & 15) * 8);
    const uint32_t od = opaque_u32((uint32_t)(tid >> 4) * (uint32_t)F + (tid & 15) * 8);
#pragma unroll
    for (int hh = 0; hh < kSwigluBwdHalves; ++hh) {
      constexpr int kN = 8 / kSwigluBwdHalves;
      u32x4 gv[kN], uv[kN], dv[kN];
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        const int jj = kN * hh + i;
        const uint16_t* hb = h + (t0 + 16 * jj) * K + c0;   // uniform
        gv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(hb + oh));
        uv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(hb + F + oh));
        dv[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(da + (t0 + 16 * jj) * F + c0 + od));
      }
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        const int jj = kN * hh + i;
        const int idx = tid + kColThreads * jj;
        const int r = idx >> 4, cc = idx & 15;
        uint4 cg, cu;
        swiglu_bwd_pair(gv[i].x, uv[i].x, dv[i].x, cg.x, cu.x);
        swiglu_bwd_pair(gv[i].y, uv[i].y, dv[i].y, cg.y, cu.y);
        swiglu_bwd_pair(gv[i].z, uv[i].z, dv[i].z, cg.z, cu.z);
        swiglu_bwd_pair(gv[i].w, uv[i].w, dv[i].w, cg.w, cu.w);
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const uint4 c = part ? cu : cg;
          const uint32_t amax = quad_max(chunk_amax_bits(c));
          const uint32_t byte = scale_byte_from_exp(amax >> 7);
          const int64_t rb = t0 * K + c0 + part * F + 16 * jj * K;   // uniform
          const uint2 e = encode_chunk(c, byte);
          *reinterpret_cast<uint2*>(q_row + rb + oh) = e;
          *reinterpret_cast<uint2*>(&lds[part][lds_off_u8(r, cc * 8)]) = e;
          if ((cc & 3) == 0) lds_sc[part][lds_sc_idx(r, cc >> 2)] = e8m0_operand(byte);
          const uint32_t bytes4 = gather_blocks4(byte);
          if ((tid & 15) == 0)
            *reinterpret_cast<uint32_t*>(s_row + (rb >> 5) + (oh >> 5)) = bytes4;
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one half's loads at a time
    }
    __syncthreads();
    requant_tile_fast<kDbias>(lds[0], lds_sc[0], T, K, c0, t0, q_col, s_col, partial);
    requant_tile_fast<kDbias>(lds[1], lds_sc[1], T, K, F + c0, t0, q_col, s_col, partial);
    __syncthreads();   // every LDS read of this tile is done before the next write
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static int grid_for(int64_t work_items, int per_block, int cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g > cap) g = cap;
  return g < 1 ? 1 : (int)g;
}

hipError_t launch_quant_rowwise(const uint16_t* x, int64_t T, int64_t K, uint8_t* q, uint8_t* s,
                                const int32_t* noop, hipStream_t st) {
  const int64_t nchunks = T * K / 8;
  const int grid = grid_for(nchunks, kRowThreads * kRowUnroll, 256 * 16);
  hipLaunchKernelGGL(quant_rowwise_kernel, dim3(grid), dim3(kRowThreads), 0, st,
                     reinterpret_cast<const uint4*>(x), reinterpret_cast<uint2*>(q), s, nchunks, noop);
  return hipGetLastError();
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus > 0 ? cus : 256;
}

// Workgroups per CU of the persistent streaming kernels.  quant_rowcol is
// bound by LDS (33 KB per workgroup: four).  requant could hold five (96
// VGPRs) but runs 5 % faster with three: more resident tiles only add
// concurrent pages and scale lines (five workgroups of quant_rowcol, with
// the LDS padding replaced by a swizzle, were 1-5 % slower as well).
constexpr int kRowcolWgPerCu = 4;
constexpr int kRequantWgPerCu = 3;
constexpr int kRowRequantWgPerCu = 4;

hipError_t launch_quant_rowcol(const uint16_t* x, int64_t T, int64_t K, uint8_t* q_row,
                               uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                               const int32_t* noop, hipStream_t st) {
  const int32_t ntt = (int32_t)(T / kTileT), ntk = (int32_t)(K / kTileK);
  const int32_t ntiles = ntt * ntk;
  const int grid = (int)std::min<int64_t>(ntiles, (int64_t)device_cus() * kRowcolWgPerCu);
  hipLaunchKernelGGL(quant_rowcol_kernel, dim3(grid), dim3(kColThreads), 0, st, x, T, K, q_row,
                     s_row, q_col, s_col, ntk, ntiles, noop);
  return hipGetLastError();
}

hipError_t launch_requant_colwise(const uint8_t* q_row, const uint8_t* s_row, int64_t T,
                                  int64_t K, uint8_t* q_col, uint8_t* s_col, float* partial,
                                  hipStream_t st) {
  const int32_t ntt = (int32_t)(T / kTileT), ntk = (int32_t)(K / kTileK);
  const int32_t ntiles = ntt * ntk;
  const int grid = (int)std::min<int64_t>(ntiles, (int64_t)device_cus() * kRequantWgPerCu);
  if (partial != nullptr)
    hipLaunchKernelGGL(requant_colwise_kernel<true>, dim3(grid), dim3(kColThreads), 0, st, q_row,
                       s_row, T, K, q_col, s_col, partial, ntk, ntiles);
  else
    hipLaunchKernelGGL(requant_colwise_kernel<false>, dim3(grid), dim3(kColThreads), 0, st,
                       q_row, s_row, T, K, q_col, s_col, partial, ntk, ntiles);
  return hipGetLastError();
}

hipError_t launch_quant_row_requant(const uint16_t* x, int64_t T, int64_t K, uint8_t* q_row,
                                   uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, float* partial,
                                   hipStream_t st) {
  const int32_t ntt = (int32_t)(T / kTileT), ntk = (int32_t)(K / kTileK);
  const int32_t ntiles = ntt * ntk;
  const int grid = (int)std::min<int64_t>(ntiles, (int64_t)device_cus() * kRowRequantWgPerCu);
  if (partial != nullptr)
    hipLaunchKernelGGL(quant_row_requant_kernel<true>, dim3(grid), dim3(kColThreads), 0, st, x, T,
                       K, q_row, s_row, q_col, s_col, partial, ntk, ntiles);
  else
    hipLaunchKernelGGL(quant_row_requant_kernel<false>, dim3(grid), dim3(kColThreads), 0, st, x,
                       T, K, q_row, s_row, q_col, s_col, partial, ntk, ntiles);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd_quant(const uint16_t* h, const uint16_t* da, int64_t T, int64_t F,
                                   uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                                   float* partial, hipStream_t st) {
  const int32_t ntt = (int32_t)(T / kTileT), ntf = (int32_t)(F / kTileK);
  const int32_t ntiles = ntt * ntf;
  const int grid = (int)std::min<int64_t>(ntiles, (int64_t)device_cus() * kSwigluBwdWgPerCu);
  if (partial != nullptr)
    hipLaunchKernelGGL(swiglu_bwd_quant_kernel<true>, dim3(grid), dim3(kColThreads), 0, st, h, da,
                       T, F, q_row, s_row, q_col, s_col, partial, ntf, ntiles);
  else
    hipLaunchKernelGGL(swiglu_bwd_quant_kernel<false>, dim3(grid), dim3(kColThreads), 0, st, h,
                       da, T, F, q_row, s_row, q_col, s_col, partial, ntf, ntiles);
  return hipGetLastError();
}

hipError_t launch_dbias_partial(const uint8_t* q_row, const uint8_t* s_row, int64_t T, int64_t N,
                                float* partial, hipStream_t st) {
  dim3 grid((unsigned)(N / 256), (unsigned)(T / kTileT));
  hipLaunchKernelGGL(dbias_partial_kernel, grid, dim3(256), 0, st, q_row, s_row, T, N, partial);
  return hipGetLastError();
}

hipError_t launch_scaled_bias_grad(const uint8_t* q_row, const uint8_t* s_row, int64_t T,
                                   int64_t N, const int64_t* m_splits, int32_t G,
                                   const float* scales, const float* bias, float* dbias,
                                   float* dscale, void* workspace, hipStream_t st) {
  // workspace: tile experts (int32, padded to 256 B), dbias partials
  // [T/128, N], dscale partials [T, N/512]
  char* ws = static_cast<char*>(workspace);
  int32_t* tile_expert = reinterpret_cast<int32_t*>(ws);
  const int64_t ntile = T / kTileT;
  float* dbp = reinterpret_cast<float*>(ws + ((ntile * 4 + 255) / 256) * 256);
  float* dsp = dbp + ntile * N;
  hipLaunchKernelGGL(tile_expert_kernel, dim3(1), dim3(256), 0, st, m_splits, G, T, tile_expert);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scaled_bias_partial_kernel, dim3((unsigned)(N / 512), (unsigned)ntile),
                     dim3(256), 0, st, q_row, s_row, T, N, scales, bias, tile_expert,
                     dbias != nullptr ? dbp : nullptr, dscale != nullptr ? dsp : nullptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dbias != nullptr) {
    e = launch_dbias_finalize(dbp, m_splits, G, T, N, dbias, st);
    if (e != hipSuccess) return e;
  }
  if (dscale != nullptr) {
    hipLaunchKernelGGL(dscale_finalize_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0,
                       st, dsp, T, N / 512, dscale);
    e = hipGetLastError();
  }
  return e;
}

size_t scaled_bias_workspace_bytes(int64_t T, int64_t N) {
  const int64_t ntile = T / kTileT;
  return (size_t)(((ntile * 4 + 255) / 256) * 256) + (size_t)ntile * N * 4 +
         (size_t)T * (N / 512) * 4;
}

hipError_t launch_dbias_finalize(const float* partial, const int64_t* m_splits, int32_t G,
                                 int64_t T, int64_t K, float* dbias, hipStream_t st) {
  dim3 grid((unsigned)G, (unsigned)((K + 63) / 64));
  hipLaunchKernelGGL(dbias_finalize_kernel, grid, dim3(256), 0, st, partial, m_splits, G, T, K,
                     dbias);
  return hipGetLastError();
}

hipError_t launch_validate_splits(const int64_t* m_splits, int32_t G, int64_t T, int32_t* flag,
                                  hipStream_t st) {
  hipLaunchKernelGGL(validate_splits_kernel, dim3(1), dim3(256), 0, st, m_splits, G, T, flag);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const uint16_t* h, int64_t T, int64_t F, uint16_t* a,
                             hipStream_t st) {
  const int grid = grid_for(T * F / 2, 256, 256 * 32);
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(grid), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(h), T, F, reinterpret_cast<uint32_t*>(a));
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* h, const uint16_t* da, int64_t T, int64_t F,
                             uint16_t* dh, hipStream_t st) {
  const int grid = grid_for(T * F / 2, 256, 256 * 32);
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(grid), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(h), reinterpret_cast<const uint32_t*>(da),
                     T, F, reinterpret_cast<uint32_t*>(dh));
  return hipGetLastError();
}

size_t convert_sweep_bytes(int32_t mode) {
  return mode == 0 ? (size_t)2 << 24 : mode == 1 ? (size_t)1 << 24 : mode == 2 ? (size_t)8 << 16 : 0;
}

hipError_t launch_convert_sweep(int32_t mode, uint8_t* out, hipStream_t st) {
  const uint32_t n = mode == 2 ? 1u << 16 : 1u << 24;
  hipLaunchKernelGGL(convert_sweep_kernel, dim3(n / 256), dim3(256), 0, st, mode, out, n);
  return hipGetLastError();
}

hipError_t launch_swiglu_quant(const uint16_t* h, int64_t T, int64_t F, uint8_t* q_row,
                               uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t st) {
  dim3 grid((unsigned)(F / kTileK), (unsigned)(T / kTileT));
  hipLaunchKernelGGL(swiglu_quant_kernel, grid, dim3(kColThreads), 0, st, h, T, F, q_row, s_row,
                     q_col, s_col);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (mxfp8_group_quantize_requant_
// noalloc): the per-128-row fp32 dbias partials that the workspace of
// mxfp8_group_quantize_requant holds, in a file-scope device array instead.
// Every GPU the library runs on holds its own copy until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host the name is
// only a stand-in for the symbol): its device address is looked up once per
// device, with that device current, and kept.
constexpr size_t kScratchBytes = MXFP8_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(float** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mx
