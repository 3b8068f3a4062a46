// Quantize helpers for 128 x 128 bf16 tiles, shared by the streaming quantize
// kernels (and, for the conversions and SwiGLU, the grouped GEMM's SwiGLU
// epilogue): row-wise blocks (1 x 32)
// from 16-byte chunks held four lanes to a block, and the column-wise pass
// (32 x 1 blocks, stored transposed) over a tile staged in LDS.  Both encode
// with the scaled conversions of mx_convert.h, so every kernel that uses them
// writes the same bytes for the same bf16 values.
#pragma once

#include "mx_convert.h"

namespace mx {

// ---------------------------------------------------------------------------
// row-wise quantize: one 16-byte chunk (8 bf16) per lane, 4 lanes per block
// ---------------------------------------------------------------------------

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte chunk
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  us2 x = __builtin_bit_cast(us2, a);
  us2 y = __builtin_bit_cast(us2, b);
  us2 m = __builtin_elementwise_max(x, y);
  return __builtin_bit_cast(uint32_t, m);
}

// Max of the bf16 magnitudes (as bit patterns) of 8 values.
__device__ __forceinline__ uint32_t chunk_amax_bits(uint4 w) {
  const uint32_t k = 0x7FFF7FFFu;
  uint32_t m = max_u16x2(max_u16x2(w.x & k, w.y & k), max_u16x2(w.z & k, w.w & k));
  uint32_t lo = m & 0xFFFFu, hi = m >> 16;
  return lo > hi ? lo : hi;
}

// Max over the 4 lanes of a quad (DPP quad permutations).
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // [1,0,3,2]
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);           // [2,3,0,1]
  return v > o ? v : o;
}

// Value of lane l + n within the lane's row of 16 (DPP row_shl; 0 past the
// end of the row).
template <int n>
__device__ __forceinline__ uint32_t row_shl(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x100 + n, 0xF, 0xF, true);
}

// The scale bytes of four consecutive 32-element blocks held by lanes l,
// l + 4, l + 8, l + 12 of a row of 16 lanes, as one word (valid in lane l).
__device__ __forceinline__ uint32_t gather_blocks4(uint32_t byte) {
  return byte | (row_shl<4>(byte) << 8) | (row_shl<8>(byte) << 16) | (row_shl<12>(byte) << 24);
}

// Encode the 8 bf16 of `w` with the block scale byte; returns 8 codes.
__device__ __forceinline__ uint2 encode_chunk(uint4 w, uint32_t byte) {
  const float sc = e8m0_operand(byte);
  return make_uint2(cvt4_bf16_e4m3(w.x, w.y, sc), cvt4_bf16_e4m3(w.z, w.w, sc));
}

// ---------------------------------------------------------------------------
// column-wise passes: tiles of 128 tokens x 128 columns staged in LDS
// ---------------------------------------------------------------------------
//
// After staging, thread t of the 256 owns the column quad q = t >> 3 (tile
// columns 4q..4q+3) and the 16-token chunk j = t & 7 (tile rows 16j..16j+15).
// A column's 32-token scale block is the chunk pair (2i, 2i+1), i.e. lanes l
// and l ^ 1; the 128 tokens of one column (one 128-byte line of the
// transposed output) belong to the eight lanes of one column quad, 16 bytes
// each, so every output store instruction writes whole lines.
//
// The tile loads are non-temporal: the streamed input would otherwise evict
// the partly written scale lines (each 128-byte line of column-wise scales
// collects 4 bytes from each of 32 tiles) before they are complete; measured
// 5-7 % faster for both kernels.  The bf16 quantize also stores its row- and
// column-wise codes non-temporally, for the same reason: its tiles write as
// many code bytes as they read, and through L2 they evicted the scale lines
// between the tiles that share one, whose partial write-backs cost 12-17 % of
// the kernel (measured by leaving the scale stores out).  Non-temporal code
// stores gain almost all of it (11 % on 131072 x 7168, 18 % on the
// 114688 x 4096 weight); the requantize, which reads a quarter as much, is
// 10 % slower with them and keeps ordinary stores.
//
// LDS rows carry 16 bytes of padding after every 16 rows: the eight chunks j
// of one read instruction (rows 16j + r) then start 4 banks apart, and the
// lanes of a half-wave read 32 distinct banks.

constexpr int kTileT = 128;       // token rows per tile
constexpr int kTileK = 128;       // hidden columns per tile
constexpr int kColThreads = 256;

__device__ __forceinline__ int lds_off_bf16(int row, int byte_col) {
  return row * 256 + (row >> 4) * 16 + byte_col;
}
constexpr int kLdsBytesBf16 = kTileT * 256 + (kTileT / 16) * 16;
__device__ __forceinline__ int lds_off_u8(int row, int col) {
  return row * 128 + (row >> 4) * 16 + col;
}
constexpr int kLdsBytesU8 = kTileT * 128 + (kTileT / 16) * 16;
// Conversion operand of tile row `row` and 32-column block `blk`, one padding
// word per 16 rows (the eight rows 16j + r of one read land in distinct banks).
__device__ __forceinline__ int lds_sc_idx(int row, int blk) { return row * 4 + blk + (row >> 4); }
constexpr int kLdsScWords = kTileT * 4 + kTileT / 16;

// Tile order: column tiles fastest (tile = row tile * ntk + column tile); of
// the orders measured (this one, row tiles fastest, bands of 32 row tiles) it
// is the fastest for the bf16 quantize and within a few percent for requant.
__device__ __forceinline__ void tile_origin(int tile, int ntk, int64_t& k0, int64_t& t0) {
  t0 = (int64_t)(tile / ntk) * kTileT;
  k0 = (int64_t)(tile % ntk) * kTileK;
}

// A per-thread LDS offset the optimizer cannot see through: computed inside
// the tile loop, so the row offsets added to it fold into the read
// instructions' immediate field instead of being hoisted out of the loop as
// one register per row.
__device__ __forceinline__ int opaque_off(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Value of lane l ^ 1 (DPP quad permutation [1, 0, 3, 2]).
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}

// Stores of one thread's column-wise results: o[c][g] holds tokens
// 16j + 4g .. 16j + 4g + 3 of tile column 4q + c, x[c] its scale byte (the
// same in lanes l and l ^ 1; the even lane stores it), s[c] the thread's sum
// of column 4q + c over its 16 tokens (kDbias only: summed over the eight
// chunks in a fixed butterfly order and stored as the tile's partial sum).
// kNT: the code stores are non-temporal (see quant_rowcol_kernel).
template <bool kDbias, bool kNT = false>
__device__ __forceinline__ void colwise_store(const uint32_t (&o)[4][4], const uint32_t (&x)[4],
                                              float (&s)[4], int64_t T, int64_t K, int64_t k0,
                                              int64_t t0, uint8_t* __restrict__ q_col,
                                              uint8_t* __restrict__ s_col,
                                              float* __restrict__ partial,
                                              const int tid = threadIdx.x) {
  const int j = tid & 7, q = tid >> 3;
  // tile bases are uniform; per-lane offsets stay 32-bit (127 * T < 2^32)
  const uint32_t ts = (uint32_t)T, ss = (uint32_t)(T / 32);
  const uint32_t od = opaque_u32(4 * q * ts + 16 * j);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4* dst = reinterpret_cast<u32x4*>(q_col + (k0 * T + t0 + c * T) + od);
    const u32x4 v = u32x4{o[c][0], o[c][1], o[c][2], o[c][3]};
    if (kNT)
      __builtin_nontemporal_store(v, dst);
    else
      *dst = v;
  }
  // lane j holds block j / 2 of the quad's four columns (lanes 2i and 2i+1
  // agree); lane 0 of the quad gathers blocks 0..3 of each column (lanes 0,
  // 2, 4, 6) and stores them as one 32-bit word per column
  const uint32_t pw = x[0] | (x[1] << 8) | (x[2] << 16) | (x[3] << 24);
  const uint32_t p2 = row_shl<2>(pw), p4 = row_shl<4>(pw), p6 = row_shl<6>(pw);
  if (j == 0) {
    const uint32_t os = opaque_u32(4 * q * ss);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t sel = (uint32_t)c | ((uint32_t)(c + 4) << 8) | 0x0C0C0000u;
      const uint32_t lo = __builtin_amdgcn_perm(p2, pw, sel);   // blocks 0, 1
      const uint32_t hi = __builtin_amdgcn_perm(p6, p4, sel);   // blocks 2, 3
      *reinterpret_cast<uint32_t*>(s_col + (k0 * (T / 32) + (t0 >> 5) + c * (T / 32)) + os) =
          __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
  }
  if (kDbias) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s[c] += __shfl_xor(s[c], 1);
      s[c] += __shfl_xor(s[c], 2);
      s[c] += __shfl_xor(s[c], 4);
    }
    if (j == 0)
      *reinterpret_cast<float4*>(partial + (t0 / kTileT) * K + k0 + 4 * q) =
          make_float4(s[0], s[1], s[2], s[3]);
  }
}

// Column-wise quantize of a staged 128 x 128 bf16 tile (columns k0.., tokens
// t0..): thread -> column quad q = tid / 8, 16-token chunk j = tid % 8.
template <bool kNT>
__device__ __forceinline__ void colwise_pass_bf16(const uint8_t* lds, int64_t T, int64_t K,
                                                  int64_t k0, int64_t t0,
                                                  uint8_t* __restrict__ q_col,
                                                  uint8_t* __restrict__ s_col,
                                                  const int tid = threadIdx.x) {
  const int j = tid & 7, q = tid >> 3;
  // row r of the chunk as bf16 pairs, columns (0, 1) and (2, 3)
  uint32_t lo[16], hi[16];
  const uint8_t* src = lds + opaque_off(lds_off_bf16(16 * j, 8 * q));   // row 16j + r at r * 256
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint2 v = *reinterpret_cast<const uint2*>(src + r * 256);
    lo[r] = v.x;
    hi[r] = v.y;
  }
  uint32_t mlo = 0, mhi = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    mlo = max_u16x2(mlo, lo[r] & 0x7FFF7FFFu);
    mhi = max_u16x2(mhi, hi[r] & 0x7FFF7FFFu);
  }
  mlo = max_u16x2(mlo, lane_xor1(mlo));   // the block's other 16 tokens
  mhi = max_u16x2(mhi, lane_xor1(mhi));
  const uint32_t xb[4] = {scale_byte_from_exp((mlo & 0xFFFFu) >> 7),
                          scale_byte_from_exp((mlo >> 16) >> 7),
                          scale_byte_from_exp((mhi & 0xFFFFu) >> 7),
                          scale_byte_from_exp((mhi >> 16) >> 7)};
  const float sc[4] = {e8m0_operand(xb[0]), e8m0_operand(xb[1]), e8m0_operand(xb[2]),
                       e8m0_operand(xb[3])};
  // a byte permute gathers the same column of two rows into one bf16 pair
  uint32_t o[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 4 * g;
    o[0][g] = cvt4_bf16_e4m3(__builtin_amdgcn_perm(lo[r + 1], lo[r], 0x05040100u),
                             __builtin_amdgcn_perm(lo[r + 3], lo[r + 2], 0x05040100u), sc[0]);
    o[1][g] = cvt4_bf16_e4m3(__builtin_amdgcn_perm(lo[r + 1], lo[r], 0x07060302u),
                             __builtin_amdgcn_perm(lo[r + 3], lo[r + 2], 0x07060302u), sc[1]);
    o[2][g] = cvt4_bf16_e4m3(__builtin_amdgcn_perm(hi[r + 1], hi[r], 0x05040100u),
                             __builtin_amdgcn_perm(hi[r + 3], hi[r + 2], 0x05040100u), sc[2]);
    o[3][g] = cvt4_bf16_e4m3(__builtin_amdgcn_perm(hi[r + 1], hi[r], 0x07060302u),
                             __builtin_amdgcn_perm(hi[r + 3], hi[r + 2], 0x07060302u), sc[3]);
  }
  float unused[4] = {0.f, 0.f, 0.f, 0.f};
  colwise_store<false, kNT>(o, xb, unused, T, K, k0, t0, q_col, s_col, nullptr, tid);
}

// ---------------------------------------------------------------------------
// SwiGLU of bf16 pairs and the row-wise quantize of a tile staged in LDS
// ---------------------------------------------------------------------------

// silu(g) = g * sigmoid(g) = g / (1 + e^-g), from the hardware base-2
// exponential and reciprocal (V_EXP_F32, V_RCP_F32; about 1 ulp each, and the
// scaling of -g by log2(e) adds a relative error below 2^-24 |g| log2 e): a
// few instructions instead of the library exp and an IEEE division, and far
// inside the half bf16 ulp that the result is rounded to.  For g below about
// -88 the exponential overflows and the result is a zero of g's sign, as with
// the library form.
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// a = silu(gate) * up of two bf16 pairs, as swiglu_fwd_kernel computes it
// (fp32 math, round to nearest even to bf16), packed as a bf16 pair.
__device__ __forceinline__ uint32_t swiglu_pair(uint32_t gw, uint32_t uw) {
  const float g0 = bf16_to_f32(gw & 0xFFFFu), g1 = bf16_to_f32(gw >> 16);
  const float u0 = bf16_to_f32(uw & 0xFFFFu), u1 = bf16_to_f32(uw >> 16);
  return f32_to_bf16(silu_f(g0) * u0) | (f32_to_bf16(silu_f(g1) * u1) << 16);
}

// Row-wise quantize of a staged 128 x 128 bf16 tile (rows t0.., columns k0..
// of a [T, K] tensor): thread t reads the 16-byte chunk t % 16 of rows
// 16 jj + t / 16 (jj = 0..7), so the quad of lanes 4b..4b+3 holds block b of
// its row, as the row-wise pass of the streaming kernels.  Called by all
// kColThreads threads; `tid` (as the column-wise helpers' `tid`) is the
// thread index, passed in by callers that must keep it from being hoisted.
__device__ __forceinline__ void rowwise_pass_bf16(const uint8_t* lds, int64_t K, int64_t k0,
                                                  int64_t t0, uint8_t* __restrict__ q_row,
                                                  uint8_t* __restrict__ s_row,
                                                  const int tid = threadIdx.x) {
  const uint32_t ro = opaque_u32((uint32_t)(tid >> 4) * (uint32_t)K + (tid & 15) * 8);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int r = 16 * jj + (tid >> 4), cc = tid & 15;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&lds[lds_off_bf16(r, cc * 16)]);
    const uint4 a = make_uint4(v.x, v.y, v.z, v.w);
    const uint32_t amax = quad_max(chunk_amax_bits(a));
    const uint32_t byte = scale_byte_from_exp(amax >> 7);
    const int64_t rb = t0 * K + k0 + 16 * jj * K;   // uniform
    *reinterpret_cast<uint2*>(q_row + rb + ro) = encode_chunk(a, byte);
    const uint32_t bytes4 = gather_blocks4(byte);
    if ((tid & 15) == 0) *reinterpret_cast<uint32_t*>(s_row + (rb >> 5) + (ro >> 5)) = bytes4;
  }
}

}  // namespace mx
