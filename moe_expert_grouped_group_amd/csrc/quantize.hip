// MXFP8 group quantize, column-wise requantize and grouped bias gradient
// kernels for gfx950.  All of them stream HBM: the design goal is full-width
// coalesced 16-byte accesses and enough bytes in flight per CU, with the
// block maxima reduced inside the wavefront (DPP) and the column-wise copies
// transposed through LDS.
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
#include "mx_device.h"
#include "kernels.h"

namespace mx {

// ---------------------------------------------------------------------------
// row-wise quantize: one 16-byte chunk (8 bf16) per lane, 4 lanes per block
// ---------------------------------------------------------------------------

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

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

// Encode the 8 bf16 of `w` with the scale 2^-X given as `inv`; returns 8 bytes.
__device__ __forceinline__ uint2 encode_chunk(uint4 w, float inv) {
  uint32_t c0 = encode_e4m3(bf16_to_f32(w.x & 0xFFFFu) * inv);
  uint32_t c1 = encode_e4m3(bf16_to_f32(w.x >> 16) * inv);
  uint32_t c2 = encode_e4m3(bf16_to_f32(w.y & 0xFFFFu) * inv);
  uint32_t c3 = encode_e4m3(bf16_to_f32(w.y >> 16) * inv);
  uint32_t c4 = encode_e4m3(bf16_to_f32(w.z & 0xFFFFu) * inv);
  uint32_t c5 = encode_e4m3(bf16_to_f32(w.z >> 16) * inv);
  uint32_t c6 = encode_e4m3(bf16_to_f32(w.w & 0xFFFFu) * inv);
  uint32_t c7 = encode_e4m3(bf16_to_f32(w.w >> 16) * inv);
  return make_uint2(pack4(c0, c1, c2, c3), pack4(c4, c5, c6, c7));
}

constexpr int kRowThreads = 256;
constexpr int kRowUnroll = 4;

// x viewed as a flat array of 16-byte chunks; chunk c holds elements
// [8c, 8c+8) and belongs to block c/4 (blocks are consecutive in the flat
// order because K % 32 == 0).  nchunks is a multiple of 256.
__global__ __launch_bounds__(kRowThreads) void quant_rowwise_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, uint8_t* __restrict__ s,
    int64_t nchunks) {
  const int64_t stride = (int64_t)gridDim.x * kRowThreads * kRowUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kRowThreads * kRowUnroll + threadIdx.x;
       base < nchunks; base += stride) {
    uint4 w[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t c = base + (int64_t)u * kRowThreads;
      w[u] = c < nchunks ? x[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t c = base + (int64_t)u * kRowThreads;
      const uint32_t amax = quad_max(chunk_amax_bits(w[u]));
      const uint32_t byte = scale_byte_from_exp(amax >> 7);
      if (c < nchunks) {
        q[c] = encode_chunk(w[u], inv_scale_from_byte(byte));
        if ((threadIdx.x & 3) == 0) s[c >> 2] = (uint8_t)byte;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fused row-wise + column-wise quantize from bf16, tile 128 rows x 128 cols
// ---------------------------------------------------------------------------

constexpr int kTileT = 128;       // token rows per tile
constexpr int kTileK = 128;       // hidden columns per tile
constexpr int kColThreads = 256;
// LDS row stride 272 B (256 B of data + 16 B pad) plus 64 B after every 32
// rows: the four 32-row blocks read in the same instruction then start
// 16 dwords apart, so a wave's column reads hit disjoint banks.
constexpr int kLdsRowBytes = 272;
__device__ __forceinline__ int lds_off_bf16(int row, int byte_col) {
  return row * kLdsRowBytes + (row >> 5) * 64 + byte_col;
}
constexpr int kLdsBytesBf16 = kTileT * kLdsRowBytes + (kTileT / 32) * 64;

__global__ __launch_bounds__(kColThreads) void quant_rowcol_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t K, uint8_t* __restrict__ q_row,
    uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytesBf16];
  const int tid = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * kTileK;
  const int64_t t0 = (int64_t)blockIdx.y * kTileT;

  // load: 128 rows x 256 B = 2048 chunks, 8 per thread; 16 chunks per row
  uint4 w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int idx = tid + kColThreads * j;
    const int r = idx >> 4, cc = idx & 15;
    w[j] = *reinterpret_cast<const uint4*>(x + (t0 + r) * K + k0 + cc * 8);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int idx = tid + kColThreads * j;
    const int r = idx >> 4, cc = idx & 15;
    *reinterpret_cast<uint4*>(&lds[lds_off_bf16(r, cc * 16)]) = w[j];
    if (q_row != nullptr) {
      // row-wise: lanes 4b..4b+3 of a quad hold the 32 values of one block
      const uint32_t amax = quad_max(chunk_amax_bits(w[j]));
      const uint32_t byte = scale_byte_from_exp(amax >> 7);
      const int64_t e = (t0 + r) * K + k0 + cc * 8;
      *reinterpret_cast<uint2*>(q_row + e) = encode_chunk(w[j], inv_scale_from_byte(byte));
      if ((tid & 3) == 0) s_row[e >> 5] = (uint8_t)byte;
    }
  }
  if (q_col == nullptr) return;
  __syncthreads();

  // column-wise: thread -> column pair p (2 columns), 32-row block rb
  const int lane = tid & 63, wave = tid >> 6;
  const int rb = lane >> 4;
  const int p = wave * 16 + (lane & 15);           // 0..63
  uint32_t v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r)
    v[r] = *reinterpret_cast<const uint32_t*>(&lds[lds_off_bf16(rb * 32 + r, p * 4)]);
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) m = max_u16x2(m, v[r] & 0x7FFF7FFFu);
  const uint32_t b0 = scale_byte_from_exp((m & 0xFFFFu) >> 7);
  const uint32_t b1 = scale_byte_from_exp((m >> 16) >> 7);
  const float inv0 = inv_scale_from_byte(b0), inv1 = inv_scale_from_byte(b1);
  uint32_t o0[8], o1[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t word = v[4 * g + i];
      a[i] = encode_e4m3(bf16_to_f32(word & 0xFFFFu) * inv0);
      b[i] = encode_e4m3(bf16_to_f32(word >> 16) * inv1);
    }
    o0[g] = pack4(a[0], a[1], a[2], a[3]);
    o1[g] = pack4(b[0], b[1], b[2], b[3]);
  }
  const int64_t kc = k0 + 2 * p;
  const int64_t tc = t0 + rb * 32;
  uint4* d0 = reinterpret_cast<uint4*>(q_col + kc * T + tc);
  uint4* d1 = reinterpret_cast<uint4*>(q_col + (kc + 1) * T + tc);
  d0[0] = make_uint4(o0[0], o0[1], o0[2], o0[3]);
  d0[1] = make_uint4(o0[4], o0[5], o0[6], o0[7]);
  d1[0] = make_uint4(o1[0], o1[1], o1[2], o1[3]);
  d1[1] = make_uint4(o1[4], o1[5], o1[6], o1[7]);
  s_col[kc * (T / 32) + (tc >> 5)] = (uint8_t)b0;
  s_col[(kc + 1) * (T / 32) + (tc >> 5)] = (uint8_t)b1;
}

// ---------------------------------------------------------------------------
// column-wise requantize of row-wise MXFP8 (+ optional dbias partials),
// tile 128 rows x 128 cols of bytes
// ---------------------------------------------------------------------------

// LDS row stride 144 B (128 + 16 pad) plus 32 B after every 32 rows: the
// four 32-row blocks of one read instruction start 8 dwords apart.
constexpr int kLdsRowBytesU8 = 144;
__device__ __forceinline__ int lds_off_u8(int row, int col) {
  return row * kLdsRowBytesU8 + (row >> 5) * 32 + col;
}
constexpr int kLdsBytesU8 = kTileT * kLdsRowBytesU8 + (kTileT / 32) * 32;

__global__ __launch_bounds__(kColThreads) void requant_colwise_kernel(
    const uint8_t* __restrict__ q_row, const uint8_t* __restrict__ s_row, int64_t T, int64_t K,
    uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col, float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytesU8];
  __shared__ uint32_t lds_s[kTileT];   // 4 scale bytes (4 blocks of 32 cols) per row
  const int tid = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * kTileK;
  const int64_t t0 = (int64_t)blockIdx.y * kTileT;
  const int64_t ks = K / 32;

  uint4 w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = tid + kColThreads * j;
    const int r = idx >> 3, cc = idx & 7;
    w[j] = *reinterpret_cast<const uint4*>(q_row + (t0 + r) * K + k0 + cc * 16);
  }
  uint32_t sv = 0;
  if (tid < kTileT)
    sv = *reinterpret_cast<const uint32_t*>(s_row + (t0 + tid) * ks + (k0 >> 5));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = tid + kColThreads * j;
    const int r = idx >> 3, cc = idx & 7;
    *reinterpret_cast<uint4*>(&lds[lds_off_u8(r, cc * 16)]) = w[j];
  }
  if (tid < kTileT) lds_s[tid] = sv;
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int rb = lane >> 4;
  const int p = wave * 16 + (lane & 15);   // column pair 0..63 -> columns 2p, 2p+1
  const int sblk = p >> 4;                 // scale block (32 columns) of both columns
  uint32_t code[32];
  int sexp[32];
  constexpr int kNone = -100000;   // no non-zero element seen
  int emax0 = kNone, emax1 = kNone;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const int row = rb * 32 + r;
    const uint32_t pair = *reinterpret_cast<const uint16_t*>(&lds[lds_off_u8(row, 2 * p)]);
    const int se = (int)((lds_s[row] >> (8 * sblk)) & 0xFFu) - 127;
    code[r] = pair;
    sexp[r] = se;
    const uint32_t m0 = pair & 0x7Fu, m1 = (pair >> 8) & 0x7Fu;
    if (m0) emax0 = max(emax0, e4m3_floor_log2(m0) + se);
    if (m1) emax1 = max(emax1, e4m3_floor_log2(m1) + se);
  }
  // X' = floor(log2 amax) - 8, clamped; all-zero column block -> -127
  const int x0 = emax0 == kNone ? -127 : min(max(emax0 - 8, -127), 127);
  const int x1 = emax1 == kNone ? -127 : min(max(emax1 - 8, -127), 127);
  uint32_t o0[8], o1[8];
  float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      const float d0 = decode_e4m3(code[r] & 0xFFu);
      const float d1 = decode_e4m3(code[r] >> 8);
      a[i] = encode_e4m3(__builtin_amdgcn_ldexpf(d0, sexp[r] - x0));
      b[i] = encode_e4m3(__builtin_amdgcn_ldexpf(d1, sexp[r] - x1));
      if (partial != nullptr) {
        sum0 += __builtin_amdgcn_ldexpf(d0, sexp[r]);
        sum1 += __builtin_amdgcn_ldexpf(d1, sexp[r]);
      }
    }
    o0[g] = pack4(a[0], a[1], a[2], a[3]);
    o1[g] = pack4(b[0], b[1], b[2], b[3]);
  }
  const int64_t kc = k0 + 2 * p;
  const int64_t tc = t0 + rb * 32;
  uint4* d0 = reinterpret_cast<uint4*>(q_col + kc * T + tc);
  uint4* d1 = reinterpret_cast<uint4*>(q_col + (kc + 1) * T + tc);
  d0[0] = make_uint4(o0[0], o0[1], o0[2], o0[3]);
  d0[1] = make_uint4(o0[4], o0[5], o0[6], o0[7]);
  d1[0] = make_uint4(o1[0], o1[1], o1[2], o1[3]);
  d1[1] = make_uint4(o1[4], o1[5], o1[6], o1[7]);
  s_col[kc * (T / 32) + (tc >> 5)] = (uint8_t)(x0 + 127);
  s_col[(kc + 1) * (T / 32) + (tc >> 5)] = (uint8_t)(x1 + 127);

  if (partial != nullptr) {
    // combine the four 32-row blocks (lanes l, l^16, l^32, l^48) in a fixed order
    sum0 += __shfl_xor(sum0, 16);
    sum1 += __shfl_xor(sum1, 16);
    sum0 += __shfl_xor(sum0, 32);
    sum1 += __shfl_xor(sum1, 32);
    if (rb == 0) {
      float* dst = partial + (t0 / kTileT) * K + kc;
      *reinterpret_cast<float2*>(dst) = make_float2(sum0, sum1);
    }
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

// dbias[g, k] = sum over the 128-row tiles of expert g of partial[tile, k],
// in tile order.  grid = (G, ceil(K / 256)).
__global__ __launch_bounds__(256) void dbias_finalize_kernel(
    const float* __restrict__ partial, const int64_t* __restrict__ m_splits, int32_t G, int64_t T,
    int64_t K, float* __restrict__ dbias) {
  __shared__ int64_t red[256];
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
  const int64_t k = (int64_t)blockIdx.y * 256 + tid;
  if (k >= K) return;
  // tiles of the expert, clipped to the token count (splits that break the
  // contract must not make the kernel read out of bounds)
  const int64_t first = min(off, T) / kTileT, last = min(off + mg, T) / kTileT;
  float s = 0.f;
  for (int64_t tile = first; tile < last; ++tile) s += partial[tile * K + k];
  dbias[(int64_t)g * K + k] = s;
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

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

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

__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint32_t* __restrict__ h,
                                                         const uint32_t* __restrict__ da,
                                                         int64_t T, int64_t F,
                                                         uint32_t* __restrict__ dh) {
  const int64_t n = T * F / 2;
  const int64_t f2 = F / 2;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / f2, c = i % f2;
    const uint32_t gw = h[row * F + c];
    const uint32_t uw = h[row * F + f2 + c];
    const uint32_t dw = da[i];
    uint32_t og = 0, ou = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float g = bf16_to_f32((gw >> (16 * j)) & 0xFFFFu);
      const float u = bf16_to_f32((uw >> (16 * j)) & 0xFFFFu);
      const float d = bf16_to_f32((dw >> (16 * j)) & 0xFFFFu);
      const float s = 1.0f / (1.0f + expf(-g));
      const float dg = d * u * s * (1.0f + g * (1.0f - s));
      const float du = d * g * s;
      og |= f32_to_bf16(dg) << (16 * j);
      ou |= f32_to_bf16(du) << (16 * j);
    }
    dh[row * F + c] = og;
    dh[row * F + f2 + c] = ou;
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
                                hipStream_t st) {
  const int64_t nchunks = T * K / 8;
  const int grid = grid_for(nchunks, kRowThreads * kRowUnroll, 256 * 16);
  hipLaunchKernelGGL(quant_rowwise_kernel, dim3(grid), dim3(kRowThreads), 0, st,
                     reinterpret_cast<const uint4*>(x), reinterpret_cast<uint2*>(q), s, nchunks);
  return hipGetLastError();
}

hipError_t launch_quant_rowcol(const uint16_t* x, int64_t T, int64_t K, uint8_t* q_row,
                               uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t st) {
  dim3 grid((unsigned)(K / kTileK), (unsigned)(T / kTileT));
  hipLaunchKernelGGL(quant_rowcol_kernel, grid, dim3(kColThreads), 0, st, x, T, K, q_row, s_row,
                     q_col, s_col);
  return hipGetLastError();
}

hipError_t launch_requant_colwise(const uint8_t* q_row, const uint8_t* s_row, int64_t T,
                                  int64_t K, uint8_t* q_col, uint8_t* s_col, float* partial,
                                  hipStream_t st) {
  dim3 grid((unsigned)(K / kTileK), (unsigned)(T / kTileT));
  hipLaunchKernelGGL(requant_colwise_kernel, grid, dim3(kColThreads), 0, st, q_row, s_row, T, K,
                     q_col, s_col, partial);
  return hipGetLastError();
}

hipError_t launch_dbias_partial(const uint8_t* q_row, const uint8_t* s_row, int64_t T, int64_t N,
                                float* partial, hipStream_t st) {
  dim3 grid((unsigned)(N / 256), (unsigned)(T / kTileT));
  hipLaunchKernelGGL(dbias_partial_kernel, grid, dim3(256), 0, st, q_row, s_row, T, N, partial);
  return hipGetLastError();
}

hipError_t launch_dbias_finalize(const float* partial, const int64_t* m_splits, int32_t G,
                                 int64_t T, int64_t K, float* dbias, hipStream_t st) {
  dim3 grid((unsigned)G, (unsigned)((K + 255) / 256));
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

}  // namespace mx
