// Grouped MXFP8 GEMM on CDNA4 block-scaled MFMA (gfx950).
//
// All three GEMMs of an expert linear reduce to one form, because every
// operand is stored with its contraction dimension contiguous and its 1x32
// scale blocks along that dimension:
//     C[m, n] = sum_k A[m, k] * B[n, k]        ("NT" in row-major letters)
//   forward (NT): A = X row-wise [T, K], B = W_g row-wise [N, K]   (per expert)
//   dgrad   (NN): A = dY row-wise [T, N], B = W_g^T from the column-wise copy
//                 [K, G*N] (rows k, columns g*N..g*N+N)
//   wgrad   (TN): A = dY column-wise [N, T], B = X column-wise [K, T], the
//                 contraction running over the expert's token columns.
// ("[Pytorch] Add support for row-wise quanted input for grouped gemm",
//  Description and Greptile Summary flowchart; "[PyTorch] Fix distributed
//  BF16 weights and trim NVFP4 saved state in the fused grouped MLP", last
//  commit message: forward reads the row-wise weight, dgrad the column-wise
//  copy, wgrad the column-wise input tiles.)
//
// Forward and dgrad are grouped along M (each expert owns a run of token
// rows, B changes per expert); wgrad is grouped along the contraction (each
// expert owns a run of token columns and its own output matrix).  The tile
// scheduler reads the device-resident m_splits ("Improve device-init grouped
// linear module with single grouped weight support", review on CUDA m_splits)
// inside every workgroup: no host synchronisation, and an expert with no
// tokens owns no forward/dgrad tile and a zero wgrad output.
//
// The MFMA used is V_MFMA_SCALE_F32_16X16X128_F8F6F4 with both operands in
// E4M3: per lane 32 contraction bytes of one row (two 16-byte runs, see the
// fragment loads), one E8M0 scale per lane (one 32-element block of the
// row), fp32 accumulators.
#include "mx_device.h"
#include "kernels.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;        // output rows per workgroup tile
constexpr int BN = 128;        // output columns per workgroup tile
constexpr int BK = 128;        // contraction bytes per stage
constexpr int kThreads = 256;  // 4 waves, 2 x 2, each 64 x 64
constexpr int kMaxGroups = 1024;

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* sa;
  const uint8_t* b;
  const uint8_t* sb;
  void* c;
  int64_t lda, ldsa, ldb, ldsb, ldc;   // row strides (bytes for a/b/scales, elements for c)
  int64_t b_gstride, sb_gstride;       // per-expert offset of B (M-grouped)
  int64_t c_gstride;                   // per-expert offset of C in elements (K-grouped)
  int64_t rows;                        // M-grouped: T; K-grouped: rows of A
  int64_t cols;                        // columns of C
  int64_t kc;                          // contraction length (M-grouped)
  const int64_t* m_splits;
  int32_t G;
  int32_t ntiles_n;                    // cols / BN
  int32_t ntiles_m;                    // K-grouped: rows / BM
};

// Exclusive scan over the experts, done by the whole workgroup: finds the
// expert that owns `target` in the running count of units(g) (tiles or
// experts), and returns (g, row offset o_g, M_g, target - first unit of g).
struct GroupHit {
  int32_t g;
  int32_t local;
  int64_t off;
  int64_t len;
};

template <bool TILES>
__device__ GroupHit find_group(const int64_t* __restrict__ m_splits, int G, int64_t target,
                               int64_t* s_units, int64_t* s_rows, GroupHit* s_hit) {
  const int tid = threadIdx.x;
  constexpr int per = kMaxGroups / kThreads;  // 4 experts per thread
  int64_t mv[per];
  int64_t u_sum = 0, r_sum = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int g = tid * per + i;
    mv[i] = g < G ? max(m_splits[g], (int64_t)0) : 0;   // negative splits count as empty
    r_sum += mv[i];
    u_sum += TILES ? (mv[i] + BM - 1) / BM : 1;
  }
  s_units[tid] = u_sum;
  s_rows[tid] = r_sum;
  if (tid == 0) s_hit->g = -1;
  __syncthreads();
  // Hillis-Steele inclusive scan of 256 pairs
  for (int d = 1; d < kThreads; d <<= 1) {
    int64_t u = 0, r = 0;
    if (tid >= d) {
      u = s_units[tid - d];
      r = s_rows[tid - d];
    }
    __syncthreads();
    s_units[tid] += u;
    s_rows[tid] += r;
    __syncthreads();
  }
  int64_t u0 = s_units[tid] - u_sum;   // exclusive prefix
  int64_t r0 = s_rows[tid] - r_sum;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int g = tid * per + i;
    const int64_t nu = g < G ? (TILES ? (mv[i] + BM - 1) / BM : 1) : 0;
    if (g < G && target >= u0 && target < u0 + nu) {
      s_hit->g = g;
      s_hit->local = (int32_t)(target - u0);
      s_hit->off = r0;
      s_hit->len = mv[i];
    }
    u0 += nu;
    r0 += mv[i];
  }
  __syncthreads();
  GroupHit h = *s_hit;
  __syncthreads();
  return h;
}

// LDS layout of one stage: A tile [BM][BK], B tile [BN][BK] (16-byte chunks
// XOR-swizzled by row so that the 16 rows read by one MFMA operand load hit
// distinct banks), then the scale tiles [BM][4] and [BN][4].
constexpr int kTileBytes = BM * BK;
constexpr int kStageBytes = 2 * kTileBytes + (BM + BN) * 4;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

template <bool KGROUPED, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile -> (expert, output block, operand pointers) -------------------
  int64_t* s_units = reinterpret_cast<int64_t*>(smem);
  int64_t* s_rows = s_units + kThreads;
  GroupHit* s_hit = reinterpret_cast<GroupHit*>(s_rows + kThreads);

  const uint8_t *a_base, *sa_base, *b_base, *sb_base;
  int64_t klen, m0, n0, valid_rows;
  char* c_base;
  const int64_t esz = OUT_BF16 ? 2 : 4;
  if (!KGROUPED) {
    const int nt = blockIdx.x % p.ntiles_n;
    const int64_t mt = blockIdx.x / p.ntiles_n;
    const GroupHit h = find_group<true>(p.m_splits, p.G, mt, s_units, s_rows, s_hit);
    if (h.g < 0) return;                        // beyond the last expert's tiles
    m0 = h.off + (int64_t)h.local * BM;
    n0 = (int64_t)nt * BN;
    // rows of the expert, never past the token count (splits that break the
    // contract must not make the kernel read or write out of bounds)
    valid_rows = min(min((int64_t)BM, h.off + h.len - m0), p.rows - m0);
    if (valid_rows <= 0) return;
    a_base = p.a + m0 * p.lda;
    sa_base = p.sa + m0 * p.ldsa;
    b_base = p.b + h.g * p.b_gstride + n0 * p.ldb;
    sb_base = p.sb + h.g * p.sb_gstride + n0 * p.ldsb;
    klen = p.kc;
    c_base = reinterpret_cast<char*>(p.c) + (m0 * p.ldc + n0) * esz;
  } else {
    const int per_group = p.ntiles_m * p.ntiles_n;
    const int gi = blockIdx.x / per_group;
    const int rem = blockIdx.x % per_group;
    const int mt = rem / p.ntiles_n, nt = rem % p.ntiles_n;
    const GroupHit h = find_group<false>(p.m_splits, p.G, gi, s_units, s_rows, s_hit);
    m0 = (int64_t)mt * BM;
    n0 = (int64_t)nt * BN;
    valid_rows = BM;
    a_base = p.a + m0 * p.lda + h.off;
    sa_base = p.sa + m0 * p.ldsa + h.off / 32;
    b_base = p.b + n0 * p.ldb + h.off;
    sb_base = p.sb + n0 * p.ldsb + h.off / 32;
    klen = h.off < p.kc ? min(h.len, p.kc - h.off) : 0;   // p.kc = T here
    c_base = reinterpret_cast<char*>(p.c) + (h.g * p.c_gstride + m0 * p.ldc + n0) * esz;
  }

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // ---- global -> register staging: 4 chunks of A and 4 of B per thread ----
  // chunk idx = tid + 256 j: row idx/8, 16-byte chunk idx%8 of the row
  const uint8_t* ga[4];
  const uint8_t* gb[4];
  int lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = tid + kThreads * j;
    const int r = idx >> 3, ch = idx & 7;
    const int ra = r < valid_rows ? r : 0;     // rows past the expert: any valid row
    ga[j] = a_base + ra * p.lda + ch * 16;
    gb[j] = b_base + r * p.ldb + ch * 16;
    lo[j] = swz(r, ch);
  }
  // scales: threads 0..127 fetch A rows' 4 bytes, 128..255 B rows' 4 bytes
  const uint8_t* gs;
  int ls;
  if (tid < BM) {
    const int r = tid < valid_rows ? tid : 0;
    gs = sa_base + r * p.ldsa;
    ls = 2 * kTileBytes + tid * 4;
  } else {
    gs = sb_base + (tid - BM) * p.ldsb;
    ls = 2 * kTileBytes + BM * 4 + (tid - BM) * 4;
  }

  const int nk = (int)(klen / BK);
  u32x4 ra[4], rb[4];
  uint32_t rs = 0;
  // fragment addresses: operand row (l % 16) of a 16-row sub-tile.  The
  // instruction takes, in lane l with q = l/16, the contraction bytes
  // [16q, 16q+16) in its first 16 bytes and [64+16q, 64+16q+16) in its last
  // 16 (16-byte chunks q and 4+q of the 128-byte stage); the lane's scale
  // byte is that of 32-element block q of its row.
  const int fr = lane & 15;
  const int fq = lane >> 4;

#define MX_GLOAD1(j, kb)                                                  \
  ra[j] = *reinterpret_cast<const u32x4*>(ga[j] + (kb));                  \
  rb[j] = *reinterpret_cast<const u32x4*>(gb[j] + (kb));
#define MX_GLOAD(kt)                                                      \
  do {                                                                    \
    const int64_t kb_ = (int64_t)(kt) * BK;                               \
    MX_GLOAD1(0, kb_) MX_GLOAD1(1, kb_) MX_GLOAD1(2, kb_) MX_GLOAD1(3, kb_) \
    rs = *reinterpret_cast<const uint32_t*>(gs + kb_ / 32);               \
  } while (0)
#define MX_LSTORE1(j, base)                                               \
  *reinterpret_cast<u32x4*>((base) + lo[j]) = ra[j];                      \
  *reinterpret_cast<u32x4*>((base) + kTileBytes + lo[j]) = rb[j];
#define MX_LSTORE(stage)                                                  \
  do {                                                                    \
    uint8_t* base_ = smem + (stage) * kStageBytes;                        \
    MX_LSTORE1(0, base_) MX_LSTORE1(1, base_) MX_LSTORE1(2, base_)        \
    MX_LSTORE1(3, base_)                                                  \
    *reinterpret_cast<uint32_t*>(base_ + ls) = rs;                        \
  } while (0)

  if (nk > 0) {
    MX_GLOAD(0);
    MX_LSTORE(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) MX_GLOAD(kt + 1);
    const uint8_t* base = smem + cur * kStageBytes;
    v8i af[4], bf[4];
    int as[4], bs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + fr;
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(base + swz(r, fq));
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(base + swz(r, 4 + fq));
      af[i] = __builtin_bit_cast(v8i, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      as[i] = base[2 * kTileBytes + r * 4 + fq];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 64 + j * 16 + fr;
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(base + kTileBytes + swz(r, fq));
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(base + kTileBytes + swz(r, 4 + fq));
      bf[j] = __builtin_bit_cast(v8i, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      bs[j] = base[2 * kTileBytes + BM * 4 + r * 4 + fq];
    }
    // D[n][m] = sum_k B[n,k] A[m,k]: srcA = B fragment, srcB = A fragment, so
    // each lane ends with 4 consecutive output columns of one output row.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i], acc[i][j], 0,
                                                                     0, 0, bs[j], 0, as[i]);
    if (kt + 1 < nk) MX_LSTORE(cur ^ 1);
    __syncthreads();
  }
#undef MX_GLOAD
#undef MX_GLOAD1
#undef MX_LSTORE
#undef MX_LSTORE1

  // ---- epilogue: lane holds C[m0 + .. + l%16][n0 + .. + 4(l/16) + 0..3] ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wm * 64 + i * 16 + fr;
    if (r >= valid_rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cidx = wn * 64 + j * 16 + 4 * fq;
      char* dst = c_base + ((int64_t)r * p.ldc + cidx) * esz;
      const v4f v = acc[i][j];
      if (OUT_BF16) {
        const uint32_t lo2 = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
        const uint32_t hi2 = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo2, hi2);
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

template <bool KG, bool BF>
static hipError_t launch_one(const GemmArgs& a, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((grouped_gemm_kernel<KG, BF>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int layout, const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                               const uint8_t* sb, void* c, bool out_bf16, int64_t T, int64_t N,
                               int64_t K, const int64_t* m_splits, int32_t G, hipStream_t st) {
  GemmArgs p{};
  p.a = a;
  p.sa = sa;
  p.b = b;
  p.sb = sb;
  p.c = c;
  p.m_splits = m_splits;
  p.G = G;
  bool kgrouped = false;
  unsigned grid = 0;
  if (layout == 0) {           // forward: C[T,N] = X[T,K] W_g[N,K]^T
    p.lda = K; p.ldsa = K / 32;
    p.ldb = K; p.ldsb = K / 32;
    p.b_gstride = N * K; p.sb_gstride = N * K / 32;
    p.ldc = N; p.rows = T; p.cols = N; p.kc = K;
  } else if (layout == 1) {    // dgrad: C[T,K] = dY[T,N] (W_g^T from [K, G*N])
    p.lda = N; p.ldsa = N / 32;
    p.ldb = (int64_t)G * N; p.ldsb = (int64_t)G * N / 32;
    p.b_gstride = N; p.sb_gstride = N / 32;
    p.ldc = K; p.rows = T; p.cols = K; p.kc = N;
  } else {                     // wgrad: C[g] [N,K] = dYc[N, rows g] Xc[K, rows g]^T
    kgrouped = true;
    p.lda = T; p.ldsa = T / 32;
    p.ldb = T; p.ldsb = T / 32;
    p.ldc = K; p.c_gstride = N * K;
    p.rows = N; p.cols = K; p.kc = T;
  }
  p.ntiles_n = (int32_t)(p.cols / BN);
  if (!kgrouped) {
    // upper bound of sum_g ceil(M_g / BM): T / BM full tiles plus one partial per expert
    const int64_t mt = T / BM + G;
    grid = (unsigned)(mt * p.ntiles_n);
  } else {
    p.ntiles_m = (int32_t)(p.rows / BM);
    grid = (unsigned)((int64_t)G * p.ntiles_m * p.ntiles_n);
  }
  if (kgrouped) return out_bf16 ? launch_one<true, true>(p, grid, st) : launch_one<true, false>(p, grid, st);
  return out_bf16 ? launch_one<false, true>(p, grid, st) : launch_one<false, false>(p, grid, st);
}

}  // namespace mx
