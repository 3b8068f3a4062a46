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
// Kernel structure (one 256 x 256 output tile per workgroup, 4 waves of
// 128 x 128):
//  * MFMA: V_MFMA_SCALE_F32_32X32X64_F8F6F4, both operands E4M3.  Lane l
//    (row l % 32 of the operand, half g = l / 32) supplies the contraction
//    bytes [16g, 16g+16) and [32+16g, 32+16g+16) of a 64-byte step, and the
//    E8M0 scale of 32-element block g of its row.  Output: lane l holds
//    column l % 32, rows 8(r/4) + 4(l/32) + r%4 for accumulator r.
//  * The MFMA's first operand is the A tile and its second the B tile, so the
//    32 lanes of a half-wave hold 32 consecutive output columns of one row:
//    a store of one accumulator register writes whole cache lines.
//  * Stages of 64 contraction bytes go HBM/L2 -> LDS by LDS DMA (no register
//    staging) into a ring of 4 buffers, so three stages are in flight while
//    one is consumed.  Each wave copies a quarter of every stage; a stage is
//    read only after every wave has waited for its own copies and passed a
//    barrier.
//  * Inside a step, the next A fragment is read while the current one's 4
//    MFMAs run; the barrier sits before the last MFMA group so that the next
//    stage's B fragments are read while that group runs.
#include <algorithm>

#include "mx_device.h"
#include "kernels.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;        // output rows per workgroup tile
constexpr int BN = 256;        // output columns per workgroup tile
constexpr int BK = 64;         // contraction bytes per stage (one MFMA step)
constexpr int kStages = 4;     // LDS ring depth
constexpr int kThreads = 256;  // 4 waves, 2 x 2, each 128 x 128
constexpr int WT = 128;        // wave tile edge
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
  int64_t kc;                          // contraction length (M-grouped); T (K-grouped)
  const int64_t* m_splits;
  int32_t G;
  int32_t ntiles_n;                    // cols / BN
  int32_t band;                        // K-grouped: row tiles per expert (rows / BM)
  int32_t ntiles;                      // K-grouped: G * band * ntiles_n tiles
};

// LDS layout of one stage: A tile [BM][BK], B tile [BN][BK], 16-byte chunk c
// of row r stored at chunk position c ^ ((r >> 1) & 3).  The LDS has 32
// banks of 4 bytes, so two 64-byte rows share one bank line; the 8
// consecutive rows of a fragment read that the LDS serves together then use
// 8 distinct 16-byte bank groups.
constexpr int kTileBytesA = BM * BK;
constexpr int kTileBytesB = BN * BK;
constexpr int kOffB = kTileBytesA;
constexpr int kStageBytes = kTileBytesA + kTileBytesB;
constexpr int kDmaPerStage = 8;    // per wave: 4 (A) + 4 (B) data copies
// E8M0 scales arrive in groups of kScaleSteps stages: 16 bytes (16 blocks of
// 32) per operand row, [BM][16] for A then [BN][16] for B, double-buffered.
// Copying a row's scale bytes one stage at a time would cost one cache-line
// request per row per stage for 2 bytes of data, as many requests as the
// operand tiles themselves.
constexpr int kScaleSteps = 8;
constexpr int kScaleRow = 2 * kScaleSteps;   // bytes per row and group
constexpr int kScOffB = BM * kScaleRow;
constexpr int kScaleBuf = (BM + BN) * kScaleRow;
constexpr int kScaleDma = 8;       // per wave and group: 4 (A) + 4 (B), 16 rows each

// Global -> LDS copies (LDS DMA) from a scalar base address plus a per-lane
// 32-bit offset (the scalar-base form streams several times faster than one
// 64-bit address per lane).  Lane i of the wave writes LDS bytes
// [lds + 16 i, lds + 16 i + 16) (dma16) or [lds + 4 i, lds + 4 i + 4) (dma4);
// `lds` is a wave-uniform LDS byte address (it goes to M0), passed as an
// integer so that no generic pointer to LDS has to be formed.  They are issued as inline asm so
// that the compiler's LDS wait-count tracking covers only the fragment reads
// (with LDS DMA it can see, it falls back to waiting for every outstanding
// LDS read before each MFMA group, which serialises the fragment prefetch).
// Ordering is kept by construction: volatile asm is not moved across the
// barriers, the explicit s_waitcnt vmcnt that precedes every read of a stage
// the DMA filled, or the scheduling barriers around the issue block; the
// copies complete in order with the compiler's own loads, so its vmcnt waits
// stay conservative.
__device__ __forceinline__ void dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(l), "v"(voff), "s"(sbase)
               : "m0");
}
__device__ __forceinline__ void dma4(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(l), "v"(voff), "s"(sbase)
               : "m0");
}

// A pointer that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* q) {
  const uint64_t v = (uint64_t)(uintptr_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only.
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Wait until this wave's copies of the needed stage have landed, given that
// `later` stages were issued after it (at most kStages - 1 = 3).  A
// stage that opens a scale group carries kScaleDma more copies; counting only
// the kDmaPerStage data copies of the later stages waits for at least as many
// completions as needed (copies complete in issue order).
__device__ __forceinline__ void wait_stage(int later) {
  if (later >= 3) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * kDmaPerStage));
  } else if (later == 2) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kDmaPerStage));
  } else if (later == 1) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerStage));
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
}

// LDS reads at integer LDS byte addresses, so that a per-lane base plus a
// per-step offset is formed once and each fragment's offset within the stage
// becomes the instruction's immediate offset.
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
__device__ __forceinline__ v8i lds_frag(uint32_t a0, uint32_t a1) {
  const u32x4 x0 = *(lds_u32x4*)a0;
  const u32x4 x1 = *(lds_u32x4*)a1;
  return __builtin_bit_cast(v8i, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ int lds_byte(uint32_t a) { return (int)*(lds_u8*)a; }

// A value the compiler must take as computed here: stops it from
// re-associating a per-step base with per-fragment constants and hoisting
// the sums out of the loop, one register each.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Expert table kept in LDS for the whole launch: exclusive prefix of tiles
// (forward/dgrad: ceil(M_g / BM) row tiles per expert) and of token rows, and
// (wgrad) the experts in decreasing order of tokens.
struct ExpertTable {
  int32_t tpre[kMaxGroups + 1];
  int64_t roff[kMaxGroups + 1];
  int16_t order[kMaxGroups];
};

// Builds the table with the whole workgroup (4 experts per thread, then a
// Hillis-Steele scan over the 256 per-thread sums in `scratch`).
template <bool KGROUPED>
__device__ void build_table(const int64_t* __restrict__ m_splits, int G, ExpertTable* t,
                            int64_t* scratch) {
  const int tid = threadIdx.x;
  constexpr int per = kMaxGroups / kThreads;
  int64_t mv[per];
  int64_t r_sum = 0;
  int32_t u_sum = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int g = tid * per + i;
    mv[i] = g < G ? max(m_splits[g], (int64_t)0) : 0;   // negative splits count as empty
    r_sum += mv[i];
    u_sum += (int32_t)((mv[i] + BM - 1) / BM);
  }
  int64_t* s_rows = scratch;
  int64_t* s_units = scratch + kThreads;
  s_rows[tid] = r_sum;
  s_units[tid] = u_sum;
  __syncthreads();
  for (int d = 1; d < kThreads; d <<= 1) {
    int64_t r = 0, u = 0;
    if (tid >= d) {
      r = s_rows[tid - d];
      u = s_units[tid - d];
    }
    __syncthreads();
    s_rows[tid] += r;
    s_units[tid] += u;
    __syncthreads();
  }
  int64_t r0 = s_rows[tid] - r_sum;
  int32_t u0 = (int32_t)(s_units[tid] - u_sum);
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int g = tid * per + i;
    if (g <= G) {
      t->roff[g] = r0;
      t->tpre[g] = u0;
    }
    r0 += mv[i];
    u0 += (int32_t)((mv[i] + BM - 1) / BM);
  }
  if (tid == kThreads - 1) {   // totals (entry G, also when G == kMaxGroups)
    t->roff[G] = s_rows[tid];
    t->tpre[G] = (int32_t)s_units[tid];
  }
  __syncthreads();
  if (KGROUPED) {
    // rank = number of experts with more tokens (ties: lower index first)
    for (int g = tid; g < G; g += kThreads) {
      const int64_t mg = t->roff[g + 1] - t->roff[g];
      int rank = 0;
      for (int h = 0; h < G; ++h) {
        const int64_t mh = t->roff[h + 1] - t->roff[h];
        rank += (mh > mg) || (mh == mg && h < g);
      }
      t->order[rank] = (int16_t)g;
    }
  }
  __syncthreads();
}

// One tile's operands.
struct TileDesc {
  const uint8_t* a;    // A rows of the tile at contraction 0
  const uint8_t* sa;
  const uint8_t* b;
  const uint8_t* sb;
  char* c;             // C[m0][n0]
  int32_t nk;          // contraction steps (BK bytes each)
  int32_t valid_rows;  // rows of A / C that belong to the tile
  int32_t nblk;        // scale blocks of the tile's contraction (nk * 2)
};

template <bool KGROUPED>
__device__ __forceinline__ TileDesc describe(const GemmArgs& p, const ExpertTable* t, int tile,
                                             int64_t esz) {
  TileDesc d;
  if (!KGROUPED) {
    const int mt = tile / p.ntiles_n, nt = tile % p.ntiles_n;
    // expert g: the last with tpre[g] <= mt (binary search over G + 1 entries)
    int lo = 0, hi = p.G;                    // tpre[lo] <= mt < tpre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (t->tpre[mid] <= mt) lo = mid; else hi = mid;
    }
    const int g = lo;
    const int64_t m0 = t->roff[g] + (int64_t)(mt - t->tpre[g]) * BM;
    const int64_t n0 = (int64_t)nt * BN;
    const int64_t end = min(t->roff[g + 1], p.rows);   // never past the token count
    d.valid_rows = (int32_t)max(min((int64_t)BM, end - m0), (int64_t)0);
    d.a = p.a + m0 * p.lda;
    d.sa = p.sa + m0 * p.ldsa;
    d.b = p.b + g * p.b_gstride + n0 * p.ldb;
    d.sb = p.sb + g * p.sb_gstride + n0 * p.ldsb;
    d.nk = d.valid_rows > 0 ? (int32_t)(p.kc / BK) : 0;
    d.nblk = (int32_t)(p.kc / 32);
    d.c = reinterpret_cast<char*>(p.c) + (m0 * p.ldc + n0) * esz;
  } else {
    const int per_expert = p.band * p.ntiles_n;
    const int g = t->order[tile / per_expert];
    const int rem = tile % per_expert;
    const int mtl = rem / p.ntiles_n, nt = rem % p.ntiles_n;
    // p.kc = T here.  Runs are multiples of 128 tokens by contract; rounding
    // down keeps every copy inside [0, T) and aligned for any split values.
    const int64_t off = min(t->roff[g], p.kc) & ~(int64_t)127;
    const int64_t len = max(min(t->roff[g + 1], p.kc) - off, (int64_t)0) & ~(int64_t)127;
    const int64_t m0 = (int64_t)mtl * BM, n0 = (int64_t)nt * BN;
    d.valid_rows = BM;
    d.a = p.a + m0 * p.lda + off;
    d.sa = p.sa + m0 * p.ldsa + off / 32;
    d.b = p.b + n0 * p.ldb + off;
    d.sb = p.sb + n0 * p.ldsb + off / 32;
    d.nk = (int32_t)(len / BK);
    d.nblk = (int32_t)(len / 32);
    d.c = reinterpret_cast<char*>(p.c) + (g * p.c_gstride + m0 * p.ldc + n0) * esz;
  }
  // every lane computed the same values: keep them in scalar registers
  d.a = uniform_ptr(d.a);
  d.sa = uniform_ptr(d.sa);
  d.b = uniform_ptr(d.b);
  d.sb = uniform_ptr(d.sb);
  d.c = (char*)uniform_ptr((const uint8_t*)d.c);
  d.nk = __builtin_amdgcn_readfirstlane(d.nk);
  d.nblk = __builtin_amdgcn_readfirstlane(d.nblk);
  d.valid_rows = __builtin_amdgcn_readfirstlane(d.valid_rows);
  return d;
}

template <bool KGROUPED, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes + 2 * kScaleBuf];
  __shared__ ExpertTable table;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t esz = OUT_BF16 ? 2 : 4;

  // the stage buffers serve as scan scratch before any copy is in flight
  build_table<KGROUPED>(p.m_splits, p.G, &table, reinterpret_cast<int64_t*>(smem));
  const int ntiles = __builtin_amdgcn_readfirstlane(KGROUPED ? p.ntiles : table.tpre[p.G] * p.ntiles_n);

  // per-lane DMA geometry: wave w copies rows [64 w, 64 w + 64) of the A and
  // B tiles, 16 rows (1 KB) per instruction: lane i -> row 16 j + i/4, LDS
  // chunk slot i%4, which holds global chunk (i%4) ^ ((row >> 1) & 3).  The
  // scale groups use the same rows, 16 rows x 16 bytes per instruction: lane
  // i -> row 16 j + i/4, bytes 4 (i%4) .. 4 (i%4) + 3 of the row's group.
  const int dr = lane >> 2;
  const int dchunk = (lane & 3) ^ ((dr >> 1) & 3);
  const int scol = (lane & 3) * 4;
  const int fr = lane & 31;   // operand row within a 32-row fragment
  const int fg = lane >> 5;   // contraction half of the lane

  uint32_t va[4], vb[4];
  const uint8_t *a_base, *b_base, *sa_base, *sb_base;
  int s_valid, s_nblk;
  auto setup = [&](const TileDesc& d) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wave * 64 + j * 16 + dr;
      const int ra = r < d.valid_rows ? r : 0;   // rows past the expert: any valid row
      va[j] = (uint32_t)(ra * p.lda + dchunk * 16);
      vb[j] = (uint32_t)(r * p.ldb + dchunk * 16);
    }
    a_base = uniform_ptr(d.a);
    b_base = uniform_ptr(d.b);
    sa_base = uniform_ptr(d.sa);
    sb_base = uniform_ptr(d.sb);
    s_valid = d.valid_rows;
    s_nblk = d.nblk;
  };
  // LDS byte addresses of the stage ring and of the scale buffers (the low
  // half of the generic address of an LDS object is its LDS address)
  const uint32_t lds_ring = (uint32_t)(uintptr_t)smem;
  const uint32_t lds_sc = lds_ring + kStages * kStageBytes;
  // Scale group `grp` (blocks [16 grp, 16 grp + 16) of every row) into buffer
  // grp % 2.  In a K-grouped tile the last group may run past the expert's
  // blocks (s_nblk, a multiple of 4): those lanes re-read the last valid word.
  // part j (0..3) of scale group grp: rows 64 w + 16 j .. + 16 of A and of B
  auto scale_part = [&](int grp, int j) {
    const uint32_t buf = lds_sc + (uint32_t)((grp & 1) * kScaleBuf);
    const int col = KGROUPED ? max(min(scol, s_nblk - 4 - 16 * grp), 0) : scol;
    const int r = wave * 64 + j * 16 + dr;
    const int ra = r < s_valid ? r : 0;
    dma4(sa_base + 16 * grp, (uint32_t)(ra * (int)p.ldsa + col),
         buf + (wave * 64 + j * 16) * kScaleRow);
    dma4(sb_base + 16 * grp, (uint32_t)(r * (int)p.ldsb + col),
         buf + kScOffB + (wave * 64 + j * 16) * kScaleRow);
  };
  // Copies of one stage: scalar source bases and LDS destination, formed
  // once per stage; part q (0..7) copies rows 64 w + 16 (q/2) .. + 16 of A
  // (q even) or B (q odd).
  struct StageCopy {
    const uint8_t* ak;
    const uint8_t* bk;
    uint32_t lds;
  };
  auto stage_copy = [&](int kt) {
    StageCopy c;
    c.ak = a_base + (int64_t)kt * BK;
    c.bk = b_base + (int64_t)kt * BK;
    c.lds = lds_ring + (uint32_t)((kt % kStages) * kStageBytes) + (uint32_t)(wave * 64 * BK);
    return c;
  };
  auto data_part = [&](const StageCopy& c, int q) {
    const int j = q >> 1;
    if ((q & 1) == 0)
      dma16(c.ak, va[j], c.lds + j * 16 * BK);
    else
      dma16(c.bk, vb[j], c.lds + kOffB + j * 16 * BK);
  };
  // a whole stage at once (first stages of a tile)
  auto issue = [&](int kt) {
    __builtin_amdgcn_sched_barrier(0);
    const StageCopy c = stage_copy(kt);
#pragma unroll
    for (int q = 0; q < 8; ++q) data_part(c, q);
    if (kt % kScaleSteps == 0)
#pragma unroll
      for (int j = 0; j < 4; ++j) scale_part(kt / kScaleSteps, j);
    __builtin_amdgcn_sched_barrier(0);
  };

  v16f acc[4][4];
  // fragments of two stages: set kt & 1 feeds the MFMAs of step kt while the
  // other set is filled from stage kt + 1
  v8i af[2][4], bf[2][4];
  int as[2][4], bs[2][4];
  // Per-lane LDS offsets of this wave's fragments inside a stage: row
  // wm WT + fr (A) or wn WT + fr (B), chunks g and 2 + g under the swizzle,
  // which for rows 32 i + fr depends on fr only; fragment i adds 32 rows =
  // 2048 bytes.  Scale bytes: row * 16 + 2 (kt % 8) + g.
  const int swzc = (fr >> 1) & 3;
  const uint32_t rA = (uint32_t)((wm * WT + fr) * BK + ((fg ^ swzc) << 4));
  const uint32_t rB = (uint32_t)(kOffB + (wn * WT + fr) * BK + ((fg ^ swzc) << 4));
  const uint32_t rX = (uint32_t)((((2 + fg) ^ swzc) - (fg ^ swzc)) << 4);   // +-32: chunk 2 + g
  const uint32_t rSA = (uint32_t)((wm * WT + fr) * kScaleRow + fg);
  const uint32_t rSB = (uint32_t)(kScOffB + (wn * WT + fr) * kScaleRow + fg);
  // this lane's LDS addresses of fragment 0 of stage kt (A chunk g, A chunk
  // 2 + g, B chunk g, B chunk 2 + g, A scale, B scale); fragment i adds an
  // immediate offset
  struct StageRead {
    uint32_t a0, a1, b0, b1, sa, sb;
  };
  auto stage_read = [&](int kt) {
    const uint32_t data = lds_ring + (uint32_t)((kt % kStages) * kStageBytes);
    const uint32_t scale = lds_sc + (uint32_t)(((kt / kScaleSteps) & 1) * kScaleBuf) +
                           (uint32_t)(2 * (kt % kScaleSteps));
    StageRead r;
    r.a0 = opaque(data + rA);
    r.a1 = opaque(r.a0 + rX);
    r.b0 = opaque(data + rB);
    r.b1 = opaque(r.b0 + rX);
    r.sa = opaque(scale + rSA);
    r.sb = opaque(scale + rSB);
    return r;
  };
  auto load_a = [&](const StageRead& r, int set, int i) {
    af[set][i] = lds_frag(r.a0 + i * 32 * BK, r.a1 + i * 32 * BK);
    as[set][i] = lds_byte(r.sa + i * 32 * kScaleRow);
  };
  auto load_b = [&](const StageRead& r, int set, int j) {
    bf[set][j] = lds_frag(r.b0 + j * 32 * BK, r.b1 + j * 32 * BK);
    bs[set][j] = lds_byte(r.sb + j * 32 * kScaleRow);
  };

  int tile = blockIdx.x;
  if (tile >= ntiles) return;
  TileDesc cur = describe<KGROUPED>(p, &table, tile, esz);
  setup(cur);
  for (int s = 0; s < kStages; ++s)
    if (s < cur.nk) issue(s);

  for (;;) {
    const int nk = cur.nk;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (nk > 0) {
      // stage 0 of this tile: its copies were issued before any later copy
      // or store of this wave, and at most 3 later stages follow them
      wait_stage(min(nk - 1, 3));
      __syncthreads();
      const StageRead r0 = stage_read(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        load_a(r0, 0, i);
        load_b(r0, 0, i);
      }
    }

    // D[m][n] = sum_k A[m,k] B[n,k]: srcA = A fragment, srcB = B fragment.
// The MFMA builtin has no side effects, so without the empty asm that takes
// its result the compiler may sink it past the uniform branches of the step
// (a scheduling barrier orders instructions only inside one basic block).
#define MX_MFMA(I, J, SET)                                                                  \
  acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                              \
      af[SET][I], bf[SET][J], acc[I][J], 0, 0, 0, as[SET][I], 0, bs[SET][J]);               \
  asm volatile("" : "+a"(acc[I][J]));                                                       \
  __builtin_amdgcn_sched_barrier(0);
#define MX_FENCE __builtin_amdgcn_sched_barrier(0);

    // One step (16 MFMAs per wave) on the fragments of stage kt, held in
    // registers (set SET) since the previous step.  The step opens with the
    // only barrier: before it this wave waits for its LDS reads of stage kt
    // and for its copies of stage kt+1; after it stage kt+1 is visible to
    // every wave and buffer kt % kStages is free.  The MFMAs then run with
    // one item of other work after each (with one wave per SIMD, anything
    // longer between two MFMAs idles the matrix pipe): the reads of stage
    // kt+1 into the other set, the 8 copies of stage kt+4 into the freed
    // buffer, and the scale group that starts at stage kt+4.
#define MX_STEP(KT, SET, FULL)                                                              \
  {                                                                                         \
    const int kt_ = (KT);                                                                   \
    const bool nx_ = (FULL) || kt_ + 1 < nk;                                                \
    const bool pf_ = (FULL) || kt_ + 4 < nk;                                                \
    const bool sg_ = pf_ && ((kt_ + 4) % kScaleSteps == 0);                                 \
    const int g_ = (kt_ + 4) / kScaleSteps;                                                 \
    __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0): this wave's reads of stage kt */    \
    if (nx_) {                                                                              \
      if (FULL)                                                                             \
        wait_stage(kStages - 2);                                                            \
      else                                                                                  \
        wait_stage(min(nk - 2 - kt_, kStages - 2));                                         \
      __syncthreads();                                                                      \
    }                                                                                       \
    const StageRead rd_ = stage_read(kt_ + 1);                                              \
    const StageCopy cp_ = stage_copy(kt_ + 4);                                              \
    MX_FENCE                                                                                \
    MX_MFMA(0, 0, SET) if (nx_) load_a(rd_, (SET) ^ 1, 0); MX_FENCE                         \
    MX_MFMA(0, 1, SET) if (pf_) data_part(cp_, 0); MX_FENCE                                 \
    MX_MFMA(0, 2, SET) if (nx_) load_b(rd_, (SET) ^ 1, 0); MX_FENCE                         \
    MX_MFMA(0, 3, SET) if (pf_) data_part(cp_, 1); MX_FENCE                                 \
    MX_MFMA(1, 0, SET) if (nx_) load_a(rd_, (SET) ^ 1, 1); MX_FENCE                         \
    MX_MFMA(1, 1, SET) if (pf_) data_part(cp_, 2); MX_FENCE                                 \
    MX_MFMA(1, 2, SET) if (nx_) load_b(rd_, (SET) ^ 1, 1); MX_FENCE                         \
    MX_MFMA(1, 3, SET) if (pf_) data_part(cp_, 3); MX_FENCE                                 \
    MX_MFMA(2, 0, SET) if (nx_) load_a(rd_, (SET) ^ 1, 2); MX_FENCE                         \
    MX_MFMA(2, 1, SET) if (pf_) data_part(cp_, 4); MX_FENCE                                 \
    MX_MFMA(2, 2, SET) if (nx_) load_b(rd_, (SET) ^ 1, 2); MX_FENCE                         \
    MX_MFMA(2, 3, SET) if (pf_) data_part(cp_, 5); MX_FENCE                                 \
    MX_MFMA(3, 0, SET) if (nx_) load_a(rd_, (SET) ^ 1, 3); if (pf_) data_part(cp_, 6);      \
    MX_FENCE                                                                                \
    MX_MFMA(3, 1, SET) if (nx_) load_b(rd_, (SET) ^ 1, 3); if (pf_) data_part(cp_, 7);      \
    MX_FENCE                                                                                \
    MX_MFMA(3, 2, SET) if (sg_) { scale_part(g_, 0); scale_part(g_, 1); } MX_FENCE          \
    MX_MFMA(3, 3, SET) if (sg_) { scale_part(g_, 2); scale_part(g_, 3); } MX_FENCE          \
  }

    // steady state (every step reads its successor and copies stage kt+4),
    // then the last 2 or 4 steps of the tile with those checks
    int kt = 0;
    for (; kt + 5 < nk; kt += 2) {
      MX_STEP(kt, 0, true)
      MX_STEP(kt + 1, 1, true)
    }
    for (; kt < nk; kt += 2) {
      MX_STEP(kt, 0, false)
      MX_STEP(kt + 1, 1, false)
    }
#undef MX_STEP
#undef MX_FENCE
#undef MX_MFMA

    // Next tile: once every wave has read the last stage (lgkmcnt(0) + the
    // barrier), all LDS buffers are free, so its first stages are copied
    // while this tile's results are stored.
    const int next = tile + gridDim.x;
    TileDesc nxt;
    nxt.nk = 0;
    if (next < ntiles) {
      nxt = describe<KGROUPED>(p, &table, next, esz);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __syncthreads();
      setup(nxt);
      for (int s = 0; s < kStages; ++s)
        if (s < nxt.nk) issue(s);
    }

    // ---- epilogue: accumulator r of acc[i][j] in lane l is C[m][n] with
    // m = wm WT + 32 i + 8 (r/4) + 4 (l/32) + r%4 and n = wn WT + 32 j + l%32,
    // so one store instruction per register writes 32 consecutive columns of
    // two rows: whole 128-byte lines for fp32 output.  The row part of the
    // address is wave-uniform (scalar base); the lane part is a 32-bit offset.
    // Global (not generic) stores: a generic store also counts on the LDS
    // wait counter, which the loop waits on for its fragment reads.
    {
      const int64_t ldc_b = p.ldc * esz;
      const int wm_u = __builtin_amdgcn_readfirstlane(wm);
      const uint32_t lane_off = (uint32_t)(4 * fg * ldc_b + (int64_t)(wn * WT + fr) * esz);
      const int vrows = cur.valid_rows;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm_u * WT + 32 * i + 8 * (r / 4) + (r % 4);
          if (vrows < BM && row + 4 * fg >= vrows) continue;
          char* rbase = cur.c + (int64_t)row * ldc_b + lane_off;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (OUT_BF16)
              *(__attribute__((address_space(1))) uint16_t*)(rbase + j * 32 * 2) =
                  (uint16_t)f32_to_bf16(acc[i][j][r]);
            else
              *(__attribute__((address_space(1))) float*)(rbase + j * 32 * 4) = acc[i][j][r];
          }
        }
      }
    }
    if (next >= ntiles) break;
    tile = next;
    cur = nxt;
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
  int64_t upper;
  if (!kgrouped) {
    // at most T / BM full row tiles plus one partial tile per expert
    upper = (T / BM + G) * p.ntiles_n;
  } else {
    p.band = (int32_t)(p.rows / BM);
    p.ntiles = G * p.band * p.ntiles_n;
    upper = p.ntiles;
  }
  // persistent grid: one workgroup per CU (the LDS ring allows one), each
  // walking the tiles with a stride of the grid size
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(upper, cus));
  if (kgrouped)
    return out_bf16 ? launch_one<true, true>(p, grid, st) : launch_one<true, false>(p, grid, st);
  return out_bf16 ? launch_one<false, true>(p, grid, st) : launch_one<false, false>(p, grid, st);
}

}  // namespace mx
