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
// Kernel structure (persistent: one workgroup per CU walks 256 x 256 output
// tiles; 4 waves of 128 x 128):
//  * MFMA: V_MFMA_SCALE_F32_32X32X64_F8F6F4, both operands E4M3.  Lane l
//    (row l % 32 of the operand, half g = l / 32) supplies the contraction
//    bytes [16g, 16g+16) and [32+16g, 32+16g+16) of a 64-byte step, and the
//    E8M0 scale of 32-element block g of its row.  Output: lane l holds
//    column l % 32, rows 8(r/4) + 4(l/32) + r%4 for accumulator r.
//  * The MFMA's first operand is the A tile and its second the B tile, so the
//    32 lanes of a half-wave hold 32 consecutive output columns of one row:
//    a store of one accumulator register writes whole cache lines.
//  * Operands go HBM/L2 -> LDS by LDS DMA (no register staging), one whole
//    128-byte line per row: an LDS stage holds 128 contraction bytes (two
//    MFMA steps) of the 256 A and 256 B rows, in two slots; E8M0 scales in
//    groups of 8 steps.
//  * The fragments of the next step are read into a second register set
//    while the current step's MFMAs run, one read per MFMA.  Odd steps open
//    with the only wait and barrier, then interleave the copies of the stage
//    two ahead with their MFMAs.
#include <type_traits>
#include <algorithm>

#include "mx_device.h"
#include "mx_tile_quant.h"
#include "kernels.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;        // output rows per workgroup tile
constexpr int BN = 256;        // output columns per workgroup tile
constexpr int BK = 128;        // contraction bytes per LDS stage: one 128-byte line per row
constexpr int KSTEP = 64;      // contraction bytes per MFMA step (two steps per stage)
constexpr int kSlots = 2;      // LDS stages
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
  int32_t split_tail;                  // M-grouped, fp32 out: split the last round's tiles
  int32_t* queue;                      // K-grouped: tile counter (dynamic order), or NULL
  // SwiGLU epilogue (forward with bf16 output only): C = h [T, 2F] holds gate
  // columns [0, F) and up columns [F, 2F); each tile pairs gate columns
  // [128 nt, 128 nt + 128) with the up columns F later, and the epilogue also
  // writes a = silu(gate) * up quantized row-wise ([T, F] + [T, F/32]) and/or
  // column-wise ([F, T] + [F, T/32]).
  int64_t f;
  uint8_t* q_row;
  uint8_t* s_row;
  uint8_t* q_col;
  uint8_t* s_col;
};

// LDS layout of one stage: A tile [BM][BK], B tile [BN][BK]; 16-byte chunk c
// of row r is stored at chunk position c ^ (r & 7).  The LDS has 32 banks of
// 4 bytes, so each 128-byte row is one bank line and the 8 consecutive rows of
// a fragment read that the LDS serves together use 8 distinct 16-byte bank
// groups.  Each row of a stage is one whole cache line of the operand: copies
// of half lines (64 contraction bytes per row and stage) fetch every line from
// memory twice and stall the copy path on the outstanding misses.
constexpr int kTileBytesA = BM * BK;
constexpr int kTileBytesB = BN * BK;
constexpr int kOffB = kTileBytesA;
constexpr int kStageBytes = kTileBytesA + kTileBytesB;
constexpr int kDmaHalf = 8;        // per wave and stage: 8 copies of A rows, then 8 of B rows
// E8M0 scales arrive in groups of kScaleSteps MFMA steps: 16 bytes (16 blocks
// of 32) per operand row, [BM][16] for A then [BN][16] for B, double-buffered.
// Copying a row's scale bytes one step at a time would cost one cache-line
// request per row per step for 2 bytes of data.
constexpr int kScaleSteps = 8;
constexpr int kScaleRow = 2 * kScaleSteps;   // bytes per row and group
constexpr int kScOffB = BM * kScaleRow;
constexpr int kScaleBuf = (BM + BN) * kScaleRow;

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
// The same for a scalar pointer stepped through a stage's copies: without it
// the compiler precomputes every step's address, one register pair each.
__device__ __forceinline__ const uint8_t* opaque_ptr(const uint8_t* q) {
  asm volatile("" : "+s"(q));
  return q;
}

// 4 x 4 transpose inside each quad of lanes: on entry lane q of the quad
// holds element (row r, column q) of a block in v_r; on exit lane q holds
// (row q, column r) in v_r.  Two exchange rounds (lanes q ^ 1, then q ^ 2),
// each swapping the off-diagonal 2 x 2 entries through a DPP quad permutation.
__device__ __forceinline__ float dpp_f(float v, int ctrl_xor) {
  const int ctrl = ctrl_xor == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  return __int_as_float(ctrl == 0xB1
      ? __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)
      : __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ void quad_transpose(float& v0, float& v1, float& v2, float& v3,
                                               bool odd, bool hi2) {
  float y = dpp_f(odd ? v0 : v1, 1);
  v0 = odd ? y : v0;
  v1 = odd ? v1 : y;
  y = dpp_f(odd ? v2 : v3, 1);
  v2 = odd ? y : v2;
  v3 = odd ? v3 : y;
  y = dpp_f(hi2 ? v0 : v2, 2);
  v0 = hi2 ? y : v0;
  v2 = hi2 ? v2 : y;
  y = dpp_f(hi2 ? v1 : v3, 2);
  v1 = hi2 ? y : v1;
  v3 = hi2 ? v3 : y;
}

// Two fp32 values -> a bf16 pair (round to nearest even; the first value in
// the low half): one V_CVT_PK_BF16_F32, the same bits as f32_to_bf16 for
// finite values.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// Expert table kept in LDS for the whole launch: exclusive prefix of tiles
// (forward/dgrad: ceil(M_g / BM) row tiles per expert) and of token rows, and
// (wgrad) the experts in decreasing order of tokens.
struct ExpertTable {
  int32_t tpre[kMaxGroups + 1];
  int64_t roff[kMaxGroups + 1];
  int16_t order[kMaxGroups];
  int32_t nempty;                      // K-grouped: experts without tokens
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
    if (tid == 0) t->nempty = 0;
    __syncthreads();
    int empties = 0;
    // rank = number of experts with more tokens (ties: lower index first)
    for (int g = tid; g < G; g += kThreads) {
      const int64_t mg = t->roff[g + 1] - t->roff[g];
      int rank = 0;
      for (int h = 0; h < G; ++h) {
        const int64_t mh = t->roff[h + 1] - t->roff[h];
        rank += (mh > mg) || (mh == mg && h < g);
      }
      t->order[rank] = (int16_t)g;
      empties += mg == 0;
    }
    if (empties) atomicAdd(&t->nempty, empties);
  }
  __syncthreads();
}

// One tile's operands.
struct TileDesc {
  const uint8_t* a;    // first copied A row of the tile at contraction 0
  const uint8_t* sa;
  const uint8_t* b;
  const uint8_t* sb;
  char* c;             // C at the first copied row, first column of the tile
  int32_t nk;          // MFMA steps (KSTEP contraction bytes each; always even)
  int32_t row_lo;      // tile rows [row_lo, row_hi) of the copied 256 belong to the tile
  int32_t row_hi;
  int32_t rows_avail;  // copied rows inside the operand (256, or T when T < 256)
  int32_t nblk;        // scale blocks of the tile's contraction (nk * 2)
  int32_t split;       // one contraction half of a split tile: add into C atomically
  int64_t m0c;         // M-grouped: first copied row (token) of the tile
  int32_t nt;          // M-grouped: column tile index
  int32_t g;           // M-grouped: the tile's expert
};

template <bool KGROUPED, bool SWIGLU = false>
__device__ __forceinline__ TileDesc describe(const GemmArgs& p, const ExpertTable* t, int tile,
                                             int64_t esz, int dynamic = 0, int g_lo = 0,
                                             int g_hi = -1) {
  TileDesc d;
  if (!KGROUPED) {
    const int mt = tile / p.ntiles_n, nt = tile % p.ntiles_n;
    // expert g: the last with tpre[g] <= mt (binary search over G + 1
    // entries, or over [g_lo, g_hi) where the caller knows that the expert
    // lies there: the tiles of a workgroup come in increasing order)
    int lo = g_lo, hi = g_hi < 0 ? p.G : g_hi;   // tpre[lo] <= mt < tpre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (t->tpre[mid] <= mt) lo = mid; else hi = mid;
    }
    const int g = lo;
    const int64_t m0 = t->roff[g] + (int64_t)(mt - t->tpre[g]) * BM;
    // SwiGLU: the tile's first B row (and C column) is gate column 128 nt;
    // its up half lies F rows (columns) further on (setup, epilogue)
    const int64_t n0 = (int64_t)nt * (SWIGLU ? BN / 2 : BN);
    const int64_t end = min(t->roff[g + 1], p.rows);   // never past the token count
    const int64_t valid = max(min((int64_t)BM, end - m0), (int64_t)0);
    // The 256 copied rows start at m0c: moved back from the tile's first row
    // m0 where the tile would run past the last token, so that every copy
    // stays inside the operand (T < 256 leaves T rows to copy).
    const int64_t m0c = min(m0, max(p.rows - BM, (int64_t)0));
    d.rows_avail = (int32_t)min((int64_t)BM, p.rows - m0c);
    d.row_lo = (int32_t)(m0 - m0c);
    d.row_hi = d.row_lo + (int32_t)valid;
    d.a = p.a + m0c * p.lda;
    d.sa = p.sa + m0c * p.ldsa;
    d.b = p.b + g * p.b_gstride + n0 * p.ldb;
    d.sb = p.sb + g * p.sb_gstride + n0 * p.ldsb;
    d.nk = valid > 0 ? (int32_t)(p.kc / KSTEP) : 0;
    d.nblk = (int32_t)(p.kc / 32);
    d.c = reinterpret_cast<char*>(p.c) + (m0c * p.ldc + n0) * esz;
    d.m0c = m0c;
    d.nt = nt;
    d.g = g;
  } else {
    // The list of tiles (experts in decreasing order of tokens) is consumed
    // from both ends at once: of the two workgroups of a pair (tiles 2q and
    // 2q + 1), one takes position q and the other position ntiles - 1 - q,
    // and they swap ends every round of the grid.  Every workgroup then
    // alternates a long tile with a short one, so the output stores of the
    // short tiles (few contraction steps, a whole 256 x 256 output) overlap
    // the other workgroups' contraction instead of all falling at the end.
    // Both tiles of a pair lie in the same round (g2 is even), so the map is
    // a bijection of [0, ntiles); with ntiles odd the last tile is the middle.
    // Dynamic order (a tile counter): the workgroups take the list in order
    // as they finish tiles, i.e. greedy longest-first placement.
    int pos = tile;
    if (!dynamic) {
      const int g2 = (int)((gridDim.x + 1) & ~1u);
      const int q = tile >> 1;
      const int from_back = (tile & 1) ^ ((tile / g2) & 1);
      pos = from_back ? p.ntiles - 1 - q : q;
    }
    const int per_expert = p.band * p.ntiles_n;
    const int g = t->order[pos / per_expert];
    const int rem = pos % per_expert;
    int mtl = rem / p.ntiles_n, nt = rem % p.ntiles_n;
    // Blocked dynamic order (dynamic == 2: the accumulating wgrad and the
    // bf16 wgrad): XCD x takes the positions congruent to x mod 8 (one
    // counter per XCD).  Where the tile grid splits into 4 x 2 blocks, those
    // positions of an expert map onto block x (a quarter of the row panels,
    // half the column panels) instead of two whole tile columns, so each dY
    // panel is read by two XCDs rather than all eight: accumulating wgrad
    // 1.60 -> 1.53 ms; the fp32 wgrad, whose output writes dominate, was 7 %
    // slower this way.  A bijection of the expert's tiles either way.
    if (dynamic == 2 && (p.band & 3) == 0 && (p.ntiles_n & 1) == 0) {
      const int x = rem & 7, k = rem >> 3;
      const int rows = p.band >> 2, cols = p.ntiles_n >> 1;
      mtl = (x >> 1) * rows + k / cols;
      nt = (x & 1) * cols + k % cols;
    }
    // p.kc = T here.  Runs are multiples of 128 tokens by contract; rounding
    // down keeps every copy inside [0, T) and aligned for any split values.
    const int64_t off = min(t->roff[g], p.kc) & ~(int64_t)127;
    const int64_t len = max(min(t->roff[g + 1], p.kc) - off, (int64_t)0) & ~(int64_t)127;
    const int64_t m0 = (int64_t)mtl * BM, n0 = (int64_t)nt * BN;
    d.row_lo = 0;
    d.row_hi = BM;
    d.rows_avail = BM;
    d.a = p.a + m0 * p.lda + off;
    d.sa = p.sa + m0 * p.ldsa + off / 32;
    d.b = p.b + n0 * p.ldb + off;
    d.sb = p.sb + n0 * p.ldsb + off / 32;
    d.nk = (int32_t)(len / KSTEP);
    d.nblk = (int32_t)(len / 32);
    d.c = reinterpret_cast<char*>(p.c) + (g * p.c_gstride + m0 * p.ldc + n0) * esz;
    d.g = 0;
  }
  // every lane computed the same values: keep them in scalar registers
  d.a = uniform_ptr(d.a);
  d.sa = uniform_ptr(d.sa);
  d.b = uniform_ptr(d.b);
  d.sb = uniform_ptr(d.sb);
  d.c = (char*)uniform_ptr((const uint8_t*)d.c);
  d.nk = __builtin_amdgcn_readfirstlane(d.nk);
  d.nblk = __builtin_amdgcn_readfirstlane(d.nblk);
  d.row_lo = __builtin_amdgcn_readfirstlane(d.row_lo);
  d.row_hi = __builtin_amdgcn_readfirstlane(d.row_hi);
  d.rows_avail = __builtin_amdgcn_readfirstlane(d.rows_avail);
  return d;
}

// Units of work of a launch.  Every unit is one tile, except in an M-grouped
// launch with fp32 output whose last round of the grid would hold at most half
// a grid of tiles: each of those `rem` tiles becomes two units, one per half
// of its contraction, so the last round runs 2 rem half-length units instead
// of rem whole tiles beside idle CUs (the dgrad of 8 experts 4096 -> 14336
// has 1040 tiles: four full rounds on 256 CUs and 16 tiles in a fifth).  Both
// halves add their partial products into C, zeroed beforehand by
// zero_split_tail_kernel: (0 + a) + b and (0 + b) + a are the same fp32 sum,
// so the result does not depend on which half lands first.
// The split saves half a tile (nk / 2 MFMA steps) and costs the zeroing
// launch and the atomic adds: measured about 32 steps plus 1.2 steps per split
// tile (dgrad above, 224 steps and 16 tiles: 0.955 -> 0.905 ms; the forward of
// the same workload, 64 steps and 56 tiles, was 7 % slower split), so a
// launch splits only where nk / 2 exceeds that.
struct UnitPlan {
  int32_t nunits;
  int32_t first_split;   // units from here on are contraction halves
  int32_t dynamic;       // K-grouped: tiles handed out through p.queue (2: blocked order)
  int32_t nq;            // counters: 8 (one per XCD) when the grid is a multiple of 8, else 1
};

// The dynamic wgrad order places long tiles well, but hands out the tiles of
// experts without tokens (stores of zeros only) all at the end, where they
// make a store-bound tail; the fixed two-ended order runs them beside the
// contraction.  Measured on the 128-expert workload with 38 empty experts the
// fixed order is 6 % faster, with 2 of 64 or none the counter is 2-22 %
// faster, so the counter is used when fewer than 1 expert in 8 is empty.
template <bool KGROUPED>
__device__ __forceinline__ UnitPlan plan_units(const GemmArgs& p, const ExpertTable* t,
                                               int ntiles, int grid) {
  UnitPlan u{ntiles, ntiles, 0, 1};
  if (KGROUPED) {
    u.dynamic = p.queue != nullptr && 8 * t->nempty < p.G;
    u.nq = grid % 8 == 0 ? 8 : 1;
    return u;
  }
  if (p.split_tail) {
    const int rem = ntiles % grid;
    const int nk = (int)(p.kc / KSTEP);
    if (rem > 0 && 2 * rem <= grid && 5 * nk > 320 + 12 * rem) {
      u.first_split = ntiles - rem;
      u.nunits = ntiles + rem;
    }
  }
  return u;
}

template <bool KGROUPED, bool SWIGLU = false>
__device__ __forceinline__ TileDesc describe_unit(const GemmArgs& p, const ExpertTable* t,
                                                  const UnitPlan& up, int unit, int64_t esz,
                                                  int g_lo = 0, int g_hi = -1) {
  if (KGROUPED || SWIGLU || unit < up.first_split) {
    TileDesc d = describe<KGROUPED, SWIGLU>(p, t, unit, esz, up.dynamic, g_lo, g_hi);
    d.split = 0;
    return d;
  }
  const int v = unit - up.first_split;
  const int half = v & 1;
  TileDesc d = describe<KGROUPED>(p, t, up.first_split + (v >> 1), esz, 0, g_lo, g_hi);
  // contraction bytes [half kc/2, (half + 1) kc/2) of the tile (kc % 1024 == 0:
  // each half is a whole number of stages and of 8-step scale groups)
  const int64_t hk = half * (p.kc / 2);
  d.a = uniform_ptr(d.a + hk);
  d.b = uniform_ptr(d.b + hk);
  d.sa = uniform_ptr(d.sa + hk / 32);
  d.sb = uniform_ptr(d.sb + hk / 32);
  d.nk >>= 1;
  d.nblk >>= 1;
  d.split = 1;
  return d;
}

// ACCUM (wgrad with fp32 output only): C += the product instead of C = it.
// SWIGLU (forward with bf16 output only): the SwiGLU + quantize epilogue
// (GemmArgs.f and the q/s outputs).
template <bool KGROUPED, bool OUT_BF16, bool ACCUM = false, bool SWIGLU = false>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs p) {
  static_assert(!SWIGLU || (!KGROUPED && OUT_BF16 && !ACCUM), "SwiGLU epilogue: forward, bf16");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSlots * kStageBytes + 2 * kScaleBuf];
  __shared__ ExpertTable table;
  __shared__ int32_t next_lds;          // dynamic order: a tile index, from thread 0
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t esz = OUT_BF16 ? 2 : 4;

  // the stage buffers serve as scan scratch before any copy is in flight
  build_table<KGROUPED>(p.m_splits, p.G, &table, reinterpret_cast<int64_t*>(smem));
  const int ntiles = __builtin_amdgcn_readfirstlane(KGROUPED ? p.ntiles : table.tpre[p.G] * p.ntiles_n);

  // Copy geometry: wave w copies rows [64 w, 64 w + 64) of the A and the B
  // tile, 8 rows x 128 bytes per instruction: lane i -> row 8 j + i/8, LDS
  // chunk position i%8, which holds the row's chunk (i%8) ^ (i/8).  The scale
  // groups use 16 rows x 16 bytes per instruction: lane i -> row 16 j + i/4,
  // bytes 4 (i%4) .. 4 (i%4) + 3 of the row's group.
  // Per-lane copy offsets: row i/8 of an 8-row part and its swizzled chunk;
  // rows of the part and of the wave go into the scalar base.  A wave whose
  // 64 rows would lie past the operand (T < 256) copies rows of the first
  // waves instead; their results are not stored.
  // Per-lane LDS offsets of this wave's fragments: row wm WT + fr (A) or
  // wn WT + fr (B), fr = lane % 32, g = lane / 32; for step half h the lane's
  // chunks are 4 h + g and 4 h + 2 + g, at positions p0 ^ 4h and p0 ^ 4h ^ 2
  // with p0 = g ^ (fr & 7) (fragment rows 32 i + fr share fr & 7); fragment
  // i adds 32 rows.
  // All of them are formed from the hardware lane id at every tile start
  // (volatile: not kept through the epilogue, where the accumulating wgrad
  // had no register left for them and spilled one; the reload's wait then
  // drained every copy once per stage).
  uint32_t ca, cb, rA, rB, rX, rH, rSA, rSB;
  auto lane_consts = [&]() {
    uint32_t ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int cr = (int)(ln >> 3), cchunk = (int)(ln & 7) ^ cr;
    ca = (uint32_t)(cr * p.lda + cchunk * 16);
    cb = (uint32_t)(cr * p.ldb + cchunk * 16);
    const int fr = (int)(ln & 31), fg = (int)(ln >> 5);
    const int p0 = fg ^ (fr & 7);
    rA = (uint32_t)((wm * WT + fr) * BK + p0 * 16);
    rB = (uint32_t)(kOffB + (wn * WT + fr) * BK + p0 * 16);
    rX = (uint32_t)(((p0 ^ 2) - p0) * 16);   // +-32: chunk 2 + g
    rH = (uint32_t)(((p0 ^ 4) - p0) * 16);   // +-64: second half of the stage
    rSA = (uint32_t)((wm * WT + fr) * kScaleRow + fg);
    rSB = (uint32_t)(kScOffB + (wn * WT + fr) * kScaleRow + fg);
  };
  const uint8_t *a_base, *b_base, *sa_base, *sb_base;
  int s_nblk;
  // LDS slot and scale-buffer parity of the current tile's stage 0 and scale
  // group 0: the copy ring runs on from one tile into the next
  int spar = 0, gpar = 0;
  auto setup = [&](const TileDesc& d) {
    const int64_t wrow = (int64_t)((wave * 64) % d.rows_avail);
    a_base = uniform_ptr(d.a + wrow * p.lda);
    sa_base = uniform_ptr(d.sa + wrow * p.ldsa);
    // SwiGLU: LDS B rows [64 w, 64 w + 64) hold the gate rows (w even) or the
    // up rows (w odd, F rows further on) of the tile's columns 64 (w / 2)..;
    // so the MFMA wave wn holds gate columns 64 wn.. in fragments 0, 1 and
    // the matching up columns in fragments 2, 3
    const int64_t brow = SWIGLU ? (int64_t)(wave & 1) * p.f + (int64_t)(wave >> 1) * 64
                                : (int64_t)wave * 64;
    b_base = uniform_ptr(d.b + brow * p.ldb);
    sb_base = uniform_ptr(d.sb + brow * p.ldsb);
    s_nblk = d.nblk;
  };
  // LDS byte addresses of the stages and of the scale buffers (the low half
  // of the generic address of an LDS object is its LDS address)
  const uint32_t lds_ring = (uint32_t)(uintptr_t)smem;
  const uint32_t lds_sc = lds_ring + kSlots * kStageBytes;
  // Part j (0..3) of scale group grp (blocks [16 grp, 16 grp + 16) of every
  // row, MFMA steps [8 grp, 8 grp + 8)) into buffer (grp + gp) % 2: rows
  // 64 w + 16 j .. + 16 of A and of B.  In a K-grouped tile the last group may
  // run past the expert's blocks (s_nblk, a multiple of 4): those lanes
  // re-read the last valid word.
  auto scale_part = [&](int grp, int j, int gp) {
    const uint32_t buf = lds_sc + (uint32_t)(((grp + gp) & 1) * kScaleBuf);
    // lane offsets formed here from the hardware lane id (volatile: not
    // kept as registers through the loop, where they were spilled)
    uint32_t ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int dr = (int)(ln >> 2), scol = (int)(ln & 3) * 4;
    const uint32_t col = (uint32_t)(KGROUPED ? max(min(scol, s_nblk - 4 - 16 * grp), 0) : scol);
    const uint32_t csa = (uint32_t)(dr * p.ldsa), csb = (uint32_t)(dr * p.ldsb);
    dma4(sa_base + (int64_t)j * 16 * p.ldsa + 16 * grp, csa + col,
         buf + (wave * 64 + j * 16) * kScaleRow);
    dma4(sb_base + (int64_t)j * 16 * p.ldsb + 16 * grp, csb + col,
         buf + kScOffB + (wave * 64 + j * 16) * kScaleRow);
  };
  // Copies of stage st (contraction bytes [128 st, 128 st + 128)) into LDS
  // slot (st + sp) % 2, part by part (rows 64 w + 8 j .. + 8, j = 0..7): a scalar
  // source pointer and LDS destination per operand, each advanced by one
  // part after its copy.
  struct StageCopy {
    const uint8_t* ak;
    const uint8_t* bk;
    uint32_t la, lb;
  };
  const int64_t a_part = 8 * p.lda, b_part = 8 * p.ldb;
  auto stage_copy = [&](int st, int sp) {
    StageCopy c;
    c.ak = a_base + (int64_t)st * BK;
    c.bk = b_base + (int64_t)st * BK;
    c.la = lds_ring + (uint32_t)(((st + sp) % kSlots) * kStageBytes) + (uint32_t)(wave * 64 * BK);
    c.lb = c.la + kOffB;
    return c;
  };
  auto copy_a = [&](StageCopy& c) {
    dma16(c.ak, ca, c.la);
    c.ak = opaque_ptr(c.ak + a_part);
    c.la += 8 * BK;
  };
  auto copy_b = [&](StageCopy& c) {
    dma16(c.bk, cb, c.lb);
    c.bk = opaque_ptr(c.bk + b_part);
    c.lb += 8 * BK;
  };

  v16f acc[4][4];
  // fragments of two MFMA steps: set kt & 1 feeds the MFMAs of step kt while
  // the other set is filled for step kt + 1
  v8i af[2][4], bf[2][4];
  int as[2][4], bs[2][4];
  // this lane's LDS addresses of fragment 0 of MFMA step kt (A chunk g, A
  // chunk 2 + g, B chunk g, B chunk 2 + g, A scale, B scale)
  struct StepRead {
    uint32_t a0, a1, b0, b1, sa, sb;
  };
  auto step_read = [&](int kt) {
    const uint32_t data = lds_ring + (uint32_t)((((kt >> 1) + spar) % kSlots) * kStageBytes) +
                          ((kt & 1) ? rH : 0u);
    const uint32_t scale = lds_sc + (uint32_t)((((kt / kScaleSteps) + gpar) & 1) * kScaleBuf) +
                           (uint32_t)(2 * (kt % kScaleSteps));
    StepRead r;
    r.a0 = opaque(data + rA);
    r.a1 = opaque(r.a0 + rX);
    r.b0 = opaque(data + rB);
    r.b1 = opaque(r.b0 + rX);
    r.sa = opaque(scale + rSA);
    r.sb = opaque(scale + rSB);
    return r;
  };
  auto load_a = [&](const StepRead& r, int set, int i) {
    af[set][i] = lds_frag(r.a0 + i * 32 * BK, r.a1 + i * 32 * BK);
    as[set][i] = lds_byte(r.sa + i * 32 * kScaleRow);
  };
  auto load_b = [&](const StepRead& r, int set, int j) {
    bf[set][j] = lds_frag(r.b0 + j * 32 * BK, r.b1 + j * 32 * BK);
    bs[set][j] = lds_byte(r.sb + j * 32 * kScaleRow);
  };
  // First copies of a tile: stages 0 (with scale group 0) and 1, into slots
  // sp, sp ^ 1 and scale buffer gp.
  auto tile_prologue = [&](int nk, int sp, int gp) {
    __builtin_amdgcn_sched_barrier(0);
    if (nk > 0) {
      StageCopy c0 = stage_copy(0, sp);
#pragma unroll
      for (int j = 0; j < kDmaHalf; ++j) {
        copy_a(c0);
        copy_b(c0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) scale_part(0, j, gp);
    }
    if (nk > 2) {
      StageCopy c1 = stage_copy(1, sp);
#pragma unroll
      for (int j = 0; j < kDmaHalf; ++j) {
        copy_a(c1);
        copy_b(c1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  UnitPlan up = plan_units<KGROUPED>(p, &table, ntiles, (int)gridDim.x);
  // blocked order (describe): the accumulating wgrad, and the bf16 wgrad
  // (fused MLP, 64 experts: FC2 wgrad 0.401 -> 0.389 ms, FC1 0.602 -> 0.592)
  if ((ACCUM || (KGROUPED && OUT_BF16)) && up.dynamic) up.dynamic = 2;
  int tile = blockIdx.x;   // unit index (a tile, or half of one: describe_unit)
  if (tile >= up.nunits) return;
  // Dynamic order (wgrad with a tile counter): the next tile must be known
  // before the current tile's last two stages, which carry its first copies.
  // Thread 0 takes the successor of the next tile from the counter at the
  // end of the current tile's contraction (and the first successor here);
  // the index reaches every wave through LDS at the next tile's start.  The
  // counters start past the workgroups' first tiles (their own indices,
  // queue_init_kernel); an index past the last tile ends the loop, so every
  // workgroup stops after finitely many tiles.  Global (not generic)
  // atomics: a generic one would also count on the LDS counter the loop
  // waits on.  With a grid that is a multiple of 8 there is one counter per
  // XCD (workgroup b runs on XCD b % 8): XCD x takes list positions x, x + 8,
  // ..., so the workgroups sharing its L2 work on neighbouring tiles of the
  // same experts (one global counter scattered them over the XCDs and raised
  // the fetched bytes by half).
  int fetched = 0;
  if (KGROUPED && up.dynamic && tid == 0)
    fetched = __hip_atomic_fetch_add(
        (__attribute__((address_space(1))) int32_t*)p.queue + (blockIdx.x & (up.nq - 1)), 1,
        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int cur_nk;   // contraction steps of the current tile
  int cur_g = 0;   // M-grouped: its expert (the next tile's lies at or after it)
  lane_consts();
  {
    const TileDesc d = describe_unit<KGROUPED, SWIGLU>(p, &table, up, tile, esz);
    setup(d);
    tile_prologue(d.nk, 0, 0);
    cur_nk = d.nk;
    cur_g = d.g;
  }
  // A tile's first wait leaves 63 vector-memory operations outstanding.  It
  // sees stages 0 and 1 land when at least 63 operations were issued after
  // them (the previous tile's stores: the counter completes in issue order),
  // and up to 63 of those stores then drain behind the first MFMA step; a
  // wait for stage 0 alone drained nearly every store before the first MFMA.
  // Where fewer operations follow them (the first tile, and after a tile
  // whose epilogue stores fewer), a full wait right after the copies or the
  // stores stands in.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  for (;;) {
    const int nk = cur_nk;
    lane_consts();
    const int ns = nk >> 1;   // stages
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (nk > 0) {
      // stages 0 and 1 landed (the wait before the tile loop explains 63)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(63));
      // dynamic order: thread 0 hands on the index it took at the end of the
      // previous tile's contraction; the previous tile's epilogue memory
      // operations (at least 64) or a full wait lie between, so this wait
      // covers the atomic too, and the barrier publishes the value
      if (KGROUPED && up.dynamic && tid == 0) next_lds = fetched;
      __syncthreads();
      // step 0 through an opaque index: with constant offsets its addresses
      // would be precomputed once and spilled, and the reload's wait counts
      // every copy and store in flight
      const StepRead r0 = step_read((int)opaque(0u));
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

    // Two MFMA steps per stage st, 16 MFMAs per wave each, every MFMA
    // followed by at most one fragment read and a copy or two (with one wave
    // per SIMD, more between two MFMAs idles the matrix pipe).  The 16 copies
    // of stage st + 2 go into slot st % 2 as soon as every wave has read it,
    // spread over a step and a half, so the copy path is never flooded by all
    // of them within one step (3-7 % faster than issuing all 16 in the odd
    // step).
    // Even step 2 st: MFMAs on set 0 (step 2 st); reads of step 2 st + 1
    // (second half of stage st) into set 1 after the first 8 MFMAs; then this
    // wave's reads are waited for and the barrier frees slot st % 2 (no wave
    // reads stage st after it); 6 copies of stage st + 2 into it.
    // Odd step 2 st + 1: this wave waits for its copies of stage st + 1 (only
    // the 6 just issued may still be in flight: the counter completes in issue
    // order), then the barrier makes stage st + 1 visible; MFMAs on set 1;
    // reads of step 2 st + 2 (stage st + 1) into set 0; the other 10 copies
    // of stage st + 2 and the scale group that starts there.  Every copy of
    // stage st + 2 has at least the whole even step 2 st + 2 to land before
    // the wait of odd step 2 st + 3.
#define MX_EVEN(ST, PF, CP)                                                                 \
  {                                                                                         \
    const int st_ = (ST);                                                                   \
    const bool pf_ = (PF);                                                                  \
    const StepRead rd_ = step_read(2 * st_ + 1);                                            \
    MX_FENCE                                                                                \
    MX_MFMA(0, 0, 0) load_a(rd_, 1, 0); MX_FENCE                                            \
    MX_MFMA(0, 1, 0) load_b(rd_, 1, 0); MX_FENCE                                            \
    MX_MFMA(0, 2, 0) load_a(rd_, 1, 1); MX_FENCE                                            \
    MX_MFMA(0, 3, 0) load_b(rd_, 1, 1); MX_FENCE                                            \
    MX_MFMA(1, 0, 0) load_a(rd_, 1, 2); MX_FENCE                                            \
    MX_MFMA(1, 1, 0) load_b(rd_, 1, 2); MX_FENCE                                            \
    MX_MFMA(1, 2, 0) load_a(rd_, 1, 3); MX_FENCE                                            \
    MX_MFMA(1, 3, 0) load_b(rd_, 1, 3); MX_FENCE                                            \
    MX_MFMA(2, 0, 0)                                                                        \
    if (pf_) {                                                                              \
      __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0): this wave's reads of stage st */  \
      __syncthreads();                    /* stage st's slot is free */                     \
    }                                                                                       \
    MX_FENCE                                                                                \
    MX_MFMA(2, 1, 0) if (pf_) copy_a(CP); MX_FENCE                                          \
    MX_MFMA(2, 2, 0) if (pf_) copy_b(CP); MX_FENCE                                          \
    MX_MFMA(2, 3, 0) MX_FENCE                                                               \
    MX_MFMA(3, 0, 0) if (pf_) copy_a(CP); MX_FENCE                                          \
    MX_MFMA(3, 1, 0) if (pf_) copy_b(CP); MX_FENCE                                          \
    MX_MFMA(3, 2, 0) MX_FENCE                                                               \
    MX_MFMA(3, 3, 0) if (pf_) copy_a(CP); if (pf_) copy_b(CP); MX_FENCE                     \
  }
#define MX_ODD(ST, NX, PF, SG, G, GP, CP)                                                   \
  {                                                                                         \
    const int st_ = (ST);                                                                   \
    const bool nx_ = (NX);                                                                  \
    const bool pf_ = (PF);                                                                  \
    const bool sg_ = (SG);                                                                  \
    const int g_ = (G);                                                                     \
    if (nx_) {                                                                              \
      /* stage st + 1 landed; only the 6 copies of stage st + 2 may be pending */          \
      if (pf_) __builtin_amdgcn_s_waitcnt(vmcnt_imm(6));                                    \
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));                                        \
      __syncthreads();                                                                      \
    }                                                                                       \
    const StepRead rd_ = step_read(2 * st_ + 2);                                            \
    MX_FENCE                                                                                \
    MX_MFMA(0, 0, 1) if (nx_) load_a(rd_, 0, 0); if (pf_) copy_a(CP); MX_FENCE              \
    MX_MFMA(0, 1, 1) if (pf_) copy_b(CP); MX_FENCE                                          \
    MX_MFMA(0, 2, 1) if (nx_) load_b(rd_, 0, 0); MX_FENCE                                   \
    MX_MFMA(0, 3, 1) if (pf_) copy_a(CP); MX_FENCE                                          \
    MX_MFMA(1, 0, 1) if (nx_) load_a(rd_, 0, 1); if (pf_) copy_b(CP); MX_FENCE              \
    MX_MFMA(1, 1, 1) MX_FENCE                                                               \
    MX_MFMA(1, 2, 1) if (nx_) load_b(rd_, 0, 1); if (pf_) copy_a(CP); MX_FENCE              \
    MX_MFMA(1, 3, 1) if (pf_) copy_b(CP); MX_FENCE                                          \
    MX_MFMA(2, 0, 1) if (nx_) load_a(rd_, 0, 2); MX_FENCE                                   \
    MX_MFMA(2, 1, 1) if (pf_) copy_a(CP); MX_FENCE                                          \
    MX_MFMA(2, 2, 1) if (nx_) load_b(rd_, 0, 2); if (pf_) copy_b(CP); MX_FENCE              \
    MX_MFMA(2, 3, 1) MX_FENCE                                                               \
    MX_MFMA(3, 0, 1) if (nx_) load_a(rd_, 0, 3); if (pf_) copy_a(CP);                       \
    if (sg_) scale_part(g_, 0, GP); MX_FENCE                                                \
    MX_MFMA(3, 1, 1) if (pf_) copy_b(CP); if (sg_) scale_part(g_, 1, GP); MX_FENCE          \
    MX_MFMA(3, 2, 1) if (nx_) load_b(rd_, 0, 3); if (sg_) scale_part(g_, 2, GP); MX_FENCE   \
    MX_MFMA(3, 3, 1) if (sg_) scale_part(g_, 3, GP); MX_FENCE                               \
  }

    // steady state (every stage has a successor two ahead)
    int st = 0;
    for (; st + 2 < ns; ++st) {
      StageCopy cp = stage_copy(st + 2, spar);
      MX_EVEN(st, true, cp)
      MX_ODD(st, true, true, ((st + 2) * 2) % kScaleSteps == 0, ((st + 2) * 2) / kScaleSteps,
             gpar, cp)
    }
    // The next tile.  Where both tiles have at least two stages, the copy
    // ring runs on into it: the last two stages of this tile carry the copies
    // of its stages 0 and 1 (and its scale group 0) in the slots and at the
    // places of the steady state, so they land under this tile's MFMAs
    // instead of being issued between the tiles (the set-up between two
    // tiles took 2-15 % of the tile time, mostly the issue of those copies).
    // Its stage 0 takes the slot after this tile's last stage, its scale
    // group 0 the buffer that this tile's last group does not use (free: the
    // group before that one was last read in the even step of stage ns - 2,
    // before its barrier).
    // (Only the next tile's step count is kept through the last stages; the
    // rest of its description is recomputed where the ring does not run on:
    // kept, it raised the register pressure enough to spill inside the loop.)
    int next = tile + (int)gridDim.x;
    if (KGROUPED && up.dynamic) {
      if (nk == 0) {   // no first wait and barrier above
        if (tid == 0) next_lds = fetched;
        __syncthreads();
      }
      next = __builtin_amdgcn_readfirstlane(next_lds) * up.nq + (int)(blockIdx.x & (up.nq - 1));
    }
    const bool has_next = next < up.nunits;
    int nk_next = 0, g_next = 0;
    if (has_next) {
      const TileDesc d = describe_unit<KGROUPED, SWIGLU>(p, &table, up, next, esz, cur_g);
      nk_next = d.nk;
      g_next = d.g;
      // this tile issues no more copies of its own: where the ring runs on,
      // its copy bases become the next tile's
      if (ns >= 2 && d.nk >= 4) setup(d);
    }
    const bool chain = has_next && ns >= 2 && nk_next >= 4;
    const int spar_n = (spar + ns) & 1;
    const int gpar_n = (gpar + (nk > 0 ? (nk - 1) / kScaleSteps : 0) + 1) & 1;
    for (; st < ns; ++st) {
      StageCopy cp = stage_copy(st + 2 - ns, spar_n);
      MX_EVEN(st, chain, cp)
      MX_ODD(st, st + 1 < ns, chain, chain && st + 2 == ns, 0, gpar_n, cp)
    }
#undef MX_EVEN
#undef MX_ODD
#undef MX_FENCE
#undef MX_MFMA
    // dynamic order: the successor of the next tile (see above)
    if (KGROUPED && up.dynamic && has_next && tid == 0)
      fetched = __hip_atomic_fetch_add(
          (__attribute__((address_space(1))) int32_t*)p.queue + (blockIdx.x & (up.nq - 1)), 1,
          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (has_next && !chain) {
      // Once every wave has read the last stage (lgkmcnt(0) + the barrier),
      // both LDS slots and both scale buffers are free: the next tile's first
      // stages are copied while this tile's results are stored.
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __syncthreads();
      const TileDesc d = describe_unit<KGROUPED, SWIGLU>(p, &table, up, next, esz, g_next,
                                                         g_next + 1);
      setup(d);
      tile_prologue(d.nk, spar_n, gpar_n);
    } else if (SWIGLU) {
      // the SwiGLU epilogue's LDS scratch: the scale buffer of this tile's
      // last group, free once every wave has read it
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __syncthreads();
    }

    // The epilogue's tile bounds and output base are recomputed from the
    // expert table (LDS) rather than kept from the tile start: held across
    // the K loop they are spilled, and the reload's wait on the vector memory
    // counter would also wait for the next tile's copies issued above.
    const TileDesc ed = describe_unit<KGROUPED, SWIGLU>(p, &table, up, tile, esz, cur_g,
                                                        cur_g + 1);

    // ---- epilogue: accumulator r of acc[i][j] in lane l is C[m][n] with
    // m = wm WT + 32 i + 8 (r/4) + 4 (l/32) + r%4 and n = wn WT + 32 j + l%32.
    // The row part of each store address is wave-uniform (scalar base), the
    // lane part a 32-bit offset.  Global (not generic) stores: a generic store
    // also counts on the LDS wait counter, which the loop waits on for its
    // fragment reads.  Non-temporal: the output is written once and not read
    // again here, and kept out of L2 it leaves room for the operand panels
    // the other workgroups on the XCD are still reading (2 % faster forward
    // and wgrad; the accumulating wgrad's old values are read the same way).
    // Forward, dgrad and the plain wgrad: one store instruction per register
    // writes 32 consecutive columns of two rows, whole 128-byte lines for
    // fp32 output (K-grouped, C is [G][N][K] and the tile's rows are N
    // rows).  With the scalar-base address form this beats the 16-byte
    // transposed form of the accumulating wgrad below, whose DPP transposes
    // cost more than the store instructions they save (wgrad 5 % faster,
    // the fused MLP's bf16 FC1 wgrad 17 %).
    // (SwiGLU: the h block is stored like any bf16 output first.)
    if (!KGROUPED || !ACCUM) {
      const int64_t ldc_b = p.ldc * esz;
      const int wm_u = __builtin_amdgcn_readfirstlane(wm);
      // SwiGLU: the wave's gate columns start 64 wn into the tile; its up
      // columns (fragments 2, 3) lie F further on
      const int64_t wcol = SWIGLU ? 64 * wn : wn * WT;
      // the lane's part of the store address, formed here from the hardware
      // lane id (volatile: not hoisted and kept through the K loop) as a
      // 32-bit offset to a scalar row base: the scalar-base store form, with
      // no 64-bit vector address arithmetic per row (forward 3 % faster)
      uint32_t ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const uint32_t lane_off =
          (ln >> 5) * 4u * (uint32_t)ldc_b + ((uint32_t)wcol + (ln & 31)) * (uint32_t)esz;
      const int lo = ed.row_lo, hi = ed.row_hi;
      const bool part = lo > 0 || hi < BM;
      // a contraction half of a split tile adds into C (branch outside the
      // store loop, which stays as it is for whole tiles)
      if (!OUT_BF16 && ed.split) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wm_u * WT + 32 * i + 8 * (r / 4) + (r % 4);
            if (part && (row < lo || row >= hi)) continue;
            char* rbase =
                (char*)uniform_ptr((const uint8_t*)(ed.c + (int64_t)row * ldc_b)) + lane_off;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              (void)__builtin_amdgcn_global_atomic_fadd_f32(
                  (__attribute__((address_space(1))) float*)(rbase + j * 32 * 4), acc[i][j][r]);
          }
        }
      } else {
        // whole tiles take a loop without the row check (a tile's rows are
        // all stored unless it is a tail tile, part); the check is uniform:
        // rows R and R + 4 of one store lie in one 8-row group, and row_lo
        // and row_hi are multiples of 128
        // bf16 with the SwiGLU epilogue: registers r and r + 1 (rows R and
        // R + 1 of one column) are converted together, as the SwiGLU below
        // converts them (the compiler shares the conversions), and lanes l
        // and l ^ 1 (neighbouring columns) swap the pair: the even lane keeps
        // row R of columns n, n + 1, the odd lane row R + 1 of columns n - 1,
        // n, so one 32-bit store per two registers writes four 64-byte row
        // pieces (FC1 + SwiGLU 5 % faster).  Other bf16 outputs keep two
        // 2-byte stores per conversion: they write as many 64-byte pieces in
        // all, and there the swap's extra VALU cost 2-7 % (so did a swap that
        // makes each store a whole 128-byte line per row: 0 to +4 %).
        const bool odd_l = (ln & 1) != 0;
        const uint32_t bsel = odd_l ? 0x03020706u : 0x05040100u;
        const uint32_t lane_off_b = lane_off + (odd_l ? (uint32_t)ldc_b - 2u : 0u);
        auto store_rows = [&](auto check) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (OUT_BF16 && SWIGLU) {
#pragma unroll
              for (int r = 0; r < 16; r += 2) {
                const int row = wm_u * WT + 32 * i + 8 * (r / 4) + (r % 4);
                if (decltype(check)::value && (row < lo || row >= hi)) continue;
                char* rbase =
                    (char*)uniform_ptr((const uint8_t*)(ed.c + (int64_t)row * ldc_b)) + lane_off_b;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const uint32_t pk = pack_bf16x2(acc[i][j][r], acc[i][j][r + 1]);
                  const uint32_t sw = (uint32_t)__builtin_amdgcn_mov_dpp((int)pk, 0xB1, 0xF, 0xF, true);
                  const int64_t jo = j >= 2 ? 2 * p.f + (j - 2) * 64 : j * 64;
                  __builtin_nontemporal_store(
                      __builtin_amdgcn_perm(sw, pk, bsel),
                      (__attribute__((address_space(1))) uint32_t*)(rbase + jo));
                }
              }
            } else if (OUT_BF16) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = wm_u * WT + 32 * i + 8 * (r / 4) + (r % 4);
                if (decltype(check)::value && (row < lo || row >= hi)) continue;
                char* rbase =
                    (char*)uniform_ptr((const uint8_t*)(ed.c + (int64_t)row * ldc_b)) + lane_off;
                // two columns 32 apart per conversion (one V_CVT_PK_BF16_F32)
#pragma unroll
                for (int j = 0; j < 4; j += 2) {
                  const uint32_t pk = pack_bf16x2(acc[i][j][r], acc[i][j + 1][r]);
                  __builtin_nontemporal_store(
                      (uint16_t)pk, (__attribute__((address_space(1))) uint16_t*)(rbase + j * 64));
                  __builtin_nontemporal_store(
                      (uint16_t)(pk >> 16),
                      (__attribute__((address_space(1))) uint16_t*)(rbase + j * 64 + 64));
                }
              }
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = wm_u * WT + 32 * i + 8 * (r / 4) + (r % 4);
                if (decltype(check)::value && (row < lo || row >= hi)) continue;
                char* rbase =
                    (char*)uniform_ptr((const uint8_t*)(ed.c + (int64_t)row * ldc_b)) + lane_off;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  __builtin_nontemporal_store(
                      acc[i][j][r], (__attribute__((address_space(1))) float*)(rbase + j * 128));
              }
            }
          }
        };
        // (one loop for the SwiGLU kernel, whose epilogue is long enough)
        if (SWIGLU || part) store_rows(std::true_type{});
        else store_rows(std::false_type{});
      }
      if (SWIGLU && (p.q_row != nullptr || p.q_col != nullptr) && 128 * wm_u >= lo &&
          128 * wm_u + 128 <= hi) {
        // SwiGLU + quantize from registers.  Fragments (i, jj) and (i, jj + 2)
        // hold gate and up for the same 32 x 32 block (rows 32 i.. of the
        // wave's 128, columns 64 wn + 32 jj.. of the tile's gate columns):
        // a = silu(gate) * up as swiglu_pair forms it from the bf16-rounded
        // h.  Column-wise: lane l holds rows 8 g + 4 (l / 32) + (0..3) of
        // column l % 32 (g = r / 4), so a 32-token block is 16 registers of
        // lanes l and l ^ 32; after two words change hands each lane stores 16
        // consecutive tokens.  Row-wise: a DPP transpose inside each quad
        // gives lane q four consecutive columns of row 8 b + 4 (l / 32) + q;
        // the row's 32-column block is the eight quads of the half-wave.
        // The encode is the streaming kernels' (scaled conversion of bf16
        // pairs with the block's E8M0 byte, saturated), so the bytes equal
        // mxfp8_swiglu_quantize of the h written above.
        const int64_t F = p.f, T = p.rows;
        const uint32_t half = ln >> 5, c = ln & 31;
        const int64_t fc0 = (int64_t)ed.nt * 128 + 64 * wn;   // the wave's first a column
        const int64_t tok0 = ed.m0c + 128 * wm_u;              // the wave's first token
        // per-lane parts of the addresses (32-bit)
        const uint32_t col_l = c * (uint32_t)T + 16 * half;
        const uint32_t scol_l = c * (uint32_t)(T / 32);
        const uint32_t row_l = (ln >> 1) * (uint32_t)F + 16 * (ln & 1);
        const uint32_t srow_l = (ln >> 1) * (uint32_t)(F / 32);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          uint32_t sbytes = 0;   // column-wise scale bytes of blocks i = 0..3
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // gate and up rounded to bf16 as the h stores round them (two
            // values per V_CVT_PK_BF16_F32), a rounded as swiglu_pair rounds it
            uint32_t a[16];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              const uint32_t gp = pack_bf16x2(acc[i][jj][r], acc[i][jj][r + 1]);
              const uint32_t up = pack_bf16x2(acc[i][jj + 2][r], acc[i][jj + 2][r + 1]);
              a[r] = f32_to_bf16(silu_f(__uint_as_float(gp << 16)) * __uint_as_float(up << 16));
              a[r + 1] = f32_to_bf16(silu_f(__uint_as_float(gp & 0xFFFF0000u)) *
                                     __uint_as_float(up & 0xFFFF0000u));
            }
            if (p.q_col != nullptr) {
              uint32_t m = 0;
#pragma unroll
              for (int r = 0; r < 16; ++r) m = max(m, a[r] & 0x7FFFu);
              {
                // lanes l and l ^ 32 through V_PERMLANE32_SWAP (lanes 32..63
                // of the first operand trade with lanes 0..31 of the second)
                const auto sw = __builtin_amdgcn_permlane32_swap(m, m, false, false);
                m = max(m, half ? (uint32_t)sw[0] : (uint32_t)sw[1]);
              }
              const uint32_t xb = scale_byte_from_exp(m >> 7);
              const float sc = e8m0_operand(xb);
              uint32_t w[4];
#pragma unroll
              for (int g = 0; g < 4; ++g)
                w[g] = cvt4_bf16_e4m3(a[4 * g] | (a[4 * g + 1] << 16),
                                      a[4 * g + 2] | (a[4 * g + 3] << 16), sc);
              // w[g]: tokens 8 g + 4 half .. + 3; lanes l and l ^ 32 trade two
              // words so that lane l holds tokens 0..15 and lane l ^ 32 16..31
              // one swap each: lane l < 32 receives the partner's w[0] / w[1],
              // lane l + 32 the partner's w[2] / w[3]
              const auto s0 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
              const auto s1 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
              const uint32_t y0 = half ? (uint32_t)s0[0] : (uint32_t)s0[1];
              const uint32_t y1 = half ? (uint32_t)s1[0] : (uint32_t)s1[1];
              const u32x4 o = half ? u32x4{y0, w[2], y1, w[3]} : u32x4{w[0], y0, w[1], y1};
              uint8_t* qb = (uint8_t*)uniform_ptr(p.q_col + (fc0 + 32 * jj) * T + tok0 + 32 * i);
              *(__attribute__((address_space(1))) u32x4*)(qb + col_l) = o;
              sbytes |= xb << (8 * i);
            }
            if (p.q_row != nullptr) {
              // row-wise through this wave's 2 KiB of the scale buffer that
              // the next tile's scale group 0 does not use (free until its K
              // loop loads group 1 there): the
              // 32 x 32 block row-major, then lane l reads half l % 2 of row
              // l / 2 (16 values of one row: one scale, 16 codes, one store)
              uint16_t* xw = reinterpret_cast<uint16_t*>(
                  smem + kSlots * kStageBytes + ((gpar_n + 1) & 1) * kScaleBuf + 2048 * wave);
#pragma unroll
              for (int r = 0; r < 16; ++r)
                xw[(8 * (r / 4) + 4 * half + (r % 4)) * 32 + c] = (uint16_t)a[r];
              const u32x4* xr = reinterpret_cast<const u32x4*>(xw + (ln >> 1) * 32 + 16 * (ln & 1));
              const u32x4 v0 = xr[0], v1 = xr[1];
              const uint32_t k7 = 0x7FFF7FFFu;
              uint32_t m2 = max_u16x2(max_u16x2(max_u16x2(v0.x & k7, v0.y & k7),
                                                max_u16x2(v0.z & k7, v0.w & k7)),
                                      max_u16x2(max_u16x2(v1.x & k7, v1.y & k7),
                                                max_u16x2(v1.z & k7, v1.w & k7)));
              uint32_t m = max(m2 & 0xFFFFu, m2 >> 16);
              m = max(m, lane_xor1(m));
              const uint32_t xb = scale_byte_from_exp(m >> 7);
              const float sc = e8m0_operand(xb);
              const u32x4 code = u32x4{cvt4_bf16_e4m3(v0.x, v0.y, sc), cvt4_bf16_e4m3(v0.z, v0.w, sc),
                                       cvt4_bf16_e4m3(v1.x, v1.y, sc), cvt4_bf16_e4m3(v1.z, v1.w, sc)};
              uint8_t* qb = (uint8_t*)uniform_ptr(p.q_row + (tok0 + 32 * i) * F + fc0 + 32 * jj);
              *(__attribute__((address_space(1))) u32x4*)(qb + row_l) = code;
              if ((ln & 1) == 0) {
                uint8_t* sb = (uint8_t*)uniform_ptr(p.s_row + (tok0 + 32 * i) * (F / 32) +
                                                    (fc0 + 32 * jj) / 32);
                *(__attribute__((address_space(1))) uint8_t*)(sb + srow_l) = (uint8_t)xb;
              }
            }
          }
          if (p.q_col != nullptr && half == 0) {
            uint8_t* sb = (uint8_t*)uniform_ptr(p.s_col + (fc0 + 32 * jj) * (T / 32) + tok0 / 32);
            *(__attribute__((address_space(1))) uint32_t*)(sb + scol_l) = sbytes;
          }
        }
      }
    }
    // wgrad accumulating into C (fp32): an expert without tokens (nk == 0)
    // leaves its C untouched, and the old values are loaded a block of 8
    // rows ahead of the stores: the wait for a load also waits for every
    // store issued before it (the counter completes in issue order), so
    // loading just before adding would serialise.  (Blocks of 16 rows held
    // 32 registers more and pushed the tile counter's claim into scratch,
    // whose spill and reload each waited for every memory operation in
    // flight.)  Registers 4b..4b+3 of a quad of
    // lanes (4 consecutive columns) hold a 4 x 4 block of C; a DPP transpose
    // inside the quad leaves lane q of it with row 8b + 4 (l/32) + q, its 4
    // columns in registers 0..3, so one 16-byte load and store per 4
    // registers cover, per instruction, 8 rows of 32 consecutive columns:
    // whole 128-byte lines, 4x fewer loads than one register at a time.  The
    // row part of the address is wave-uniform (scalar base); the lane part is
    // a 32-bit offset.
    else if (nk > 0) {
      static_assert(!ACCUM || !OUT_BF16, "the accumulating wgrad adds into fp32");
      const int64_t ldc_b = p.ldc * esz;
      const int wm_u = __builtin_amdgcn_readfirstlane(wm);
      // per-lane values derived here from the hardware lane id (volatile
      // mbcnt, so it is not hoisted): from a value computed at the kernel
      // entry they would stay live through the K loop, where no register is
      // left
      uint32_t ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const uint32_t cq = (ln & 31) >> 2;       // column quad of the 32-column fragment
      const bool odd = (ln & 1) != 0, hi2 = (ln & 2) != 0;
      const uint32_t my_row = 4 * (ln >> 5) + (ln & 3);   // within an 8-row group
      // 32-bit lane offset (7 rows of at most a few hundred KB plus a column)
      const uint32_t lane_off =
          my_row * (uint32_t)ldc_b + (uint32_t)(wn * WT) * (uint32_t)esz + 4 * cq * (uint32_t)esz;
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      // Sixteen blocks h of 8 rows (8-row group h % 4 of 32-row fragment row
      // h / 4): the old values of block h + 1 are loaded before block h is
      // stored, so the wait for block h + 1's loads leaves block h's stores
      // in flight.  Two blocks of old values are live (32 registers).
      f32x4 old[2][4];
      auto load_block = [&](int h, f32x4 (&o)[4]) {
        const int row = wm_u * WT + 32 * (h >> 2) + 8 * (h & 3);
        const char* rb = (const char*)uniform_ptr((const uint8_t*)(ed.c + (int64_t)row * ldc_b)) + lane_off;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = __builtin_nontemporal_load(
              (__attribute__((address_space(1))) const f32x4*)(rb + j * 32 * 4));
      };
      load_block(0, old[0]);
#pragma unroll
      for (int h = 0; h < 16; ++h) {
        if (h + 1 < 16) load_block(h + 1, old[(h + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        const int i = h >> 2, b = h & 3;
        const int row = wm_u * WT + 32 * i + 8 * b;   // uniform
        char* rbase = (char*)uniform_ptr((const uint8_t*)(ed.c + (int64_t)row * ldc_b)) + lane_off;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v0 = acc[i][j][4 * b], v1 = acc[i][j][4 * b + 1];
          float v2 = acc[i][j][4 * b + 2], v3 = acc[i][j][4 * b + 3];
          quad_transpose(v0, v1, v2, v3, odd, hi2);
          const f32x4 ov = old[h & 1][j];
          v0 += ov.x;
          v1 += ov.y;
          v2 += ov.z;
          v3 += ov.w;
          __builtin_nontemporal_store(f32x4{v0, v1, v2, v3},
              (__attribute__((address_space(1))) f32x4*)(rbase + j * 32 * 4));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!has_next) break;
    // the store loops above issue one operation per register (256 per wave
    // for every row inside the tile) or, accumulating, 64 loads and 64
    // stores
    if (!(KGROUPED ? (!ACCUM || nk > 0) : (ed.row_lo == 0 && ed.row_hi == BM)))
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    tile = next;
    cur_nk = nk_next;
    cur_g = g_next;
    spar = spar_n;
    gpar = gpar_n;
  }
}

// Zeroes the output rows of the tiles that describe_unit splits in two (the
// same plan, from the same device m_splits and grid), before the GEMM adds
// both halves into them.  fp32 output only.
__global__ __launch_bounds__(kThreads) void zero_split_tail_kernel(GemmArgs p, int32_t grid) {
  __shared__ ExpertTable table;
  __shared__ int64_t scan[2 * kThreads];
  build_table<false>(p.m_splits, p.G, &table, scan);
  const int ntiles = table.tpre[p.G] * p.ntiles_n;
  const UnitPlan up = plan_units<false>(p, &table, ntiles, grid);
  const int rem = up.nunits - ntiles;
  for (int b = blockIdx.x; b < rem; b += gridDim.x) {
    const TileDesc d = describe<false>(p, &table, up.first_split + b, 4);
    float* c = reinterpret_cast<float*>(d.c);
    const int rows = d.row_hi - d.row_lo;
    for (int idx = threadIdx.x; idx < rows * (BN / 4); idx += kThreads) {
      const int r = d.row_lo + idx / (BN / 4);
      *reinterpret_cast<float4*>(c + (int64_t)r * p.ldc + 4 * (idx % (BN / 4))) =
          make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// Sets the wgrad's tile counters before the GEMM on the same stream: the
// first tiles are the workgroups' own indices, so with one counter per XCD
// (grid a multiple of 8) each starts at grid / 8, else the one counter at
// the grid size.
__global__ void queue_init_kernel(int32_t* queue, int32_t grid) {
  if (grid % 8 == 0) {
    if (threadIdx.x < 8) queue[threadIdx.x] = grid / 8;
  } else if (threadIdx.x == 0) {
    queue[0] = grid;
  }
}

template <bool KG, bool BF, bool ACC = false, bool SW = false>
static hipError_t launch_one(const GemmArgs& a, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((grouped_gemm_kernel<KG, BF, ACC, SW>), dim3(grid), dim3(kThreads), 0, st,
                     a);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int layout, const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                               const uint8_t* sb, void* c, bool out_bf16, int64_t T, int64_t N,
                               int64_t K, const int64_t* m_splits, int32_t G, bool accumulate,
                               hipStream_t st, int32_t* queue) {
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
  // contraction halves of the last round's tiles (describe_unit): fp32
  // output, M-grouped, and halves that are whole stages and scale groups
  // (and only where the contraction is long enough to split one tile:
  // plan_units with rem = 1; otherwise the zeroing launch is left out)
  p.split_tail = (!kgrouped && !out_bf16 && p.kc % 1024 == 0 &&
                  5 * (p.kc / KSTEP) > 320 + 12) ? 1 : 0;
  if (p.split_tail) {
    hipLaunchKernelGGL(zero_split_tail_kernel, dim3(std::max(1u, grid / 2)), dim3(kThreads), 0,
                       st, p, (int32_t)grid);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (kgrouped && queue != nullptr) {
    hipLaunchKernelGGL(queue_init_kernel, dim3(1), dim3(64), 0, st, queue, (int32_t)grid);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.queue = queue;
  }
  if (kgrouped && accumulate) return launch_one<true, false, true>(p, grid, st);
  if (kgrouped)
    return out_bf16 ? launch_one<true, true>(p, grid, st) : launch_one<true, false>(p, grid, st);
  return out_bf16 ? launch_one<false, true>(p, grid, st) : launch_one<false, false>(p, grid, st);
}

// Forward (NT) with bf16 h [T, 2F] and the SwiGLU + quantize epilogue.
hipError_t launch_grouped_gemm_swiglu(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                                      const uint8_t* sb, uint16_t* h, int64_t T, int64_t F,
                                      int64_t K, const int64_t* m_splits, int32_t G,
                                      uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                      uint8_t* s_col, hipStream_t st) {
  GemmArgs p{};
  p.a = a;
  p.sa = sa;
  p.b = b;
  p.sb = sb;
  p.c = h;
  p.m_splits = m_splits;
  p.G = G;
  const int64_t N = 2 * F;
  p.lda = K; p.ldsa = K / 32;
  p.ldb = K; p.ldsb = K / 32;
  p.b_gstride = N * K; p.sb_gstride = N * K / 32;
  p.ldc = N; p.rows = T; p.cols = N; p.kc = K;
  p.ntiles_n = (int32_t)(N / BN);
  p.f = F;
  p.q_row = q_row;
  p.s_row = s_row;
  p.q_col = q_col;
  p.s_col = s_col;
  const int64_t upper = (T / BM + G) * p.ntiles_n;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(upper, cus));
  return launch_one<false, true, false, true>(p, grid, st);
}

}  // namespace mx
