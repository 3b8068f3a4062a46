/*
 * mxfp8moe.h -- C ABI of the MXFP8 MoE expert grouped-GEMM library (gfx950).
 *
 * The hot path of an MoE expert linear layer on MXFP8 data, as described on
 * the NVIDIA TransformerEngine pull-request pages
 *   [P3244] "[Pytorch] Add support for row-wise quanted input for grouped gemm"
 *   [P3545] "[PyTorch] Fix distributed BF16 weights and trim NVFP4 saved state
 *            in the fused grouped MLP"
 *   [P3224] "Improve device-init grouped linear module with single grouped
 *            weight support"
 * with the MXFP8 arithmetic of the OCP Microscaling Formats (MX) v1.0
 * specification (sections 5 and 6.3), which the pages leave unstated.
 *
 * Formats and conventions used by every entry point
 * -------------------------------------------------
 *  - bf16 tensors are passed as their 16-bit patterns (uint16_t).
 *  - MXFP8 data bytes are E4M3 ("FN": max 448, no infinity) and scale bytes
 *    are E8M0 (value 2^(u-127)).  A block of 32 values shares one scale:
 *      X = floor(log2(max|v|)) - 8, clamped to [-127, 127] (0 for an all-zero
 *      block, i.e. byte 0); each element is the E4M3 value nearest to v/2^X,
 *      ties to the even code, saturating at +-448; the sign of zero is kept.
 *  - Row-wise data of a [R, C] tensor: bytes [R, C] row-major, scales
 *    [R, C/32] row-major, blocks of 1 x 32 along C ([P3244] Description).
 *  - Column-wise data of a [R, C] tensor (blocks of 32 x 1 along R) is stored
 *    transposed: bytes [C, R] and scales [C, R/32], both row-major.  It is the
 *    copy the wgrad GEMM reads ([P3244] Greptile Summary flowchart;
 *    [P3545] Description: every wgrad path takes the column-wise tiles).
 *  - bf16 inputs must be finite.  Neither the pages nor the OCP rule give a
 *    scale for a block that holds Inf or NaN; the bytes written for such a
 *    block are unspecified (they are not NaN-propagating), and there the
 *    fused mxfp8_group_quantize_requant may differ from the separate
 *    quantize and requantize calls.  No entry point checks for this.
 *  - Scale arrays have exactly the shape (T, K/32): the page's padded shape
 *    (round_up(T,128), round_up(K/32,4)) ([P3244] review thread on
 *    scale_shape) has no padding under the alignment contract below.
 *  - Alignment contract ([P3244] review thread on scale_shape: per-expert
 *    128-token alignment from the dispatch, hidden % 512 == 0, assert rather
 *    than pad): T % 128 == 0, every m_splits[g] % 128 == 0 and >= 0,
 *    sum(m_splits) == T, K % 512 == 0, N % 512 == 0.  Host-checkable parts
 *    are checked (MXFP8_EINVAL); the device-resident splits are checked only
 *    by mxfp8_validate_splits.  Under this contract column-wise blocks never
 *    straddle an expert boundary, so the quantize/requant bytes do not depend
 *    on the split.
 *  - m_splits is a DEVICE array of int64 ([P3224] review: the native grouped
 *    path requires CUDA int64 m_splits and errors on host splits).  A host
 *    pointer is rejected with MXFP8_EINVAL.
 *  - Every buffer is caller-owned device memory.  Outputs are fully
 *    overwritten in place (the output= reuse of [P3224] Greptile Summary).
 *    No entry point allocates, frees or synchronizes; all work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream), so the calls can
 *    be captured in a HIP graph.  Kernels never fill memory with a memset
 *    node.
 *  - T = 0 (no token routed to any expert) is valid everywhere: the buffers
 *    whose size is a multiple of T are empty and may be NULL; outputs that
 *    do not depend on T (the wgrad's [G, N, K], dbias [G, N]) must still be
 *    given and are written as for experts without tokens (zeros), and an
 *    accumulated main_grad is left as it is.
 *  - Errors: the return value is a status code; mxfp8_last_error() gives a
 *    message for the last failing call on this thread.  MXFP8_EINVAL mirrors
 *    the pages' ValueError (bad shapes, NULL pointers, host m_splits),
 *    MXFP8_ENOTSUP their NotImplementedError (unsupported format requests),
 *    MXFP8_EHIP their RuntimeError (a HIP launch failure).
 */
#ifndef MXFP8MOE_H
#define MXFP8MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mxfp8_status {
  MXFP8_OK = 0,
  MXFP8_EINVAL = 1,
  MXFP8_ENOTSUP = 2,
  MXFP8_EHIP = 3
} mxfp8_status;

/* GEMM layouts, row-major letters: NT: C = A B^T, NN: C = A B, TN: C = A^T B. */
typedef enum mxfp8_layout {
  MXFP8_LAYOUT_NT = 0, /* forward  */
  MXFP8_LAYOUT_NN = 1, /* dgrad    */
  MXFP8_LAYOUT_TN = 2  /* wgrad    */
} mxfp8_layout;

typedef enum mxfp8_out_dtype {
  MXFP8_OUT_F32 = 0,
  MXFP8_OUT_BF16 = 1
} mxfp8_out_dtype;

#define MXFP8_ROWWISE 1u
#define MXFP8_COLWISE 2u

/* Message for the last failing call on this thread ("" if none). */
const char* mxfp8_last_error(void);

/* ABI version of this header (incremented on any signature change). */
int32_t mxfp8_abi_version(void);

/*
 * mxfp8_group_quantize -- bf16 grouped token tensor -> MXFP8.
 * Row-wise ([P3244] Description: the grouped GEMM takes input already
 * quantized row-wise) and/or column-wise ([P3244] review: the column-wise
 * scales come from the group quantize kernel) in one pass over x.
 *
 *   x      [T, K] bf16, row-major (device)
 *   usage  MXFP8_ROWWISE | MXFP8_COLWISE (at least one)
 *   q_row  [T, K] u8,  s_row [T, K/32] u8        (required iff ROWWISE)
 *   q_col  [K, T] u8,  s_col [K, T/32] u8        (required iff COLWISE)
 *   noop_flag  NULL, or a device int32 read when the kernels run: non-zero
 *          makes the call write nothing, so the outputs keep their previous
 *          contents ([P3224] Greptile Summary and its test list: the group
 *          quantize's noop flag, replayed in a CUDA graph).  A captured
 *          graph can thereby skip re-quantizing weights that did not change;
 *          the flag is set or cleared by the caller's own kernels.
 * The same call quantizes a grouped weight [G, N, K] viewed as [G*N, K]
 * (T = G*N); its column-wise copy is then [K, G*N], expert g being columns
 * [g*N, (g+1)*N).
 * Errors: EINVAL for NULL required pointers, T % 128, K % 512, usage == 0.
 */
mxfp8_status mxfp8_group_quantize(const uint16_t* x, int64_t T, int64_t K, uint32_t usage,
                                  uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                  uint8_t* s_col, const int32_t* noop_flag, void* stream);

/*
 * Bytes of device workspace that mxfp8_requant_colwise (with dbias) and
 * mxfp8_grouped_dbias need for a [T, N] operand: one fp32 partial sum per
 * 128-row tile and column, i.e. (T/128) * N * 4.
 */
size_t mxfp8_dbias_workspace_bytes(int64_t T, int64_t N);

/*
 * mxfp8_requant_colwise -- row-wise MXFP8 -> exact dequantize -> column-wise
 * MXFP8, optionally with the fused grouped bias gradient
 * ([P3244] Description: dequant + requant with col-wise to save for
 * backward / for wgrad; Greptile Summary: dbias reduced directly from the
 * dequantized gradient).
 *
 *   q_row [T, K] u8, s_row [T, K/32] u8     (device)
 *   q_col [K, T] u8, s_col [K, T/32] u8     (device, written)
 *   dbias NULL, or [G, K] fp32 (device, written): dbias[g, k] = sum over the
 *         rows r of expert g of dequant(q_row)[r, k]; 0 for an empty expert.
 *         Needs m_splits (device int64 [G]) and a workspace of
 *         mxfp8_dbias_workspace_bytes(T, K) bytes; the sum order is fixed, so
 *         results are bitwise reproducible.
 * Errors: EINVAL for NULL pointers, T % 128, K % 512, G < 1, host m_splits,
 * a workspace smaller than required.
 */
mxfp8_status mxfp8_requant_colwise(const uint8_t* q_row, const uint8_t* s_row, int64_t T,
                                   int64_t K, uint8_t* q_col, uint8_t* s_col,
                                   const int64_t* m_splits, int32_t G, float* dbias,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * mxfp8_group_quantize_requant -- mxfp8_group_quantize(ROWWISE) followed by
 * mxfp8_requant_colwise (with its optional dbias) in one pass over x: the
 * backward's gradient is quantized row-wise for dgrad, and its column-wise
 * copy for wgrad is requantized from those row-wise values, not quantized
 * from bf16 ([P3244] Description and Greptile flowchart: dequantize, then
 * column-wise requantize, with the bias reductions from the dequantized
 * grad).  x is read once instead of the row-wise codes being read back.
 *  x: bf16 [T, K]; q_row/s_row: [T, K] + [T, K/32]; q_col/s_col: the
 *  transposed column-wise copy [K, T] + [K, T/32]; dbias, m_splits, G,
 *  workspace as for mxfp8_requant_colwise.
 *  For finite x every output byte (and dbias, bit for bit) equals what the
 *  two calls give.
 * Errors: EINVAL for NULL pointers (T > 0), T % 128, K % 512, and as
 * mxfp8_requant_colwise for dbias.
 */
mxfp8_status mxfp8_group_quantize_requant(const uint16_t* x, int64_t T, int64_t K,
                                          uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                          uint8_t* s_col, const int64_t* m_splits, int32_t G,
                                          float* dbias, void* workspace, size_t workspace_bytes,
                                          void* stream);

/*
 * mxfp8_group_quantize_requant_noalloc -- mxfp8_group_quantize_requant for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same work and
 * the same bytes, with no workspace argument.  The dbias partial sums live in
 * a static device array of MXFP8_NOALLOC_SCRATCH_BYTES bytes inside the
 * library (one per GPU, held until the process ends; its address is looked
 * up on the first call on each device).  The call allocates and frees
 * nothing.
 *  Arguments as mxfp8_group_quantize_requant, without workspace.
 *  Limit: with dbias, (T/128) * K * 4 bytes of partials must fit the array,
 *  i.e. mxfp8_dbias_workspace_bytes(T, K) <= MXFP8_NOALLOC_SCRATCH_BYTES
 *  (32 MiB: for K = 14336, T up to 74880; for K = 7168, up to 149760);
 *  without dbias there is no limit.
 *  Every call on one GPU shares that GPU's array, and the array keeps the
 *  last call's partials: calls with dbias that may overlap on one GPU (on
 *  different streams, or from different threads) race on it and give wrong
 *  dbias.  Stream-ordered calls, graph replays included, are safe.  Nothing
 *  needs clearing: each call writes every partial its finalize reads.
 * Errors: as mxfp8_group_quantize_requant, and EINVAL when the partials of
 * the requested dbias exceed the static array.
 */
#define MXFP8_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
mxfp8_status mxfp8_group_quantize_requant_noalloc(const uint16_t* x, int64_t T, int64_t K,
                                                  uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                                  uint8_t* s_col, const int64_t* m_splits,
                                                  int32_t G, float* dbias, void* stream);

/*
 * mxfp8_grouped_dbias -- grouped bias gradient from row-wise MXFP8 dY with no
 * column-wise copy (the frozen-weight case: [P3244] Greptile Summary, dbias
 * reduced without a wgrad stage).
 *   q_row [T, N] u8, s_row [T, N/32] u8; dbias [G, N] fp32 (written).
 * Same workspace and errors as mxfp8_requant_colwise.
 */
mxfp8_status mxfp8_grouped_dbias(const uint8_t* q_row, const uint8_t* s_row, int64_t T,
                                 int64_t N, const int64_t* m_splits, int32_t G, float* dbias,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * mxfp8_grouped_scaled_bias_grad -- gradients of a bias scaled by each
 * token's routing scale, from row-wise MXFP8 dY ([P3244] Greptile Summary:
 * scaled-bias gradient reductions; its flowchart takes the bias and
 * routing-scale reductions from the dequantized gradient).  With the forward
 * out_r = x_r W_g^T + s_r b_g for row r of expert g:
 *   dbias[g, n] = sum over rows r of expert g of s_r * dY[r, n]
 *   dscales[r]  = sum over n of dY[r, n] * b[g, n]
 * dY is dequantized exactly; sums in fp32 in a fixed order (bitwise
 * reproducible).  An expert with no rows gets dbias[g] = 0.
 *   q_row [T, N] + s_row [T, N/32]: row-wise dY; m_splits: device int64 [G];
 *   scales: device fp32 [T] (needed for dbias); bias: device fp32 [G, N]
 *   (needed for dscales); dbias: fp32 [G, N] or NULL; dscales: fp32 [T] or
 *   NULL (at least one); workspace: device, at least
 *   mxfp8_scaled_bias_workspace_bytes(T, N) bytes.
 * Errors: EINVAL for NULL inputs, neither output requested, an output without
 * its input, T % 128, N % 512, host m_splits, a small workspace.
 */
size_t mxfp8_scaled_bias_workspace_bytes(int64_t T, int64_t N);
mxfp8_status mxfp8_grouped_scaled_bias_grad(const uint8_t* q_row, const uint8_t* s_row,
                                            int64_t T, int64_t N, const int64_t* m_splits,
                                            int32_t G, const float* scales, const float* bias,
                                            float* dbias, float* dscales, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * mxfp8_grouped_gemm -- the three grouped GEMMs of an expert linear
 * y = x W^T (in_features K, out_features N, grouped weight [G, N, K],
 * [P3224] Greptile Summary) on MXFP8 operands, fp32 accumulation.
 * Expert g owns token rows [o_g, o_g + m_splits[g]), o_g = sum of the
 * previous splits.
 *
 *  NT (forward, [P3244] Description: row-wise data goes straight to the
 *      forward grouped GEMM):
 *      a = X row-wise  [T, K] + [T, K/32]
 *      b = W row-wise  [G, N, K] + [G, N, K/32]
 *      c [T, N]:  c[r] = X[r] W_g^T for r in expert g
 *  NN (dgrad, [P3244] Description backward paragraph; [P3545] last commit
 *      message: the column-wise weight copy exists for dgrad):
 *      a = dY row-wise [T, N] + [T, N/32]
 *      b = W column-wise copy [K, G*N] + [K, G*N/32]
 *      c [T, K]:  c[r] = dY[r] W_g
 *  TN (wgrad, [P3244] flowchart: column-wise requantize feeds the wgrad
 *      grouped GEMM):
 *      a = dY column-wise copy [N, T] + [N, T/32]
 *      b = X column-wise copy  [K, T] + [K, T/32]
 *      c [G, N, K]: c[g] = sum over r in expert g of dY[r]^T X[r];
 *      an expert with no rows gets c[g] = 0.
 *  c_dtype: MXFP8_OUT_F32 or MXFP8_OUT_BF16 (round to nearest even).
 *  Rows of c that belong to no expert (none under the contract) are not
 *  written by NT/NN.
 *  With fp32 output, an NT/NN call may split the few long tiles of its
 *  grid's last round into two contraction halves: it then enqueues a small
 *  kernel that zeroes those tiles' rows of c, and the two halves add into
 *  them.  The result is deterministic (two fp32 adds onto zero commute) and
 *  the launches stay stream-ordered and graph-capturable; their rounding
 *  differs from the unsplit sum only by the order of the fp32 additions.
 * Errors: EINVAL for NULL pointers, bad layout, T % 128, N % 512, K % 512,
 * G < 1, host m_splits; ENOTSUP for another c_dtype.
 */
mxfp8_status mxfp8_grouped_gemm(int32_t layout, const uint8_t* a_data, const uint8_t* a_scale,
                                const uint8_t* b_data, const uint8_t* b_scale, void* c,
                                int32_t c_dtype, int64_t T, int64_t N, int64_t K,
                                const int64_t* m_splits, int32_t G, void* stream);

/*
 * mxfp8_grouped_gemm_swiglu_quantize -- the forward (NT) grouped GEMM of the
 * fused expert MLP's first linear, FC1, with its activation and the MXFP8
 * quantize of the activation in the GEMM's epilogue ([P3545] Description:
 * the fused grouped MLP runs FC1 -> activation -> FC2 as one op; its
 * saved-state commit: the FC2 forward reads the row-wise tiles of the
 * activation and the FC2 wgrad the column-wise ones).  The activation is
 * SwiGLU (not defined on the pages): gate = columns [0, F) of h, up =
 * columns [F, 2F).
 *      h[r] = X[r] W1_g^T  (bf16, round to nearest even), r in expert g
 *      a    = silu(gate) * up from the bf16 h, fp32 math, bf16 rounding
 *      a quantized row-wise and/or column-wise
 *  The outputs are byte-identical to mxfp8_grouped_gemm (NT, bf16 output)
 *  followed by mxfp8_swiglu_quantize on its h; a itself is never written.
 *   a_data/a_scale  X row-wise [T, K] + [T, K/32]
 *   b_data/b_scale  W1 row-wise [G, 2F, K] + [G, 2F, K/32]
 *   h               [T, 2F] bf16, written (the SwiGLU backward reads it)
 *   usage           MXFP8_ROWWISE | MXFP8_COLWISE (at least one)
 *   q_row [T, F] u8, s_row [T, F/32] u8     (required iff ROWWISE)
 *   q_col [F, T] u8, s_col [F, T/32] u8     (required iff COLWISE)
 * Errors: EINVAL for NULL required pointers, T % 128, F % 512, K % 512,
 * G < 1 or G > 1024, host m_splits, usage == 0.
 */
mxfp8_status mxfp8_grouped_gemm_swiglu_quantize(const uint8_t* a_data, const uint8_t* a_scale,
                                                const uint8_t* b_data, const uint8_t* b_scale,
                                                uint16_t* h, int64_t T, int64_t F, int64_t K,
                                                const int64_t* m_splits, int32_t G,
                                                uint32_t usage, uint8_t* q_row, uint8_t* s_row,
                                                uint8_t* q_col, uint8_t* s_col, void* stream);

/*
 * mxfp8_grouped_gemm_wgrad_accumulate -- the TN (wgrad) product of
 * mxfp8_grouped_gemm added into an existing fp32 weight-gradient buffer
 * instead of overwriting it, the form a training step uses when the weight
 * gradient accumulates into an fp32 main_grad ([P3545] last commit message:
 * the fused grouped MLP's weight gradients are checked in main_grad):
 *      main_grad[g] += sum over r in expert g of dY[r]^T X[r]
 *  a, b, T, N, K, m_splits, G as for the TN layout of mxfp8_grouped_gemm;
 *  main_grad: caller-owned device fp32 [G, N, K], read and written.  The sum
 *  of an expert's product is formed in fp32 as for mxfp8_grouped_gemm and
 *  added to main_grad once (one fp32 rounding).  An expert with no rows
 *  leaves its main_grad[g] untouched (bit for bit).
 * Errors: EINVAL for NULL pointers, T % 128, N % 512, K % 512, G < 1 or
 * G > 1024, host m_splits.
 */
mxfp8_status mxfp8_grouped_gemm_wgrad_accumulate(const uint8_t* a_data, const uint8_t* a_scale,
                                                 const uint8_t* b_data, const uint8_t* b_scale,
                                                 float* main_grad, int64_t T, int64_t N, int64_t K,
                                                 const int64_t* m_splits, int32_t G,
                                                 void* stream);

/*
 * mxfp8_grouped_gemm_ws, mxfp8_grouped_gemm_wgrad_accumulate_ws -- the same
 * calls with a caller-owned device workspace holding a tile counter, through
 * which the TN (wgrad) tiles are handed out in order as workgroups finish
 * theirs: greedy longest-first placement of the experts' tiles, instead of a
 * fixed assignment that, under skewed routing, lets a few workgroups with the
 * largest experts' tiles run long after the rest (the routing skew of the
 * [P3224] m_splits use case; [P3545]'s fused grouped MLP).  The outputs are
 * bit-identical to those of the calls without a workspace (each tile is
 * computed the same way, by whichever workgroup takes it).  NT/NN ignore the
 * workspace.
 *  The kernel keeps the fixed order when 1 expert in 8 or more has no token:
 *  those experts' tiles store zeros only, and the fixed order runs them
 *  beside the contraction instead of last.
 *  workspace: device memory of at least mxfp8_grouped_gemm_workspace_bytes()
 *  bytes, owned by the caller; its contents need no initialisation (the call
 *  enqueues a one-thread kernel that sets the counter before the GEMM) and
 *  are meaningless afterwards.  Calls that may run at the same time (other
 *  streams) need workspaces of their own; stream-ordered calls, graph replays
 *  included, can share one.
 * Errors: as the calls without a workspace, and EINVAL for a NULL or too
 * small workspace.
 */
size_t mxfp8_grouped_gemm_workspace_bytes(void);
mxfp8_status mxfp8_grouped_gemm_ws(int32_t layout, const uint8_t* a_data, const uint8_t* a_scale,
                                   const uint8_t* b_data, const uint8_t* b_scale, void* c,
                                   int32_t c_dtype, int64_t T, int64_t N, int64_t K,
                                   const int64_t* m_splits, int32_t G, void* workspace,
                                   size_t workspace_bytes, void* stream);
mxfp8_status mxfp8_grouped_gemm_wgrad_accumulate_ws(const uint8_t* a_data,
                                                    const uint8_t* a_scale, const uint8_t* b_data,
                                                    const uint8_t* b_scale, float* main_grad,
                                                    int64_t T, int64_t N, int64_t K,
                                                    const int64_t* m_splits, int32_t G,
                                                    void* workspace, size_t workspace_bytes,
                                                    void* stream);

/*
 * mxfp8_validate_splits -- device-side check of the alignment contract on the
 * device splits ([P3224] review: an alignment check must accompany device
 * m_splits).  Writes *flag (device int32) = bitmask: 1 = a negative split,
 * 2 = a split not a multiple of 128, 4 = sum != T.  0 means valid.  The host
 * reads the flag only when it wants to (no synchronization here).
 */
mxfp8_status mxfp8_validate_splits(const int64_t* m_splits, int32_t G, int64_t T, int32_t* flag,
                                   void* stream);

/*
 * SwiGLU between the two linears of the fused expert MLP ([P3545]
 * Description: FC1 -> activation -> FC2; the activation is not defined on
 * the pages).  Gate = columns [0, F), up = columns [F, 2F) of h:
 *   a = silu(gate) * up;  fp32 math, bf16 in and out (round to nearest even).
 *   h [T, 2F] bf16, a [T, F] bf16.  Errors: EINVAL for NULL, T < 0, F % 8.
 */
mxfp8_status mxfp8_swiglu_fwd(const uint16_t* h, int64_t T, int64_t F, uint16_t* a,
                              void* stream);

/*
 * mxfp8_swiglu_quantize -- SwiGLU fused with the MXFP8 quantize of its output,
 * the FC2 input of the fused expert MLP ([P3545] Description: FC1 ->
 * activation -> FC2 as one op; its saved-state commit: the FC2 wgrad reads
 * the column-wise tiles of that input, the FC2 forward the row-wise ones).
 * The bf16 activation a = silu(h[:, :F]) * h[:, F:] is formed in registers
 * (exactly the bf16 values mxfp8_swiglu_fwd writes) and quantized as
 * mxfp8_group_quantize quantizes a [T, F] tensor, without writing a:
 * the outputs are byte-identical to mxfp8_swiglu_fwd followed by
 * mxfp8_group_quantize.
 *
 *   h      [T, 2F] bf16 (device)
 *   usage  MXFP8_ROWWISE | MXFP8_COLWISE (at least one)
 *   q_row  [T, F] u8,  s_row [T, F/32] u8        (required iff ROWWISE)
 *   q_col  [F, T] u8,  s_col [F, T/32] u8        (required iff COLWISE)
 * Errors: EINVAL for NULL required pointers, T % 128, F % 512, usage == 0.
 */
mxfp8_status mxfp8_swiglu_quantize(const uint16_t* h, int64_t T, int64_t F, uint32_t usage,
                                   uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                   uint8_t* s_col, void* stream);

/*
 * Backward of mxfp8_swiglu_fwd: given h [T, 2F] and da [T, F] (bf16), writes
 * dh [T, 2F] bf16: d gate = da * up * s * (1 + gate * (1 - s)), s = sigmoid(gate);
 * d up = da * silu(gate).  Errors as mxfp8_swiglu_fwd.
 */
mxfp8_status mxfp8_swiglu_bwd(const uint16_t* h, const uint16_t* da, int64_t T, int64_t F,
                              uint16_t* dh, void* stream);

/*
 * mxfp8_swiglu_bwd_quantize -- the SwiGLU backward fused with the quantize of
 * its output for the FC1 backward of the fused expert MLP ([P3545]
 * Description: FC1 -> activation -> FC2 as one op; the FC1 dgrad reads the
 * row-wise and its wgrad the column-wise copy of dh, and [P3244] Description
 * and Greptile flowchart: the column-wise copy requantized from the
 * dequantized row-wise values, the bias gradient reduced from them).  dh =
 * mxfp8_swiglu_bwd(h, da) is formed in registers and handled exactly as
 * mxfp8_group_quantize_requant handles a [T, 2F] tensor, without writing dh:
 * every output byte, and dbias bit for bit, equals mxfp8_swiglu_bwd followed
 * by mxfp8_group_quantize_requant.
 *   h      [T, 2F] bf16 (gate | up, device);  da [T, F] bf16 (device)
 *   q_row  [T, 2F] u8,  s_row [T, 2F/32] u8
 *   q_col  [2F, T] u8,  s_col [2F, T/32] u8
 *   m_splits, G, dbias [G, 2F] fp32, workspace: as mxfp8_group_quantize_requant
 *   with K = 2F (dbias optional: NULL skips it and needs no workspace).
 * Errors: EINVAL for NULL pointers (T > 0), T % 128, F % 256, and as
 * mxfp8_requant_colwise for dbias.
 */
mxfp8_status mxfp8_swiglu_bwd_quantize(const uint16_t* h, const uint16_t* da, int64_t T,
                                       int64_t F, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                       uint8_t* s_col, const int64_t* m_splits, int32_t G,
                                       float* dbias, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * mxfp8_convert_sweep -- diagnostic: runs the device's E4M3 / E8M0 conversion
 * helpers (the ones every quantize kernel encodes and decodes with) over
 * every (value, scale byte) pair, so that a test can compare them with an
 * independent encoder (OCP Microscaling Formats v1.0, sections 5.3-5.4 and
 * 6.3: E4M3 round to nearest even, saturated to 448; value = code * 2^X).
 * Not a step of the hot path.
 *   mode 0: out holds 2^24 u16; entry 65536 * s + h = the codes of the bf16
 *           values (h, h ^ 0x8000) encoded with scale byte s (byte 0 is h).
 *   mode 1: out holds 2^24 u8; entry 65536 * x + 256 * s + c = code c decoded
 *           with scale byte s and encoded again with scale byte x.
 *   mode 2: out holds 2^16 pairs of fp32 bit patterns; entry 256 * s + c =
 *           the codes (c, c ^ 0x80) decoded with scale byte s.
 * out: device buffer of at least mxfp8_convert_sweep_bytes(mode) bytes,
 * written asynchronously on `stream`.  Errors: EINVAL for an unknown mode, a
 * NULL or too small buffer.
 */
size_t mxfp8_convert_sweep_bytes(int32_t mode);
mxfp8_status mxfp8_convert_sweep(int32_t mode, void* out, size_t out_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8MOE_H */
