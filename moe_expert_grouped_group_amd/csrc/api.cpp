// C-ABI entry points of libmxfp8moe.so: argument validation, then kernel
// launches on the caller's stream.  Nothing here allocates, frees or
// synchronizes.  The contracts are documented in include/mxfp8moe.h.
#include "../../include/mxfp8moe.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

mxfp8_status fail(mxfp8_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

mxfp8_status ok() {
  g_err[0] = '\0';
  return MXFP8_OK;
}

mxfp8_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MXFP8_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define REQUIRE(cond, ...)                                 \
  do {                                                     \
    if (!(cond)) return fail(MXFP8_EINVAL, __VA_ARGS__);   \
  } while (0)

// The native grouped path takes device-resident int64 splits; a host array is
// an error (mirrors the ValueError for host m_splits in "Improve device-init
// grouped linear module with single grouped weight support").
mxfp8_status check_device_splits(const int64_t* m_splits, int32_t G, const char* fn) {
  if (m_splits == nullptr) return fail(MXFP8_EINVAL, "%s: m_splits is NULL", fn);
  if (G < 1) return fail(MXFP8_EINVAL, "%s: G = %d must be >= 1", fn, (int)G);
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  const hipError_t e = hipPointerGetAttributes(&attr, m_splits);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return fail(MXFP8_EINVAL,
                "%s: m_splits must be a device int64 array (pointer query failed: %s)", fn,
                hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(MXFP8_EINVAL, "%s: m_splits must be a device int64 array, got a host pointer",
                fn);
  return MXFP8_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* mxfp8_last_error(void) { return g_err; }

int32_t mxfp8_abi_version(void) { return 4; }

size_t mxfp8_dbias_workspace_bytes(int64_t T, int64_t N) {
  if (T <= 0 || N <= 0) return 0;
  return (size_t)((T + 127) / 128) * (size_t)N * sizeof(float);
}

mxfp8_status mxfp8_group_quantize(const uint16_t* x, int64_t T, int64_t K, uint32_t usage,
                                  uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                  uint8_t* s_col, const int32_t* noop_flag, void* stream) {
  const char* fn = "mxfp8_group_quantize";
  REQUIRE(x != nullptr || T == 0, "%s: x is NULL", fn);
  REQUIRE(usage != 0 && (usage & ~(MXFP8_ROWWISE | MXFP8_COLWISE)) == 0,
          "%s: usage must be a non-empty combination of MXFP8_ROWWISE and MXFP8_COLWISE", fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(K > 0 && K % 512 == 0, "%s: K = %lld must be a positive multiple of 512", fn,
          (long long)K);
  if (T == 0) return ok();   // nothing to read or write: every buffer is empty
  const bool row = usage & MXFP8_ROWWISE, col = usage & MXFP8_COLWISE;
  REQUIRE(!row || (q_row && s_row), "%s: ROWWISE requested but q_row/s_row is NULL", fn);
  REQUIRE(!col || (q_col && s_col), "%s: COLWISE requested but q_col/s_col is NULL", fn);
  hipError_t e;
  if (col)
    e = mx::launch_quant_rowcol(x, T, K, row ? q_row : nullptr, row ? s_row : nullptr, q_col,
                                s_col, noop_flag, as_stream(stream));
  else
    e = mx::launch_quant_rowwise(x, T, K, q_row, s_row, noop_flag, as_stream(stream));
  return hip_status(e, fn);
}

mxfp8_status mxfp8_requant_colwise(const uint8_t* q_row, const uint8_t* s_row, int64_t T,
                                   int64_t K, uint8_t* q_col, uint8_t* s_col,
                                   const int64_t* m_splits, int32_t G, float* dbias,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mxfp8_requant_colwise";
  REQUIRE(T == 0 || (q_row && s_row && q_col && s_col), "%s: NULL data/scale pointer", fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(K > 0 && K % 512 == 0, "%s: K = %lld must be a positive multiple of 512", fn,
          (long long)K);
  float* partial = nullptr;
  if (dbias != nullptr) {
    mxfp8_status st = check_device_splits(m_splits, G, fn);
    if (st != MXFP8_OK) return st;
    REQUIRE((workspace != nullptr || T == 0) &&
                workspace_bytes >= mxfp8_dbias_workspace_bytes(T, K),
            "%s: dbias needs a workspace of %zu bytes", fn, mxfp8_dbias_workspace_bytes(T, K));
    partial = static_cast<float*>(workspace);
  }
  hipStream_t st = as_stream(stream);
  hipError_t e = hipSuccess;
  if (T > 0) e = mx::launch_requant_colwise(q_row, s_row, T, K, q_col, s_col, partial, st);
  if (e == hipSuccess && dbias != nullptr)
    e = mx::launch_dbias_finalize(partial, m_splits, G, T, K, dbias, st);
  return hip_status(e, fn);
}

mxfp8_status mxfp8_group_quantize_requant(const uint16_t* x, int64_t T, int64_t K,
                                          uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                          uint8_t* s_col, const int64_t* m_splits, int32_t G,
                                          float* dbias, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  const char* fn = "mxfp8_group_quantize_requant";
  REQUIRE(T == 0 || (x && q_row && s_row && q_col && s_col), "%s: NULL data/scale pointer", fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(K > 0 && K % 512 == 0, "%s: K = %lld must be a positive multiple of 512", fn,
          (long long)K);
  float* partial = nullptr;
  if (dbias != nullptr) {
    mxfp8_status st = check_device_splits(m_splits, G, fn);
    if (st != MXFP8_OK) return st;
    REQUIRE((workspace != nullptr || T == 0) &&
                workspace_bytes >= mxfp8_dbias_workspace_bytes(T, K),
            "%s: dbias needs a workspace of %zu bytes", fn, mxfp8_dbias_workspace_bytes(T, K));
    partial = static_cast<float*>(workspace);
  }
  hipStream_t st = as_stream(stream);
  hipError_t e = hipSuccess;
  if (T > 0) e = mx::launch_quant_row_requant(x, T, K, q_row, s_row, q_col, s_col, partial, st);
  if (e == hipSuccess && dbias != nullptr)
    e = mx::launch_dbias_finalize(partial, m_splits, G, T, K, dbias, st);
  return hip_status(e, fn);
}

mxfp8_status mxfp8_group_quantize_requant_noalloc(const uint16_t* x, int64_t T, int64_t K,
                                                  uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                                  uint8_t* s_col, const int64_t* m_splits,
                                                  int32_t G, float* dbias, void* stream) {
  const char* fn = "mxfp8_group_quantize_requant_noalloc";
  REQUIRE(T == 0 || (x && q_row && s_row && q_col && s_col), "%s: NULL data/scale pointer", fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(K > 0 && K % 512 == 0, "%s: K = %lld must be a positive multiple of 512", fn,
          (long long)K);
  float* partial = nullptr;
  if (dbias != nullptr) {
    const size_t need = mxfp8_dbias_workspace_bytes(T, K);
    REQUIRE(need <= mx::noalloc_scratch_bytes(),
            "%s: dbias of a [%lld, %lld] operand needs %zu bytes of partial sums, more than the "
            "%zu-byte static scratch (MXFP8_NOALLOC_SCRATCH_BYTES); use "
            "mxfp8_group_quantize_requant with a workspace",
            fn, (long long)T, (long long)K, need, mx::noalloc_scratch_bytes());
    mxfp8_status st = check_device_splits(m_splits, G, fn);
    if (st != MXFP8_OK) return st;
    if (T > 0) {
      const hipError_t e = mx::noalloc_scratch(&partial);
      if (e != hipSuccess) return hip_status(e, fn);
    }
  }
  hipStream_t st = as_stream(stream);
  hipError_t e = hipSuccess;
  if (T > 0) e = mx::launch_quant_row_requant(x, T, K, q_row, s_row, q_col, s_col, partial, st);
  if (e == hipSuccess && dbias != nullptr)
    e = mx::launch_dbias_finalize(partial, m_splits, G, T, K, dbias, st);
  return hip_status(e, fn);
}

mxfp8_status mxfp8_grouped_dbias(const uint8_t* q_row, const uint8_t* s_row, int64_t T,
                                 int64_t N, const int64_t* m_splits, int32_t G, float* dbias,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mxfp8_grouped_dbias";
  REQUIRE(dbias && (T == 0 || (q_row && s_row)), "%s: NULL pointer", fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(N > 0 && N % 512 == 0, "%s: N = %lld must be a positive multiple of 512", fn,
          (long long)N);
  mxfp8_status s = check_device_splits(m_splits, G, fn);
  if (s != MXFP8_OK) return s;
  REQUIRE((workspace != nullptr || T == 0) &&
              workspace_bytes >= mxfp8_dbias_workspace_bytes(T, N),
          "%s: needs a workspace of %zu bytes", fn, mxfp8_dbias_workspace_bytes(T, N));
  float* partial = static_cast<float*>(workspace);
  hipStream_t st = as_stream(stream);
  hipError_t e = hipSuccess;
  if (T > 0) e = mx::launch_dbias_partial(q_row, s_row, T, N, partial, st);
  if (e == hipSuccess) e = mx::launch_dbias_finalize(partial, m_splits, G, T, N, dbias, st);
  return hip_status(e, fn);
}

size_t mxfp8_scaled_bias_workspace_bytes(int64_t T, int64_t N) {
  if (T <= 0 || N <= 0) return 0;
  return mx::scaled_bias_workspace_bytes(T, N);
}

mxfp8_status mxfp8_grouped_scaled_bias_grad(const uint8_t* q_row, const uint8_t* s_row,
                                            int64_t T, int64_t N, const int64_t* m_splits,
                                            int32_t G, const float* scales, const float* bias,
                                            float* dbias, float* dscales, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  const char* fn = "mxfp8_grouped_scaled_bias_grad";
  REQUIRE(T == 0 || (q_row && s_row), "%s: NULL data/scale pointer", fn);
  REQUIRE(dbias || dscales, "%s: neither dbias nor dscales requested", fn);
  REQUIRE(!dbias || scales || T == 0, "%s: dbias needs the routing scales", fn);
  REQUIRE(!dscales || bias || T == 0, "%s: dscales needs the bias", fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(N > 0 && N % 512 == 0, "%s: N = %lld must be a positive multiple of 512", fn,
          (long long)N);
  mxfp8_status s = check_device_splits(m_splits, G, fn);
  if (s != MXFP8_OK) return s;
  if (T == 0) {
    // no rows: dbias is zero for every expert, dscales is empty
    if (dbias != nullptr)
      return hip_status(mx::launch_dbias_finalize(nullptr, m_splits, G, 0, N, dbias,
                                                  as_stream(stream)), fn);
    return ok();
  }
  REQUIRE(workspace != nullptr && workspace_bytes >= mx::scaled_bias_workspace_bytes(T, N),
          "%s: needs a workspace of %zu bytes", fn, mx::scaled_bias_workspace_bytes(T, N));
  return hip_status(mx::launch_scaled_bias_grad(q_row, s_row, T, N, m_splits, G, scales, bias,
                                                dbias, dscales, workspace, as_stream(stream)),
                    fn);
}

static mxfp8_status grouped_gemm_impl(const char* fn, int32_t layout, const uint8_t* a_data,
                                      const uint8_t* a_scale, const uint8_t* b_data,
                                      const uint8_t* b_scale, void* c, int32_t c_dtype, int64_t T,
                                      int64_t N, int64_t K, const int64_t* m_splits, int32_t G,
                                      int32_t* queue, void* stream) {
  REQUIRE(layout == MXFP8_LAYOUT_NT || layout == MXFP8_LAYOUT_NN || layout == MXFP8_LAYOUT_TN,
          "%s: layout %d is not NT(0), NN(1) or TN(2)", fn, (int)layout);
  if (c_dtype != MXFP8_OUT_F32 && c_dtype != MXFP8_OUT_BF16)
    return fail(MXFP8_ENOTSUP, "%s: output dtype %d is not supported (f32 = 0, bf16 = 1)", fn,
                (int)c_dtype);
  // with no tokens nothing is read, and the forward/dgrad output is empty too
  REQUIRE(T == 0 || (a_data && a_scale && b_data && b_scale && c), "%s: NULL operand pointer",
          fn);
  REQUIRE(c || layout != MXFP8_LAYOUT_TN, "%s: NULL output", fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(N > 0 && N % 512 == 0, "%s: N = %lld must be a positive multiple of 512", fn,
          (long long)N);
  REQUIRE(K > 0 && K % 512 == 0, "%s: K = %lld must be a positive multiple of 512", fn,
          (long long)K);
  REQUIRE(G <= 1024, "%s: G = %d exceeds the supported 1024 experts", fn, (int)G);
  mxfp8_status s = check_device_splits(m_splits, G, fn);
  if (s != MXFP8_OK) return s;
  if (T == 0 && layout != MXFP8_LAYOUT_TN) return ok();
  const hipError_t e = mx::launch_grouped_gemm(layout, a_data, a_scale, b_data, b_scale, c,
                                               c_dtype == MXFP8_OUT_BF16, T, N, K, m_splits, G,
                                               false, as_stream(stream), queue);
  return hip_status(e, fn);
}

mxfp8_status mxfp8_grouped_gemm_swiglu_quantize(const uint8_t* a_data, const uint8_t* a_scale,
                                                const uint8_t* b_data, const uint8_t* b_scale,
                                                uint16_t* h, int64_t T, int64_t F, int64_t K,
                                                const int64_t* m_splits, int32_t G,
                                                uint32_t usage, uint8_t* q_row, uint8_t* s_row,
                                                uint8_t* q_col, uint8_t* s_col, void* stream) {
  const char* fn = "mxfp8_grouped_gemm_swiglu_quantize";
  REQUIRE(usage != 0 && (usage & ~(MXFP8_ROWWISE | MXFP8_COLWISE)) == 0,
          "%s: usage must be a non-empty combination of MXFP8_ROWWISE and MXFP8_COLWISE", fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(F > 0 && F % 512 == 0, "%s: F = %lld must be a positive multiple of 512", fn,
          (long long)F);
  REQUIRE(K > 0 && K % 512 == 0, "%s: K = %lld must be a positive multiple of 512", fn,
          (long long)K);
  REQUIRE(G <= 1024, "%s: G = %d exceeds the supported 1024 experts", fn, (int)G);
  if (T > 0) {
    REQUIRE(a_data && a_scale && b_data && b_scale && h, "%s: NULL operand pointer", fn);
    const bool row = usage & MXFP8_ROWWISE, col = usage & MXFP8_COLWISE;
    REQUIRE(!row || (q_row && s_row), "%s: ROWWISE requested but q_row/s_row is NULL", fn);
    REQUIRE(!col || (q_col && s_col), "%s: COLWISE requested but q_col/s_col is NULL", fn);
  }
  mxfp8_status s = check_device_splits(m_splits, G, fn);
  if (s != MXFP8_OK) return s;
  if (T == 0) return ok();   // no rows: every output is empty
  const bool row = usage & MXFP8_ROWWISE, col = usage & MXFP8_COLWISE;
  return hip_status(mx::launch_grouped_gemm_swiglu(a_data, a_scale, b_data, b_scale, h, T, F, K,
                                                   m_splits, G, row ? q_row : nullptr,
                                                   row ? s_row : nullptr, col ? q_col : nullptr,
                                                   col ? s_col : nullptr, as_stream(stream)),
                    fn);
}

static mxfp8_status wgrad_accumulate_impl(const char* fn, const uint8_t* a_data,
                                          const uint8_t* a_scale, const uint8_t* b_data,
                                          const uint8_t* b_scale, float* main_grad, int64_t T,
                                          int64_t N, int64_t K, const int64_t* m_splits,
                                          int32_t G, int32_t* queue, void* stream) {
  REQUIRE(main_grad && (T == 0 || (a_data && a_scale && b_data && b_scale)), "%s: NULL pointer",
          fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(N > 0 && N % 512 == 0, "%s: N = %lld must be a positive multiple of 512", fn,
          (long long)N);
  REQUIRE(K > 0 && K % 512 == 0, "%s: K = %lld must be a positive multiple of 512", fn,
          (long long)K);
  REQUIRE(G <= 1024, "%s: G = %d exceeds the supported 1024 experts", fn, (int)G);
  mxfp8_status s = check_device_splits(m_splits, G, fn);
  if (s != MXFP8_OK) return s;
  if (T == 0) return ok();   // every expert is empty: main_grad stays as it is
  const hipError_t e =
      mx::launch_grouped_gemm(MXFP8_LAYOUT_TN, a_data, a_scale, b_data, b_scale, main_grad, false,
                              T, N, K, m_splits, G, true, as_stream(stream), queue);
  return hip_status(e, fn);
}

// A workspace must hold the tile counter: at least mxfp8_grouped_gemm_workspace_bytes().
static mxfp8_status check_gemm_workspace(const char* fn, void* workspace, size_t bytes) {
  REQUIRE(workspace != nullptr && bytes >= mxfp8_grouped_gemm_workspace_bytes(),
          "%s: needs a device workspace of %zu bytes", fn, mxfp8_grouped_gemm_workspace_bytes());
  return MXFP8_OK;
}

size_t mxfp8_grouped_gemm_workspace_bytes(void) { return 256; }

mxfp8_status mxfp8_grouped_gemm(int32_t layout, const uint8_t* a_data, const uint8_t* a_scale,
                                const uint8_t* b_data, const uint8_t* b_scale, void* c,
                                int32_t c_dtype, int64_t T, int64_t N, int64_t K,
                                const int64_t* m_splits, int32_t G, void* stream) {
  return grouped_gemm_impl("mxfp8_grouped_gemm", layout, a_data, a_scale, b_data, b_scale, c,
                           c_dtype, T, N, K, m_splits, G, nullptr, stream);
}

mxfp8_status mxfp8_grouped_gemm_ws(int32_t layout, const uint8_t* a_data, const uint8_t* a_scale,
                                   const uint8_t* b_data, const uint8_t* b_scale, void* c,
                                   int32_t c_dtype, int64_t T, int64_t N, int64_t K,
                                   const int64_t* m_splits, int32_t G, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const char* fn = "mxfp8_grouped_gemm_ws";
  const mxfp8_status s = check_gemm_workspace(fn, workspace, workspace_bytes);
  if (s != MXFP8_OK) return s;
  return grouped_gemm_impl(fn, layout, a_data, a_scale, b_data, b_scale, c, c_dtype, T, N, K,
                           m_splits, G, static_cast<int32_t*>(workspace), stream);
}

mxfp8_status mxfp8_grouped_gemm_wgrad_accumulate(const uint8_t* a_data, const uint8_t* a_scale,
                                                 const uint8_t* b_data, const uint8_t* b_scale,
                                                 float* main_grad, int64_t T, int64_t N, int64_t K,
                                                 const int64_t* m_splits, int32_t G,
                                                 void* stream) {
  return wgrad_accumulate_impl("mxfp8_grouped_gemm_wgrad_accumulate", a_data, a_scale, b_data,
                               b_scale, main_grad, T, N, K, m_splits, G, nullptr, stream);
}

mxfp8_status mxfp8_grouped_gemm_wgrad_accumulate_ws(const uint8_t* a_data,
                                                    const uint8_t* a_scale, const uint8_t* b_data,
                                                    const uint8_t* b_scale, float* main_grad,
                                                    int64_t T, int64_t N, int64_t K,
                                                    const int64_t* m_splits, int32_t G,
                                                    void* workspace, size_t workspace_bytes,
                                                    void* stream) {
  const char* fn = "mxfp8_grouped_gemm_wgrad_accumulate_ws";
  const mxfp8_status s = check_gemm_workspace(fn, workspace, workspace_bytes);
  if (s != MXFP8_OK) return s;
  return wgrad_accumulate_impl(fn, a_data, a_scale, b_data, b_scale, main_grad, T, N, K, m_splits,
                               G, static_cast<int32_t*>(workspace), stream);
}

mxfp8_status mxfp8_validate_splits(const int64_t* m_splits, int32_t G, int64_t T, int32_t* flag,
                                   void* stream) {
  const char* fn = "mxfp8_validate_splits";
  REQUIRE(flag != nullptr, "%s: flag is NULL", fn);
  REQUIRE(G <= 1 << 20, "%s: G = %d is too large", fn, (int)G);
  mxfp8_status s = check_device_splits(m_splits, G, fn);
  if (s != MXFP8_OK) return s;
  return hip_status(mx::launch_validate_splits(m_splits, G, T, flag, as_stream(stream)), fn);
}

mxfp8_status mxfp8_swiglu_fwd(const uint16_t* h, int64_t T, int64_t F, uint16_t* a,
                              void* stream) {
  const char* fn = "mxfp8_swiglu_fwd";
  REQUIRE(T == 0 || (h && a), "%s: NULL pointer", fn);
  REQUIRE(T >= 0, "%s: T < 0", fn);
  REQUIRE(F > 0 && F % 8 == 0, "%s: F = %lld must be a positive multiple of 8", fn, (long long)F);
  if (T == 0) return ok();
  return hip_status(mx::launch_swiglu_fwd(h, T, F, a, as_stream(stream)), fn);
}

mxfp8_status mxfp8_swiglu_quantize(const uint16_t* h, int64_t T, int64_t F, uint32_t usage,
                                   uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                   uint8_t* s_col, void* stream) {
  const char* fn = "mxfp8_swiglu_quantize";
  REQUIRE(h != nullptr || T == 0, "%s: h is NULL", fn);
  REQUIRE(usage != 0 && (usage & ~(MXFP8_ROWWISE | MXFP8_COLWISE)) == 0,
          "%s: usage must be a non-empty combination of MXFP8_ROWWISE and MXFP8_COLWISE", fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(F > 0 && F % 512 == 0, "%s: F = %lld must be a positive multiple of 512", fn,
          (long long)F);
  if (T == 0) return ok();   // nothing to read or write: every buffer is empty
  const bool row = usage & MXFP8_ROWWISE, col = usage & MXFP8_COLWISE;
  REQUIRE(!row || (q_row && s_row), "%s: ROWWISE requested but q_row/s_row is NULL", fn);
  REQUIRE(!col || (q_col && s_col), "%s: COLWISE requested but q_col/s_col is NULL", fn);
  return hip_status(mx::launch_swiglu_quant(h, T, F, row ? q_row : nullptr, row ? s_row : nullptr,
                                            col ? q_col : nullptr, col ? s_col : nullptr,
                                            as_stream(stream)),
                    fn);
}

mxfp8_status mxfp8_swiglu_bwd(const uint16_t* h, const uint16_t* da, int64_t T, int64_t F,
                              uint16_t* dh, void* stream) {
  const char* fn = "mxfp8_swiglu_bwd";
  REQUIRE(T == 0 || (h && da && dh), "%s: NULL pointer", fn);
  REQUIRE(T >= 0, "%s: T < 0", fn);
  REQUIRE(F > 0 && F % 8 == 0, "%s: F = %lld must be a positive multiple of 8", fn, (long long)F);
  if (T == 0) return ok();
  return hip_status(mx::launch_swiglu_bwd(h, da, T, F, dh, as_stream(stream)), fn);
}

mxfp8_status mxfp8_swiglu_bwd_quantize(const uint16_t* h, const uint16_t* da, int64_t T,
                                       int64_t F, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                       uint8_t* s_col, const int64_t* m_splits, int32_t G,
                                       float* dbias, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  const char* fn = "mxfp8_swiglu_bwd_quantize";
  REQUIRE(T == 0 || (h && da && q_row && s_row && q_col && s_col), "%s: NULL pointer", fn);
  REQUIRE(T >= 0 && T % 128 == 0, "%s: T = %lld must be a multiple of 128", fn, (long long)T);
  REQUIRE(F > 0 && F % 256 == 0, "%s: F = %lld must be a positive multiple of 256", fn,
          (long long)F);
  const int64_t K = 2 * F;
  float* partial = nullptr;
  if (dbias != nullptr) {
    mxfp8_status st = check_device_splits(m_splits, G, fn);
    if (st != MXFP8_OK) return st;
    REQUIRE((workspace != nullptr || T == 0) &&
                workspace_bytes >= mxfp8_dbias_workspace_bytes(T, K),
            "%s: dbias needs a workspace of %zu bytes", fn, mxfp8_dbias_workspace_bytes(T, K));
    partial = static_cast<float*>(workspace);
  }
  hipStream_t st = as_stream(stream);
  hipError_t e = hipSuccess;
  if (T > 0)
    e = mx::launch_swiglu_bwd_quant(h, da, T, F, q_row, s_row, q_col, s_col, partial, st);
  if (e == hipSuccess && dbias != nullptr)
    e = mx::launch_dbias_finalize(partial, m_splits, G, T, K, dbias, st);
  return hip_status(e, fn);
}

size_t mxfp8_convert_sweep_bytes(int32_t mode) { return mx::convert_sweep_bytes(mode); }

mxfp8_status mxfp8_convert_sweep(int32_t mode, void* out, size_t out_bytes, void* stream) {
  const char* fn = "mxfp8_convert_sweep";
  const size_t need = mx::convert_sweep_bytes(mode);
  REQUIRE(need != 0, "%s: unknown mode %d", fn, (int)mode);
  REQUIRE(out != nullptr && out_bytes >= need, "%s: mode %d needs a buffer of %zu bytes", fn,
          (int)mode, need);
  return hip_status(mx::launch_convert_sweep(mode, static_cast<uint8_t*>(out), as_stream(stream)),
                    fn);
}

}  // extern "C"
