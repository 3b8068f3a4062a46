// Internal launcher declarations (host side).  Each launcher enqueues its
// kernels on `st` and returns hipGetLastError(); shapes are validated by the
// C-ABI layer before any launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// noop: NULL, or a device int32 that, when non-zero as the kernel runs, makes
// the launch write nothing.
hipError_t launch_quant_rowwise(const uint16_t* x, int64_t T, int64_t K, uint8_t* q, uint8_t* s,
                                const int32_t* noop, hipStream_t st);
hipError_t launch_quant_rowcol(const uint16_t* x, int64_t T, int64_t K, uint8_t* q_row,
                               uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                               const int32_t* noop, hipStream_t st);
hipError_t launch_quant_row_requant(const uint16_t* x, int64_t T, int64_t K, uint8_t* q_row,
                                   uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, float* partial,
                                   hipStream_t st);
hipError_t launch_requant_colwise(const uint8_t* q_row, const uint8_t* s_row, int64_t T,
                                  int64_t K, uint8_t* q_col, uint8_t* s_col, float* partial,
                                  hipStream_t st);
hipError_t launch_dbias_partial(const uint8_t* q_row, const uint8_t* s_row, int64_t T, int64_t N,
                                float* partial, hipStream_t st);
hipError_t launch_scaled_bias_grad(const uint8_t* q_row, const uint8_t* s_row, int64_t T,
                                   int64_t N, const int64_t* m_splits, int32_t G,
                                   const float* scales, const float* bias, float* dbias,
                                   float* dscale, void* workspace, hipStream_t st);
size_t scaled_bias_workspace_bytes(int64_t T, int64_t N);
hipError_t launch_dbias_finalize(const float* partial, const int64_t* m_splits, int32_t G,
                                 int64_t T, int64_t K, float* dbias, hipStream_t st);
hipError_t launch_validate_splits(const int64_t* m_splits, int32_t G, int64_t T, int32_t* flag,
                                  hipStream_t st);
hipError_t launch_swiglu_fwd(const uint16_t* h, int64_t T, int64_t F, uint16_t* a,
                             hipStream_t st);
hipError_t launch_swiglu_quant(const uint16_t* h, int64_t T, int64_t F, uint8_t* q_row,
                               uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t st);
hipError_t launch_swiglu_bwd(const uint16_t* h, const uint16_t* da, int64_t T, int64_t F,
                             uint16_t* dh, hipStream_t st);
hipError_t launch_swiglu_bwd_quant(const uint16_t* h, const uint16_t* da, int64_t T, int64_t F,
                                   uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                                   float* partial, hipStream_t st);
size_t convert_sweep_bytes(int32_t mode);   // 0 for an unknown mode
// The file-scope device scratch of quantize.hip: its size, and its address on
// the current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(float** out);
hipError_t launch_convert_sweep(int32_t mode, uint8_t* out, hipStream_t st);
hipError_t launch_grouped_gemm(int layout, const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                               const uint8_t* sb, void* c, bool out_bf16, int64_t T, int64_t N,
                               int64_t K, const int64_t* m_splits, int32_t G, bool accumulate,
                               hipStream_t st, int32_t* queue = nullptr);
// Forward NT with bf16 h [T, 2F] (gate | up), fused with the SwiGLU of h and
// the row- and/or column-wise quantize of a = silu(gate) * up [T, F].
hipError_t launch_grouped_gemm_swiglu(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                                      const uint8_t* sb, uint16_t* h, int64_t T, int64_t F,
                                      int64_t K, const int64_t* m_splits, int32_t G,
                                      uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                      uint8_t* s_col, hipStream_t st);

}  // namespace mx
