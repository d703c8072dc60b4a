// Host-side launchers of the MBOK kernels; called by the C ABI after it has
// validated every argument.  Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mbok.h"

namespace mbok {

int launch_residual_binarize(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs,
                             void* alpha, int32_t* flag, hipStream_t stream);
int launch_residual_energy(const mbok_desc* d, const float* W, int64_t ldw, double* rows,
                           double* layer, hipStream_t stream);
int launch_refit(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs, void* alpha,
                 int rounds, hipStream_t stream);
int refit_max_rounds();
int launch_pack(const mbok_desc* d, const int8_t* signs, const void* alpha, void* packed,
                hipStream_t stream);
int launch_gemv(const mbok_desc* d, const void* packed, const void* x, int32_t x_dtype,
                float* y, void* workspace, hipStream_t stream);
size_t gemv_workspace_bytes(const mbok_desc* d);
int launch_gemv_f4(const mbok_desc* d, const void* packed, const void* x, float* y,
                   hipStream_t stream);
// the same matrix-core product for 1..gemm_f4_max_tokens() bf16 tokens
int launch_gemm_f4(const mbok_desc* d, const void* packed, const void* X, int64_t T,
                   int64_t ldx, float* Y, int64_t ldy, hipStream_t stream);
int gemm_f4_max_tokens();
// 1..gemm_f4g_max_tokens() tokens with one product per group (8 tokens each)
int launch_gemm_f4g(const mbok_desc* d, const void* packed, const void* X, int64_t T,
                    int64_t ldx, float* Y, int64_t ldy, hipStream_t stream);
int gemm_f4g_max_tokens();
int launch_gemvt(const mbok_desc* d, const void* packed, const void* grad, int32_t g_dtype,
                 float* dx, void* ws, hipStream_t stream);
size_t gemvt_workspace_bytes(const mbok_desc* d);
int launch_gemvt_noalloc(const mbok_desc* d, const void* packed, const void* grad,
                         int32_t g_dtype, float* dx, hipStream_t stream);
size_t gemvt_scratch_bytes();
int launch_skinny(const mbok_desc* d, const void* packed, const void* X, int64_t T, int64_t ldx,
                  float* Y, int64_t ldy, hipStream_t stream);
int skinny_max_tokens();
size_t svid_workspace_bytes(const mbok_desc* d);
int launch_svid_decompose(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs,
                          void* s_out, void* s_in, int iters, void* ws, hipStream_t stream);
int launch_svid_pack(const mbok_desc* d, const int8_t* signs, const void* s_out, void* packed,
                     hipStream_t stream);
int launch_svid_skinny(const mbok_desc* d, const void* packed, const void* x, int32_t x_dtype,
                       const void* s_in, float* y, hipStream_t stream);
// the same product on the fp4 x fp8 decode kernel (gemv_f4.hip)
int launch_svid_f4(const mbok_desc* d, const void* packed, const void* x, int32_t x_dtype,
                   const void* s_in, float* y, hipStream_t stream);
int allocate_kernels(int L, const int64_t* sizes, const double* errors, int kmax, int64_t budget,
                     int32_t* K_out);
// passes: 1 = prefill levels rounded to bf16; 2 = plus a second pass with
// the bf16 residues of the levels (T <= 16 runs the same kernels either way)
int launch_gemm(const mbok_desc* d, const void* packed, const void* X, int64_t T, int64_t ldx,
                float* Y, int64_t ldy, int passes, hipStream_t stream);

}  // namespace mbok
