// C ABI of the MBOK library: argument validation and dispatch.  Every check
// runs on the host before anything is enqueued; nothing here allocates,
// synchronises or keeps state.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>

#include "../../include/mbok.h"
#include "mbok_launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Checks a descriptor that may have been filled by hand.
int check_desc(const mbok_desc* d) {
  if (!d) return MBOK_ERR_INVALID_ARG;
  if (d->m < 1 || d->m > (1 << 24)) return MBOK_ERR_SHAPE;
  if (d->n < MBOK_GROUP || d->n > (1 << 20) || d->n % MBOK_GROUP) return MBOK_ERR_SHAPE;
  if (d->K < 1 || d->K > MBOK_MAX_K) return MBOK_ERR_UNSUPPORTED;
  if (d->group != MBOK_GROUP) return MBOK_ERR_UNSUPPORTED;
  if (d->alpha_dtype != MBOK_F32 && d->alpha_dtype != MBOK_F16) return MBOK_ERR_DTYPE;
  if (d->layout != MBOK_LAYOUT_L64) return MBOK_ERR_UNSUPPORTED;
  return MBOK_OK;
}

size_t alpha_size(int32_t dt) { return dt == MBOK_F16 ? 2 : 4; }

}  // namespace

extern "C" {

int mbok_desc_init(mbok_desc* d, int32_t m, int32_t n, int32_t K, int32_t alpha_dtype) {
  if (!d) return MBOK_ERR_INVALID_ARG;
  mbok_desc t;
  t.m = m;
  t.n = n;
  t.K = K;
  t.group = MBOK_GROUP;
  t.alpha_dtype = alpha_dtype;
  t.layout = MBOK_LAYOUT_L64;
  const int st = check_desc(&t);
  if (st != MBOK_OK) return st;
  *d = t;
  return MBOK_OK;
}

size_t mbok_packed_bytes(const mbok_desc* d) {
  if (check_desc(d) != MBOK_OK) return 0;
  const size_t m_pad = ((size_t)d->m + MBOK_ROW_BLOCK - 1) / MBOK_ROW_BLOCK * MBOK_ROW_BLOCK;
  const size_t G = (size_t)d->n / MBOK_GROUP;
  return (size_t)d->K * m_pad * (size_t)d->n / 8 +
         (size_t)d->K * m_pad * G * alpha_size(d->alpha_dtype);
}

size_t mbok_alpha_bytes(const mbok_desc* d) {
  if (check_desc(d) != MBOK_OK) return 0;
  return (size_t)d->K * (size_t)d->m * ((size_t)d->n / MBOK_GROUP) * alpha_size(d->alpha_dtype);
}

int mbok_residual_binarize(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs,
                           void* alpha, int32_t* flag, void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!W || !signs || !alpha) return MBOK_ERR_INVALID_ARG;
  if (ldw < d->n) return MBOK_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(signs, 16) || !aligned(alpha, 16) || (ldw % 4) != 0)
    return MBOK_ERR_ALIGN;
  if (flag && !aligned(flag, 4)) return MBOK_ERR_ALIGN;
  return mbok::launch_residual_binarize(d, W, ldw, signs, alpha, flag, (hipStream_t)stream);
}

int mbok_residual_energy(const mbok_desc* d, const float* W, int64_t ldw, double* row_energy,
                         double* layer_energy, void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!W || !row_energy || !layer_energy) return MBOK_ERR_INVALID_ARG;
  if (ldw < d->n) return MBOK_ERR_INVALID_ARG;
  if (!aligned(W, 16) || (ldw % 4) != 0 || !aligned(row_energy, 8) || !aligned(layer_energy, 8))
    return MBOK_ERR_ALIGN;
  return mbok::launch_residual_energy(d, W, ldw, row_energy, layer_energy, (hipStream_t)stream);
}

int mbok_allocate_kernels(int32_t L, const int64_t* sizes, const double* errors, int32_t kmax,
                          int64_t budget, int32_t* K_out) {
  if (!sizes || !errors || !K_out || L < 1 || kmax < 1 || kmax > MBOK_MAX_K || budget < 0)
    return MBOK_ERR_INVALID_ARG;
  for (int32_t l = 0; l < L; ++l) {
    if (sizes[l] < 1 || sizes[l] > (int64_t(1) << 44)) return MBOK_ERR_INVALID_ARG;
    for (int32_t k = 0; k < kmax; ++k) {
      const double e = errors[(size_t)l * kmax + k];
      if (!std::isfinite(e) || e < 0.0) return MBOK_ERR_INVALID_ARG;
    }
  }
  return mbok::allocate_kernels(L, sizes, errors, kmax, budget, K_out);
}

size_t mbok_svid_workspace_bytes(const mbok_desc* d) {
  if (check_desc(d) != MBOK_OK) return 0;
  return mbok::svid_workspace_bytes(d);
}

int mbok_svid_decompose(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs,
                        void* s_out, void* s_in, int32_t iters, void* workspace, void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!W || !signs || !s_out || !s_in || !workspace) return MBOK_ERR_INVALID_ARG;
  if (ldw < d->n || iters < 1 || iters > MBOK_MAX_SVID_ITERS) return MBOK_ERR_INVALID_ARG;
  if (!aligned(W, 16) || (ldw % 4) != 0 || !aligned(signs, 16) || !aligned(s_out, 4) ||
      !aligned(s_in, 4) || !aligned(workspace, 256))
    return MBOK_ERR_ALIGN;
  return mbok::launch_svid_decompose(d, W, ldw, signs, s_out, s_in, iters, workspace,
                                     (hipStream_t)stream);
}

int mbok_svid_pack(const mbok_desc* d, const int8_t* signs, const void* s_out, void* packed,
                   void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!signs || !s_out || !packed) return MBOK_ERR_INVALID_ARG;
  if (!aligned(signs, 16) || !aligned(s_out, 4) || !aligned(packed, 16)) return MBOK_ERR_ALIGN;
  return mbok::launch_svid_pack(d, signs, s_out, packed, (hipStream_t)stream);
}

size_t mbok_svid_gemv_workspace_bytes(const mbok_desc* d) {
  (void)d;
  return 0;
}

int mbok_svid_gemv(const mbok_desc* d, const void* packed, const void* s_in, const void* x,
                   int32_t x_dtype, float* y, void* workspace, void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!packed || !s_in || !x || !y) return MBOK_ERR_INVALID_ARG;
  if (x_dtype != MBOK_BF16 && x_dtype != MBOK_F32) return MBOK_ERR_DTYPE;
  if (!aligned(packed, 16) || !aligned(s_in, 16) || !aligned(x, 16) || !aligned(y, 4) ||
      (workspace && !aligned(workspace, 256)))
    return MBOK_ERR_ALIGN;
  // the fp4 x fp8 form by default; MBOK_SVID_VARIANT=skinny selects the bf16
  // +-1 form (measurements)
  const char* v = getenv("MBOK_SVID_VARIANT");
  if (v && strcmp(v, "skinny") == 0)
    return mbok::launch_svid_skinny(d, packed, x, x_dtype, s_in, y, (hipStream_t)stream);
  return mbok::launch_svid_f4(d, packed, x, x_dtype, s_in, y, (hipStream_t)stream);
}

int mbok_refit(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs, void* alpha,
               int32_t rounds, void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!W || !signs || !alpha) return MBOK_ERR_INVALID_ARG;
  if (ldw < d->n) return MBOK_ERR_INVALID_ARG;
  if (rounds < 0 || rounds > MBOK_MAX_REFIT_ROUNDS || rounds > mbok::refit_max_rounds())
    return MBOK_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(signs, 16) || !aligned(alpha, 16) || (ldw % 4) != 0)
    return MBOK_ERR_ALIGN;
  return mbok::launch_refit(d, W, ldw, signs, alpha, rounds, (hipStream_t)stream);
}

int mbok_pack(const mbok_desc* d, const int8_t* signs, const void* alpha, void* packed,
              void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!signs || !alpha || !packed) return MBOK_ERR_INVALID_ARG;
  if (!aligned(signs, 16) || !aligned(alpha, 16) || !aligned(packed, 16)) return MBOK_ERR_ALIGN;
  return mbok::launch_pack(d, signs, alpha, packed, (hipStream_t)stream);
}

size_t mbok_gemv_workspace_bytes(const mbok_desc* d) {
  if (check_desc(d) != MBOK_OK) return 0;
  return mbok::gemv_workspace_bytes(d);
}

int mbok_gemv(const mbok_desc* d, const void* packed, const void* x, int32_t x_dtype, float* y,
              void* workspace, void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!packed || !x || !y) return MBOK_ERR_INVALID_ARG;
  if (x_dtype != MBOK_BF16 && x_dtype != MBOK_F32) return MBOK_ERR_DTYPE;
  if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(y, 4)) return MBOK_ERR_ALIGN;
  if (workspace && !aligned(workspace, 256)) return MBOK_ERR_ALIGN;
  return mbok::launch_gemv(d, packed, x, x_dtype, y, workspace, (hipStream_t)stream);
}

size_t mbok_gemvt_workspace_bytes(const mbok_desc* d) {
  if (check_desc(d) != MBOK_OK) return 0;
  return mbok::gemvt_workspace_bytes(d);
}

int mbok_gemvt(const mbok_desc* d, const void* packed, const void* g, int32_t g_dtype, float* dx,
               void* workspace, void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!packed || !g || !dx) return MBOK_ERR_INVALID_ARG;
  if (g_dtype != MBOK_BF16 && g_dtype != MBOK_F32) return MBOK_ERR_DTYPE;
  if (!aligned(packed, 16) || !aligned(g, g_dtype == MBOK_BF16 ? 2 : 4) || !aligned(dx, 4))
    return MBOK_ERR_ALIGN;
  if (workspace && !aligned(workspace, 256)) return MBOK_ERR_ALIGN;
  return mbok::launch_gemvt(d, packed, g, g_dtype, dx, workspace, (hipStream_t)stream);
}

size_t mbok_gemvt_scratch_bytes(void) { return mbok::gemvt_scratch_bytes(); }

int mbok_gemvt_noalloc(const mbok_desc* d, const void* packed, const void* g, int32_t g_dtype,
                       float* dx, void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!packed || !g || !dx) return MBOK_ERR_INVALID_ARG;
  if (g_dtype != MBOK_BF16 && g_dtype != MBOK_F32) return MBOK_ERR_DTYPE;
  if (!aligned(packed, 16) || !aligned(g, g_dtype == MBOK_BF16 ? 2 : 4) || !aligned(dx, 4))
    return MBOK_ERR_ALIGN;
  return mbok::launch_gemvt_noalloc(d, packed, g, g_dtype, dx, (hipStream_t)stream);
}

static int gemm_checked(const mbok_desc* d, const void* packed, const void* X, int32_t x_dtype,
                        int64_t T, int64_t ldx, float* Y, int64_t ldy, int passes,
                        void* stream) {
  int st = check_desc(d);
  if (st != MBOK_OK) return st;
  if (!packed || !X || !Y) return MBOK_ERR_INVALID_ARG;
  if (T < 1 || T > MBOK_MAX_T) return MBOK_ERR_SHAPE;
  if (ldx < d->n || ldy < d->m) return MBOK_ERR_INVALID_ARG;
  if (x_dtype != MBOK_BF16) return MBOK_ERR_DTYPE;
  if (!aligned(packed, 16) || !aligned(X, 16) || (ldx % 8) != 0 || !aligned(Y, 4))
    return MBOK_ERR_ALIGN;
  return mbok::launch_gemm(d, packed, X, T, ldx, Y, ldy, passes, (hipStream_t)stream);
}

int mbok_gemm(const mbok_desc* d, const void* packed, const void* X, int32_t x_dtype, int64_t T,
              int64_t ldx, float* Y, int64_t ldy, void* stream) {
  return gemm_checked(d, packed, X, x_dtype, T, ldx, Y, ldy, 1, stream);
}

int mbok_gemm_precise(const mbok_desc* d, const void* packed, const void* X, int32_t x_dtype,
                      int64_t T, int64_t ldx, float* Y, int64_t ldy, void* stream) {
  return gemm_checked(d, packed, X, x_dtype, T, ldx, Y, ldy, 2, stream);
}

const char* mbok_status_str(int status) {
  switch (status) {
    case MBOK_OK: return "MBOK_OK: success";
    case MBOK_ERR_INVALID_ARG: return "MBOK_ERR_INVALID_ARG: null pointer, unknown enum or bad leading dimension";
    case MBOK_ERR_SHAPE: return "MBOK_ERR_SHAPE: m, n or T out of range, or n not a multiple of 128";
    case MBOK_ERR_DTYPE: return "MBOK_ERR_DTYPE: element type not accepted by this call";
    case MBOK_ERR_ALIGN: return "MBOK_ERR_ALIGN: pointer or leading dimension misaligned";
    case MBOK_ERR_HIP: return "MBOK_ERR_HIP: the HIP runtime rejected a launch";
    case MBOK_ERR_UNSUPPORTED: return "MBOK_ERR_UNSUPPORTED: K, group or layout outside what the library runs";
    case MBOK_ERR_INFEASIBLE: return "MBOK_ERR_INFEASIBLE: no kernel allocation fits the bit budget";
    case MBOK_ERR_SCRATCH: return "MBOK_ERR_SCRATCH: the call needs more scratch than the library's static scratch holds";
  }
  return "unknown status";
}

const char* mbok_version(void) { return "mbok 0.1.0 gfx950"; }

}  // extern "C"
