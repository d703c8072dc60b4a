// Multi-token product Y = X . W_hat^T (interim: one decode launch per token).
#include "mbok_device.h"
#include "mbok_launch.h"

namespace mbok {

int launch_gemm(const mbok_desc* d, const void* packed, const void* X, int64_t T, int64_t ldx,
                float* Y, int64_t ldy, hipStream_t stream) {
  const uint16_t* Xb = reinterpret_cast<const uint16_t*>(X);
  for (int64_t t = 0; t < T; ++t) {
    const int st = launch_gemv(d, packed, Xb + t * ldx, MBOK_BF16, Y + t * ldy, nullptr, stream);
    if (st != MBOK_OK) return st;
  }
  return MBOK_OK;
}

}  // namespace mbok
