// Greedy residual binarization on the GPU: W (fp32) -> K sign planes (int8)
// and group scales (fp16 or fp32), float64 residual arithmetic.
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// Paper-Notes reading note, 训练策略 (kernels initialised from the pretrained
// weight by greedy search) and 关键设计 (closed-form least-squares scale for
// fixed signs); the gist.science summaries' "Successive SVID" (each kernel is
// fitted to the residual of the previous ones).
//
// One wavefront per (row, group): lane l holds columns 2l and 2l+1 of the
// group.  The group sum of |R| is reduced as an unevaluated float64 pair
// (sum, error) with error-free additions in a fixed order, then rounded once
// to float64, so the scale equals round(fsum(|R|) / 128) in the scale dtype.
#include "mbok_device.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

template <bool F16>
__global__ void __launch_bounds__(256) residual_binarize_kernel(
    const float* __restrict__ W, int64_t ldw, int m, int n, int K,
    int8_t* __restrict__ signs, void* __restrict__ alpha, int32_t* __restrict__ flag) {
  const int lane = threadIdx.x & (kWave - 1);
  const int G = n / kGroup;
  const int64_t task = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (task >= (int64_t)m * G) return;  // whole wave exits together
  const int i = (int)(task / G);
  const int g = (int)(task % G);
  const int64_t col = (int64_t)g * kGroup + 2 * lane;

  const float2 w2 = *reinterpret_cast<const float2*>(W + (int64_t)i * ldw + col);
  double r0 = (double)w2.x, r1 = (double)w2.y;
  if (flag && (!isfinite(w2.x) || !isfinite(w2.y))) {
    __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int k = 0; k < K; ++k) {
    const double s0 = (r0 >= 0.0) ? 1.0 : -1.0;  // sign(0) = sign(-0) = +1
    const double s1 = (r1 >= 0.0) ? 1.0 : -1.0;
    double hi, lo;
    two_sum(fabs(r0), fabs(r1), hi, lo);
    wave_sum_dd(hi, lo, lane);
    const double a = (hi + lo) / (double)kGroup;  // one rounding, then exact /128
    double a_st;
    const int64_t aidx = ((int64_t)k * m + i) * G + g;
    if (F16) {
      const uint16_t h = f64_to_f16_rne(a);
      a_st = (double)f16_bits_to_f32(h);
      if (lane == 0) reinterpret_cast<uint16_t*>(alpha)[aidx] = h;
    } else {
      const float f = (float)a;  // v_cvt_f32_f64: nearest-even
      a_st = (double)f;
      if (lane == 0) reinterpret_cast<float*>(alpha)[aidx] = f;
    }
    const int64_t sidx = ((int64_t)k * m + i) * n + col;
    char2 sv;
    sv.x = (int8_t)s0;
    sv.y = (int8_t)s1;
    *reinterpret_cast<char2*>(signs + sidx) = sv;
    r0 = r0 - a_st * s0;
    r1 = r1 - a_st * s1;
  }
}

}  // namespace

int launch_residual_binarize(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs,
                             void* alpha, int32_t* flag, hipStream_t stream) {
  const int G = d->n / kGroup;
  const int64_t tasks = (int64_t)d->m * G;
  const int waves_per_block = 4;
  const int64_t blocks = (tasks + waves_per_block - 1) / waves_per_block;
  if (blocks > 0x7fffffff) return MBOK_ERR_SHAPE;
  dim3 grid((unsigned)blocks), block(waves_per_block * kWave);
  if (d->alpha_dtype == MBOK_F16)
    hipLaunchKernelGGL(residual_binarize_kernel<true>, grid, block, 0, stream, W, ldw, d->m,
                       d->n, d->K, signs, alpha, flag);
  else
    hipLaunchKernelGGL(residual_binarize_kernel<false>, grid, block, 0, stream, W, ldw, d->m,
                       d->n, d->K, signs, alpha, flag);
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

}  // namespace mbok
