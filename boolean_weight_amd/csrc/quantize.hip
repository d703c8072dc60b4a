// Greedy residual binarization on the GPU: W (fp32) -> K sign planes (int8)
// and group scales (fp16 or fp32), float64 residual arithmetic.
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// Paper-Notes reading note, 训练策略 (kernels initialised from the pretrained
// weight by greedy search) and 关键设计 (closed-form least-squares scale for
// fixed signs); the gist.science summaries' "Successive SVID" (each kernel is
// fitted to the residual of the previous ones).
//
// Four lanes per (row, group), 32 columns each; the weights stay in
// registers and each residual R_k is recomputed from them in kernel order.
// The group sum of |R| is formed exactly as an unevaluated float64 pair
// (sum, error) with error-free additions, then rounded once to float64, so
// the scale equals round(fsum(|R|) / 128) in the scale dtype.  (The pair sum
// is exact when the group's residual magnitudes lie within about 2^48 of
// one another; the residuals of a group share the scales' quantum, so this
// holds for any trained layer.)
#include "mbok_device.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

template <bool F16, int K>
__global__ void __launch_bounds__(256) residual_binarize_kernel(
    const float* __restrict__ W, int64_t ldw, int m, int n, int8_t* __restrict__ signs,
    void* __restrict__ alpha, int32_t* __restrict__ flag) {
  const int G = n / kGroup;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t task = tid >> 2;
  const int q = (int)(tid & 3);
  if (task >= (int64_t)m * G) return;  // whole quads exit together
  const int i = (int)(task / G);
  const int g = (int)(task % G);
  const int64_t col = (int64_t)g * kGroup + 32 * q;

  float w[32];
  load_weights32(W + (int64_t)i * ldw + col, w);
  if (flag) {
    bool finite = true;
#pragma unroll
    for (int j = 0; j < 32; ++j) finite = finite && isfinite(w[j]);
    if (!finite) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  uint32_t bits[K];  // bit j: column 32q + j is +1
  double a_st[K];    // stored (rounded) scales
#pragma unroll
  for (int k = 0; k < K; ++k) {
    // R_k of each column, recomputed from W in kernel order:
    // r = (((w - a_0 s_0) - a_1 s_1) - ...), each step one float64 rounding
    double h0 = 0.0, l0 = 0.0, h1 = 0.0, l1 = 0.0;
    uint32_t b = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      double r = (double)w[j];
#pragma unroll
      for (int p = 0; p < k; ++p) r = ((bits[p] >> j) & 1u) ? r - a_st[p] : r + a_st[p];
      b |= (uint32_t)(r >= 0.0) << j;  // sign(0) = sign(-0) = +1
      if (j & 1)
        dd_acc(h1, l1, fabs(r));
      else
        dd_acc(h0, l0, fabs(r));
    }
    bits[k] = b;
    two_sum(h0, l0, h0, l0);
    two_sum(h1, l1, h1, l1);
    dd_add(h0, l0, h1, l1);
    quad_sum_dd(h0, l0, q);
    const double a = (h0 + l0) / (double)kGroup;  // one rounding, then exact /128
    a_st[k] = F16 ? (double)f16_bits_to_f32(f64_to_f16_rne(a))
                  : (double)(float)a;  // v_cvt_f32_f64: nearest-even
  }
#pragma unroll
  for (int k = 0; k < K; ++k)
    store_sign_bits32(signs + ((int64_t)k * m + i) * n + col, bits[k]);
  if (q < K) {
    // lane q stores scale q (its value is bit-identical in every lane)
    double aq = a_st[0];
#pragma unroll
    for (int k = 1; k < K; ++k) aq = (q == k) ? a_st[k] : aq;
    const int64_t aidx = ((int64_t)q * m + i) * G + g;
    if (F16)
      reinterpret_cast<uint16_t*>(alpha)[aidx] = f64_to_f16_rne(aq);  // exact: aq is fp16
    else
      reinterpret_cast<float*>(alpha)[aidx] = (float)aq;
  }
}

template <bool F16>
int launch_dt(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs, void* alpha,
              int32_t* flag, hipStream_t stream) {
  const int G = d->n / kGroup;
  const int64_t tasks = (int64_t)d->m * G;
  const int block = 256;
  const int64_t blocks = (4 * tasks + block - 1) / block;
  if (blocks > 0x7fffffff) return MBOK_ERR_SHAPE;
  dim3 grid((unsigned)blocks);
  switch (d->K) {
    case 1:
      hipLaunchKernelGGL((residual_binarize_kernel<F16, 1>), grid, dim3(block), 0, stream, W, ldw,
                         d->m, d->n, signs, alpha, flag);
      break;
    case 2:
      hipLaunchKernelGGL((residual_binarize_kernel<F16, 2>), grid, dim3(block), 0, stream, W, ldw,
                         d->m, d->n, signs, alpha, flag);
      break;
    case 3:
      hipLaunchKernelGGL((residual_binarize_kernel<F16, 3>), grid, dim3(block), 0, stream, W, ldw,
                         d->m, d->n, signs, alpha, flag);
      break;
    case 4:
      hipLaunchKernelGGL((residual_binarize_kernel<F16, 4>), grid, dim3(block), 0, stream, W, ldw,
                         d->m, d->n, signs, alpha, flag);
      break;
    default:
      return MBOK_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

}  // namespace

int launch_residual_binarize(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs,
                             void* alpha, int32_t* flag, hipStream_t stream) {
  if (d->alpha_dtype == MBOK_F16) return launch_dt<true>(d, W, ldw, signs, alpha, flag, stream);
  return launch_dt<false>(d, W, ldw, signs, alpha, flag, stream);
}

}  // namespace mbok
