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
// Every float64 operation in this file is an exact or a once-rounded IEEE
// operation: no multiply may be fused into a following add (that would
// break the error-free sums), so contraction is off for the whole file.
#pragma clang fp contract(off)

#include "mbok_exact.h"
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

// Residual energies of the greedy chain, per row: rows[k * m + i] = the
// float64 nearest to sum_j R_k[i, j]^2 for k = 0..K (R_0 = W).  One
// workgroup per row; quad t of the workgroup takes the row's groups t, t + Q,
// ...  Each lane recomputes R_0..R_K of its 32 columns in the quantizer's
// order (the scales come out bit-identical to residual_binarize_kernel's)
// and accumulates the exact squares (a product and its fused-multiply-add
// error) into float64 pairs; the quads' pairs are then added in quad order.
constexpr int kEnergyMaxQuads = 64;

template <bool F16, int K>
__global__ void __launch_bounds__(256) residual_energy_kernel(const float* __restrict__ W,
                                                              int64_t ldw, int m, int n,
                                                              double* __restrict__ rows) {
  __shared__ double sh_hi[kEnergyMaxQuads][K + 1];
  __shared__ double sh_lo[kEnergyMaxQuads][K + 1];
  const int i = blockIdx.x;
  const int G = n / kGroup;
  const int nquads = blockDim.x >> 2;
  const int quad = threadIdx.x >> 2;
  const int q = threadIdx.x & 3;
  double eh[K + 1], el[K + 1];
#pragma unroll
  for (int k = 0; k <= K; ++k) eh[k] = el[k] = 0.0;

  for (int g = quad; g < G; g += nquads) {  // the same trip count in a quad
    float w[32];
    load_weights32(W + (int64_t)i * ldw + (int64_t)g * kGroup + 32 * q, w);
    uint32_t bits[K];
    double a_st[K];
#pragma unroll
    for (int k = 0; k <= K; ++k) {
      double h0 = 0.0, l0 = 0.0, h1 = 0.0, l1 = 0.0;
      uint32_t b = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        double r = (double)w[j];
#pragma unroll
        for (int p = 0; p < k; ++p) r = ((bits[p] >> j) & 1u) ? r - a_st[p] : r + a_st[p];
        const double sq = r * r, sqe = __fma_rn(r, r, -sq);
        dd_acc(eh[k], el[k], sq);
        el[k] += sqe;
        if (k < K) {
          b |= (uint32_t)(r >= 0.0) << j;
          if (j & 1)
            dd_acc(h1, l1, fabs(r));
          else
            dd_acc(h0, l0, fabs(r));
        }
      }
      if (k < K) {
        bits[k] = b;
        two_sum(h0, l0, h0, l0);
        two_sum(h1, l1, h1, l1);
        dd_add(h0, l0, h1, l1);
        quad_sum_dd(h0, l0, q);
        const double a = (h0 + l0) / (double)kGroup;
        a_st[k] = F16 ? (double)f16_bits_to_f32(f64_to_f16_rne(a)) : (double)(float)a;
      }
    }
  }
#pragma unroll
  for (int k = 0; k <= K; ++k) {
    two_sum(eh[k], el[k], eh[k], el[k]);
    quad_sum_dd(eh[k], el[k], q);
    if (q == 0) {
      sh_hi[quad][k] = eh[k];
      sh_lo[quad][k] = el[k];
    }
  }
  __syncthreads();
  if (threadIdx.x <= K) {
    const int k = threadIdx.x;
    double h = sh_hi[0][k], l = sh_lo[0][k];
    for (int t = 1; t < nquads; ++t) dd_add(h, l, sh_hi[t][k], sh_lo[t][k]);
    rows[(int64_t)k * m + i] = h;  // h = RN(h + l)
  }
}

// layer[k] = the float64 nearest to sum_i rows[k * m + i]: per thread a
// strided pair sum, then a fixed tree over the workgroup.
__global__ void __launch_bounds__(256) energy_layer_kernel(const double* __restrict__ rows, int m,
                                                           int kcount,
                                                           double* __restrict__ layer) {
  __shared__ double sh_hi[256], sh_lo[256];
  const int t = threadIdx.x;
  for (int k = 0; k < kcount; ++k) {
    double h = 0.0, l = 0.0;
    for (int i = t; i < m; i += 256) dd_acc(h, l, rows[(int64_t)k * m + i]);
    two_sum(h, l, h, l);
    sh_hi[t] = h;
    sh_lo[t] = l;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (t < s) {
        double a = sh_hi[t], b = sh_lo[t];
        dd_add(a, b, sh_hi[t + s], sh_lo[t + s]);
        sh_hi[t] = a;
        sh_lo[t] = b;
      }
      __syncthreads();
    }
    if (t == 0) layer[k] = sh_hi[0];
    __syncthreads();
  }
}

template <bool F16>
int launch_energy_dt(const mbok_desc* d, const float* W, int64_t ldw, double* rows, double* layer,
                     hipStream_t stream) {
  const int G = d->n / kGroup;
  const int nquads = G < kEnergyMaxQuads ? G : kEnergyMaxQuads;
  const int threads = (4 * nquads + kWave - 1) / kWave * kWave;
  dim3 grid((unsigned)d->m), block(threads);
  switch (d->K) {
    case 1:
      hipLaunchKernelGGL((residual_energy_kernel<F16, 1>), grid, block, 0, stream, W, ldw, d->m,
                         d->n, rows);
      break;
    case 2:
      hipLaunchKernelGGL((residual_energy_kernel<F16, 2>), grid, block, 0, stream, W, ldw, d->m,
                         d->n, rows);
      break;
    case 3:
      hipLaunchKernelGGL((residual_energy_kernel<F16, 3>), grid, block, 0, stream, W, ldw, d->m,
                         d->n, rows);
      break;
    case 4:
      hipLaunchKernelGGL((residual_energy_kernel<F16, 4>), grid, block, 0, stream, W, ldw, d->m,
                         d->n, rows);
      break;
    default:
      return MBOK_ERR_UNSUPPORTED;
  }
  if (hipGetLastError() != hipSuccess) return MBOK_ERR_HIP;
  hipLaunchKernelGGL(energy_layer_kernel, dim3(1), dim3(256), 0, stream, rows, d->m, d->K + 1,
                     layer);
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

}  // namespace

int launch_residual_binarize(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs,
                             void* alpha, int32_t* flag, hipStream_t stream) {
  if (d->alpha_dtype == MBOK_F16) return launch_dt<true>(d, W, ldw, signs, alpha, flag, stream);
  return launch_dt<false>(d, W, ldw, signs, alpha, flag, stream);
}

int launch_residual_energy(const mbok_desc* d, const float* W, int64_t ldw, double* rows,
                           double* layer, hipStream_t stream) {
  if (d->alpha_dtype == MBOK_F16) return launch_energy_dt<true>(d, W, ldw, rows, layer, stream);
  return launch_energy_dt<false>(d, W, ldw, rows, layer, stream);
}

}  // namespace mbok
