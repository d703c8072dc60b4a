// Successive sign-value-independent decomposition (SVID) on the GPU.  (Its
// product runs in the few-token kernel, skinny.hip.)
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// gist.science summaries, "Riformulazione Booleana e SVID" (Italian),
// "Successive SVID" (Dutch), "Descomposición SVID" (Spanish): a weight is
// approximated by sign(W) (.) (s_out s_in^T) where s_out s_in^T is the rank-1
// SVD of |W|, and every further kernel is fitted the same way to the residual
// left by the previous ones:
//     W ~ sum_k B_k (.) (s_out^k s_in^k^T).
//
// Kernel k on the device:
//   1. signs: B_k = sign(R_{k-1}) with sign(0) = +1;
//   2. the top singular triple of |R_{k-1}| by power iteration in float64,
//      from v = 1/sqrt(n): u = |R| v, u /= |u|; v = |R|^T u, sigma = |v|,
//      v /= sigma (a fixed number of rounds);
//   3. s_out = sqrt(sigma) u and s_in = sqrt(sigma) v, rounded once to the
//      scale dtype.
// R_{k-1} is never stored: every pass recomputes each entry from W and the
// earlier kernels' signs and rounded scale vectors, in kernel order with one
// float64 rounding per kernel, exactly as the residual is defined.  |R| has
// nonnegative entries, so the iterates stay nonnegative (the Perron vectors).
// All sums run in a fixed order, so the decomposition is bit-reproducible.
//
// Every float64 operation here is an IEEE operation rounded on its own; no
// multiply may be fused into an add, so contraction is off for the file.
#pragma clang fp contract(off)

#include "mbok_exact.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

constexpr int kSvidBlock = 256;
constexpr int kSvidMaxSlices = 64;
constexpr int kSvidRowsPerSlice = 256;
constexpr int kSvidScalars = 8;  // [0] = |u|, [1] = sigma

template <typename AT>
__device__ __forceinline__ double scale_f64(const AT* s, int64_t idx) {
  return (double)alpha_to_f32<AT>(s[idx]);
}

// R_kc[i, j]: W minus the first kc kernels, in kernel order.
template <typename AT>
__device__ __forceinline__ double residual_at(float w, const int8_t* __restrict__ signs,
                                              const AT* __restrict__ s_out,
                                              const AT* __restrict__ s_in, int m, int n, int i,
                                              int j, int kc) {
  double r = (double)w;
  for (int k = 0; k < kc; ++k) {
    const double p = scale_f64<AT>(s_out, (int64_t)k * m + i) * scale_f64<AT>(s_in, (int64_t)k * n + j);
    r = signs[((int64_t)k * m + i) * n + j] >= 0 ? r - p : r + p;
  }
  return r;
}

// Fixed-order sum of one value per thread of a 256-thread block; the result
// is valid in thread 0.
__device__ __forceinline__ double block_sum(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = kSvidBlock / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] = sh[threadIdx.x] + sh[threadIdx.x + s];
    __syncthreads();
  }
  return sh[0];
}

// signs[kc][i][j] = sign(R_kc[i, j]), 0 -> +1.  One thread per 4 columns.
template <typename AT>
__global__ void __launch_bounds__(kSvidBlock) svid_sign_kernel(
    const float* __restrict__ W, int64_t ldw, int m, int n, int kc, int8_t* __restrict__ signs,
    const AT* __restrict__ s_out, const AT* __restrict__ s_in) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = n / 4;
  if (t >= (int64_t)m * per_row) return;
  const int i = (int)(t / per_row);
  const int j0 = (int)(t % per_row) * 4;
  const float4 w = *reinterpret_cast<const float4*>(W + (int64_t)i * ldw + j0);
  const float wv[4] = {w.x, w.y, w.z, w.w};
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double r = residual_at<AT>(wv[e], signs, s_out, s_in, m, n, i, j0 + e, kc);
    packed |= (uint32_t)(r >= 0.0 ? 0x01u : 0xffu) << (8 * e);
  }
  *reinterpret_cast<uint32_t*>(signs + ((int64_t)kc * m + i) * n + j0) = packed;
}

// u[i] = sum_j |R_kc[i, j]| v[j]; one workgroup per row.
template <typename AT>
__global__ void __launch_bounds__(kSvidBlock) svid_row_kernel(
    const float* __restrict__ W, int64_t ldw, int m, int n, int kc,
    const int8_t* __restrict__ signs, const AT* __restrict__ s_out, const AT* __restrict__ s_in,
    const double* __restrict__ v, double* __restrict__ u) {
  __shared__ double sh[kSvidBlock];
  const int i = blockIdx.x;
  double acc = 0.0;
  for (int j = threadIdx.x; j < n; j += kSvidBlock) {
    const double r = residual_at<AT>(W[(int64_t)i * ldw + j], signs, s_out, s_in, m, n, i, j, kc);
    acc = acc + fabs(r) * v[j];
  }
  const double tot = block_sum(acc, sh);
  if (threadIdx.x == 0) u[i] = tot;
}

// partial[s * n + j] = sum over rows of slice s of |R_kc[i, j]| u[i]; one
// thread per column, workgroups over (column blocks, row slices).
template <typename AT>
__global__ void __launch_bounds__(kSvidBlock) svid_col_kernel(
    const float* __restrict__ W, int64_t ldw, int m, int n, int kc,
    const int8_t* __restrict__ signs, const AT* __restrict__ s_out, const AT* __restrict__ s_in,
    const double* __restrict__ u, int rows_per_slice, double* __restrict__ partial) {
  const int j = blockIdx.x * kSvidBlock + threadIdx.x;
  const int s = blockIdx.y;
  if (j >= n) return;
  const int i0 = s * rows_per_slice;
  const int i1 = min(i0 + rows_per_slice, m);
  double acc = 0.0;
  for (int i = i0; i < i1; ++i) {
    const double r = residual_at<AT>(W[(int64_t)i * ldw + j], signs, s_out, s_in, m, n, i, j, kc);
    acc = acc + fabs(r) * u[i];
  }
  partial[(int64_t)s * n + j] = acc;
}

// v[j] = sum over slices (in order) of partial[s * n + j]
__global__ void __launch_bounds__(kSvidBlock) svid_col_reduce_kernel(
    const double* __restrict__ partial, int S, int n, double* __restrict__ v) {
  const int j = blockIdx.x * kSvidBlock + threadIdx.x;
  if (j >= n) return;
  double acc = partial[j];
  for (int s = 1; s < S; ++s) acc = acc + partial[(int64_t)s * n + j];
  v[j] = acc;
}

// x /= |x| (Euclidean, fixed-order sum); the norm goes to *norm.  One
// workgroup.
__global__ void __launch_bounds__(kSvidBlock) svid_normalize_kernel(double* __restrict__ x,
                                                                    int len,
                                                                    double* __restrict__ norm) {
  __shared__ double sh[kSvidBlock];
  double acc = 0.0;
  for (int t = threadIdx.x; t < len; t += kSvidBlock) acc = acc + x[t] * x[t];
  const double nrm = sqrt(block_sum(acc, sh));
  for (int t = threadIdx.x; t < len; t += kSvidBlock) x[t] = nrm > 0.0 ? x[t] / nrm : 0.0;
  if (threadIdx.x == 0) *norm = nrm;
}

__global__ void __launch_bounds__(kSvidBlock) svid_fill_kernel(double* __restrict__ x, int len,
                                                               double value) {
  const int t = blockIdx.x * kSvidBlock + threadIdx.x;
  if (t < len) x[t] = value;
}

template <typename AT>
__device__ __forceinline__ AT round_scale(double v);
template <>
__device__ __forceinline__ uint16_t round_scale<uint16_t>(double v) { return f64_to_f16_rne(v); }
template <>
__device__ __forceinline__ float round_scale<float>(double v) { return (float)v; }

// s_out[kc][i] = round(sqrt(sigma) u[i]), s_in[kc][j] = round(sqrt(sigma) v[j])
template <typename AT>
__global__ void __launch_bounds__(kSvidBlock) svid_scales_kernel(
    const double* __restrict__ u, const double* __restrict__ v,
    const double* __restrict__ scalars, int m, int n, int kc, AT* __restrict__ s_out,
    AT* __restrict__ s_in) {
  const int t = blockIdx.x * kSvidBlock + threadIdx.x;
  const double root = sqrt(scalars[1]);
  if (t < m) s_out[(int64_t)kc * m + t] = round_scale<AT>(root * u[t]);
  if (t < n) s_in[(int64_t)kc * n + t] = round_scale<AT>(root * v[t]);
}

int slices_for(int m) {
  int S = (m + kSvidRowsPerSlice - 1) / kSvidRowsPerSlice;
  return S > kSvidMaxSlices ? kSvidMaxSlices : S;
}

template <typename AT>
int decompose(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs, AT* s_out,
              AT* s_in, int iters, double* ws, hipStream_t stream) {
  const int m = d->m, n = d->n;
  const int S = slices_for(m);
  const int rows_per_slice = (m + S - 1) / S;
  double* u = ws;
  double* v = u + m;
  double* scalars = v + n;
  double* partial = scalars + kSvidScalars;
  const dim3 blk(kSvidBlock);
  const int64_t sign_threads = (int64_t)m * (n / 4);
  const unsigned sign_blocks = (unsigned)((sign_threads + kSvidBlock - 1) / kSvidBlock);
  const unsigned col_blocks = (unsigned)((n + kSvidBlock - 1) / kSvidBlock);
  const unsigned vec_blocks = (unsigned)(((m > n ? m : n) + kSvidBlock - 1) / kSvidBlock);
  for (int kc = 0; kc < d->K; ++kc) {
    hipLaunchKernelGGL(svid_sign_kernel<AT>, dim3(sign_blocks), blk, 0, stream, W, ldw, m, n, kc,
                       signs, s_out, s_in);
    hipLaunchKernelGGL(svid_fill_kernel, dim3(col_blocks), blk, 0, stream, v, n,
                       1.0 / sqrt((double)n));
    for (int it = 0; it < iters; ++it) {
      hipLaunchKernelGGL(svid_row_kernel<AT>, dim3((unsigned)m), blk, 0, stream, W, ldw, m, n, kc,
                         signs, s_out, s_in, v, u);
      hipLaunchKernelGGL(svid_normalize_kernel, dim3(1), blk, 0, stream, u, m, scalars);
      hipLaunchKernelGGL(svid_col_kernel<AT>, dim3(col_blocks, (unsigned)S), blk, 0, stream, W,
                         ldw, m, n, kc, signs, s_out, s_in, u, rows_per_slice, partial);
      hipLaunchKernelGGL(svid_col_reduce_kernel, dim3(col_blocks), blk, 0, stream, partial, S, n,
                         v);
      hipLaunchKernelGGL(svid_normalize_kernel, dim3(1), blk, 0, stream, v, n, scalars + 1);
    }
    hipLaunchKernelGGL(svid_scales_kernel<AT>, dim3(vec_blocks), blk, 0, stream, u, v, scalars, m,
                       n, kc, s_out, s_in);
    if (hipGetLastError() != hipSuccess) return MBOK_ERR_HIP;
  }
  return MBOK_OK;
}

}  // namespace

size_t svid_workspace_bytes(const mbok_desc* d) {
  const size_t S = (size_t)slices_for(d->m);
  return sizeof(double) * ((size_t)d->m + (size_t)d->n + kSvidScalars + S * (size_t)d->n);
}

int launch_svid_decompose(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs,
                          void* s_out, void* s_in, int iters, void* ws, hipStream_t stream) {
  double* w = reinterpret_cast<double*>(ws);
  if (d->alpha_dtype == MBOK_F16)
    return decompose<uint16_t>(d, W, ldw, signs, reinterpret_cast<uint16_t*>(s_out),
                               reinterpret_cast<uint16_t*>(s_in), iters, w, stream);
  return decompose<float>(d, W, ldw, signs, reinterpret_cast<float*>(s_out),
                          reinterpret_cast<float*>(s_in), iters, w, stream);
}

}  // namespace mbok
