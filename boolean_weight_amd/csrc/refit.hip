// Alternating least-squares refit of the K Boolean kernels of a layer for the
// weight itself: scales, then signs, then scales again, `rounds` times.
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// Paper-Notes reading note, 关键设计 (efficient scale optimisation): with the
// Boolean matrices fixed the scales have a closed-form least-squares
// solution, and the two are optimised in turn, one fixed while the other is
// updated.
//
// One wavefront per (row, group) of 128 columns; lane l holds columns 2l and
// 2l+1.  Per group:
//   scale step  (B^T B) a = B^T w solved exactly and rounded once.  The Gram
//               matrix is integer (popcounts of sign ballots); with its
//               adjugate C and determinant D, a_k = sum_j c_kj w_j / D where
//               c_kj = sum_l C_kl b_lj is an integer below 2^23, so each
//               product c_kj w_j is an exact float64 and the sum over the
//               group is exact as a float64 pair.  The quotient is rounded to
//               odd in float64 (exact remainder signs), then to nearest-even
//               in the scale dtype, which equals one rounding of the exact
//               rational.  A singular Gram matrix keeps the scales.
//   sign step   each weight takes the pattern of its nearest level
//               sum_k a_k b_k (levels and distances in float64; ties go to
//               the larger level, then to the larger pattern index
//               sum_k [b_k = +1] 2^k).
// The pair sums are exact when, within a group, the nonzero weights'
// magnitudes lie within a factor 2^48 of one another (any trained layer);
// beyond that the quotient before its rounding is accurate to about 2^-100.
#include "mbok_device.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

constexpr int kMaxRefitRounds = 64;

// Exact sign (-1, 0, +1) of a + b + c + d (no overflow): the terms are merged
// into a nonoverlapping expansion of increasing magnitude with error-free
// additions (Shewchuk's grow-expansion); its largest nonzero component
// carries the sign of the sum.
__device__ __forceinline__ int sign_of_sum4(double a, double b, double c, double d) {
  double e[4] = {a, 0.0, 0.0, 0.0};
  const double t[3] = {b, c, d};
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    double q = t[i];
#pragma unroll
    for (int j = 0; j <= i; ++j) {
      double s, h;
      two_sum(q, e[j], s, h);
      e[j] = h;
      q = s;
    }
    e[i + 1] = q;
  }
  int sgn = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (e[j] != 0.0) sgn = e[j] > 0.0 ? 1 : -1;
  return sgn;
}

// Sign of (nh + nl) - c * D, exactly (c * D split by a fused multiply-add).
__device__ __forceinline__ int remainder_sign(double nh, double nl, double c, double D) {
  const double p = c * D;
  const double pe = __fma_rn(c, D, -p);
  return sign_of_sum4(nh, nl, -p, -pe);
}

// Step the magnitude of a nonzero float64 by one unit in the last place.
__device__ __forceinline__ double step_away(double v) {
  return __longlong_as_double(__double_as_longlong(v) + 1);
}
__device__ __forceinline__ double step_toward(double v) {
  return __longlong_as_double(__double_as_longlong(v) - 1);
}

// (nh + nl) / D rounded to odd in float64, for an exact pair (nh, nl) with
// |nl| <= ulp(nh) / 2 and a positive integer D < 2^53.  Rounding this once
// more to a format of at most 51 significant bits gives the nearest-even
// rounding of the exact quotient.
__device__ double div_round_odd(double nh, double nl, double D) {
  if (nh == 0.0) return 0.0;
  const double sgn = nh > 0.0 ? 1.0 : -1.0;
  const double q0 = nh / D;
  double q = q0 + (__fma_rn(-q0, D, nh) + nl) / D;  // within two units of the truth
  int rs = remainder_sign(nh, nl, q, D);
  // q too large in magnitude: step toward zero until it is not
  for (int it = 0; it < 4 && rs * sgn < 0; ++it) {
    q = step_toward(q);
    rs = remainder_sign(nh, nl, q, D);
  }
  // q below the truth: step away while the next value still is not above it
  for (int it = 0; it < 4 && rs * sgn > 0; ++it) {
    const double q2 = step_away(q);
    const int r2 = remainder_sign(nh, nl, q2, D);
    if (r2 * sgn < 0) break;
    q = q2;
    rs = r2;
  }
  // q is now the truncation of the quotient; an inexact one gets an odd last bit
  if (rs != 0) q = __longlong_as_double(__double_as_longlong(q) | 1);
  return q;
}

// Determinant of the 3x3 matrix formed by rows r0, r1, r2 and columns c0, c1,
// c2 of the 4x4 integer matrix A.
__device__ __forceinline__ int64_t det3(const int64_t A[4][4], int r0, int r1, int r2, int c0,
                                        int c1, int c2) {
  return A[r0][c0] * (A[r1][c1] * A[r2][c2] - A[r1][c2] * A[r2][c1]) -
         A[r0][c1] * (A[r1][c0] * A[r2][c2] - A[r1][c2] * A[r2][c0]) +
         A[r0][c2] * (A[r1][c0] * A[r2][c1] - A[r1][c1] * A[r2][c0]);
}

// Adjugate and determinant of the K x K Gram matrix, taken as the 4x4 matrix
// diag(Gram, I): its determinant is det(Gram) and the top-left K x K block
// of its adjugate is adj(Gram).  adj[k][l] = (-1)^(k+l) * minor(l, k).
template <int K>
__device__ __forceinline__ int64_t adjugate(const int Gm[K][K], int64_t adj[K][K]) {
  int64_t A[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) A[r][c] = (r < K && c < K) ? Gm[r < K ? r : 0][c < K ? c : 0] : (r == c);
  int64_t cof[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int rs[3], cs[3], nr = 0, nc = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t != r) rs[nr++] = t;
        if (t != c) cs[nc++] = t;
      }
      const int64_t mnr = det3(A, rs[0], rs[1], rs[2], cs[0], cs[1], cs[2]);
      cof[r][c] = ((r + c) & 1) ? -mnr : mnr;
    }
  }
  int64_t det = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) det += A[0][c] * cof[0][c];
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int l = 0; l < K; ++l) adj[k][l] = cof[l][k];
  return det;
}

template <bool F16>
__device__ __forceinline__ double load_alpha(const void* alpha, int64_t idx) {
  if (F16) return (double)f16_bits_to_f32(reinterpret_cast<const uint16_t*>(alpha)[idx]);
  return (double)reinterpret_cast<const float*>(alpha)[idx];
}

template <bool F16, int K>
__global__ void __launch_bounds__(256) refit_kernel(const float* __restrict__ W, int64_t ldw,
                                                    int m, int n, int8_t* __restrict__ signs,
                                                    void* __restrict__ alpha, int rounds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int G = n / kGroup;
  const int64_t task = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (task >= (int64_t)m * G) return;  // whole wave exits together
  const int i = (int)(task / G);
  const int g = (int)(task % G);
  const int64_t col = (int64_t)g * kGroup + 2 * lane;

  const float2 w2 = *reinterpret_cast<const float2*>(W + (int64_t)i * ldw + col);
  const double w0 = (double)w2.x, w1 = (double)w2.y;
  bool p0[K], p1[K];  // current signs of the lane's two columns (true = +1)
  double a[K];        // current scales, values of the scale dtype
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const char2 sv = *reinterpret_cast<const char2*>(signs + ((int64_t)k * m + i) * n + col);
    p0[k] = sv.x >= 0;
    p1[k] = sv.y >= 0;
    a[k] = load_alpha<F16>(alpha, ((int64_t)k * m + i) * G + g);
  }

  for (int step = 0; step < 2 * rounds + 1; ++step) {
    if ((step & 1) == 0) {
      // ---- scale step
      uint64_t ev[K], od[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        ev[k] = __ballot(p0[k]);
        od[k] = __ballot(p1[k]);
      }
      int Gm[K][K];
#pragma unroll
      for (int k = 0; k < K; ++k)
#pragma unroll
        for (int l = 0; l < K; ++l)
          Gm[k][l] = kGroup - 2 * (__popcll(ev[k] ^ ev[l]) + __popcll(od[k] ^ od[l]));
      int64_t adj[K][K];
      const int64_t det = adjugate<K>(Gm, adj);
      if (det == 0) continue;  // singular: the scales stay
      const double D = (double)det;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        int64_t c0 = 0, c1 = 0;
#pragma unroll
        for (int l = 0; l < K; ++l) {
          c0 += p0[l] ? adj[k][l] : -adj[k][l];
          c1 += p1[l] ? adj[k][l] : -adj[k][l];
        }
        double hi, lo;
        two_sum((double)c0 * w0, (double)c1 * w1, hi, lo);  // both products exact
        wave_sum_dd(hi, lo, lane);
        const double q = div_round_odd(hi, lo, D);
        if (F16)
          a[k] = (double)f16_bits_to_f32(f64_to_f16_rne(q));
        else
          a[k] = (double)(float)q;  // v_cvt_f32_f64: nearest-even
      }
    } else {
      // ---- sign step: nearest of the 2^K levels, scanned in pattern order
      double b0d = 0.0, b0l = 0.0, b1d = 0.0, b1l = 0.0;
      int b0i = -1, b1i = -1;
#pragma unroll
      for (int idx = 0; idx < (1 << K); ++idx) {
        double lev = 0.0;
#pragma unroll
        for (int k = 0; k < K; ++k) lev = lev + (((idx >> k) & 1) ? a[k] : -a[k]);
        const double d0 = fabs(w0 - lev), d1 = fabs(w1 - lev);
        if (b0i < 0 || d0 < b0d || (d0 == b0d && lev >= b0l)) {
          b0d = d0;
          b0l = lev;
          b0i = idx;
        }
        if (b1i < 0 || d1 < b1d || (d1 == b1d && lev >= b1l)) {
          b1d = d1;
          b1l = lev;
          b1i = idx;
        }
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        p0[k] = (b0i >> k) & 1;
        p1[k] = (b1i >> k) & 1;
      }
    }
  }

#pragma unroll
  for (int k = 0; k < K; ++k) {
    char2 sv;
    sv.x = p0[k] ? 1 : -1;
    sv.y = p1[k] ? 1 : -1;
    *reinterpret_cast<char2*>(signs + ((int64_t)k * m + i) * n + col) = sv;
    const int64_t aidx = ((int64_t)k * m + i) * G + g;
    if (lane == 0) {
      if (F16)
        reinterpret_cast<uint16_t*>(alpha)[aidx] = f64_to_f16_rne(a[k]);  // exact: a is fp16
      else
        reinterpret_cast<float*>(alpha)[aidx] = (float)a[k];
    }
  }
}

template <bool F16>
int launch_refit_dt(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs, void* alpha,
                    int rounds, hipStream_t stream) {
  const int G = d->n / kGroup;
  const int64_t tasks = (int64_t)d->m * G;
  const int waves_per_block = 4;
  const int64_t blocks = (tasks + waves_per_block - 1) / waves_per_block;
  if (blocks > 0x7fffffff) return MBOK_ERR_SHAPE;
  dim3 grid((unsigned)blocks), block(waves_per_block * kWave);
  switch (d->K) {
    case 1:
      hipLaunchKernelGGL((refit_kernel<F16, 1>), grid, block, 0, stream, W, ldw, d->m, d->n,
                         signs, alpha, rounds);
      break;
    case 2:
      hipLaunchKernelGGL((refit_kernel<F16, 2>), grid, block, 0, stream, W, ldw, d->m, d->n,
                         signs, alpha, rounds);
      break;
    case 3:
      hipLaunchKernelGGL((refit_kernel<F16, 3>), grid, block, 0, stream, W, ldw, d->m, d->n,
                         signs, alpha, rounds);
      break;
    case 4:
      hipLaunchKernelGGL((refit_kernel<F16, 4>), grid, block, 0, stream, W, ldw, d->m, d->n,
                         signs, alpha, rounds);
      break;
    default:
      return MBOK_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

}  // namespace

int refit_max_rounds() { return kMaxRefitRounds; }

int launch_refit(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs, void* alpha,
                 int rounds, hipStream_t stream) {
  if (rounds < 0 || rounds > kMaxRefitRounds) return MBOK_ERR_INVALID_ARG;
  if (d->alpha_dtype == MBOK_F16) return launch_refit_dt<true>(d, W, ldw, signs, alpha, rounds, stream);
  return launch_refit_dt<false>(d, W, ldw, signs, alpha, rounds, stream);
}

}  // namespace mbok
