// Alternating least-squares refit of the K Boolean kernels of a layer for the
// weight itself: scales, then signs, then scales again, `rounds` times.
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// Paper-Notes reading note, 关键设计 (efficient scale optimisation): with the
// Boolean matrices fixed the scales have a closed-form least-squares
// solution, and the two are optimised in turn, one fixed while the other is
// updated.
//
// Four lanes per (row, group) of 128 columns, 32 columns each: the weights
// stay in registers and the signs are kept as one word of bits per kernel
// and lane.  Per group:
//   scale step  (B^T B) a = B^T w solved exactly and rounded once.  The Gram
//               matrix is integer (popcounts of sign-bit differences); with
//               its adjugate C and determinant D, a_k = sum_l C_kl r_l / D,
//               where r_l = sum_j b_lj w_j is summed exactly as a float64
//               pair and each C_kl r_l is split exactly by fused multiply-
//               adds.  The quotient is rounded to odd in float64 (exact
//               remainder signs), then to nearest-even in the scale dtype,
//               which equals one rounding of the exact rational.  A singular
//               Gram matrix keeps the scales.
//   sign step   each weight takes the pattern of its nearest level
//               sum_k a_k b_k (levels and distances in float64; ties go to
//               the larger level, then to the larger pattern index
//               sum_k [b_k = +1] 2^k).
// The pair sums are exact when, within a group, the nonzero weights'
// magnitudes lie within a factor 2^48 of one another (any trained layer);
// beyond that the quotient before its rounding is accurate to about 2^-100.
// Every float64 operation in this file is an exact or a once-rounded IEEE
// operation: no multiply may be fused into a following add (that would
// break the error-free sums), so contraction is off for the whole file.
#pragma clang fp contract(off)

#include "mbok_exact.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

constexpr int kMaxRefitRounds = 64;
constexpr int kRefitBlock = 256;  // threads per workgroup, four per (row, group)

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
__device__ __forceinline__ int det3(const int A[4][4], int r0, int r1, int r2, int c0, int c1,
                                    int c2) {
  return A[r0][c0] * (A[r1][c1] * A[r2][c2] - A[r1][c2] * A[r2][c1]) -
         A[r0][c1] * (A[r1][c0] * A[r2][c2] - A[r1][c2] * A[r2][c0]) +
         A[r0][c2] * (A[r1][c0] * A[r2][c1] - A[r1][c1] * A[r2][c0]);
}

// Adjugate and determinant of the K x K Gram matrix, taken as the 4x4 matrix
// diag(Gram, I): its determinant is det(Gram) and the top-left K x K block
// of its adjugate is adj(Gram).  adj[k][l] = (-1)^(k+l) * minor(l, k).
// 32-bit integers suffice: a Gram matrix of +-1 vectors of length 128 is
// positive semidefinite with diagonal 128, so (Hadamard) its determinant is
// at most 2^28, every cofactor at most 2^21 in magnitude, and each product
// formed here stays below 2^31.
template <int K>
__device__ __forceinline__ int adjugate(const int Gm[K][K], int adj[K][K]) {
  int A[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) A[r][c] = (r < K && c < K) ? Gm[r < K ? r : 0][c < K ? c : 0] : (r == c);
  int cof[4][4];
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
      const int mnr = det3(A, rs[0], rs[1], rs[2], cs[0], cs[1], cs[2]);
      cof[r][c] = ((r + c) & 1) ? -mnr : mnr;
    }
  }
  int det = 0;
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

// Lanes 4t .. 4t+3 (a quad) share one (row, group): lane q holds columns
// 32q .. 32q+31.

// Exact pair sum over the lane's 32 columns of b_j w_j (bit j of `bits`),
// in two chains.
__device__ __forceinline__ void signed_sum32(const float w[32], uint32_t bits, double& hi,
                                             double& lo) {
  double h0 = 0.0, l0 = 0.0, h1 = 0.0, l1 = 0.0;
#pragma unroll
  for (int j = 0; j < 32; j += 2) {
    const float v0 = ((bits >> j) & 1u) ? w[j] : -w[j];
    const float v1 = ((bits >> (j + 1)) & 1u) ? w[j + 1] : -w[j + 1];
    dd_acc(h0, l0, (double)v0);
    dd_acc(h1, l1, (double)v1);
  }
  two_sum(h0, l0, h0, l0);
  two_sum(h1, l1, h1, l1);
  dd_add(h0, l0, h1, l1);
  hi = h0;
  lo = l0;
}

template <bool F16, int K>
__global__ void __launch_bounds__(256) refit_kernel(const float* __restrict__ W, int64_t ldw,
                                                    int m, int n, int8_t* __restrict__ signs,
                                                    void* __restrict__ alpha, int rounds) {
  constexpr int M = 1 << K;  // levels
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
  uint32_t bits[K];  // bit j: column 32q + j is +1
  double a[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    bits[k] = load_sign_bits32(signs + ((int64_t)k * m + i) * n + col);
    a[k] = load_alpha<F16>(alpha, ((int64_t)k * m + i) * G + g);
  }

  for (int step = 0; step < 2 * rounds + 1; ++step) {
    if ((step & 1) == 0) {
      // ---- scale step.  Gram matrix: 128 - 2 * (differing signs), the
      // differences of the K(K-1)/2 pairs packed 8 bits each for the quad sum
      int Gm[K][K];
      {
        int packed[2] = {0, 0};
        int slot = 0;
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
          for (int l = k + 1; l < K; ++l, ++slot)
            packed[slot >> 2] |= __popc(bits[k] ^ bits[l]) << (8 * (slot & 3));
        packed[0] = quad_sum_i(packed[0]);
        if (K * (K - 1) / 2 > 4) packed[1] = quad_sum_i(packed[1]);
        slot = 0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          Gm[k][k] = kGroup;
#pragma unroll
          for (int l = k + 1; l < K; ++l, ++slot) {
            const int diff = (packed[slot >> 2] >> (8 * (slot & 3))) & 0xff;
            Gm[k][l] = Gm[l][k] = kGroup - 2 * diff;
          }
        }
      }
      int adj[K][K];
      const int det = adjugate<K>(Gm, adj);
      if (det == 0) continue;  // singular: the scales stay
      double rh[K], rl[K];
#pragma unroll
      for (int l = 0; l < K; ++l) {
        signed_sum32(w, bits[l], rh[l], rl[l]);
        quad_sum_dd(rh[l], rl[l], q);
      }
      // lane q solves for scale k = q (lanes beyond K repeat the last one)
      const int kq = q < K ? q : K - 1;
      double nh = 0.0, nl = 0.0;
#pragma unroll
      for (int l = 0; l < K; ++l) {
        int cq = adj[0][l];
#pragma unroll
        for (int k = 1; k < K; ++k) cq = (kq == k) ? adj[k][l] : cq;
        const double c = (double)cq;  // |c| < 2^22: exact
        const double p = c * rh[l], pe = __fma_rn(c, rh[l], -p);
        const double pl = c * rl[l], ple = __fma_rn(c, rl[l], -pl);
        dd_add(nh, nl, p, pe);
        dd_add(nh, nl, pl, ple);
      }
      const double qt = div_round_odd(nh, nl, (double)det);
      const double aq = F16 ? (double)f16_bits_to_f32(f64_to_f16_rne(qt))
                            : (double)(float)qt;  // v_cvt_f32_f64: nearest-even
      a[0] = quad_perm_d<0x00>(aq);
      if (K > 1) a[1 < K ? 1 : 0] = quad_perm_d<0x55>(aq);
      if (K > 2) a[2 < K ? 2 : 0] = quad_perm_d<0xaa>(aq);
      if (K > 3) a[3 < K ? 3 : 0] = quad_perm_d<0xff>(aq);
    } else {
      // ---- sign step.  The levels, each summed in kernel order, are sorted
      // ascending by (level, pattern); scanning them in that order and
      // taking every level whose distance is <= the best so far ends on the
      // nearest level, the larger one on a tie, the larger pattern on equal
      // levels.
      double lev[M];
      int pat[M];
#pragma unroll
      for (int idx = 0; idx < M; ++idx) {
        double v = 0.0;
#pragma unroll
        for (int k = 0; k < K; ++k) v = v + (((idx >> k) & 1) ? a[k] : -a[k]);
        lev[idx] = v;
        pat[idx] = idx;
      }
      // odd-even transposition sort: M passes of compare-exchange
#pragma unroll
      for (int pass = 0; pass < M; ++pass) {
#pragma unroll
        for (int x = pass & 1; x + 1 < M; x += 2) {
          const bool swap = lev[x] > lev[x + 1] || (lev[x] == lev[x + 1] && pat[x] > pat[x + 1]);
          const double l0 = lev[x], l1 = lev[x + 1];
          const int p0 = pat[x], p1 = pat[x + 1];
          lev[x] = swap ? l1 : l0;
          lev[x + 1] = swap ? l0 : l1;
          pat[x] = swap ? p1 : p0;
          pat[x + 1] = swap ? p0 : p1;
        }
      }
      uint32_t nb[K];
#pragma unroll
      for (int k = 0; k < K; ++k) nb[k] = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const double wj = (double)w[j];
        double bd = fabs(wj - lev[0]);
        int bp = pat[0];
#pragma unroll
        for (int x = 1; x < M; ++x) {
          const double dx = fabs(wj - lev[x]);
          const bool take = dx <= bd;
          bd = take ? dx : bd;
          bp = take ? pat[x] : bp;
        }
#pragma unroll
        for (int k = 0; k < K; ++k) nb[k] |= (uint32_t)((bp >> k) & 1) << j;
      }
#pragma unroll
      for (int k = 0; k < K; ++k) bits[k] = nb[k];
    }
  }

#pragma unroll
  for (int k = 0; k < K; ++k) {
    store_sign_bits32(signs + ((int64_t)k * m + i) * n + col, bits[k]);
  }
  if (q < K) {
    // lane q stores scale q (its value is bit-identical in every lane)
    double aq = a[0];
#pragma unroll
    for (int k = 1; k < K; ++k) aq = (q == k) ? a[k] : aq;
    const int64_t aidx = ((int64_t)q * m + i) * G + g;
    if (F16)
      reinterpret_cast<uint16_t*>(alpha)[aidx] = f64_to_f16_rne(aq);  // exact: aq is fp16
    else
      reinterpret_cast<float*>(alpha)[aidx] = (float)aq;
  }
}

template <bool F16>
int launch_refit_dt(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs, void* alpha,
                    int rounds, hipStream_t stream) {
  const int G = d->n / kGroup;
  const int64_t tasks = (int64_t)d->m * G;
  const int64_t blocks = (4 * tasks + kRefitBlock - 1) / kRefitBlock;
  if (blocks > 0x7fffffff) return MBOK_ERR_SHAPE;
  dim3 grid((unsigned)blocks), block(kRefitBlock);
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
