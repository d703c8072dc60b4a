// Helpers of the exact-arithmetic kernels (quantizer, refit, residual
// energies, SVID) and of the SVID activation fragments: error-free float64
// sums, DPP exchanges inside lane quads, and per-lane loads of 32 weights and
// their sign bits.  Internal header.
#pragma once

#include "mbok_device.h"

namespace mbok {

// ------------------------------------------------ error-free float64 sums

// error-free a + b = s + e (Knuth's TwoSum).  The helpers below hold only
// when each add is rounded on its own: with contraction a caller's product
// could be fused into them, so it is switched off inside them.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
#pragma clang fp contract(off)
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// (hi, lo) += (bhi, blo), renormalised to hi = RN(hi + lo).  Exact whenever
// the exact sum, and every pair involved, are multiples of one power of two
// q with magnitudes below about 2^100 q (|lo| <= 16 ulp(hi) allowed).  The
// final renormalisation is a full TwoSum, so cancellation between hi and bhi
// (a small s next to a larger e) stays exact.
__device__ __forceinline__ void dd_add(double& hi, double& lo, double bhi, double blo) {
#pragma clang fp contract(off)
  double s, e;
  two_sum(hi, bhi, s, e);
  e += lo + blo;
  two_sum(s, e, hi, lo);
}

// Sum of the (hi, lo) pairs of all 64 lanes by a butterfly; every lane ends
// with the same bits because each combine puts the lower lane's pair first.
__device__ __forceinline__ void wave_sum_dd(double& hi, double& lo, int lane) {
#pragma unroll
  for (int mask = 1; mask < kWave; mask <<= 1) {
    double ohi = __shfl_xor(hi, mask, kWave);
    double olo = __shfl_xor(lo, mask, kWave);
    if (lane & mask) {
      double th = ohi, tl = olo;
      dd_add(th, tl, hi, lo);
      hi = th;
      lo = tl;
    } else {
      dd_add(hi, lo, ohi, olo);
    }
  }
}

// ------------------------------------------- four lanes per (row, group)

// Lanes 4t .. 4t+3 (a quad) exchange values with DPP quad permutations.
template <int CTRL>
__device__ __forceinline__ int quad_perm_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ double quad_perm_d(double v) {
  const int lo = quad_perm_i<CTRL>(__double2loint(v));
  const int hi = quad_perm_i<CTRL>(__double2hiint(v));
  return __hiloint2double(hi, lo);
}
constexpr int kQuadXor1 = 0xb1;  // [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4e;  // [2, 3, 0, 1]

// Sum of an exact pair over the quad; every lane ends with the same bits
// because each combine puts the lower lane's pair first.
__device__ __forceinline__ void quad_sum_dd(double& hi, double& lo, int q) {
  double oh = quad_perm_d<kQuadXor1>(hi), ol = quad_perm_d<kQuadXor1>(lo);
  if (q & 1) {
    dd_add(oh, ol, hi, lo);
    hi = oh;
    lo = ol;
  } else {
    dd_add(hi, lo, oh, ol);
  }
  oh = quad_perm_d<kQuadXor2>(hi);
  ol = quad_perm_d<kQuadXor2>(lo);
  if (q & 2) {
    dd_add(oh, ol, hi, lo);
    hi = oh;
    lo = ol;
  } else {
    dd_add(hi, lo, oh, ol);
  }
}

__device__ __forceinline__ int quad_sum_i(int v) {
  v += quad_perm_i<kQuadXor1>(v);
  return v + quad_perm_i<kQuadXor2>(v);
}

// The lane's 32 consecutive weights into registers (8 16-byte loads).
__device__ __forceinline__ void load_weights32(const float* __restrict__ src, float w[32]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float4 v = reinterpret_cast<const float4*>(src)[t];
    w[4 * t] = v.x;
    w[4 * t + 1] = v.y;
    w[4 * t + 2] = v.z;
    w[4 * t + 3] = v.w;
  }
}

// 32 int8 signs -> one word, bit j set where entry j is >= 0.  Four entries
// per dword: their inverted top bits 7, 15, 23, 31 gather into bits 0..3.
__device__ __forceinline__ uint32_t load_sign_bits32(const int8_t* __restrict__ src) {
  uint32_t b = 0;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint4 v = reinterpret_cast<const uint4*>(src)[t];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = ~d[e] & 0x80808080u;
      const uint32_t nib = ((x >> 7) | (x >> 14) | (x >> 21) | (x >> 28)) & 0xfu;
      b |= nib << (16 * t + 4 * e);
    }
  }
  return b;
}

// One word of bits -> 32 int8 signs (+1 for a set bit, -1 otherwise).
__device__ __forceinline__ void store_sign_bits32(int8_t* __restrict__ dst, uint32_t bits) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint32_t d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t nib = (bits >> (16 * t + 4 * e)) & 0xfu;
      // one bit per byte, then 0x01 for a set bit and 0xff for a clear one
      const uint32_t x = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
      d[e] = 0xffffffffu ^ (x * 0xfeu);
    }
    reinterpret_cast<uint4*>(dst)[t] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

// (hi, lo) += v for a float64 v, error-free; exact under the same condition
// as dd_add.  The pair is renormalised only by the caller (dd_add).
__device__ __forceinline__ void dd_acc(double& hi, double& lo, double v) {
#pragma clang fp contract(off)
  double s, e;
  two_sum(hi, v, s, e);
  hi = s;
  lo += e;
}

// float32 -> bf16 bits, one rounding to nearest-even (the compiler's
// conversion, as the prefill unpack uses)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

}  // namespace mbok
