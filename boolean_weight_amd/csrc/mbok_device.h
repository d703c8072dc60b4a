// Device helpers shared by the MBOK kernels (gfx950).  Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mbok.h"

namespace mbok {

constexpr int kGroup = MBOK_GROUP;         // input columns per scale
constexpr int kRowBlock = MBOK_ROW_BLOCK;  // rows per packed row block
constexpr int kWave = 64;                  // CDNA wavefront width

// Geometry of one layer in the L64 layout.
struct Geom {
  int m, n, K, G, RB;    // G = n / 128 groups, RB = row blocks of 64
  int64_t bits_bytes;    // size of the sign region
};

inline Geom make_geom(const mbok_desc* d) {
  Geom g;
  g.m = d->m;
  g.n = d->n;
  g.K = d->K;
  g.G = d->n / kGroup;
  g.RB = (d->m + kRowBlock - 1) / kRowBlock;
  g.bits_bytes = (int64_t)d->K * g.RB * kRowBlock * (d->n / 8);
  return g;
}

// 16-row tile of work item b.  Workgroup b runs on XCD b % 8, so within each
// full set of 32 tiles (8 row blocks of 64 rows) the items b = 8j + xcd,
// j = 4u + quarter, take quarter `quarter` of row block 8u + xcd: the four
// tiles of a row block share one XCD and its L2 lines of scales.  A trailing
// partial set keeps b.
__device__ __forceinline__ int tile16_of(int b, int tiles) {
  const int full = tiles & ~31;
  if (b >= full) return b;
  const int xcd = b & 7, j = b >> 3;
  return (((j >> 2) << 3) + xcd) * 4 + (j & 3);
}

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

// ----------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float32 -> bf16 bits, one rounding to nearest-even (the compiler's
// conversion, as the prefill unpack uses)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

template <typename AT>
__device__ __forceinline__ float alpha_to_f32(AT a);
template <>
__device__ __forceinline__ float alpha_to_f32<float>(float a) { return a; }
template <>
__device__ __forceinline__ float alpha_to_f32<uint16_t>(uint16_t a) { return f16_bits_to_f32(a); }

// float64 -> IEEE binary16, one rounding, nearest-even (subnormals and
// overflow to infinity included).  Converting through float32 would round
// twice, so this works on the float64 bits directly.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  int e = (int)((u >> 52) & 0x7ff);
  uint64_t frac = u & 0xfffffffffffffull;
  if (e == 0x7ff) return sign | (frac ? 0x7e00u : 0x7c00u);
  if (e == 0 && frac == 0) return sign;
  // value = 1.frac * 2^(e-1023) for normals (e > 0); float64 subnormals are
  // far below the fp16 range and round to zero below.
  int exp = e - 1023;
  uint64_t sig = (e ? (frac | (1ull << 52)) : frac);  // 53-bit significand
  if (exp > 15) return sign | 0x7c00u;
  int shift;  // bits of sig to drop
  uint32_t hexp;
  if (exp >= -14) {  // normal fp16: keep 11 significant bits
    shift = 52 - 10;
    hexp = (uint32_t)(exp + 15);
  } else {  // subnormal fp16: quantum 2^-24
    shift = 52 - 10 + (-14 - exp);
    hexp = 0;
    if (shift > 63) return sign;
  }
  uint64_t kept = sig >> shift;
  uint64_t rem = sig & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (kept & 1))) kept += 1;
  uint32_t out;
  if (hexp) {
    // kept holds 1.xxxx (11 bits); a carry to 2^11 bumps the exponent
    if (kept >> 11) {
      kept >>= 1;
      hexp += 1;
    }
    if (hexp >= 31) return sign | 0x7c00u;
    out = (hexp << 10) | (uint32_t)(kept & 0x3ff);
  } else {
    // subnormal: kept < 2^10, or == 2^10 which is the smallest normal
    out = (uint32_t)kept;
  }
  return sign | (uint16_t)out;
}

}  // namespace mbok
