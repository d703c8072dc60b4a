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

// ----------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
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
