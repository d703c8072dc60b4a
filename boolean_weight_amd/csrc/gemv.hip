// Decode product y = sum_k (alpha_k (.) B_k) x for one token, gfx950.
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// Paper-Notes reading note, 关键设计: Wx splits into K Boolean matrix-vector
// products, so every weight multiply becomes an add or a subtract of an
// activation; group-wise scales (one per 128 input columns) are applied per
// group.  局限与展望: activations stay full precision.
//
// Design (lut variant, the default):
//  * one workgroup per block of 64 output rows; lane l of every wavefront owns
//    row 64*blockIdx + l, so a wavefront reads one (group, kernel) sign plane
//    of its row block with a single 16-byte load per lane: 1 KB contiguous.
//  * the activations are staged in LDS as signed-sum tables: nibble a of
//    sign word w holds the 4 columns c0, c0+4, c0+8, c0+12 of the group, with
//    c0 = 32w + 16(a%2) + a/2 (the L64 bit order), and its table holds the 16
//    values sum_t (+-x[c0+4t]), one per sign pattern.  A nibble then selects
//    its entry: one LDS read and one fp32 add per 4 weights instead of 4
//    adds.  All 64 lanes read the same 16-entry table at the same time, so
//    the read is a conflict-free broadcast within 16 banks.
//  * per (group, kernel) the 32 lookups of a row are summed, then scaled by
//    the group's alpha with one FMA; wavefronts split the groups; a fixed-order
//    sum over wavefronts in LDS gives y (deterministic, no atomics).
//  * long rows are processed in column slabs so that the tables stay within
//    80 KB of LDS (two workgroups per compute unit).
//
// Variant "direct" (for comparison): the same mapping without tables, one
// select and add per sign bit.
#include <stdlib.h>
#include <string.h>

#include "mbok_device.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

constexpr int kChunksPerGroup = kGroup / 4;   // 32 nibbles (tables) per group
constexpr int kTableFloats = 16;              // entries per 4-column table
constexpr int kMaxSlabGroups = 40;            // 40 * 32 * 16 * 4 B = 80 KB
constexpr int kGpwMax = 3;                    // groups per wavefront per slab

template <typename XT>
__device__ __forceinline__ void load_x4(const XT* __restrict__ x, int64_t col, float& x0,
                                        float& x1, float& x2, float& x3);

template <typename XT>
__device__ __forceinline__ void load_x16(const XT* __restrict__ x, int64_t col, float* v);

template <>
__device__ __forceinline__ void load_x4<float>(const float* __restrict__ x, int64_t col,
                                               float& x0, float& x1, float& x2, float& x3) {
  const float4 v = *reinterpret_cast<const float4*>(x + col);
  x0 = v.x;
  x1 = v.y;
  x2 = v.z;
  x3 = v.w;
}

template <>
__device__ __forceinline__ void load_x4<uint16_t>(const uint16_t* __restrict__ x, int64_t col,
                                                  float& x0, float& x1, float& x2, float& x3) {
  const uint2 v = *reinterpret_cast<const uint2*>(x + col);
  x0 = bf16_bits_to_f32(v.x & 0xffffu);
  x1 = bf16_bits_to_f32(v.x >> 16);
  x2 = bf16_bits_to_f32(v.y & 0xffffu);
  x3 = bf16_bits_to_f32(v.y >> 16);
}

template <>
__device__ __forceinline__ void load_x16<float>(const float* __restrict__ x, int64_t col,
                                                float* v) {
  const float4* p = reinterpret_cast<const float4*>(x + col);
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float4 f = p[h];
    v[4 * h] = f.x;
    v[4 * h + 1] = f.y;
    v[4 * h + 2] = f.z;
    v[4 * h + 3] = f.w;
  }
}

template <>
__device__ __forceinline__ void load_x16<uint16_t>(const uint16_t* __restrict__ x,
                                                   int64_t col, float* v) {
  const uint4* p = reinterpret_cast<const uint4*>(x + col);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint4 u = p[h];
    const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * h + 2 * j] = bf16_bits_to_f32(d[j] & 0xffffu);
      v[8 * h + 2 * j + 1] = bf16_bits_to_f32(d[j] >> 16);
    }
  }
}

// The 16 signed sums of 4 activations: entry p = sum_t (bit t of p ? x_t : -x_t).
__device__ __forceinline__ void build_table4(float x0, float x1, float x2, float x3,
                                             float* __restrict__ dst) {
  const float lo[4] = {-x0 - x1, x0 - x1, -x0 + x1, x0 + x1};
  const float hi[4] = {-x2 - x3, x2 - x3, -x2 + x3, x2 + x3};
  float4* d4 = reinterpret_cast<float4*>(dst);
#pragma unroll
  for (int h = 0; h < 4; ++h)
    d4[h] = make_float4(lo[0] + hi[h], lo[1] + hi[h], lo[2] + hi[h], lo[3] + hi[h]);
}

// Sum over the 128 columns of one (row, group, kernel): sign word nibbles
// select entries of the group's 32 tables.  `tab` is the byte address of the
// group's tables in LDS (2 KB aligned), so the entry address is
// (nibble * 4) | tab plus a per-nibble constant that the compiler folds into
// the ds_read offset: one shift, one and-or and one fp32 add per nibble.
__device__ __forceinline__ float lut_dot128(const uint4 b, uint32_t tab) {
  typedef __attribute__((address_space(3))) const float lds_f32;
  const uint32_t wv[4] = {b.x, b.y, b.z, b.w};
  float part[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t sh = q == 0 ? (wv[w] << 2) : (wv[w] >> (4 * q - 2));
      uint32_t addr;  // ((sh & 0x3c) | tab): tab has no bits in 2..5
      asm("v_and_or_b32 %0, %1, 60, %2" : "=v"(addr) : "v"(sh), "v"(tab));
      s += reinterpret_cast<lds_f32*>((uintptr_t)addr)[(w * 8 + q) * kTableFloats];
    }
    part[w] = s;
  }
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const float* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const float*)p;
}

template <typename XT, typename AT, int K, int NW>
__global__ void __launch_bounds__(NW * kWave) gemv_lut_kernel(
    const uint4* __restrict__ bits, const AT* __restrict__ scales, const XT* __restrict__ x,
    float* __restrict__ y, int m, int G, int slab_groups) {
  extern __shared__ float lds[];
  const int rb = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float yacc = 0.f;
  for (int g0 = 0; g0 < G; g0 += slab_groups) {
    const int sg = min(slab_groups, G - g0);
    // issue this wavefront's sign and scale loads for the slab first, so they
    // are in flight while the tables are built
    uint4 b[kGpwMax][K];
    float a[kGpwMax][K];
#pragma unroll
    for (int j = 0; j < kGpwMax; ++j) {
      const int gl = wave + j * NW;
      if (gl < sg) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int64_t c = (((int64_t)rb * G + g0 + gl) * K + k) * kRowBlock + lane;
          b[j][k] = bits[c];
          a[j][k] = alpha_to_f32<AT>(scales[c]);
        }
      }
    }
    if (g0 > 0) __syncthreads();  // every wavefront is done with the previous slab
    // one thread per 16-column block (block b of group gl = words w = b/2,
    // nibbles a = 2e + b%2): it builds the 4 tables of columns b*16 + e + 4t
    for (int blk = threadIdx.x; blk < sg * 8; blk += NW * kWave) {
      float v[16];
      load_x16<XT>(x, (int64_t)g0 * kGroup + 16 * blk, v);
      const int gl = blk >> 3, b = blk & 7;
      float* tab = lds + (gl * kChunksPerGroup + 8 * (b >> 1) + (b & 1)) * kTableFloats;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        build_table4(v[e], v[4 + e], v[8 + e], v[12 + e], tab + 2 * e * kTableFloats);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kGpwMax; ++j) {
      const int gl = wave + j * NW;
      if (gl < sg) {
        const uint32_t tab = lds_addr(lds + gl * kChunksPerGroup * kTableFloats);
#pragma unroll
        for (int k = 0; k < K; ++k) yacc = fmaf(a[j][k], lut_dot128(b[j][k], tab), yacc);
      }
    }
  }
  __syncthreads();  // tables no longer needed: reuse LDS for the partial sums
  lds[wave * kWave + lane] = yacc;
  __syncthreads();
  if (wave == 0) {
    float s = lds[lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += lds[w * kWave + lane];
    const int i = rb * kRowBlock + lane;
    if (i < m) y[i] = s;
  }
}

// Reference-style variant: no tables, x staged in LDS as fp32, one select and
// one add per sign bit.
template <typename XT, typename AT, int K, int NW>
__global__ void __launch_bounds__(NW * kWave) gemv_direct_kernel(
    const uint4* __restrict__ bits, const AT* __restrict__ scales, const XT* __restrict__ x,
    float* __restrict__ y, int m, int G, int slab_groups) {
  extern __shared__ float lds[];
  const int rb = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float yacc = 0.f;
  for (int g0 = 0; g0 < G; g0 += slab_groups) {
    const int sg = min(slab_groups, G - g0);
    if (g0 > 0) __syncthreads();
    for (int c4 = threadIdx.x; c4 < sg * kGroup / 4; c4 += NW * kWave) {
      float x0, x1, x2, x3;
      load_x4<XT>(x, (int64_t)g0 * kGroup + 4 * c4, x0, x1, x2, x3);
      *reinterpret_cast<float4*>(lds + 4 * c4) = make_float4(x0, x1, x2, x3);
    }
    __syncthreads();
    for (int gl = wave; gl < sg; gl += NW) {
      for (int k = 0; k < K; ++k) {
        const int64_t c = (((int64_t)rb * G + g0 + gl) * K + k) * kRowBlock + lane;
        const uint4 b = bits[c];
        const float a = alpha_to_f32<AT>(scales[c]);
        const uint32_t wv[4] = {b.x, b.y, b.z, b.w};
        float s = 0.f;
        for (int w = 0; w < 4; ++w)
          for (int t = 0; t < 32; ++t) {
            // bit t = 8e + q of word w is column 32w + 4q + e
            const float xv = lds[gl * kGroup + 32 * w + 4 * (t & 7) + (t >> 3)];
            s += ((wv[w] >> t) & 1u) ? xv : -xv;
          }
        yacc = fmaf(a, s, yacc);
      }
    }
  }
  __syncthreads();
  lds[wave * kWave + lane] = yacc;
  __syncthreads();
  if (wave == 0) {
    float s = lds[lane];
    for (int w = 1; w < NW; ++w) s += lds[w * kWave + lane];
    const int i = rb * kRowBlock + lane;
    if (i < m) y[i] = s;
  }
}

enum Variant { kLut = 0, kDirect = 1 };

int variant_from_env() {
  const char* v = getenv("MBOK_GEMV_VARIANT");
  if (v && strcmp(v, "direct") == 0) return kDirect;
  return kLut;
}

template <typename XT, typename AT, int K>
int launch_typed(const Geom& geo, const void* packed, const void* x, float* y,
                 hipStream_t stream) {
  constexpr int NW = 16;
  const uint4* bits = reinterpret_cast<const uint4*>(packed);
  const AT* scales = reinterpret_cast<const AT*>(reinterpret_cast<const char*>(packed) +
                                                 geo.bits_bytes);
  const int nslabs = (geo.G + kMaxSlabGroups - 1) / kMaxSlabGroups;
  const int slab = (geo.G + nslabs - 1) / nslabs;
  dim3 grid(geo.RB), block(NW * kWave);
  if (variant_from_env() == kDirect) {
    const size_t lds = (size_t)(slab * kGroup > NW * kWave ? slab * kGroup : NW * kWave) *
                       sizeof(float);
    hipLaunchKernelGGL((gemv_direct_kernel<XT, AT, K, NW>), grid, block, lds, stream, bits,
                       scales, reinterpret_cast<const XT*>(x), y, geo.m, geo.G, slab);
  } else {
    const size_t tab = (size_t)slab * kChunksPerGroup * kTableFloats * sizeof(float);
    const size_t lds = tab > NW * kWave * sizeof(float) ? tab : NW * kWave * sizeof(float);
    hipLaunchKernelGGL((gemv_lut_kernel<XT, AT, K, NW>), grid, block, lds, stream, bits,
                       scales, reinterpret_cast<const XT*>(x), y, geo.m, geo.G, slab);
  }
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

template <typename XT, typename AT>
int launch_k(const Geom& geo, const void* packed, const void* x, float* y, hipStream_t s) {
  switch (geo.K) {
    case 1: return launch_typed<XT, AT, 1>(geo, packed, x, y, s);
    case 2: return launch_typed<XT, AT, 2>(geo, packed, x, y, s);
    case 3: return launch_typed<XT, AT, 3>(geo, packed, x, y, s);
    case 4: return launch_typed<XT, AT, 4>(geo, packed, x, y, s);
  }
  return MBOK_ERR_UNSUPPORTED;
}

}  // namespace

int launch_gemv(const mbok_desc* d, const void* packed, const void* x, int32_t x_dtype,
                float* y, hipStream_t stream) {
  const Geom geo = make_geom(d);
  const bool f16a = d->alpha_dtype == MBOK_F16;
  if (x_dtype == MBOK_BF16)
    return f16a ? launch_k<uint16_t, uint16_t>(geo, packed, x, y, stream)
                : launch_k<uint16_t, float>(geo, packed, x, y, stream);
  return f16a ? launch_k<float, uint16_t>(geo, packed, x, y, stream)
              : launch_k<float, float>(geo, packed, x, y, stream);
}

}  // namespace mbok
