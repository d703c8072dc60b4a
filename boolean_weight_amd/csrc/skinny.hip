// Few-token product Y = X . W_hat^T, 1..16 tokens, on the matrix cores
// without rounding W_hat (gfx950).
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// Paper-Notes reading note, 关键设计: W ~ sum_k alpha_k B_k, one scale per
// (row, 128-column group, kernel).  Per group the product splits exactly as
//     y[t, row] = sum_g sum_k alpha_k[row, g] * S_k[t, row, g],
//     S_k[t, row, g] = sum_{c in g} B_k[row, c] * x[t, c],
// and S_k is a sum of +-x: the signs become bf16 +-1 (exact), the matrix cores
// add and subtract the bf16 activations with fp32 accumulation, and alpha_k is
// applied per group in fp32.  Unlike the prefill kernel nothing is rounded to
// bf16 beyond the activations themselves, so results match the fp64
// definition to fp32 accumulation error.
//
// One v_mfma_f32_16x16x32_bf16 covers 16 tokens x 16 rows x 32 columns:
//   A (tokens x columns): lane (i, q) = (lane % 16, lane / 16) holds token i,
//     columns 128g + 32q + 8s + 0..7 at step s (natural order, one 16-byte load);
//   B (columns x rows): lane (i, q) holds row i of the tile, the same columns;
//     they are word q of the row's 16-byte chunk for (g, k), where bit 8e + p
//     is column 32q + 4p + e.  Two byte permutes spread the word into
//     P01 = [b0, b0, b1, b1] and P23 = [b2, b2, b3, b3]; shifting each left by
//     7 - p brings the bits of columns 4p + {0, 1} (P01) or 4p + {2, 3} (P23)
//     to bits 15 and 31, and one v_and_or_b32 per dword makes them the sign
//     bits of two bf16 ones.  The packed bit is 1 for +1, which gives a set
//     sign bit, so the kernel accumulates -S_k and subtracts alpha_k * S.
//   C: lane (i, q), register r = token 4q + r, row i.
//
// A workgroup owns 16 rows and all columns; its NW wavefronts take
// contiguous ranges of groups and walk them 4 groups at a time.  For each
// kernel, 16-lane block q loads the 16-byte chunks of the 16 rows for group
// g + q (one 16-byte load per lane, four 256-byte runs per wavefront);
// v_permlane32_swap + v_permlane16_swap then transpose the 4 x 4 (16-lane
// block, word) matrix so that register j holds word q of group g + j, the B
// operand of group g + j.  The scales are spread the same way (3 swaps).  The
// partial sums of the wavefronts are added in LDS in a fixed wave order, so
// results are deterministic.
#include <stdlib.h>
#include <string.h>

#include "mbok_exact.h"
#include "mbok_lanes.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kMaxSkinnyTokens = 16;

// Two bf16 values of magnitude 1 whose sign bits are bits 15 and 31 of src:
// (src & mask) | ones in one v_and_or_b32, mask = 0x80008000 in an SGPR and
// ones = 0x3F803F80 in a VGPR (a VOP3 encoding takes no literal constants).
__device__ __forceinline__ uint32_t signed_ones(uint32_t src, uint32_t mask, uint32_t ones) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(src), "s"(mask), "v"(ones));
  return d;
}

template <typename AT>
__device__ __forceinline__ uint32_t scale_bits(AT a);
template <>
__device__ __forceinline__ uint32_t scale_bits<float>(float a) { return __float_as_uint(a); }
template <>
__device__ __forceinline__ uint32_t scale_bits<uint16_t>(uint16_t a) { return a; }

template <typename AT>
__device__ __forceinline__ float scale_value(uint32_t b);
template <>
__device__ __forceinline__ float scale_value<float>(uint32_t b) { return __uint_as_float(b); }
template <>
__device__ __forceinline__ float scale_value<uint16_t>(uint32_t b) {
  return f16_bits_to_f32((uint16_t)b);
}

template <typename AT, int K>
__global__ void __launch_bounds__(1024) gemm_skinny_kernel(
    const u32x4* __restrict__ bits, const AT* __restrict__ scales,
    const uint16_t* __restrict__ X, int64_t ldx, float* __restrict__ Y, int64_t ldy, int T,
    int m, int G) {
  extern __shared__ float red[];  // [NW][4][64] partial sums
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int NW = blockDim.x >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int tile = blockIdx.x;  // rows 16 * tile .. + 15, inside row block tile / 4
  const int rb = tile >> 2;
  const int rin = ((tile & 3) << 4) + i;
  const int g0 = (int)((int64_t)wave * G / NW);
  const int g1 = (int)((int64_t)(wave + 1) * G / NW);
  const bool tok_ok = i < T;
  const uint16_t* xrow = X + (int64_t)(tok_ok ? i : 0) * ldx + 32 * q;

  const uint32_t mask = __builtin_amdgcn_readfirstlane(0x80008000u);
  uint32_t ones;
  asm("v_mov_b32 %0, 0x3f803f80" : "=v"(ones));

  f32x4 yacc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int gb = g0; gb < g1; gb += 4) {
    const int nj = g1 - gb < 4 ? g1 - gb : 4;  // groups in this block
    const int gq = gb + (q < nj ? q : nj - 1);  // group loaded by block q
    const int64_t c = (int64_t)(rb * G + gq) * K * 64 + rin;
    u32x4 wv[K];
    AT av[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      wv[k] = bits[c + k * 64];
      av[k] = scales[c + k * 64];
    }
    u32x4 xv[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        xv[j][s] = (tok_ok && j < nj)
                       ? *reinterpret_cast<const u32x4*>(xrow + (int64_t)kGroup * (gb + j) + 8 * s)
                       : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < K; ++k) {
      uint32_t w[4] = {wv[k].x, wv[k].y, wv[k].z, wv[k].w};
      transpose4(w);  // w[j] = word q of row i, group gb + j
      uint32_t a[4];
      spread4(scale_bits<AT>(av[k]), a);  // a[j] = scale of row i, group gb + j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j >= nj) break;
        const uint32_t p01 = __builtin_amdgcn_perm(w[j], w[j], 0x01010000u);
        const uint32_t p23 = __builtin_amdgcn_perm(w[j], w[j], 0x03030202u);
        f32x4 S = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int se = 7 - 2 * s, so = 6 - 2 * s;  // columns 8s + 0..3, 8s + 4..7
          const u32x4 b = u32x4{signed_ones(p01 << se, mask, ones),
                                signed_ones(p23 << se, mask, ones),
                                signed_ones(p01 << so, mask, ones),
                                signed_ones(p23 << so, mask, ones)};
          S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[j][s]),
                                                      __builtin_bit_cast(bf16x8, b), S, 0, 0,
                                                      0);
        }
        const float sc = scale_value<AT>(a[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[r] = __builtin_fmaf(-sc, S[r], yacc[r]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = yacc[r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 256; idx += blockDim.x) {
    float sum = 0.f;
    for (int w = 0; w < NW; ++w) sum += red[w * 256 + idx];
    const int l = idx & 63, r = idx >> 6;
    const int tok = 4 * (l >> 4) + r;
    const int row = tile * 16 + (l & 15);
    if (tok < T && row < m) Y[(int64_t)tok * ldy + row] = sum;
  }
}

// Streaming form (the default): one persistent workgroup per compute unit.
// Wavefront w owns group block w of the slab (groups 4w .. 4w+3, at most 8
// blocks: slabs of up to 32 groups), loads the activation fragments of its
// groups once per slab, and walks the workgroup's 16-row tiles (b, b + grid,
// ... through tile16_of), loading the sign chunks and scales of tile t + 1
// while tile t is expanded and multiplied.  So the weight stream overlaps the
// expansion and the MFMAs, and activations are read once per workgroup
// instead of once per tile.  Partial sums of up to JMAX tiles stay in
// registers; each tile is summed over wavefronts in a fixed order at the end.
template <typename AT, int K>
struct SkinnyLoads {
  u32x4 w[K];
  AT a[K];
};

// The SVID product's activations for one wavefront's block of 4 groups:
// frag[((j * K + k) * 2 + part) * 128 + c] (bf16) is the hi (part 0) or lo
// (part 1) part of v = s_in^k[col] * x[col], col = 128 (gb + j) + c, formed
// in fp32 (exact for fp16 scales and bf16 x); hi = RNE(v), lo = RNE(v - hi),
// so hi + lo is v to about 2^-17 relative.  The 64 lanes share the values.
template <typename AT, int K>
__device__ __forceinline__ void svid_block_fragments(const void* __restrict__ x, int x_f32,
                                                     const AT* __restrict__ s_in, int n, int gb,
                                                     int nj, int lane,
                                                     uint16_t* __restrict__ frag) {
  // lane takes columns c = lane and lane + 64 of each group; all loads first
  float xv[4][2];
  AT sv[4][K][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t col = (int64_t)kGroup * (gb + (j < nj ? j : 0)) + lane + 64 * h;
      xv[j][h] = x_f32 ? reinterpret_cast<const float*>(x)[col]
                       : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[col]);
#pragma unroll
      for (int k = 0; k < K; ++k) sv[j][k][h] = s_in[(int64_t)k * n + col];
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j >= nj) break;
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = lane + 64 * h;
        const float v = alpha_to_f32<AT>(sv[j][k][h]) * xv[j][h];
        const uint16_t hi = f32_to_bf16_rne(v);
        frag[((j * K + k) * 2) * kGroup + c] = hi;
        frag[((j * K + k) * 2 + 1) * kGroup + c] = f32_to_bf16_rne(v - bf16_bits_to_f32(hi));
      }
  }
}

// SV: the SVID product.  Token row 2k + part holds the hi / lo bf16 part of
// s_in^k (.) x (svid_block_fragments, formed by each wavefront for its own
// groups in a private LDS area after the partial-sum area), the scale slots hold
// s_out^k of the row (the same in every group), so kernel k is applied to its
// two token rows only and the output is the sum of all token rows:
// y = sum_k s_out^k (.) (B_k (s_in^k (.) x)).  X and ldx are unused then.
//
// The arguments the first loads need come first (the first 14 argument dwords
// arrive in SGPRs at launch); the grid size and tw = tiles per workgroup
// (bits 0..3, one more for workgroups below tw >> 8) | wavefronts (bits
// 4..7) are arguments, so no address waits on a dispatch-packet load and
// nothing is divided.
template <typename AT, int K, int JMAX, bool SV>
__global__ void __launch_bounds__(512) gemm_skinny_stream_kernel(
    const u32x4* __restrict__ bits, const AT* __restrict__ scales,
    const uint16_t* __restrict__ X, int64_t ldx, int T, int G, int slab_groups, int tiles,
    int grid, int tw, float* __restrict__ Y, int64_t ldy, int m, const void* __restrict__ sv_x,
    int sv_xf32, const AT* __restrict__ sv_sin) {
  extern __shared__ float red[];  // [JMAX][NW][4][64] partial sums
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int NW = (tw >> 4) & 15;
  const int i = lane & 15, q = lane >> 4;
  const int ntl = (tw & 15) + ((int)blockIdx.x < (tw >> 8) ? 1 : 0);  // <= JMAX
  const bool tok_ok = i < T;
  const uint16_t* xrow = SV ? nullptr : X + (int64_t)(tok_ok ? i : 0) * ldx + 32 * q;
  uint16_t* frag = SV ? reinterpret_cast<uint16_t*>(red + JMAX * NW * 256) +
                            wave * (4 * K * 2 * kGroup)
                      : nullptr;
  const uint32_t mask = __builtin_amdgcn_readfirstlane(0x80008000u);
  uint32_t ones;
  asm("v_mov_b32 %0, 0x3f803f80" : "=v"(ones));

  f32x4 yacc[JMAX];
#pragma unroll
  for (int t = 0; t < JMAX; ++t) yacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g0 = 0; g0 < G; g0 += slab_groups) {
    const int sg = min(slab_groups, G - g0);
    const int nj = min(4, sg - 4 * wave);  // groups of this wavefront's block
    if (nj <= 0) continue;                 // uniform per wavefront
    const int gb = g0 + 4 * wave;
    const int gq = gb + (q < nj ? q : nj - 1);  // group loaded by 16-lane block q
    u32x4 xv[4][4];
    if constexpr (SV) {
      svid_block_fragments<AT, K>(sv_x, sv_xf32, sv_sin, G * kGroup, gb, nj, lane, frag);
      // the area is this wavefront's own, and its LDS operations complete in order
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xv[j][s] = (tok_ok && j < nj)
                         ? *reinterpret_cast<const u32x4*>(
                               frag + ((j * K + (i >> 1)) * 2 + (i & 1)) * kGroup + 32 * q + 8 * s)
                         : u32x4{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xv[j][s] = (tok_ok && j < nj) ? *reinterpret_cast<const u32x4*>(
                                              xrow + (int64_t)kGroup * (gb + j) + 8 * s)
                                        : u32x4{0u, 0u, 0u, 0u};
    }
    auto load = [&](int t, SkinnyLoads<AT, K>& L) {
      // opaque to the compiler, so each tile's address is formed where it is
      // loaded instead of every tile's ahead of the first load
      int tb = (int)blockIdx.x + t * grid;
      asm volatile("" : "+s"(tb));
      const int row = tile16_of(tb, tiles) * 16 + i;
      const int64_t c = ((int64_t)(row / kRowBlock) * G + gq) * K * kRowBlock + row % kRowBlock;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        L.w[k] = bits[c + k * kRowBlock];
        L.a[k] = scales[c + k * kRowBlock];
      }
    };
    auto compute = [&](const SkinnyLoads<AT, K>& L, f32x4 acc) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        uint32_t w[4] = {L.w[k].x, L.w[k].y, L.w[k].z, L.w[k].w};
        transpose4(w);  // w[j] = word q of row i, group gb + j
        uint32_t a[4];
        spread4(scale_bits<AT>(L.a[k]), a);  // a[j] = scale of row i, group gb + j
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j >= nj) break;
          const uint32_t p01 = __builtin_amdgcn_perm(w[j], w[j], 0x01010000u);
          const uint32_t p23 = __builtin_amdgcn_perm(w[j], w[j], 0x03030202u);
          f32x4 S = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int se = 7 - 2 * s, so = 6 - 2 * s;
            const u32x4 bb = u32x4{signed_ones(p01 << se, mask, ones),
                                   signed_ones(p23 << se, mask, ones),
                                   signed_ones(p01 << so, mask, ones),
                                   signed_ones(p23 << so, mask, ones)};
            S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[j][s]),
                                                        __builtin_bit_cast(bf16x8, bb), S, 0, 0,
                                                        0);
          }
          const float sc = scale_value<AT>(a[j]);
          if constexpr (SV) {
            // token 4q + r belongs to kernel (4q + r) / 2
            const float sc0 = (2 * q == k) ? sc : 0.f, sc1 = (2 * q + 1 == k) ? sc : 0.f;
            acc[0] = __builtin_fmaf(-sc0, S[0], acc[0]);
            acc[1] = __builtin_fmaf(-sc0, S[1], acc[1]);
            acc[2] = __builtin_fmaf(-sc1, S[2], acc[2]);
            acc[3] = __builtin_fmaf(-sc1, S[3], acc[3]);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(-sc, S[r], acc[r]);
          }
        }
      }
      return acc;
    };
    SkinnyLoads<AT, K> LA, LB;
    load(0, LA);
#pragma unroll
    for (int t = 0; t < JMAX; t += 2) {
      if (t >= ntl) break;
      if (t + 1 < ntl) load(t + 1, LB);
      yacc[t] = compute(LA, yacc[t]);
      if (t + 1 >= ntl) break;
      if (t + 2 < ntl) load(t + 2, LA);
      yacc[t + 1] = compute(LB, yacc[t + 1]);
    }
  }

#pragma unroll
  for (int t = 0; t < JMAX; ++t) {
    if (t >= ntl) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(((t * NW) + wave) * 4 + r) * 64 + lane] = yacc[t][r];
  }
  __syncthreads();
  if constexpr (SV) {
    // one output per row: the token rows in order, each summed over wavefronts
    for (int idx = threadIdx.x; idx < ntl * 16; idx += NW * 64) {
      const int t = idx >> 4, ri = idx & 15;
      float sum = 0.f;
      for (int tok = 0; tok < T; ++tok) {
        const int e = (tok & 3) * 64 + (tok >> 2) * 16 + ri;
        float part = 0.f;
        for (int w = 0; w < NW; ++w) part += red[(t * NW + w) * 256 + e];
        sum += part;
      }
      const int row = tile16_of((int)blockIdx.x + t * grid, tiles) * 16 + ri;
      if (row < m) Y[row] = sum;
    }
  } else {
    for (int idx = threadIdx.x; idx < ntl * 256; idx += NW * 64) {
      const int t = idx >> 8, e = idx & 255;
      float sum = 0.f;
      for (int w = 0; w < NW; ++w) sum += red[(t * NW + w) * 256 + e];
      const int l = e & 63, r = e >> 6;
      const int tok = 4 * (l >> 4) + r;
      const int row = tile16_of((int)blockIdx.x + t * grid, tiles) * 16 + (l & 15);
      if (tok < T && row < m) Y[(int64_t)tok * ldy + row] = sum;
    }
  }
}

int env_int(const char* name, int fallback) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : fallback;
}

template <typename AT, int K>
void launch_k(const Geom& geo, const u32x4* bits, const AT* scales, const uint16_t* X,
              int64_t ldx, float* Y, int64_t ldy, int T, int NW, hipStream_t stream) {
  const size_t lds = (size_t)NW * 256 * sizeof(float);
  hipLaunchKernelGGL((gemm_skinny_kernel<AT, K>), dim3(geo.RB * 4), dim3(64 * NW), lds, stream,
                     bits, scales, X, ldx, Y, ldy, T, geo.m, geo.G);
}

constexpr int kSkinnyJ = 8;  // tiles per persistent workgroup (registers)

template <typename AT, int K, bool SV = false>
void launch_stream_k(const Geom& geo, const u32x4* bits, const AT* scales, const uint16_t* X,
                     int64_t ldx, float* Y, int64_t ldy, int T, hipStream_t stream,
                     const void* sv_x = nullptr, int sv_xf32 = 0, const AT* sv_sin = nullptr) {
  // slabs of at most 32 groups: one wavefront per block of 4 groups, at most 8
  const int nslabs = (geo.G + 31) / 32;
  const int slab = (geo.G + nslabs - 1) / nslabs;
  const int NW = (slab + 3) / 4;
  const int tiles = geo.RB * 4;
  int grid = tiles < 256 ? tiles : 256;
  if (grid * kSkinnyJ < tiles) grid = (tiles + kSkinnyJ - 1) / kSkinnyJ;
  size_t lds = (size_t)kSkinnyJ * NW * 256 * sizeof(float);
  if (SV) lds += (size_t)NW * 4 * K * 2 * kGroup * sizeof(uint16_t);
  static_assert(kSkinnyJ <= 15, "tiles per workgroup are packed in 4 bits");
  const int tw = tiles / grid | NW << 4 | (tiles % grid) << 8;
  hipLaunchKernelGGL((gemm_skinny_stream_kernel<AT, K, kSkinnyJ, SV>), dim3(grid), dim3(64 * NW), lds,
                     stream, bits, scales, X, ldx, T, geo.G, slab, tiles, grid, tw, Y, ldy, geo.m,
                     sv_x, sv_xf32, sv_sin);
}

template <typename AT>
int launch_at(const Geom& geo, const void* packed, const void* X, int64_t ldx, float* Y,
              int64_t ldy, int T, hipStream_t stream) {
  const u32x4* bits = reinterpret_cast<const u32x4*>(packed);
  const AT* scales = reinterpret_cast<const AT*>(reinterpret_cast<const char*>(packed) +
                                                 geo.bits_bytes);
  const uint16_t* Xb = reinterpret_cast<const uint16_t*>(X);
  // streaming pays off when workgroups get several tiles of one slab (many
  // rows, at most 32 groups) or when 16 tokens make the activation fragments
  // worth keeping; MBOK_SKINNY_VARIANT=stream|blocks overrides
  const char* v = getenv("MBOK_SKINNY_VARIANT");
  bool streaming = (geo.G <= 32 && geo.m >= 8192) || T >= 16;
  if (v && strcmp(v, "blocks") == 0) streaming = false;
  if (v && strcmp(v, "stream") == 0) streaming = true;
  if (streaming) {
    switch (geo.K) {
      case 1: launch_stream_k<AT, 1>(geo, bits, scales, Xb, ldx, Y, ldy, T, stream); break;
      case 2: launch_stream_k<AT, 2>(geo, bits, scales, Xb, ldx, Y, ldy, T, stream); break;
      case 3: launch_stream_k<AT, 3>(geo, bits, scales, Xb, ldx, Y, ldy, T, stream); break;
      default: launch_stream_k<AT, 4>(geo, bits, scales, Xb, ldx, Y, ldy, T, stream); break;
    }
    return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
  }
  // about 4800 wavefronts over the chip (~5 per SIMD), at most 16 per
  // workgroup; measured best for 4096 to 27648 rows
  const int tiles = geo.RB * 4;
  int NW = env_int("MBOK_SKINNY_NW", (4800 + tiles / 2) / tiles);
  if (NW > 16) NW = 16;
  if (NW > geo.G) NW = geo.G;
  if (NW < 1) NW = 1;
  switch (geo.K) {
    case 1: launch_k<AT, 1>(geo, bits, scales, Xb, ldx, Y, ldy, T, NW, stream); break;
    case 2: launch_k<AT, 2>(geo, bits, scales, Xb, ldx, Y, ldy, T, NW, stream); break;
    case 3: launch_k<AT, 3>(geo, bits, scales, Xb, ldx, Y, ldy, T, NW, stream); break;
    default: launch_k<AT, 4>(geo, bits, scales, Xb, ldx, Y, ldy, T, NW, stream); break;
  }
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

}  // namespace

int skinny_max_tokens() { return kMaxSkinnyTokens; }

// The SVID product: 2K token rows formed from x and s_in in the kernel.
int launch_svid_skinny(const mbok_desc* d, const void* packed, const void* x, int32_t x_dtype,
                       const void* s_in, float* y, hipStream_t stream) {
  const Geom geo = make_geom(d);
  const u32x4* bits = reinterpret_cast<const u32x4*>(packed);
  const int T = 2 * geo.K;
  const int xf = x_dtype == MBOK_F32 ? 1 : 0;
  if (d->alpha_dtype == MBOK_F16) {
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(
        reinterpret_cast<const char*>(packed) + geo.bits_bytes);
    const uint16_t* si = reinterpret_cast<const uint16_t*>(s_in);
    switch (geo.K) {
      case 1: launch_stream_k<uint16_t, 1, true>(geo, bits, sc, nullptr, 0, y, geo.m, T, stream, x, xf, si); break;
      case 2: launch_stream_k<uint16_t, 2, true>(geo, bits, sc, nullptr, 0, y, geo.m, T, stream, x, xf, si); break;
      case 3: launch_stream_k<uint16_t, 3, true>(geo, bits, sc, nullptr, 0, y, geo.m, T, stream, x, xf, si); break;
      default: launch_stream_k<uint16_t, 4, true>(geo, bits, sc, nullptr, 0, y, geo.m, T, stream, x, xf, si); break;
    }
  } else {
    const float* sc =
        reinterpret_cast<const float*>(reinterpret_cast<const char*>(packed) + geo.bits_bytes);
    const float* si = reinterpret_cast<const float*>(s_in);
    switch (geo.K) {
      case 1: launch_stream_k<float, 1, true>(geo, bits, sc, nullptr, 0, y, geo.m, T, stream, x, xf, si); break;
      case 2: launch_stream_k<float, 2, true>(geo, bits, sc, nullptr, 0, y, geo.m, T, stream, x, xf, si); break;
      case 3: launch_stream_k<float, 3, true>(geo, bits, sc, nullptr, 0, y, geo.m, T, stream, x, xf, si); break;
      default: launch_stream_k<float, 4, true>(geo, bits, sc, nullptr, 0, y, geo.m, T, stream, x, xf, si); break;
    }
  }
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

int launch_skinny(const mbok_desc* d, const void* packed, const void* X, int64_t T, int64_t ldx,
                  float* Y, int64_t ldy, hipStream_t stream) {
  if (T < 1 || T > kMaxSkinnyTokens) return MBOK_ERR_SHAPE;
  const Geom geo = make_geom(d);
  if (d->alpha_dtype == MBOK_F16)
    return launch_at<uint16_t>(geo, packed, X, ldx, Y, ldy, (int)T, stream);
  return launch_at<float>(geo, packed, X, ldx, Y, ldy, (int)T, stream);
}

}  // namespace mbok
