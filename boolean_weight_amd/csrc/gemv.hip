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

// byte k of v added to base: one VOP2 add with a byte-select operand
#define MBOK_ADD_BYTE(out, base, v, k)                                              \
  asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD " \
      "src1_sel:BYTE_" #k                                                           \
      : "=v"(out)                                                                   \
      : "v"(base), "v"(v))

// As lut_dot128, with the nibble addresses formed per word: the even nibbles
// shifted to bits 2..5 of each byte with one shift and one mask, the odd ones
// likewise, then each entry address is one add of a selected byte to `tab`
// (any table base works: it is an ordinary register operand).  2.5 VALU
// operations per 4 weights.
// 8 table addresses of one sign word (nibbles 0..7), one VOP2 add each.
__device__ __forceinline__ void word_addresses(uint32_t w, uint32_t tab, uint32_t* a) {
  const uint32_t ev = (w << 2) & 0x3c3c3c3cu;  // byte k: nibble 2k, times 4
  const uint32_t od = (w >> 2) & 0x3c3c3c3cu;  // byte k: nibble 2k+1, times 4
  asm("v_add_u32_sdwa %0, %8, %9 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0\n\t"
      "v_add_u32_sdwa %1, %8, %10 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0\n\t"
      "v_add_u32_sdwa %2, %8, %9 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1\n\t"
      "v_add_u32_sdwa %3, %8, %10 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1\n\t"
      "v_add_u32_sdwa %4, %8, %9 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2\n\t"
      "v_add_u32_sdwa %5, %8, %10 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2\n\t"
      "v_add_u32_sdwa %6, %8, %9 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3\n\t"
      "v_add_u32_sdwa %7, %8, %10 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
        "=&v"(a[6]), "=&v"(a[7])
      : "v"(tab), "v"(ev), "v"(od));
}

// Sum of the 16 lookups of two sign words (w0 = word 2h, w1 = word 2h+1 of
// the chunk): 16 addresses, then 16 LDS reads in flight, then a tree sum.
__device__ __forceinline__ float lut_dot64_sdwa(uint32_t w0, uint32_t w1, uint32_t tab, int h) {
  typedef __attribute__((address_space(3))) const float lds_f32;
  uint32_t ad[16];
  word_addresses(w0, tab, ad);
  word_addresses(w1, tab, ad + 8);
  float v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q)
    v[q] = reinterpret_cast<lds_f32*>((uintptr_t)ad[q])[(16 * h + q) * kTableFloats];
#pragma unroll
  for (int s = 8; s >= 1; s >>= 1)
#pragma unroll
    for (int q = 0; q < s; ++q) v[q] += v[q + s];
  return v[0];
}

// The scheduling barriers keep the batches of successive half chunks apart,
// so at most 16 lookups are in flight per wavefront (about what the LDS
// counter tracks anyway) and register use stays low enough for 4+ waves per
// SIMD.
__device__ __forceinline__ float lut_dot128_sdwa(const uint4 b, uint32_t tab) {
  const float lo = lut_dot64_sdwa(b.x, b.y, tab, 0);
  __builtin_amdgcn_sched_barrier(0);
  const float hi = lut_dot64_sdwa(b.z, b.w, tab, 1);
  __builtin_amdgcn_sched_barrier(0);
  return lo + hi;
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
        for (int k = 0; k < K; ++k) yacc = fmaf(a[j][k], lut_dot128_sdwa(b[j][k], tab), yacc);
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

// Row-slice variant: a wavefront covers R = 64/NS rows and NS column slices
// (lane = c*R + r), a workgroup covers R rows and every column, so no
// cross-workgroup step is needed and small layers still give m/R workgroups.
// The NW*NS slices ("streams") of a workgroup take groups p, p+NW*NS, ...;
// all streams of the workgroup read the same slab of tables.  Group tables
// are kGroupStride = 2112 bytes apart (33 x 64): the NS slices of a
// wavefront read consecutive groups, whose tables then start 16 banks apart,
// so one ds_read of the whole wavefront stays free of bank conflicts.  The
// next group's sign planes are loaded before the current one is summed.
constexpr int kGroupStride = 2112;  // bytes between the tables of two groups

// Per slab of groups, each thread of the first 8*sg loads one 16-column
// block of activations, then the sign planes are requested, then the thread
// builds the four tables of its block straight from registers.
template <typename XT, typename AT, int K, int NW, int NS>
__global__ void __launch_bounds__(NW * kWave) gemv_rows_kernel(
    const uint4* __restrict__ bits, const AT* __restrict__ scales, const XT* __restrict__ x,
    float* __restrict__ y, int m, int G, int slab_groups) {
  constexpr int R = kWave / NS;
  constexpr int NP = NW * NS;
  extern __shared__ float lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c = lane / R, r = lane % R;
  const int p = wave * NS + c;
  const int i = blockIdx.x * R + r;  // < m_pad: R divides the 64-row block
  const int rb = i / kRowBlock, rr = i % kRowBlock;
  // chunk (g, k) of this row: bits_row[(g * K + k) * 64], 32-bit offsets
  const uint4* bits_row = bits + (int64_t)rb * G * K * kRowBlock + rr;
  const AT* scales_row = scales + (int64_t)rb * G * K * kRowBlock + rr;
  const uint32_t lbase = lds_addr(lds);
  float yacc = 0.f;
  for (int g0 = 0; g0 < G; g0 += slab_groups) {
    const int sg = min(slab_groups, G - g0);
    // Activations first: the table build waits only for these (loads return
    // in order), while the sign planes issued next are still in flight.
    // Thread b < 8 sg loads the 16-column block b of the slab.
    const bool hx = (int)threadIdx.x < sg * 8;
    float v[16];
    if (hx) load_x16<XT>(x, (int64_t)g0 * kGroup + 16 * threadIdx.x, v);
    uint4 bA[K], bB[K];
    float aA[K], aB[K];
    if (p < sg) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const uint32_t o = (uint32_t)((g0 + p) * K + k) * kRowBlock;
        bA[k] = bits_row[o];
        aA[k] = alpha_to_f32<AT>(scales_row[o]);
      }
    }
    if (g0 > 0) __syncthreads();  // the previous slab's tables are no longer read
    if (hx) {
      // block bb of group gl holds the columns of tables 8(bb/2) + 2e + bb%2
      const int gl = threadIdx.x >> 3, bb = threadIdx.x & 7;
      float* tabs = lds + (gl * kGroupStride) / 4 + (8 * (bb >> 1) + (bb & 1)) * kTableFloats;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        build_table4(v[e], v[4 + e], v[8 + e], v[12 + e], tabs + 2 * e * kTableFloats);
    }
    __syncthreads();
    for (int gl = p; gl < sg; gl += 2 * NP) {
      const int g1 = gl + NP, g2 = gl + 2 * NP;
      if (g1 < sg) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const uint32_t o = (uint32_t)((g0 + g1) * K + k) * kRowBlock;
          bB[k] = bits_row[o];
          aB[k] = alpha_to_f32<AT>(scales_row[o]);
        }
      }
      {
        const uint32_t tab = lbase + gl * kGroupStride;
#pragma unroll
        for (int k = 0; k < K; ++k) yacc = fmaf(aA[k], lut_dot128_sdwa(bA[k], tab), yacc);
      }
      if (g2 < sg) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const uint32_t o = (uint32_t)((g0 + g2) * K + k) * kRowBlock;
          bA[k] = bits_row[o];
          aA[k] = alpha_to_f32<AT>(scales_row[o]);
        }
      }
      if (g1 < sg) {
        const uint32_t tab = lbase + g1 * kGroupStride;
#pragma unroll
        for (int k = 0; k < K; ++k) yacc = fmaf(aB[k], lut_dot128_sdwa(bB[k], tab), yacc);
      }
    }
  }
  // fixed-order sum over the NS slices of the wavefront, then over wavefronts
#pragma unroll
  for (int off = R; off < kWave; off <<= 1) yacc += __shfl_xor(yacc, off, kWave);
  if (NW > 1) {
    __syncthreads();
    if (c == 0) lds[wave * R + r] = yacc;
    __syncthreads();
    if (wave != 0 || c != 0) return;
    yacc = lds[r];
#pragma unroll
    for (int w = 1; w < NW; ++w) yacc += lds[w * R + r];
  } else if (c != 0) {
    return;
  }
  if (i < m) y[i] = yacc;
}

// Streaming variant: one persistent workgroup per compute unit.  Wavefront w
// owns group block w (groups 4w .. 4w+3 of the slab); lane (j, r) =
// (lane / 16, lane % 16) handles row r of the tile and group 4w + j, so one
// 16-byte load per lane covers 16 rows x 4 groups (four 256-byte runs of a
// plane).  The workgroup builds the tables of a slab once and then walks its
// 16-row tiles (b, b + grid, ... through words_tile), loading tile t + 1 while
// tile t is summed, so the stream of sign planes overlaps the lookups instead
// of alternating with them workgroup by workgroup.  Group tables are
// kGroupStride = 2112 bytes apart, so the 4 groups of one ds_read hit 16-bank
// windows 16 banks apart.  Partial sums of up to JMAX tiles stay in registers
// across slabs; each tile is finally summed over the 4 groups of a block and
// over wavefronts in a fixed order.
template <typename AT, int K>
struct BlockLoads {
  uint4 b[K];
  float a[K];
};

template <typename XT, typename AT, int K, int JMAX>
// The arguments the first loads need come first, so that they are among
// the ones preloaded into SGPRs at launch; the scales are found from the
// packed buffer (they follow the 4 G K tiles 16-byte sign chunks).
// The grid size, the wavefront count and the tiles per workgroup (tpw, plus
// one for the first textra workgroups) are arguments, so that no address
// waits on a load from the dispatch packet and nothing is divided; the output
// arguments come last (the first 14 argument dwords arrive in SGPRs).
__global__ void __launch_bounds__(16 * kWave) gemv_stream_kernel(
    const uint4* __restrict__ bits, const XT* __restrict__ x, int G, int tiles, int slab_groups,
    int grid, int nw, int tpw, int textra, float* __restrict__ y, int m) {
  const AT* __restrict__ scales =
      reinterpret_cast<const AT*>(bits + (int64_t)tiles * 16 * G * K);
  extern __shared__ float lds[];
  const int NW = nw;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, j = lane >> 4;
  const int ntl = tpw + ((int)blockIdx.x < textra ? 1 : 0);  // <= JMAX
  float yacc[JMAX];
#pragma unroll
  for (int t = 0; t < JMAX; ++t) yacc[t] = 0.f;

  auto load = [&](int t, int g0, int gl, BlockLoads<AT, K>& L) {
    // opaque to the compiler, so each tile's address is formed where it is
    // loaded instead of every tile's ahead of the first load
    int tb = (int)blockIdx.x + t * grid;
    asm volatile("" : "+s"(tb));
    const int i = tile16_of(tb, tiles) * 16 + r;
    const int64_t ch = (((int64_t)(i / kRowBlock) * G + g0 + gl) * K) * kRowBlock + i % kRowBlock;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      L.b[k] = bits[ch + k * kRowBlock];
      L.a[k] = alpha_to_f32<AT>(scales[ch + k * kRowBlock]);
    }
  };

  for (int g0 = 0; g0 < G; g0 += slab_groups) {
    const int sg = min(slab_groups, G - g0);
    const int gl = 4 * wave + j;  // this lane's group within the slab
    const bool active = gl < sg;
    const int glc = active ? gl : sg - 1;  // clamped: loads stay in bounds
    const bool hx = (int)threadIdx.x < sg * 8;
    float v[16];
    if (hx) load_x16<XT>(x, (int64_t)g0 * kGroup + 16 * threadIdx.x, v);
    BlockLoads<AT, K> LA, LB;
    load(0, g0, glc, LA);
    if (g0 > 0) __syncthreads();  // the previous slab's tables are no longer read
    if (hx) {
      const int tg = threadIdx.x >> 3, bb = threadIdx.x & 7;
      float* tabs = lds + (tg * kGroupStride) / 4 + (8 * (bb >> 1) + (bb & 1)) * kTableFloats;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        build_table4(v[e], v[4 + e], v[8 + e], v[12 + e], tabs + 2 * e * kTableFloats);
    }
    __syncthreads();
    const uint32_t tab = lds_addr(lds) + glc * kGroupStride;
    auto sum = [&](const BlockLoads<AT, K>& L, float acc) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < K; ++k) s = fmaf(L.a[k], lut_dot128_sdwa(L.b[k], tab), s);
      return active ? acc + s : acc;
    };
#pragma unroll
    for (int t = 0; t < JMAX; t += 2) {
      if (t >= ntl) break;
      if (t + 1 < ntl) load(t + 1, g0, glc, LB);
      yacc[t] = sum(LA, yacc[t]);
      if (t + 1 >= ntl) break;
      if (t + 2 < ntl) load(t + 2, g0, glc, LA);
      yacc[t + 1] = sum(LB, yacc[t + 1]);
    }
  }

  // per tile: fixed-order sum over the 4 groups of a block, then over wavefronts
  __syncthreads();  // tables are no longer read: reuse LDS
#pragma unroll
  for (int t = 0; t < JMAX; ++t) {
    if (t >= ntl) break;
    float u = yacc[t];
    u += __shfl_xor(u, 16, kWave);
    u += __shfl_xor(u, 32, kWave);
    if (j == 0) lds[(t * NW + wave) * 16 + r] = u;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < ntl * 16; idx += NW * kWave) {
    const int t = idx >> 4, rr = idx & 15;
    float u = lds[(t * NW) * 16 + rr];
    for (int w = 1; w < NW; ++w) u += lds[(t * NW + w) * 16 + rr];
    const int i = tile16_of(blockIdx.x + t * grid, tiles) * 16 + rr;
    if (i < m) y[i] = u;
  }
}

// Column-split variant (the default when a workspace is given): workgroup
// (rb, s) covers the 64 rows of row block rb and the GPW*NW groups of column
// slice s; its wavefronts own GPW groups each and build only their slice's
// tables, so a layer becomes RB*S workgroups spread over every compute unit
// while each table is still shared by 64 rows.  With S > 1 slices each
// workgroup stores its 64 partial sums to partials[s][row]; gemv_reduce_kernel,
// launched next on the same stream, adds them in slice order 0..S-1 (a fixed
// order: the result does not depend on scheduling).  The kernel boundary
// orders the two, so no device-wide fence or atomic is needed.
template <typename XT, typename AT, int K, int NW, int GPW>
__global__ void __launch_bounds__(NW * kWave) gemv_split_kernel(
    const uint4* __restrict__ bits, const AT* __restrict__ scales, const XT* __restrict__ x,
    float* __restrict__ y, int m, int m_pad, int G, int S, float* __restrict__ partials) {
  extern __shared__ float lds[];
  const int rb = blockIdx.x / S;
  const int s = blockIdx.x - rb * S;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g0 = s * (NW * GPW);
  const int ng = min(NW * GPW, G - g0);
  uint4 b[GPW][K];
  float a[GPW][K];
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    const int gl = wave * GPW + j;
    if (gl < ng) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t c = (((int64_t)rb * G + g0 + gl) * K + k) * kRowBlock + lane;
        b[j][k] = bits[c];
        a[j][k] = alpha_to_f32<AT>(scales[c]);
      }
    }
  }
  for (int blk = threadIdx.x; blk < ng * 8; blk += NW * kWave) {
    float v[16];
    load_x16<XT>(x, (int64_t)g0 * kGroup + 16 * blk, v);
    const int gl = blk >> 3, bb = blk & 7;
    float* tab = lds + (gl * kChunksPerGroup + 8 * (bb >> 1) + (bb & 1)) * kTableFloats;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      build_table4(v[e], v[4 + e], v[8 + e], v[12 + e], tab + 2 * e * kTableFloats);
  }
  __syncthreads();
  float yacc = 0.f;
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    const int gl = wave * GPW + j;
    if (gl < ng) {
      const uint32_t tab = lds_addr(lds + gl * kChunksPerGroup * kTableFloats);
#pragma unroll
      for (int k = 0; k < K; ++k) yacc = fmaf(a[j][k], lut_dot128_sdwa(b[j][k], tab), yacc);
    }
  }
  if (NW > 1) {
    __syncthreads();
    lds[wave * kWave + lane] = yacc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < NW; ++w) yacc += lds[w * kWave + lane];
  }
  const int i = rb * kRowBlock + lane;
  if (S == 1) {
    if (i < m) y[i] = yacc;
  } else {
    partials[(int64_t)s * m_pad + i] = yacc;
  }
}

// y[i] = sum over slices s = 0..S-1 of partials[s][i], in that order.
__global__ void __launch_bounds__(256) gemv_reduce_kernel(const float* __restrict__ partials,
                                                          float* __restrict__ y, int m,
                                                          int m_pad, int S) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  float t = partials[i];
  for (int q = 1; q < S; ++q) t += partials[(int64_t)q * m_pad + i];
  y[i] = t;
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

enum Variant { kSplit = 0, kFullRow = 1, kDirect = 2, kRows = 3, kStream = 4 };

// Kernel choice by shape, from measurements on MI355X (per-launch times in
// HIP graphs over a rotating pool): row slices of 16 rows for small layers
// with K <= 2, column slices plus the reduce kernel for wide layers
// (n >= 2m), whole-row workgroups otherwise.  MBOK_GEMV_VARIANT overrides
// ("rows", "split", "fullrow", "direct") for measurements.
// bf16 activations may take the matrix-core kernel of the few-token product
// (one token); MBOK_GEMV_VARIANT=skinny selects it.
bool use_skinny_for_gemv(const Geom&) {
  const char* v = getenv("MBOK_GEMV_VARIANT");
  return v && strcmp(v, "skinny") == 0;
}

// The fp4 x fp8 matrix-core kernel (gemv_f4.hip) for bf16 activations: the
// default when a row carries at least 8192 sign bits (K n), the layer at
// least 2^25 (K m n), or K = 4.  Measured per call against the table kernel:
// 4096 x 4096 K = 2 3.98 against 4.10 us, 2048 x 4096 K = 3 4.02 / 4.43,
// 512 x 4096 K = 2 3.66 / 3.80, 8192 x 4096 K = 1 4.31 / 4.95, 4096 x 1024
// K = 4 3.36 / 3.70, every workload shape of K = 3 5-20% faster; the table
// kernel stays ahead for short rows (1024 x 1024 K = 2 2.89 against 3.10,
// 4096 x 4096 K = 1 3.66 / 3.76, 300 x 1024 K = 1 2.52 / 2.96).
// MBOK_GEMV_VARIANT=f4 selects it for every shape; any other value of the
// variable selects that table variant instead.
bool use_f4_for_gemv(const Geom& geo) {
  const char* v = getenv("MBOK_GEMV_VARIANT");
  if (v) return strcmp(v, "f4") == 0;
  const int64_t K = geo.K, kn = K * geo.n;
  return kn >= 8192 || kn * geo.m >= (int64_t(1) << 25) || K >= 4;
}

int variant_for(const Geom&) {
  const char* v = getenv("MBOK_GEMV_VARIANT");
  if (v && strcmp(v, "direct") == 0) return kDirect;
  if (v && strcmp(v, "fullrow") == 0) return kFullRow;
  if (v && strcmp(v, "split") == 0) return kSplit;
  if (v && strcmp(v, "rows") == 0) return kRows;
  if (v && strcmp(v, "stream") == 0) return kStream;
  return kStream;
}

constexpr int kSplitNW = 4;           // wavefronts per split workgroup
constexpr int kTargetWaves = 4096;    // 16 per compute unit

}  // namespace

// Column slices of the split kernel: groups per wavefront (1..4) and slices.
void gemv_split_shape(int RB, int G, int* gpw, int* S) {
  int s_target = (kTargetWaves + RB * kSplitNW - 1) / (RB * kSplitNW);
  if (s_target < 1) s_target = 1;
  const int per_slice = (G + s_target - 1) / s_target;
  int g = (per_slice + kSplitNW - 1) / kSplitNW;
  if (g < 1) g = 1;
  if (g > 4) g = 4;
  *gpw = g;
  *S = (G + kSplitNW * g - 1) / (kSplitNW * g);
}

size_t gemv_workspace_bytes(const mbok_desc* d) {
  const Geom geo = make_geom(d);
  if (variant_for(geo) != kSplit) return 0;
  int gpw, S;
  gemv_split_shape(geo.RB, geo.G, &gpw, &S);
  if (S <= 1) return 0;
  return (size_t)S * geo.RB * kRowBlock * sizeof(float);  // partials[S][m_pad]
}

namespace {

template <typename XT, typename AT, int K, int GPW>
int launch_split(const Geom& geo, int S, const uint4* bits, const AT* scales, const void* x,
                 float* y, void* ws, hipStream_t stream) {
  constexpr int NW = kSplitNW;
  float* partials = reinterpret_cast<float*>(ws);
  const int m_pad = geo.RB * kRowBlock;
  const size_t tab = (size_t)NW * GPW * kChunksPerGroup * kTableFloats * sizeof(float);
  const size_t lds = tab > NW * kWave * sizeof(float) ? tab : NW * kWave * sizeof(float);
  hipLaunchKernelGGL((gemv_split_kernel<XT, AT, K, NW, GPW>), dim3(geo.RB * S), dim3(NW * kWave),
                     lds, stream, bits, scales, reinterpret_cast<const XT*>(x), y, geo.m, m_pad,
                     geo.G, S, partials);
  if (hipGetLastError() != hipSuccess) return MBOK_ERR_HIP;
  if (S > 1) {
    hipLaunchKernelGGL(gemv_reduce_kernel, dim3((geo.m + 255) / 256), dim3(256), 0, stream,
                       partials, y, geo.m, m_pad, S);
    if (hipGetLastError() != hipSuccess) return MBOK_ERR_HIP;
  }
  return MBOK_OK;
}

// Rows per workgroup for the row-slice kernel: the largest R in {64, 32, 16}
// that still gives at least one workgroup per compute unit (MBOK_GEMV_R
// overrides, for measurements).
int rows_per_workgroup(int m) {
  const char* v = getenv("MBOK_GEMV_R");
  if (v) {
    const int r = atoi(v);
    if (r == 16 || r == 32 || r == 64) return r;
  }
  if (m >= 64 * 256) return 64;
  if (m >= 32 * 256) return 32;
  return 16;
}

int rows_waves() {
  const char* v = getenv("MBOK_GEMV_NW");
  const int nw = v ? atoi(v) : 16;
  return (nw == 4 || nw == 8 || nw == 16) ? nw : 16;
}

template <typename XT, typename AT, int K, int NW, int NS>
int launch_rows_nw(const Geom& geo, const uint4* bits, const AT* scales, const void* x, float* y,
                   hipStream_t stream) {
  constexpr int R = kWave / NS;
  // slabs of at most 32 groups: 32 * 2112 B = 66 KB of tables
  const int nslabs = (geo.G + 31) / 32;
  const int slab = (geo.G + nslabs - 1) / nslabs;
  size_t lds = (size_t)slab * kGroupStride;
  if (lds < NW * R * sizeof(float)) lds = NW * R * sizeof(float);
  const int blocks = (geo.m + R - 1) / R;
  hipLaunchKernelGGL((gemv_rows_kernel<XT, AT, K, NW, NS>), dim3(blocks), dim3(NW * kWave), lds,
                     stream, bits, scales, reinterpret_cast<const XT*>(x), y, geo.m, geo.G, slab);
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

constexpr int kStreamJ = 8;  // tiles per persistent workgroup (registers)

template <typename XT, typename AT, int K>
int launch_stream(const Geom& geo, const uint4* bits, const AT* scales, const void* x, float* y,
                  hipStream_t stream) {
  // slabs of at most 64 groups (135 KB of tables), one wavefront per block of
  // 4 groups; one workgroup per compute unit, more when the tiles would not
  // fit kStreamJ per workgroup
  const int nslabs = (geo.G + 63) / 64;
  const int slab = (geo.G + nslabs - 1) / nslabs;
  const int NW = (slab + 3) / 4;
  const int tiles = geo.RB * (kRowBlock / 16);
  int grid = tiles < 256 ? tiles : 256;
  if (grid * kStreamJ < tiles) grid = (tiles + kStreamJ - 1) / kStreamJ;
  size_t lds = (size_t)slab * kGroupStride;
  const size_t red = (size_t)kStreamJ * NW * 16 * sizeof(float);
  if (lds < red) lds = red;
  if ((const void*)(bits + (int64_t)tiles * 16 * geo.G * K) != (const void*)scales)
    return MBOK_ERR_UNSUPPORTED;  // the kernel finds the scales after the signs
  hipLaunchKernelGGL((gemv_stream_kernel<XT, AT, K, kStreamJ>), dim3(grid), dim3(NW * kWave),
                     lds, stream, bits, reinterpret_cast<const XT*>(x), geo.G, tiles, slab, grid,
                     NW, tiles / grid, tiles % grid, y, geo.m);
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

template <typename XT, typename AT, int K, int NS>
int launch_rows(const Geom& geo, const uint4* bits, const AT* scales, const void* x, float* y,
                hipStream_t stream) {
  // 16 wavefronts leave 128 VGPRs per lane, which K >= 3 exceeds (it would
  // spill to scratch): those use at most 8
  const int nw = rows_waves();
  if (nw == 4) return launch_rows_nw<XT, AT, K, 4, NS>(geo, bits, scales, x, y, stream);
  if constexpr (K <= 2) {
    if (nw == 16) return launch_rows_nw<XT, AT, K, 16, NS>(geo, bits, scales, x, y, stream);
  }
  return launch_rows_nw<XT, AT, K, 8, NS>(geo, bits, scales, x, y, stream);
}

template <typename XT, typename AT, int K>
int launch_typed(const Geom& geo, const void* packed, const void* x, float* y, void* ws,
                 hipStream_t stream) {
  constexpr int NW = 16;
  const uint4* bits = reinterpret_cast<const uint4*>(packed);
  const AT* scales = reinterpret_cast<const AT*>(reinterpret_cast<const char*>(packed) +
                                                 geo.bits_bytes);
  const int variant = variant_for(geo);
  if (variant == kStream) return launch_stream<XT, AT, K>(geo, bits, scales, x, y, stream);
  if (variant == kRows) {
    switch (rows_per_workgroup(geo.m)) {
      case 64: return launch_rows<XT, AT, K, 1>(geo, bits, scales, x, y, stream);
      case 32: return launch_rows<XT, AT, K, 2>(geo, bits, scales, x, y, stream);
      default: return launch_rows<XT, AT, K, 4>(geo, bits, scales, x, y, stream);
    }
  }
  if (variant == kSplit) {
    int gpw, S;
    gemv_split_shape(geo.RB, geo.G, &gpw, &S);
    if (S == 1 || ws != nullptr) {
      switch (gpw) {
        case 1: return launch_split<XT, AT, K, 1>(geo, S, bits, scales, x, y, ws, stream);
        case 2: return launch_split<XT, AT, K, 2>(geo, S, bits, scales, x, y, ws, stream);
        case 3: return launch_split<XT, AT, K, 3>(geo, S, bits, scales, x, y, ws, stream);
        default: return launch_split<XT, AT, K, 4>(geo, S, bits, scales, x, y, ws, stream);
      }
    }
    // no workspace: whole rows per workgroup
  }
  const int nslabs = (geo.G + kMaxSlabGroups - 1) / kMaxSlabGroups;
  const int slab = (geo.G + nslabs - 1) / nslabs;
  dim3 grid(geo.RB), block(NW * kWave);
  if (variant == kDirect) {
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
int launch_k(const Geom& geo, const void* packed, const void* x, float* y, void* ws,
             hipStream_t s) {
  switch (geo.K) {
    case 1: return launch_typed<XT, AT, 1>(geo, packed, x, y, ws, s);
    case 2: return launch_typed<XT, AT, 2>(geo, packed, x, y, ws, s);
    case 3: return launch_typed<XT, AT, 3>(geo, packed, x, y, ws, s);
    case 4: return launch_typed<XT, AT, 4>(geo, packed, x, y, ws, s);
  }
  return MBOK_ERR_UNSUPPORTED;
}

}  // namespace

int launch_gemv(const mbok_desc* d, const void* packed, const void* x, int32_t x_dtype,
                float* y, void* ws, hipStream_t stream) {
  const Geom geo = make_geom(d);
  const bool f16a = d->alpha_dtype == MBOK_F16;
  if (x_dtype == MBOK_BF16 && use_skinny_for_gemv(geo))
    return launch_skinny(d, packed, x, 1, d->n, y, d->m, stream);
  if (x_dtype == MBOK_BF16 && use_f4_for_gemv(geo)) return launch_gemv_f4(d, packed, x, y, stream);
  if (x_dtype == MBOK_BF16)
    return f16a ? launch_k<uint16_t, uint16_t>(geo, packed, x, y, ws, stream)
                : launch_k<uint16_t, float>(geo, packed, x, y, ws, stream);
  return f16a ? launch_k<float, uint16_t>(geo, packed, x, y, ws, stream)
              : launch_k<float, float>(geo, packed, x, y, ws, stream);
}

}  // namespace mbok
