// Decode product y = W_hat x for one bf16 token on the matrix cores (gfx950).
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// Paper-Notes reading note, 关键设计: W x splits into K Boolean products, one
// per kernel, each scaled per group of 128 input columns; 局限与展望: the
// activations stay in full precision.
//
// Each Boolean product of a 16-row tile is done by the scaled matrix-core
// instruction v_mfma_scale_f32_16x16x128_f8f6f4 with an fp8 (e4m3) A operand
// and an fp4 (e2m1) B operand:
//  * B (128 columns x 16 rows of W): the signs.  Each becomes the fp4 nibble
//    0b?010 (magnitude 1.0) whose sign bit ? is the stored bit, so B holds -b
//    (the sum is negated once at the end).  Lane 16q + r holds row r's sign
//    word q (32 columns) as four dwords of nibbles, one shift and one and-or
//    each; nibble p of dword d takes bit 4p + d of the word, so product term
//    k = 32q + 8d + p is column 32q + 16(p & 1) + 4d + (p >> 1) of the group
//    (the packed bit order).
//  * A (16 x 128): the activations of group j of the wavefront, a high fp8
//    part in row 4j and a low fp8 part in row 4j + 1 (all other rows zero).
//    With one E8M0 scale per 32 columns (the block's
//    largest exponent minus 7) the high part keeps 4 significant bits and the
//    low part (scale 2^-4 of it) the next 4, so together they hold the bf16
//    activation exactly when it lies within 13 binades of its block's largest
//    (below that the low part is rounded).
//  * D: the four groups of a wavefront use disjoint rows of A, so their
//    products of one kernel chain through one accumulator: D row 4j + e,
//    column r (lane 16j + r, register e) is group j's high (e = 0) or low
//    (e = 1) sum for row r.  That lane loaded alpha_k of (row r, group j)
//    itself and adds alpha_k (hi + lo) to its fp32 sum.
// The matrix cores add the 128 products of one block exactly when they span
// a narrow range (small integers; bf16 values within 6 binades) and
// otherwise drop bits far below the largest product: measured up to 1e-4 of
// the sum of |products| with fp8 values over the whole e4m3 range, about
// 1e-7 of the bound sum |W_hat| |x| on the workloads' Gaussian activations.
//
// Work split: one persistent workgroup per compute unit walks 16-row tiles
// (XCD-aware order); wavefront w owns groups 4w .. 4w+3 of a column slab of
// at most 64 groups.  Per (tile, kernel) a wavefront issues one 16-byte sign
// load per lane (16-lane block j: the 16 rows of group j, 256 contiguous
// bytes) and one 2-byte scale load, and transposes the (16-lane block, word)
// matrix with two v_permlane32_swap and two v_permlane16_swap; tile t+3 is
// loaded while tile t is multiplied.  Each wavefront first stages its own
// groups' activations: each lane takes 8 columns, finds its 32-column
// block's scale with two lane exchanges and writes the fp8 bytes of both
// parts to the wavefront's part of LDS (no workgroup barrier).  A
// fixed-order sum over wavefronts in LDS gives y (no atomics).  A NaN or infinite activation makes every output NaN.
#include "mbok_device.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kF4GroupsPerWave = 4;
constexpr int kF4MaxWaves = 16;
constexpr int kF4MaxSlab = kF4GroupsPerWave * kF4MaxWaves;  // 64 groups
// wavefronts per workgroup, so that four tile buffers fit in registers: 16
// (128 VGPRs each) for K <= 2, 12 (168) for K = 3, 8 (256) for K = 4
constexpr int f4_max_waves(int K) { return K >= 4 ? 8 : (K == 3 ? 12 : kF4MaxWaves); }
constexpr int kF4J = 8;         // tiles per workgroup (sums in registers)
constexpr int kE8M0One = 127;   // E8M0 code of 1.0
constexpr int kOpBytes = 256;   // fp8 A bytes per group: 2 parts x 4 lane blocks x 32

// Scale code of the low parts of a block whose high parts use `code`: 2^-4
// of the high scale (the low part is at most half an e4m3 step of the high
// part), clamped at the smallest code.
__device__ __forceinline__ int lo_code(int code) { return code > 4 ? code - 4 : 0; }

// Constants kept in registers (an SGPR and a VGPR), so that one v_and_or_b32
// takes both: a VOP3 instruction has no literal operand on this target.
__device__ __forceinline__ uint32_t sgpr_const(uint32_t v) {
  uint32_t r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
  return r;
}
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// The wavefront's own LDS writes are complete and visible to its lanes: its
// LDS operations finish in order, so waiting for all of them suffices (the
// compiler is kept from moving LDS accesses across the wait).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
// 4 x 4 transpose of (16-lane block, register): afterwards r[j] in block q is
// what r[q] held in block j.
__device__ __forceinline__ void transpose4(uint32_t (&r)[4]) {
  swap32(r[0], r[2]);
  swap32(r[1], r[3]);
  swap16(r[0], r[1]);
  swap16(r[2], r[3]);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// A streaming load: the signs are read once, so they are marked
// nontemporal (measured faster for read streams on this part).
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int K, typename AT>
struct F4Loads {
  uint4 s[K];  // lane 16j + r: the 4 sign words of (row r, group j, kernel k)
  AT a[K];     // and its scale
};

// Where column w (0..31) of 32-column block blk goes in a group's A operand
// bytes of one part: it is product term k = 32 blk + 8 ((w >> 2) & 3) +
// 2 (w & 3) + (w >> 4), and term k sits in lane block (k & 63) >> 4, byte
// (k & 15) + 16 [k >= 64] of that lane's 32.
__device__ __forceinline__ int op_byte(int blk, int w) {
  const int k = 32 * blk + 8 * ((w >> 2) & 3) + 2 * (w & 3) + (w >> 4);
  return ((k & 63) >> 4) * 32 + (k & 15) + (k >= 64 ? 16 : 0);
}

template <typename AT, int K, int JMAX>
__global__ void __launch_bounds__(f4_max_waves(K) * kWave) gemv_f4_kernel(
    const uint4* __restrict__ bits, const uint16_t* __restrict__ x, int G, int tiles,
    int slab_groups, float* __restrict__ y, int m) {
  // the scales follow the sign region: tiles * 16 rows x G groups x K chunks
  const AT* __restrict__ scales =
      reinterpret_cast<const AT*>(bits + (int64_t)tiles * 16 * G * K);
  __shared__ __attribute__((aligned(16))) uint8_t ops[kF4MaxSlab * kOpBytes];  // 16 KB
  __shared__ uint8_t codes[kF4MaxSlab * 4];
  __shared__ float red[JMAX * kF4MaxWaves * 16];
  const int NW = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane & 15;   // row of the tile (B column, D column)
  const int q = lane >> 4;   // lane block: the wavefront's group j at load time
  const int ntl = (tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;  // <= JMAX
  int nonfinite = 0;  // this thread saw a NaN or infinite activation
  const uint32_t sgn = sgpr_const(0x88888888u);  // fp4 sign bits
  const uint32_t one = vgpr_const(0x22222222u);  // fp4 1.0 in every nibble

  for (int g0 = 0; g0 < G; g0 += slab_groups) {
    const int sg = min(slab_groups, G - g0);
    // this lane's load group (block q), clamped so loads stay in bounds; a
    // group past the slab has a zero A operand and adds nothing
    const int gq = min(kF4GroupsPerWave * wave + q, sg - 1);
    auto load = [&](int t, F4Loads<K, AT>& L) {
      const int i0 = tile16_of(blockIdx.x + t * gridDim.x, tiles) * 16;
      const int rb = i0 / kRowBlock, r0 = i0 % kRowBlock;
      const int64_t ch = ((int64_t)rb * G + g0 + gq) * K * kRowBlock + r0 + r;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        L.s[k] = load_stream(bits + ch + k * kRowBlock);
        L.a[k] = scales[ch + k * kRowBlock];
      }
    };
    // the activations first, then the first tiles' signs: loads complete in
    // order, so the activations' conversion waits only for them while the
    // signs are still in flight
    const int xt = threadIdx.x;  // 8 columns per thread, 4 threads per 32-column block
    const bool has_x = xt < sg * 16;
    const uint4 u = has_x ? *reinterpret_cast<const uint4*>(x + (int64_t)g0 * kGroup + 8 * xt)
                          : make_uint4(0, 0, 0, 0);
    F4Loads<K, AT> L0, L1, L2, L3;
    load(0, L0);
    if (ntl > 1) load(1, L1);
    if (ntl > 2) load(2, L2);

    // ---- activations -> fp8 operand bytes.  Thread xt converts columns
    // 8 xt .. 8 xt + 7 of the slab, so wavefront w converts exactly its own
    // groups 4w .. 4w+3 into its own part of the LDS operand bytes: only the
    // wavefront's own LDS accesses need ordering, never the workgroup's.
    // (Its reads of the previous slab's bytes were consumed before the first
    // product of that slab.)
    if (has_x) {
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
      uint32_t mx = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, max(wv[e] & 0x7fffu, (wv[e] >> 16) & 0x7fffu));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1, kWave));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2, kWave));
      const int eb = (int)(mx >> 7);  // biased exponent of the block's largest |x|
      if (eb == 0xff) nonfinite = 1;
      const int code = mx == 0 ? kE8M0One : (eb > 7 ? eb - 7 : 0);
      const int lcode = lo_code(code);
      const int gl = xt >> 4, blk = (xt >> 2) & 3, sub = xt & 3;
      if (sub == 0) codes[gl * 4 + blk] = (uint8_t)code;
      uint8_t* hi = ops + gl * kOpBytes;
      uint8_t* lo = hi + kOpBytes / 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bb = (e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xffffu);
        const float v = __builtin_ldexpf(bf16_bits_to_f32(bb), kE8M0One - code);
        const int h8 = __builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false);
        const float l = __builtin_ldexpf(v - __builtin_amdgcn_cvt_f32_fp8(h8, 0), code - lcode);
        const int l8 = __builtin_amdgcn_cvt_pk_fp8_f32(l, 0.f, 0, false);
        const int pos = op_byte(blk, 8 * sub + e);
        hi[pos] = (uint8_t)h8;
        lo[pos] = (uint8_t)l8;
      }
    }
    wave_lds_sync();
    // ---- A operands, one per group j of the wavefront: lane (row rho = r,
    // block q) holds the high part of group j if rho == 4j, its low part if
    // rho == 4j + 1, else zeros.  The four have disjoint nonzero rows, so the
    // products of one kernel chain through one accumulator.
    v8i_t A[kF4GroupsPerWave];
    int ascale;
    {
      const int j = r >> 2, part = r & 3;
      const int gl = kF4GroupsPerWave * wave + j;
      const bool live = part < 2 && gl < sg;
      const int glc = min(gl, sg - 1);
      const uint4* src = reinterpret_cast<const uint4*>(ops + glc * kOpBytes +
                                                        (part & 1) * (kOpBytes / 2) + q * 32);
      const uint4 d0 = src[0], d1 = src[1];
      const v8i_t data = {(int)d0.x, (int)d0.y, (int)d0.z, (int)d0.w,
                          (int)d1.x, (int)d1.y, (int)d1.z, (int)d1.w};
#pragma unroll
      for (int jj = 0; jj < kF4GroupsPerWave; ++jj) {
        A[jj] = (live && jj == j) ? data : v8i_t{0, 0, 0, 0, 0, 0, 0, 0};
        // keep the operands in registers: recomputing the selects at every
        // product would cost eight VALU instructions each
        asm volatile("" : "+v"(A[jj]));
      }
      const int code = (int)codes[glc * 4 + q];
      ascale = !live ? kE8M0One : (part == 0 ? code : lo_code(code));
    }

    // Per kernel: the four groups' products chained; lane 16j + r then holds
    // group j's high and low sums for row r in registers 0 and 1.
    auto mul = [&](F4Loads<K, AT>& L, float a) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        uint32_t w[4] = {L.s[k].x, L.s[k].y, L.s[k].z, L.s[k].w};
        transpose4(w);  // w[j] in block q: word q of (row r, group j)
        v4f_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kF4GroupsPerWave; ++j) {
          v8i_t B;
          B[0] = (int)(((w[j] << 3) & sgn) | one);
          B[1] = (int)(((w[j] << 2) & sgn) | one);
          B[2] = (int)(((w[j] << 1) & sgn) | one);
          B[3] = (int)((w[j] & sgn) | one);
          B[4] = B[5] = B[6] = B[7] = 0;
          d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[j], B, d, 0, 4, 0, ascale, 0,
                                                               kE8M0One);
        }
        a = fmaf(alpha_to_f32<AT>(L.a[k]), d[0] + d[1], a);
      }
      return a;
    };

    // tile t + 3 is loaded while tile t is multiplied; each tile's sums (the
    // wavefront's four groups are its four lane blocks) go to LDS
    auto step = [&](int t, F4Loads<K, AT>& L) {
      float u = mul(L, 0.f);
      u += __shfl_xor(u, 16, kWave);
      u += __shfl_xor(u, 32, kWave);
      if (q == 0) {
        float* dst = red + (t * NW + wave) * 16 + r;
        *dst = g0 == 0 ? u : *dst + u;  // slabs in order
      }
    };
    for (int t = 0; t < ntl; t += 4) {
      if (t + 3 < ntl) load(t + 3, L3);
      step(t, L0);
      if (t + 1 >= ntl) break;
      if (t + 4 < ntl) load(t + 4, L0);
      step(t + 1, L1);
      if (t + 2 >= ntl) break;
      if (t + 5 < ntl) load(t + 5, L1);
      step(t + 2, L2);
      if (t + 3 >= ntl) break;
      if (t + 6 < ntl) load(t + 6, L2);
      step(t + 3, L3);
    }
  }

  const bool bad = __syncthreads_or(nonfinite) != 0;
  for (int idx = threadIdx.x; idx < ntl * 16; idx += blockDim.x) {
    const int t = idx >> 4, rr = idx & 15;
    float u = red[(t * NW) * 16 + rr];
    for (int w = 1; w < NW; ++w) u += red[(t * NW + w) * 16 + rr];
    const int i = tile16_of(blockIdx.x + t * gridDim.x, tiles) * 16 + rr;
    if (i < m) y[i] = bad ? __builtin_nanf("") : -u;  // B held -b
  }
}

template <typename AT, int K>
int launch_f4_k(const Geom& geo, const void* packed, const void* x, float* y,
                hipStream_t stream) {
  const int max_slab = kF4GroupsPerWave * f4_max_waves(K);
  const int nslabs = (geo.G + max_slab - 1) / max_slab;
  const int slab = (geo.G + nslabs - 1) / nslabs;
  const int NW = (slab + kF4GroupsPerWave - 1) / kF4GroupsPerWave;
  const int tiles = geo.RB * (kRowBlock / 16);
  int grid = tiles < 256 ? tiles : 256;
  if (grid * kF4J < tiles) grid = (tiles + kF4J - 1) / kF4J;
  hipLaunchKernelGGL((gemv_f4_kernel<AT, K, kF4J>), dim3(grid), dim3(NW * kWave), 0, stream,
                     reinterpret_cast<const uint4*>(packed),
                     reinterpret_cast<const uint16_t*>(x), geo.G, tiles, slab, y, geo.m);
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

template <typename AT>
int launch_f4_t(const Geom& geo, const void* packed, const void* x, float* y,
                hipStream_t stream) {
  switch (geo.K) {
    case 1: return launch_f4_k<AT, 1>(geo, packed, x, y, stream);
    case 2: return launch_f4_k<AT, 2>(geo, packed, x, y, stream);
    case 3: return launch_f4_k<AT, 3>(geo, packed, x, y, stream);
    case 4: return launch_f4_k<AT, 4>(geo, packed, x, y, stream);
  }
  return MBOK_ERR_UNSUPPORTED;
}

}  // namespace

int launch_gemv_f4(const mbok_desc* d, const void* packed, const void* x, float* y,
                   hipStream_t stream) {
  const Geom geo = make_geom(d);
  return d->alpha_dtype == MBOK_F16 ? launch_f4_t<uint16_t>(geo, packed, x, y, stream)
                                    : launch_f4_t<float>(geo, packed, x, y, stream);
}

}  // namespace mbok
