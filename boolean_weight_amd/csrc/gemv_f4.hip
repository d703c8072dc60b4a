// Decode product y = W_hat x for one bf16 token on the matrix cores (gfx950).
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// Paper-Notes reading note, 关键设计: W x splits into K Boolean products, one
// per kernel, each scaled per group of 128 input columns; 局限与展望: the
// activations stay in full precision.
//
// Each Boolean product of a 16-row tile is done by the scaled matrix-core
// instruction v_mfma_scale_f32_16x16x128_f8f6f4 with an fp8 (e4m3) A operand
// and an fp4 (e2m1) B operand, four instructions (one per 32-column word i of
// a group) per (tile, kernel):
//  * B (128 product terms x 16 rows of W): lane 16q + r loads the 16-byte
//    chunk of (row r, group q of the wavefront, kernel k) and gives product i
//    its word i, so K-block q of product i is word i of group q.  Nibble p of
//    B dword d takes bit 4p + d of the word in place (one and-or per dword,
//    no shift): product term kk = 8d + p of a word is column
//    16 (p & 1) + 4d + (p >> 1) (the packed bit order), and its value is
//    c_d + b for d < 3 (nibble bases 4.0/6.0, 2.0/4.0, 0/2.0: c = 5, 3, 1) and
//    -b for d = 3 (1.0/-1.0), b = +1 for a set bit.
//  * A (16 x 128): row 4q + e holds part e (0 high, 1 low) of the activations
//    of group q's word i, nonzero only in K-block q; columns of class d = 3 are
//    negated, so every product term is b x plus c_d x.  With one E8M0 scale
//    per (row, 32-term block) (the word's largest exponent minus 7) the high
//    part keeps 4 significant bits and the low part (scale 2^-4 of it) the
//    next 4, so together they hold the bf16 activation exactly when it lies
//    within 13 binades of its word's largest (below that the low part is
//    rounded).
//  * D: lane 16j + r, registers 0 and 1, accumulate over the four words group
//    j's high and low sums for row r, each sum_j b x + C_j where C_j =
//    sum (5 x, 3 x, x) over the group's columns of classes 0, 1, 2.  C_j is
//    formed once per group in fp32 while the activations are converted, and
//    the lane adds alpha_k (hi + lo - C_j) to its fp32 sum; the kernels'
//    product chains are interleaved.
// The matrix cores add the products of one instruction exactly when they span
// a narrow range (small integers; bf16 values within a few binades) and
// otherwise drop bits far below the largest product: about 1e-6 of the bound
// sum |W_hat| |x| on the workloads' Gaussian activations.
//
// Work split: one persistent workgroup per compute unit walks 16-row tiles
// (XCD-aware order); wavefront w owns groups 4w .. 4w+3 of a column slab of
// at most 64 groups.  Per (tile, kernel) a wavefront issues one 16-byte sign
// load per lane (16-lane block j: the 16 rows of group j, 256 contiguous
// bytes) and one 2-byte scale load; tile t+2 is loaded while tile t is
// multiplied, and only the first tile's loads go out before the activations
// are converted.  The grid size, wavefront count and tiles per workgroup are
// kernel arguments (preloaded), so no address waits on a dispatch-packet
// load.  Each wavefront first stages its own groups' activations: each lane
// takes 8 columns, finds its 32-column word's scale with two lane exchanges
// and writes the fp8 bytes of both parts to the wavefront's part of LDS (no
// workgroup barrier).  A fixed-order sum over wavefronts in LDS gives y (no
// atomics).  A NaN or infinite activation makes every output NaN.
#include <stdint.h>

#include <type_traits>

#include "mbok_device.h"
#include "mbok_lanes.h"
#include "mbok_launch.h"

namespace mbok {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
// the raw buffer loads, declared under the compiler's intrinsic names
__device__ u32x4_t raw_buffer_load_b128(i32x4_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ uint16_t raw_buffer_load_b16(i32x4_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.i16");
__device__ float raw_buffer_load_f32(i32x4_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.f32");

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kF4GroupsPerWave = 4;
constexpr int kF4MaxWaves = 16;
constexpr int kF4MaxSlab = kF4GroupsPerWave * kF4MaxWaves;  // 64 groups
// wavefronts per workgroup, so that the tile buffers fit in registers: 16
// (128 VGPRs each) for K <= 2, 12 (168) for K = 3, 8 (256) for K = 4
constexpr int f4_max_waves(int K) { return K >= 4 ? 8 : (K == 3 ? 12 : kF4MaxWaves); }
// with 2..4 tokens the A operands and sums take ~16 more registers per token
// pair and kernel: 12 wavefronts for K = 1, 8 otherwise
constexpr int f4_max_waves(int K, int TT) {
  return TT == 1 ? f4_max_waves(K) : (K == 1 ? 12 : 8);
}
constexpr int kF4J = 8;         // most tiles per workgroup
constexpr int kF4MaxTokens = 4;  // tokens of one few-token call (2 per token pair)
// tiles loaded ahead of the one multiplied (measured, 27648 x 5120 K = 3:
// 13.0 us two ahead, 13.4-13.7 three, 13.6 four)
constexpr int kF4Ahead = 2;
constexpr int kE8M0One = 127;   // E8M0 code of 1.0
constexpr int kOpBytes = 256;   // fp8 A bytes per group: 2 parts x 4 lane blocks x 32

// Scale code of the low parts of a block whose high parts use `code`: 2^-4
// of the high scale (the low part is at most half an e4m3 step of the high
// part), clamped at the smallest code.
__device__ __forceinline__ int lo_code(int code) { return code > 4 ? code - 4 : 0; }

// One thread's 8 activations of a 32-column word (wv[d] holds columns 2d,
// 2d + 1 as bf16) as fp8 high and low parts: H[d], L[d] bytes 0 and 1 for
// columns 2d, 2d + 1; class-3 columns (d >= 2 of an odd thread) negated; and
// corr += c(class) x over the 8 columns (c_lo for d < 2, c_hi for d >= 2).
// The scaled conversions divide by 2^(code - 127) (the high part) and
// 2^(lo_code - 127) (the low part) and round once, nearest-even: the same
// bytes as scaling with ldexp and converting (checked bit for bit over every
// finite bf16 value and every code the word scale takes), and the high
// part converts straight from the bf16 pair.
__device__ __forceinline__ void convert_word8(const uint32_t (&wv)[4], int code, bool odd,
                                              float c_lo, float c_hi, uint32_t (&H)[4],
                                              uint32_t (&L)[4], float& corr) {
  typedef short v2i16 __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
  const float s_hi = __builtin_ldexpf(1.f, code - kE8M0One);
  const float s_lo = __builtin_ldexpf(1.f, lo_code(code) - kE8M0One);
  const uint32_t neg3 = odd ? 0x80008000u : 0u;  // sign flips of a class-3 pair
  const v2i16 zero = {0, 0};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // class 3 (d >= 2 of an odd thread) negated; its c is 0, so the
    // correction may take the negated values too
    const uint32_t pair = d >= 2 ? wv[d] ^ neg3 : wv[d];
    const float x0 = bf16_bits_to_f32(pair & 0xffffu);
    const float x1 = bf16_bits_to_f32(pair >> 16);
    corr = fmaf(d < 2 ? c_lo : c_hi, x0, corr);
    corr = fmaf(d < 2 ? c_lo : c_hi, x1, corr);
    const v2i16 h = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
        zero, __builtin_bit_cast(v2bf16, pair), s_hi, false);
    const int hb = __builtin_bit_cast(int, h);
    const auto back = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb, s_hi, false);
    // exact: the bits the high part left (the bytes above 1 are never read)
    const v2i16 l =
        __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(zero, x0 - back[0], x1 - back[1], s_lo, false);
    H[d] = (uint32_t)hb;
    L[d] = (uint32_t)__builtin_bit_cast(int, l);
  }
}

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

// DPP lane exchanges within a quad / a 16-lane row (no LDS round trip).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kRowMirror = 0x140;     // lane i <- lane 15 - i of its row
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7 - i of its half-row
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

// The 8 term bytes this thread writes for one part: P[d] holds the fp8 bytes
// of its columns 2d, 2d + 1 in bytes 0, 1; the partner thread (sub ^ 2, the
// other h) holds the interleaved ones.  h = 0 returns dwords [A2d B2d A2d+1
// B2d+1] for d = 0, 1; h = 1 for d = 2, 3 (A: the h = 0 thread, B: h = 1).
__device__ __forceinline__ uint2 pair_terms(const uint32_t (&P)[4], bool h) {
  const uint32_t r1 = dpp_u32<kQuadXor2>(h ? P[0] : P[2]);
  const uint32_t r2 = dpp_u32<kQuadXor2>(h ? P[1] : P[3]);
  // v_perm_b32 selector bytes 0..3 take the second operand's bytes, 4..7 the first's
  constexpr uint32_t kInterleave = 0x05010400u;  // [s1.b0, s0.b0, s1.b1, s0.b1]
  const uint32_t w0 = __builtin_amdgcn_perm(h ? P[2] : r1, h ? r1 : P[0], kInterleave);
  const uint32_t w1 = __builtin_amdgcn_perm(h ? P[3] : r2, h ? r2 : P[1], kInterleave);
  return make_uint2(w0, w1);
}

__device__ __forceinline__ uint4 as_uint4(u32x4_t v) { return make_uint4(v.x, v.y, v.z, v.w); }

// Sign and scale loads go through buffer resources (V#) built in SGPRs per
// tile.  A tile past the workgroup's last gets a resource of size 0, so its
// loads return zeros without touching memory: every tile slot issues the same
// loads whether or not it holds a tile, the count of loads in flight is the
// same on every path through the tile loop, and the compiler's wait counts
// before each tile's products cover that tile's loads only (with the loads
// skipped by a branch, it waited for every load in flight, the tiles issued
// ahead included).
constexpr int kAuxNt = 2;  // cache-policy bit: nontemporal (the signs are read once)
// raw (stride 0) buffer over p: bytes [0, 2^32 - 1) if live, none otherwise;
// word 3 holds the gfx9 data format the raw loads ignore
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* p, bool live) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4_t v;
  v.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  v.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
  v.z = __builtin_amdgcn_readfirstlane(live ? -1 : 0);
  v.w = 0x00020000;
  return v;
}
template <typename AT>
__device__ __forceinline__ AT load_scale(i32x4_t rsrc, int voffset);
template <>
__device__ __forceinline__ uint16_t load_scale<uint16_t>(i32x4_t rsrc, int voffset) {
  return raw_buffer_load_b16(rsrc, voffset, 0, 0);
}
template <>
__device__ __forceinline__ float load_scale<float>(i32x4_t rsrc, int voffset) {
  return raw_buffer_load_f32(rsrc, voffset, 0, 0);
}

// A scale as the 32-bit lane value the spreading exchanges move, and back
template <typename AT>
__device__ __forceinline__ uint32_t scale_bits_f4(AT a);
template <>
__device__ __forceinline__ uint32_t scale_bits_f4<float>(float a) { return __float_as_uint(a); }
template <>
__device__ __forceinline__ uint32_t scale_bits_f4<uint16_t>(uint16_t a) { return a; }
template <typename AT>
__device__ __forceinline__ float scale_value_f4(uint32_t b);
template <>
__device__ __forceinline__ float scale_value_f4<float>(uint32_t b) { return __uint_as_float(b); }
template <>
__device__ __forceinline__ float scale_value_f4<uint16_t>(uint32_t b) {
  return f16_bits_to_f32((uint16_t)b);
}

template <int K, typename AT>
struct F4Loads {
  uint4 s[K];  // lane 16j + r: the 4 sign words of (row r, group j, kernel k)
  AT a[K];     // and its scale
};

// A 32-column word's column c (0..31) is its product term kk =
// 8 ((c >> 2) & 3) + 2 (c & 3) + (c >> 4): B dword d, nibble p holds bit 4p + d
// of the word, i.e. column 16 (p & 1) + 4 d + (p >> 1), as term 8d + p.  The
// converted activations are stored in LDS in term order.

template <typename AT, int K, int NT, bool EARLY>
__global__ void __launch_bounds__(f4_max_waves(K) * kWave) gemv_f4_kernel(
    const uint4* __restrict__ bits, const uint16_t* __restrict__ x, int G, int tiles,
    int slab_groups, int grid, int nw, int tpw, int textra, float* __restrict__ y, int m) {
  // the scales follow the sign region: tiles * 16 rows x G groups x K chunks
  const AT* __restrict__ scales =
      reinterpret_cast<const AT*>(bits + (int64_t)tiles * 16 * G * K);
  // converted activations: [group][part][word][32 terms]
  __shared__ __attribute__((aligned(16))) uint8_t ops[kF4MaxSlab * kOpBytes];  // 16 KB
  __shared__ __attribute__((aligned(4))) uint8_t codes[kF4MaxSlab * 4];
  __shared__ float red[NT * kF4MaxWaves * 16];
  const int NW = nw;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane & 15;   // row of the tile (B column, D column; A row at A time)
  const int q = lane >> 4;   // lane block: K-block q holds group 4 wave + q
  const int b = blockIdx.x;
  const int ntl = tpw + (b < textra ? 1 : 0);  // tiles of this workgroup, <= NT (tile slots)
  int nonfinite = 0;  // this thread saw a NaN or infinite activation
  // B dword d, nibble p: bit 4p + d of the word at nibble bit d, over a base
  // nibble: d = 0 {4.0, 6.0}, d = 1 {2.0, 4.0}, d = 2 {0, 2.0}, d = 3
  // {1.0, -1.0}, i.e. c_d + b with c = 5, 3, 1 and -b for d = 3
  const uint32_t m0 = sgpr_const(0x11111111u), m1 = sgpr_const(0x22222222u);
  const uint32_t m2 = sgpr_const(0x44444444u), m3 = sgpr_const(0x88888888u);
  const uint32_t b0 = vgpr_const(0x66666666u), b1 = vgpr_const(0x44444444u);
  const uint32_t b3 = vgpr_const(0x22222222u);

  for (int g0 = 0; g0 < G; g0 += slab_groups) {
    const int sg = min(slab_groups, G - g0);
    // this lane's load group (block q), clamped so loads stay in bounds; a
    // group past the slab has a zero A operand and adds nothing
    const int gq = min(kF4GroupsPerWave * wave + q, sg - 1);
    // this lane's byte offsets inside a tile's sign and scale blocks
    const int vs = (gq * K * kRowBlock + r) * 16;
    const int va = (gq * K * kRowBlock + r) * (int)sizeof(AT);
    auto load = [&](int t, F4Loads<K, AT>& L) {
      // opaque to the compiler, so each tile's address is formed where it is
      // loaded instead of every tile's ahead of the first load
      int tb = b + t * grid;
      asm volatile("" : "+s"(tb));
      const int i0 = tile16_of(tb, tiles) * 16;
      const int rb = i0 / kRowBlock, r0 = i0 % kRowBlock;
      const int64_t c0 = ((int64_t)rb * G + g0) * K * kRowBlock + r0;  // the tile's first chunk
      const i32x4_t rs = buffer_rsrc(bits + c0, t < ntl);
      const i32x4_t ra = buffer_rsrc(scales + c0, t < ntl);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        L.s[k] = as_uint4(raw_buffer_load_b128(rs, vs + k * kRowBlock * 16, 0, kAuxNt));
        L.a[k] = load_scale<AT>(ra, va + k * kRowBlock * (int)sizeof(AT));
      }
    };
    // The activations first.  Every compute unit asks for them at once, and
    // each sign load issued before they arrive sits in the same memory
    // queues ahead of other wavefronts' activation loads, so only the first
    // tile's signs go out now (EARLY: some workgroup has more than one tile
    // to keep the stream going, or the layer has several column slabs;
    // else right after the activations arrive), the rest once this
    // wavefront has converted its activations (measured: 11008 x 4096 7.9
    // -> 7.1 us, 4096 x 4096 K = 2 4.65 -> 4.09 us).  With one tile per
    // workgroup: 4096 x 4096, K = 2 (one slab) 3.57 us waiting for the
    // activations against 3.81 us with the signs right behind them; 4096 x
    // 11008, K = 3 (two slabs) 6.82 against 6.50 us.  EARLY is a
    // compile-time choice so that the conversion waits for the activations
    // alone (a runtime condition made the compiler wait for every load in
    // flight).
    const int xt = threadIdx.x;  // 8 columns per thread, 4 threads per 32-column word
    const bool has_x = xt < sg * 16;
    const uint4 u = has_x ? *reinterpret_cast<const uint4*>(x + (int64_t)g0 * kGroup + 8 * xt)
                          : make_uint4(0, 0, 0, 0);
    F4Loads<K, AT> Lb[kF4Ahead + 1];  // tile t in Lb[t % (kF4Ahead + 1)]
    F4Loads<K, AT>& L0 = Lb[0];
    if (EARLY) {
      load(0, L0);
    } else {
      // one tile per workgroup: its signs go out as soon as the activations
      // are in, ahead of the conversion (3.96 -> 3.86 us for 4096 x 4096)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      load(0, L0);
    }

    // ---- activations -> fp8 operand bytes.  Thread xt converts columns
    // 8 xt .. 8 xt + 7 of the slab, so wavefront w converts exactly its own
    // groups 4w .. 4w+3 into its own part of the LDS operand bytes: only the
    // wavefront's own LDS accesses need ordering, never the workgroup's.
    // (Its reads of the previous slab's bytes were consumed before the first
    // product of that slab.)
    float corr = 0.f;  // sum over this thread's columns of c(class) x
    if (has_x) {
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
      uint32_t mx = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, max(wv[e] & 0x7fffu, (wv[e] >> 16) & 0x7fffu));
      // the word's 4 threads are a quad of lanes
      mx = max(mx, dpp_u32<kQuadXor1>(mx));
      mx = max(mx, dpp_u32<kQuadXor2>(mx));
      const int eb = (int)(mx >> 7);  // biased exponent of the word's largest |x|
      if (eb == 0xff) nonfinite = 1;
      const int code = mx == 0 ? kE8M0One : (eb > 7 ? eb - 7 : 0);
      const int gl = xt >> 4, word = (xt >> 2) & 3, sub = xt & 3;
      if (sub == 0) codes[gl * 4 + word] = (uint8_t)code;
      // column 8 sub + e is in sign class ((8 sub + e) >> 2) & 3 = 2 (sub & 1) + (e >> 2)
      const bool odd = (sub & 1) != 0;
      const float c_lo = odd ? 1.f : 5.f, c_hi = odd ? 0.f : 3.f;  // e < 4, e >= 4
      uint32_t H[4], L[4];  // fp8 bytes of columns 2d, 2d + 1 in bytes 0, 1
      convert_word8(wv, code, odd, c_lo, c_hi, H, L, corr);
      // Threads sub and sub ^ 2 fill the word's terms 16 (sub & 1) ..
      // +15: term byte 2e + h is column 8 sub + e of the thread with h =
      // sub >> 1.  The h = 0 thread writes bytes 0..7 (columns e = 0..3 of
      // both), the h = 1 thread bytes 8..15, after one exchange in the quad.
      const bool h = (sub >> 1) != 0;
      uint8_t* hi = ops + gl * kOpBytes + word * 32 + 16 * (sub & 1) + 8 * (int)h;
      uint8_t* lo = hi + kOpBytes / 2;
      *reinterpret_cast<uint2*>(hi) = pair_terms(H, h);
      *reinterpret_cast<uint2*>(lo) = pair_terms(L, h);
    }
    // the group's correction: lanes 16j .. 16j+15 converted group 4w + j
    corr = corr + __uint_as_float(dpp_u32<kQuadXor1>(__float_as_uint(corr)));
    corr = corr + __uint_as_float(dpp_u32<kQuadXor2>(__float_as_uint(corr)));
    corr = corr + __uint_as_float(dpp_u32<kRowHalfMirror>(__float_as_uint(corr)));
    corr = corr + __uint_as_float(dpp_u32<kRowMirror>(__float_as_uint(corr)));
    // a tile past the last loads zeros, reading nothing
#pragma unroll
    for (int j = 1; j < kF4Ahead; ++j)
      if (j < NT) load(j, Lb[j]);
    wave_lds_sync();
    // ---- A operands, one per word i.  K-block q of product i holds word i
    // of the wavefront's group q (the B operand of lane 16q + r is word i of
    // its own loaded chunk), and A row 4q + e holds part e of that group
    // (e = 0 high, 1 low), nonzero only in K-block q.  Lane 16c + rho holds
    // A row rho, terms 16c .. 16c+15 (bytes 0..15) and 64 + 16c .. (bytes
    // 16..31): K-block q sits in lane blocks 2 (q & 1) and 2 (q & 1) + 1,
    // bytes 16 (q >> 1) ... of them.  The E8M0 scale of (row rho, K-block c)
    // is lane 16c + rho's.
    v8i_t A[4];
    int ascale[4];
    {
      const int qa = r >> 2, part = r & 3;  // this lane's A row 4 qa + part
      const int gl = kF4GroupsPerWave * wave + qa;
      const bool live = part < 2 && gl < sg && (qa & 1) == (q >> 1);
      const int glc = min(gl, sg - 1);
      const uint8_t* base = ops + glc * kOpBytes + (part & 1) * (kOpBytes / 2) + 16 * (q & 1);
      const bool upper = (qa >> 1) != 0;
      // every read goes out before the first wait, and the zero half (or the
      // whole operand of a dead row) is masked, not branched around
      uint4 dd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dd[i] = *reinterpret_cast<const uint4*>(base + 32 * i);
      // scale of (row r, K-block q): nonzero rows of K-block q are 4q, 4q + 1
      const int sq = min(kF4GroupsPerWave * wave + q, sg - 1);
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + sq * 4);
      const uint32_t keep = live ? ~0u : 0u;
      const uint32_t klo = upper ? 0u : keep, khi = upper ? keep : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A[i] = v8i_t{(int)(dd[i].x & klo), (int)(dd[i].y & klo), (int)(dd[i].z & klo),
                     (int)(dd[i].w & klo), (int)(dd[i].x & khi), (int)(dd[i].y & khi),
                     (int)(dd[i].z & khi), (int)(dd[i].w & khi)};
        asm volatile("" : "+v"(A[i]));
      }
      const bool srow = (r >> 2) == q && part < 2 && kF4GroupsPerWave * wave + q < sg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int code = (int)((cw >> (8 * i)) & 0xffu);
        ascale[i] = !srow ? kE8M0One : (part == 0 ? code : lo_code(code));
      }
    }

    // Per kernel: the four words' products chained (interleaved over the
    // kernels); lane 16j + r then holds group j's high and low sums for row r
    // in registers 0 and 1.
    auto mul = [&](F4Loads<K, AT>& L, float a) {
      v4f_t d[K];
#pragma unroll
      for (int k = 0; k < K; ++k) d[k] = v4f_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const uint32_t w = i == 0 ? L.s[k].x : i == 1 ? L.s[k].y : i == 2 ? L.s[k].z : L.s[k].w;
          v8i_t B;
          B[0] = (int)((w & m0) | b0);
          B[1] = (int)((w & m1) | b1);
          B[2] = (int)(w & m2);
          B[3] = (int)((w & m3) | b3);
          B[4] = B[5] = B[6] = B[7] = 0;
          d[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[i], B, d[k], 0, 4, 0,
                                                                  ascale[i], 0, kE8M0One);
        }
      }
#pragma unroll
      for (int k = 0; k < K; ++k) a = fmaf(alpha_to_f32<AT>(L.a[k]), (d[k][0] + d[k][1]) - corr, a);
      return a;
    };

    // tile t + kF4Ahead is loaded while tile t is multiplied; each tile's sums (the
    // wavefront's four groups are its four lane blocks) go to LDS
    auto step = [&](int t, F4Loads<K, AT>& L) {
      float uu = mul(L, 0.f);
      // sum over the four lane blocks (groups): 16-lane rows 0+1, 2+3, then
      // the two halves, with lane swaps instead of LDS permutes
      {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(uu), __float_as_uint(uu),
                                                        false, false);
        uu = __uint_as_float(a[0]) + __uint_as_float(a[1]);
        const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(uu), __float_as_uint(uu),
                                                        false, false);
        uu = __uint_as_float(c[0]) + __uint_as_float(c[1]);
      }
      if (q == 0) {
        float* dst = red + (t * NW + wave) * 16 + r;
        *dst = g0 == 0 ? uu : *dst + uu;  // slabs in order
      }
    };
    // Unrolled over the tile slots, with every load issued whether or not
    // its tile exists: a workgroup's last tile leaves the chain, no path that
    // skipped a load merges back into the steps, and the wait before tile
    // t's products covers tile t's loads alone (with the loads skipped by a
    // branch, the compiler waited for every load in flight, the tiles issued
    // ahead included).
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntl) break;
      if (t + kF4Ahead < NT) load(t + kF4Ahead, Lb[(t + kF4Ahead) % (kF4Ahead + 1)]);
      step(t, Lb[t % (kF4Ahead + 1)]);
    }
  }

  const bool bad = __syncthreads_or(nonfinite) != 0;
  for (int idx = threadIdx.x; idx < ntl * 16; idx += NW * kWave) {
    const int t = idx >> 4, rr = idx & 15;
    float uu = red[(t * NW) * 16 + rr];
    for (int w = 1; w < NW; ++w) uu += red[(t * NW + w) * 16 + rr];
    const int i = tile16_of(b + t * grid, tiles) * 16 + rr;
    if (i < m) y[i] = bad ? __builtin_nanf("") : uu;
  }
}

// The few-token form of the kernel above, TT = 2..4 tokens (EARLY as above:
// here whenever a workgroup has more than one tile): token t's
// activations are row t of x (ldx elements apart) and its outputs row t of y
// (ldy apart).  A row 4q + s of a product holds part s & 1 of token
// 2p + (s >> 1) for token pair p (the one-token kernel leaves rows 4q + 2,
// 4q + 3 zero), so 2 tokens take one instruction per (tile, kernel, word) and
// 3 or 4 tokens two.
template <typename AT, int K, int NT, int TT, bool EARLY>
__device__ __forceinline__ void f4_tokens_body(const uint4* __restrict__ bits,
                                               const uint16_t* __restrict__ x, int64_t ldx,
                                               int G, int tiles, int slab_groups, int grid,
                                               int nw, int tpw, int textra,
                                               float* __restrict__ y, int64_t ldy, int m) {
  constexpr int TP = (TT + 1) / 2;  // token pairs
  static_assert(TT >= 2 && TT <= 4, "2..4 tokens");
  constexpr int kSlabMax = kF4GroupsPerWave * f4_max_waves(K, TT);
  constexpr int kRedWaves = f4_max_waves(K, TT);
  // the scales follow the sign region: tiles * 16 rows x G groups x K chunks
  const AT* __restrict__ scales =
      reinterpret_cast<const AT*>(bits + (int64_t)tiles * 16 * G * K);
  // converted activations: [group][token][part][word][32 terms]
  __shared__ __attribute__((aligned(16))) uint8_t ops[kSlabMax * TT * kOpBytes];  // up to 32 KB
  __shared__ __attribute__((aligned(4))) uint8_t codes[kSlabMax * TT * 4];
  __shared__ float red[NT * kRedWaves * TT * 16];
  const int NW = nw;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane & 15;   // row of the tile (B column, D column; A row at A time)
  const int q = lane >> 4;   // lane block: K-block q holds group 4 wave + q
  const int b = blockIdx.x;
  const int ntl = tpw + (b < textra ? 1 : 0);  // tiles of this workgroup, <= NT
  int nonfinite = 0;  // bit t: this thread saw a NaN or infinite activation of token t
  // B dword d, nibble p: bit 4p + d of the word at nibble bit d, over a base
  // nibble: d = 0 {4.0, 6.0}, d = 1 {2.0, 4.0}, d = 2 {0, 2.0}, d = 3
  // {1.0, -1.0}, i.e. c_d + b with c = 5, 3, 1 and -b for d = 3
  const uint32_t m0 = sgpr_const(0x11111111u), m1 = sgpr_const(0x22222222u);
  const uint32_t m2 = sgpr_const(0x44444444u), m3 = sgpr_const(0x88888888u);
  const uint32_t b0 = vgpr_const(0x66666666u), b1 = vgpr_const(0x44444444u);
  const uint32_t b3 = vgpr_const(0x22222222u);

  for (int g0 = 0; g0 < G; g0 += slab_groups) {
    const int sg = min(slab_groups, G - g0);
    // this lane's load group (block q), clamped so loads stay in bounds; a
    // group past the slab has a zero A operand and adds nothing
    const int gq = min(kF4GroupsPerWave * wave + q, sg - 1);
    // this lane's byte offsets inside a tile's sign and scale blocks
    const int vs = (gq * K * kRowBlock + r) * 16;
    const int va = (gq * K * kRowBlock + r) * (int)sizeof(AT);
    auto load = [&](int t, F4Loads<K, AT>& L) {
      // opaque to the compiler, so each tile's address is formed where it is
      // loaded instead of every tile's ahead of the first load
      int tb = b + t * grid;
      asm volatile("" : "+s"(tb));
      const int i0 = tile16_of(tb, tiles) * 16;
      const int rb = i0 / kRowBlock, r0 = i0 % kRowBlock;
      const int64_t c0 = ((int64_t)rb * G + g0) * K * kRowBlock + r0;  // the tile's first chunk
      const i32x4_t rs = buffer_rsrc(bits + c0, t < ntl);
      const i32x4_t ra = buffer_rsrc(scales + c0, t < ntl);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        L.s[k] = as_uint4(raw_buffer_load_b128(rs, vs + k * kRowBlock * 16, 0, kAuxNt));
        L.a[k] = load_scale<AT>(ra, va + k * kRowBlock * (int)sizeof(AT));
      }
    };
    // The activations first.  Every compute unit asks for them at once, and
    // each sign load issued before they arrive sits in the same memory
    // queues ahead of other wavefronts' activation loads, so only the first
    // tile's signs go out now (EARLY: some workgroup has more than one tile
    // to keep the stream going; else right after the activations arrive),
    // the rest once this wavefront has converted its activations (measured:
    // 11008 x 4096 7.9 -> 7.1 us, 4096 x 4096 K = 2 4.65 -> 4.09 us).  EARLY
    // is a compile-time choice so that the conversion waits for the
    // activations alone (a runtime condition made the compiler wait for
    // every load in flight).
    const int xt = threadIdx.x;  // 8 columns per thread, 4 threads per 32-column word
    const bool has_x = xt < sg * 16;
    uint4 u[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      u[tt] = has_x ? *reinterpret_cast<const uint4*>(x + tt * ldx + (int64_t)g0 * kGroup + 8 * xt)
                    : make_uint4(0, 0, 0, 0);
    F4Loads<K, AT> Lb[kF4Ahead + 1];  // tile t in Lb[t % (kF4Ahead + 1)]
    F4Loads<K, AT>& L0 = Lb[0];
    if (EARLY) {
      load(0, L0);
    } else {
      // one tile per workgroup: its signs go out as soon as the activations
      // are in, ahead of the conversion (3.96 -> 3.86 us for 4096 x 4096)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      load(0, L0);
    }

    // ---- activations -> fp8 operand bytes.  Thread xt converts columns
    // 8 xt .. 8 xt + 7 of the slab, so wavefront w converts exactly its own
    // groups 4w .. 4w+3 into its own part of the LDS operand bytes: only the
    // wavefront's own LDS accesses need ordering, never the workgroup's.
    // (Its reads of the previous slab's bytes were consumed before the first
    // product of that slab.)
    float corr[TT];  // sum over this thread's columns of c(class) x, per token
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) corr[tt] = 0.f;
    if (has_x) {
      const int gl = xt >> 4, word = (xt >> 2) & 3, sub = xt & 3;
      // column 8 sub + e is in sign class ((8 sub + e) >> 2) & 3 = 2 (sub & 1) + (e >> 2)
      const bool odd = (sub & 1) != 0;
      const float c_lo = odd ? 1.f : 5.f, c_hi = odd ? 0.f : 3.f;  // e < 4, e >= 4
      // Threads sub and sub ^ 2 fill the word's terms 16 (sub & 1) ..
      // +15: term byte 2e + h is column 8 sub + e of the thread with h =
      // sub >> 1.  The h = 0 thread writes bytes 0..7 (columns e = 0..3 of
      // both), the h = 1 thread bytes 8..15, after one exchange in the quad.
      const bool h = (sub >> 1) != 0;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const uint32_t wv[4] = {u[tt].x, u[tt].y, u[tt].z, u[tt].w};
        uint32_t mx = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = max(mx, max(wv[e] & 0x7fffu, (wv[e] >> 16) & 0x7fffu));
        // the word's 4 threads are a quad of lanes
        mx = max(mx, dpp_u32<kQuadXor1>(mx));
        mx = max(mx, dpp_u32<kQuadXor2>(mx));
        const int eb = (int)(mx >> 7);  // biased exponent of the word's largest |x|
        if (eb == 0xff) nonfinite |= 1 << tt;
        const int code = mx == 0 ? kE8M0One : (eb > 7 ? eb - 7 : 0);
          if (sub == 0) codes[(gl * TT + tt) * 4 + word] = (uint8_t)code;
        uint32_t H[4], L[4];  // fp8 bytes of columns 2d, 2d + 1 in bytes 0, 1
        convert_word8(wv, code, odd, c_lo, c_hi, H, L, corr[tt]);
        uint8_t* hi = ops + (gl * TT + tt) * kOpBytes + word * 32 + 16 * (sub & 1) + 8 * (int)h;
        uint8_t* lo = hi + kOpBytes / 2;
        *reinterpret_cast<uint2*>(hi) = pair_terms(H, h);
        *reinterpret_cast<uint2*>(lo) = pair_terms(L, h);
      }
    }
    // the group's correction: lanes 16j .. 16j+15 converted group 4w + j
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      float c = corr[tt];
      c = c + __uint_as_float(dpp_u32<kQuadXor1>(__float_as_uint(c)));
      c = c + __uint_as_float(dpp_u32<kQuadXor2>(__float_as_uint(c)));
      c = c + __uint_as_float(dpp_u32<kRowHalfMirror>(__float_as_uint(c)));
      c = c + __uint_as_float(dpp_u32<kRowMirror>(__float_as_uint(c)));
      corr[tt] = c;
    }
    // a tile past the last loads zeros, reading nothing
#pragma unroll
    for (int j = 1; j < kF4Ahead; ++j)
      if (j < NT) load(j, Lb[j]);
    wave_lds_sync();
    // ---- A operands, one per word i.  K-block q of product i holds word i
    // of the wavefront's group q (the B operand of lane 16q + r is word i of
    // its own loaded chunk), and A row 4q + e holds part e of that group
    // (e = 0 high, 1 low), nonzero only in K-block q.  Lane 16c + rho holds
    // A row rho, terms 16c .. 16c+15 (bytes 0..15) and 64 + 16c .. (bytes
    // 16..31): K-block q sits in lane blocks 2 (q & 1) and 2 (q & 1) + 1,
    // bytes 16 (q >> 1) ... of them.  The E8M0 scale of (row rho, K-block c)
    // is lane 16c + rho's.
    // With several tokens, A row 4q + s holds part s & 1 of token 2p + (s >> 1)
    // in the operands of token pair p.
    v8i_t A[TP][4];
    int ascale[TP][4];
    {
      const int qa = r >> 2, slot = r & 3;  // this lane's A row 4 qa + slot
      const int part = slot & 1;
      const int gl = kF4GroupsPerWave * wave + qa;
      const int glc = min(gl, sg - 1);
      const bool upper = (qa >> 1) != 0;
      // scale of (row r, K-block q): nonzero rows of K-block q are 4q .. 4q + 3
      const int sq = min(kF4GroupsPerWave * wave + q, sg - 1);
#pragma unroll
      for (int p = 0; p < TP; ++p) {
        const int tt = 2 * p + (slot >> 1);
        const int ttc = min(tt, TT - 1);
        const bool live = tt < TT && gl < sg && (qa & 1) == (q >> 1);
        const uint8_t* base =
            ops + (glc * TT + ttc) * kOpBytes + part * (kOpBytes / 2) + 16 * (q & 1);
        // every read goes out before the first wait, and the zero half (or the
        // whole operand of a dead row) is masked, not branched around
        uint4 dd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dd[i] = *reinterpret_cast<const uint4*>(base + 32 * i);
        const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + (sq * TT + ttc) * 4);
        const uint32_t keep = live ? ~0u : 0u;
        const uint32_t klo = upper ? 0u : keep, khi = upper ? keep : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          A[p][i] = v8i_t{(int)(dd[i].x & klo), (int)(dd[i].y & klo), (int)(dd[i].z & klo),
                          (int)(dd[i].w & klo), (int)(dd[i].x & khi), (int)(dd[i].y & khi),
                          (int)(dd[i].z & khi), (int)(dd[i].w & khi)};
          asm volatile("" : "+v"(A[p][i]));
        }
        const bool srow = (r >> 2) == q && tt < TT && kF4GroupsPerWave * wave + q < sg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int code = (int)((cw >> (8 * i)) & 0xffu);
          ascale[p][i] = !srow ? kE8M0One : (part == 0 ? code : lo_code(code));
        }
      }
    }

    // Per kernel: the four words' products chained (interleaved over the
    // kernels); lane 16j + r then holds group j's high and low sums for row r
    // in registers 0 and 1.
    // Per kernel: the four words' products chained (interleaved over the
    // kernels); lane 16j + r then holds group j's high and low sums for row r
    // in registers 0 and 1 (token 2p of pair p) and 2 and 3 (token 2p + 1).
    auto mul = [&](F4Loads<K, AT>& L, float (&a)[TT]) {
      v4f_t d[K][TP];
#pragma unroll
      for (int k = 0; k < K; ++k)
#pragma unroll
        for (int p = 0; p < TP; ++p) d[k][p] = v4f_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const uint32_t w = i == 0 ? L.s[k].x : i == 1 ? L.s[k].y : i == 2 ? L.s[k].z : L.s[k].w;
          v8i_t B;
          B[0] = (int)((w & m0) | b0);
          B[1] = (int)((w & m1) | b1);
          B[2] = (int)(w & m2);
          B[3] = (int)((w & m3) | b3);
          B[4] = B[5] = B[6] = B[7] = 0;
#pragma unroll
          for (int p = 0; p < TP; ++p)
            d[k][p] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[p][i], B, d[k][p], 0, 4, 0,
                                                                       ascale[p][i], 0, kE8M0One);
        }
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float al = alpha_to_f32<AT>(L.a[k]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const v4f_t& dk = d[k][tt >> 1];
          const float hl = (tt & 1) ? dk[2] + dk[3] : dk[0] + dk[1];
          a[tt] = fmaf(al, hl - corr[tt], a[tt]);
        }
      }
    };

    // tile t + kF4Ahead is loaded while tile t is multiplied; each tile's sums (the
    // wavefront's four groups are its four lane blocks) go to LDS
    auto step = [&](int t, F4Loads<K, AT>& L) {
      float uu[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) uu[tt] = 0.f;
      mul(L, uu);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        // sum over the four lane blocks (groups): 16-lane rows 0+1, 2+3, then
        // the two halves, with lane swaps instead of LDS permutes
        float v = uu[tt];
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                        false, false);
        v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
        const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                        false, false);
        v = __uint_as_float(c[0]) + __uint_as_float(c[1]);
        if (q == 0) {
          float* dst = red + ((t * NW + wave) * TT + tt) * 16 + r;
          *dst = g0 == 0 ? v : *dst + v;  // slabs in order
        }
      }
    };
    // Unrolled over the tile slots, with every load issued whether or not
    // its tile exists: a workgroup's last tile leaves the chain, no path that
    // skipped a load merges back into the steps, and the wait before tile
    // t's products covers tile t's loads alone (with the loads skipped by a
    // branch, the compiler waited for every load in flight, the tiles issued
    // ahead included).
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntl) break;
      if (t + kF4Ahead < NT) load(t + kF4Ahead, Lb[(t + kF4Ahead) % (kF4Ahead + 1)]);
      step(t, Lb[t % (kF4Ahead + 1)]);
    }
  }

  int bad = 0;  // bit t: some thread saw a non-finite activation of token t
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
    if (__syncthreads_or(nonfinite & (1 << tt))) bad |= 1 << tt;
  for (int idx = threadIdx.x; idx < ntl * 16 * TT; idx += NW * kWave) {
    const int tt = idx / (ntl * 16), e = idx - tt * (ntl * 16);
    const int t = e >> 4, rr = e & 15;
    float uu = red[((t * NW) * TT + tt) * 16 + rr];
    for (int w = 1; w < NW; ++w) uu += red[((t * NW + w) * TT + tt) * 16 + rr];
    const int i = tile16_of(b + t * grid, tiles) * 16 + rr;
    if (i < m) y[tt * ldy + i] = ((bad >> tt) & 1) ? __builtin_nanf("") : uu;
  }
}


// 2..4 tokens; the token strides follow the arguments of the one-token kernel
template <typename AT, int K, int NT, int TT, bool EARLY>
__global__ void __launch_bounds__(f4_max_waves(K, TT) * kWave) gemm_f4_kernel(
    const uint4* __restrict__ bits, const uint16_t* __restrict__ x, int G, int tiles,
    int slab_groups, int grid, int nw, int tpw, int textra, float* __restrict__ y, int m,
    int ldx, int ldy) {
  f4_tokens_body<AT, K, NT, TT, EARLY>(bits, x, ldx, G, tiles, slab_groups, grid, nw, tpw, textra, y,
                                     ldy, m);
}

// ---------------------------------------------------------------------------
// Several tokens, one product per group.  The kernels above give each
// product one 32-column word of four groups (K-block q = group q), so an A
// row is nonzero in one K-block only and holds one part of one token: at most
// two tokens per instruction.  Here a product covers the four words of ONE
// group (K-block c = word c), so every A row is dense: row 2 tt + e holds part
// e of token 8 o + tt of token octet o, and one instruction per (tile,
// group, kernel, octet) takes 8 tokens.
//  * B: lane 16q + r loads the chunk of (row r, group q) as above; a 4 x 4
//    transpose of (16-lane block, word) gives lane 16c + r word c of every
//    group g (the B operand of group g's product), and the scales are spread
//    so that every lane holds alpha of its row r for the four groups.
//  * A (per group and octet, from the wavefront's LDS staging): lane 16c + rho
//    holds row rho, terms 16c .. 16c+15 (word c >> 1) and 64 + 16c .. (word
//    2 + (c >> 1)), at byte offset 16 (c & 1) of those words; the E8M0 scale
//    of (row rho, K-block c) is the code of word c of that token and part.
//  * D: lane 16j + r holds rows 4j .. 4j+3: tokens 2j (registers 0, 1: high
//    and low parts) and 2j + 1 (2, 3) of the octet, row r of W.  The lane adds
//    alpha (hi + lo - C) for its two tokens over the four groups and the K
//    kernels, so no lane exchange is needed to sum over groups.
// The correction C of (token, group) is formed while converting and handed
// to the lanes that need it through the wavefront's LDS.
constexpr int kF4gTokens = 8;  // tokens per octet (16 A rows: 8 tokens x 2 parts)
constexpr int kF4gMaxOctets = 2;
constexpr int kF4gMaxTokens = kF4gTokens * kF4gMaxOctets;
// wavefronts per workgroup (4 groups each): 12 for one octet (<= 168
// registers), 8 for two (the A operands of 16 tokens take 64)
constexpr int f4g_waves(int NO) { return NO == 1 ? 12 : 8; }
constexpr int kF4gOpsPerWave = kF4GroupsPerWave * kF4gTokens * kOpBytes;  // 8 KB

template <typename AT, int K, int NT, int NO, bool EARLY>
__global__ void __launch_bounds__(f4g_waves(NO) * kWave) gemm_f4g_kernel(
    const uint4* __restrict__ bits, const uint16_t* __restrict__ X, int G, int tiles,
    int slab_groups, int grid, int nw, int tpw, int textra, float* __restrict__ Y, int m, int T,
    int ldx, int ldy) {
  constexpr int NWM = f4g_waves(NO);
  constexpr int TO = kF4gTokens * NO;  // token slots
  const AT* __restrict__ scales =
      reinterpret_cast<const AT*>(bits + (int64_t)tiles * 16 * G * K);
  // per wavefront: [group j][token tt][part][word][32 terms] of one octet
  __shared__ __attribute__((aligned(16))) uint8_t ops[NWM * kF4gOpsPerWave];
  __shared__ __attribute__((aligned(4))) uint8_t codes[NWM * kF4GroupsPerWave * kF4gTokens * 4];
  __shared__ float cs[NWM * kF4GroupsPerWave * kF4gTokens];  // corrections [j][tt]
  __shared__ float red[NT * NWM * TO * 16];
  __shared__ int bad_tokens;
  const int NW = nw;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane & 15;
  const int q = lane >> 4;
  const int b = blockIdx.x;
  const int ntl = tpw + (b < textra ? 1 : 0);
  if (threadIdx.x == 0) bad_tokens = 0;
  int nonfinite = 0;  // bit t: this thread saw a NaN or infinite activation of token t
  const uint32_t m0 = sgpr_const(0x11111111u), m1 = sgpr_const(0x22222222u);
  const uint32_t m2 = sgpr_const(0x44444444u), m3 = sgpr_const(0x88888888u);
  const uint32_t b0 = vgpr_const(0x66666666u), b1 = vgpr_const(0x44444444u);
  const uint32_t b3 = vgpr_const(0x22222222u);
  uint8_t* const wops = ops + wave * kF4gOpsPerWave;
  uint8_t* const wcodes = codes + wave * (kF4GroupsPerWave * kF4gTokens * 4);
  float* const wcs = cs + wave * (kF4GroupsPerWave * kF4gTokens);

  for (int g0 = 0; g0 < G; g0 += slab_groups) {
    const int sg = min(slab_groups, G - g0);
    const int gq = min(kF4GroupsPerWave * wave + q, sg - 1);
    const int vs = (gq * K * kRowBlock + r) * 16;
    const int va = (gq * K * kRowBlock + r) * (int)sizeof(AT);
    auto load = [&](int t, F4Loads<K, AT>& L) {
      int tb = b + t * grid;
      asm volatile("" : "+s"(tb));
      const int i0 = tile16_of(tb, tiles) * 16;
      const int rb = i0 / kRowBlock, r0 = i0 % kRowBlock;
      const int64_t c0 = ((int64_t)rb * G + g0) * K * kRowBlock + r0;
      const i32x4_t rs = buffer_rsrc(bits + c0, t < ntl);
      const i32x4_t ra = buffer_rsrc(scales + c0, t < ntl);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        L.s[k] = as_uint4(raw_buffer_load_b128(rs, vs + k * kRowBlock * 16, 0, kAuxNt));
        L.a[k] = load_scale<AT>(ra, va + k * kRowBlock * (int)sizeof(AT));
      }
    };
    // this lane converts 8 columns of group j = lane >> 4 of the wavefront
    const int gl = kF4GroupsPerWave * wave + q;
    const bool has_g = gl < sg;
    const int word = (lane >> 2) & 3, sub = lane & 3;
    const bool odd = (sub & 1) != 0;
    const float c_lo = odd ? 1.f : 5.f, c_hi = odd ? 0.f : 3.f;
    const bool h = (sub >> 1) != 0;
    const uint16_t* xg = X + (int64_t)(g0 + (has_g ? gl : 0)) * kGroup + 8 * (lane & 15);

    F4Loads<K, AT> Lb[kF4Ahead + 1];
    v8i_t A[kF4GroupsPerWave][NO];
    int ascale[kF4GroupsPerWave][NO];
    float C[NO][kF4GroupsPerWave][2];  // corrections of this lane's two tokens
    // every token's activations first, then the first tile's signs (as for
    // one token: behind the activations, or once they are in)
    uint4 u[NO][kF4gTokens];
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int tt = 0; tt < kF4gTokens; ++tt) {
        const int t = kF4gTokens * o + tt;
        u[o][tt] = (has_g && t < T) ? *reinterpret_cast<const uint4*>(xg + t * ldx)
                                    : make_uint4(0, 0, 0, 0);
      }
    if (EARLY) {
      load(0, Lb[0]);
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      load(0, Lb[0]);
    }
#pragma unroll
    for (int o = 0; o < NO; ++o) {
#pragma unroll
      for (int tt = 0; tt < kF4gTokens; ++tt) {
        // tokens past T are not converted: their A rows are masked below
        if (kF4gTokens * o + tt >= T) break;
        const uint32_t wv[4] = {u[o][tt].x, u[o][tt].y, u[o][tt].z, u[o][tt].w};
        uint32_t mx = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = max(mx, max(wv[e] & 0x7fffu, (wv[e] >> 16) & 0x7fffu));
        mx = max(mx, dpp_u32<kQuadXor1>(mx));
        mx = max(mx, dpp_u32<kQuadXor2>(mx));
        const int eb = (int)(mx >> 7);
        if (eb == 0xff) nonfinite |= 1 << (kF4gTokens * o + tt);
        const int code = mx == 0 ? kE8M0One : (eb > 7 ? eb - 7 : 0);
          if (sub == 0) wcodes[(q * kF4gTokens + tt) * 4 + word] = (uint8_t)code;
        float corr = 0.f;
        uint32_t H[4], L[4];  // fp8 bytes of columns 2d, 2d + 1 in bytes 0, 1
        convert_word8(wv, code, odd, c_lo, c_hi, H, L, corr);
        uint8_t* hi = wops + (q * kF4gTokens + tt) * kOpBytes + word * 32 + 16 * (sub & 1) +
                      8 * (int)h;
        *reinterpret_cast<uint2*>(hi) = pair_terms(H, h);
        *reinterpret_cast<uint2*>(hi + kOpBytes / 2) = pair_terms(L, h);
        // the group's correction: sum over its 16 lanes
        corr = corr + __uint_as_float(dpp_u32<kQuadXor1>(__float_as_uint(corr)));
        corr = corr + __uint_as_float(dpp_u32<kQuadXor2>(__float_as_uint(corr)));
        corr = corr + __uint_as_float(dpp_u32<kRowHalfMirror>(__float_as_uint(corr)));
        corr = corr + __uint_as_float(dpp_u32<kRowMirror>(__float_as_uint(corr)));
        if (r == 0) wcs[q * kF4gTokens + tt] = corr;
      }
      if (o == 0) {
#pragma unroll
        for (int j = 1; j < kF4Ahead; ++j)
          if (j < NT) load(j, Lb[j]);
      }
      wave_lds_sync();
      // A operands of the octet: lane 16c + rho, row rho = 2 tt + part
      {
        const int tt = r >> 1, part = r & 1;
        const int w1 = q >> 1;
        const int Tl = T - kF4gTokens * o;  // live tokens of the octet (may exceed 8)
        const uint32_t keep = tt < Tl ? ~0u : 0u;
        const bool c0 = 2 * q < Tl, c1 = 2 * q + 1 < Tl;
#pragma unroll
        for (int j = 0; j < kF4GroupsPerWave; ++j) {
          const uint8_t* base =
              wops + (j * kF4gTokens + tt) * kOpBytes + part * (kOpBytes / 2) + 16 * (q & 1);
          const uint4 lo4 = *reinterpret_cast<const uint4*>(base + 32 * w1);
          const uint4 hi4 = *reinterpret_cast<const uint4*>(base + 32 * (w1 + 2));
          A[j][o] = v8i_t{(int)(lo4.x & keep), (int)(lo4.y & keep), (int)(lo4.z & keep),
                          (int)(lo4.w & keep), (int)(hi4.x & keep), (int)(hi4.y & keep),
                          (int)(hi4.z & keep), (int)(hi4.w & keep)};
          const int code = keep ? wcodes[(j * kF4gTokens + tt) * 4 + q] : kE8M0One;
          ascale[j][o] = part == 0 ? code : lo_code(code);
          C[o][j][0] = c0 ? wcs[j * kF4gTokens + 2 * q] : 0.f;
          C[o][j][1] = c1 ? wcs[j * kF4gTokens + 2 * q + 1] : 0.f;
        }
      }
      // the reads are in registers before the next octet overwrites the staging
      wave_lds_sync();
    }

    // Per kernel: the chunk's words transposed into the four groups' B
    // operands, the scales spread, one product per (group, octet); lane
    // 16j + r adds alpha (hi + lo - C) for tokens 2j, 2j + 1 of each octet.
    auto mul = [&](F4Loads<K, AT>& L, float (&acc)[NO][2]) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        uint32_t w[4] = {L.s[k].x, L.s[k].y, L.s[k].z, L.s[k].w};
        transpose4(w);  // w[g] = word q of (row r, group g)
        uint32_t ab[4];
        spread4(scale_bits_f4<AT>(L.a[k]), ab);  // ab[g] = alpha of (row r, group g)
#pragma unroll
        for (int g = 0; g < kF4GroupsPerWave; ++g) {
          v8i_t B;
          B[0] = (int)((w[g] & m0) | b0);
          B[1] = (int)((w[g] & m1) | b1);
          B[2] = (int)(w[g] & m2);
          B[3] = (int)((w[g] & m3) | b3);
          B[4] = B[5] = B[6] = B[7] = 0;
          const float al = scale_value_f4<AT>(ab[g]);
#pragma unroll
          for (int o = 0; o < NO; ++o) {
            const v4f_t d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A[g][o], B, v4f_t{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, ascale[g][o], 0, kE8M0One);
            acc[o][0] = fmaf(al, (d[0] + d[1]) - C[o][g][0], acc[o][0]);
            acc[o][1] = fmaf(al, (d[2] + d[3]) - C[o][g][1], acc[o][1]);
          }
        }
      }
    };
    auto step = [&](int t, F4Loads<K, AT>& L) {
      float acc[NO][2];
#pragma unroll
      for (int o = 0; o < NO; ++o) acc[o][0] = acc[o][1] = 0.f;
      mul(L, acc);
#pragma unroll
      for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int tok = kF4gTokens * o + 2 * q + e;
          float* dst = red + ((t * NW + wave) * TO + tok) * 16 + r;
          *dst = g0 == 0 ? acc[o][e] : *dst + acc[o][e];  // slabs in order
        }
    };
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntl) break;
      if (t + kF4Ahead < NT) load(t + kF4Ahead, Lb[(t + kF4Ahead) % (kF4Ahead + 1)]);
      step(t, Lb[t % (kF4Ahead + 1)]);
    }
  }

  __syncthreads();
  if (nonfinite) atomicOr(&bad_tokens, nonfinite);
  __syncthreads();
  const int bad = bad_tokens;
  for (int idx = threadIdx.x; idx < ntl * 16 * T; idx += NW * kWave) {
    const int tok = idx / (ntl * 16), e = idx - tok * (ntl * 16);
    const int t = e >> 4, rr = e & 15;
    float uu = red[((t * NW) * TO + tok) * 16 + rr];
    for (int w = 1; w < NW; ++w) uu += red[((t * NW + w) * TO + tok) * 16 + rr];
    const int i = tile16_of(b + t * grid, tiles) * 16 + rr;
    if (i < m) Y[(int64_t)tok * ldy + i] = ((bad >> tok) & 1) ? __builtin_nanf("") : uu;
  }
}

// ---------------------------------------------------------------------------
// The SVID scale variant's product y = sum_k s_out^k (.) (B_k (s_in^k (.) x))
// ("Successive SVID" of the gist.science summaries: each kernel's scales are
// an outer product s_out^k s_in^k^T) on the decode kernel above.  The packed
// layer holds s_out^k[i] in every group's scale slot, so the per-(tile,
// kernel) epilogue is the decode's.  What changes is the activation side:
// kernel k contracts with its own vector v_k = s_in^k (.) x (one fp32
// product, exact for fp16 scales and bf16 x), split into four fp8 parts with
// per-word scales 2^(code - 127 - 4p), p = 0..3: 16 significant bits of the
// word's largest |v|, as the bf16 hi/lo split of the bf16 +-1 product keeps.
// The four parts fill A rows 4q .. 4q + 3 of group q, so each (tile, kernel,
// word) is still one instruction; D registers 0..3 of lane 16j + r are the
// four parts' sums of group j and row r.  Every workgroup converts K vectors
// (x and the K rows of s_in it needs) per column slab; slabs of at most 32
// groups (8 wavefronts: the A operands of K kernels take 32 K registers).
constexpr int kF4sMaxWaves = 8;
constexpr int kF4sMaxSlab = kF4GroupsPerWave * kF4sMaxWaves;  // 32 groups
constexpr int kF4sOpBytes = 4 * kGroup;  // 4 parts x 128 terms per (kernel, group)

template <typename AT>
__device__ __forceinline__ void load8_f32(const AT* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8_f32<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = f16_bits_to_f32((uint16_t)(w[e] & 0xffffu));
    v[2 * e + 1] = f16_bits_to_f32((uint16_t)(w[e] >> 16));
  }
}
template <>
__device__ __forceinline__ void load8_f32<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w;
  v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
}
// 8 bf16 (XF = false) or fp32 (XF = true) activations
template <bool XF>
__device__ __forceinline__ void load8_x(const void* x, int64_t col, float (&v)[8]) {
  if constexpr (XF) {
    load8_f32<float>(reinterpret_cast<const float*>(x) + col, v);
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + col);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
      v[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
    }
  }
}

// Part scale codes 2^-4 apart, clamped at the smallest code.
__device__ __forceinline__ int part_code(int code, int p) {
  return code > 4 * p ? code - 4 * p : 0;
}

template <typename AT, int K, int NT, bool XF, bool EARLY>
__global__ void __launch_bounds__(kF4sMaxWaves * kWave) gemv_f4_svid_kernel(
    const uint4* __restrict__ bits, const void* __restrict__ x, const AT* __restrict__ s_in,
    int G, int tiles, int slab_groups, int grid, int nw, int tpw, int textra,
    float* __restrict__ y, int m) {
  typedef short v2i16 __attribute__((ext_vector_type(2)));
  const AT* __restrict__ scales =
      reinterpret_cast<const AT*>(bits + (int64_t)tiles * 16 * G * K);
  const int n = G * kGroup;
  // converted vectors: [kernel][group][part][word][32 terms]
  __shared__ __attribute__((aligned(16))) uint8_t ops[K * kF4sMaxSlab * kF4sOpBytes];
  __shared__ __attribute__((aligned(4))) uint8_t codes[K * kF4sMaxSlab * 4];
  __shared__ float red[NT * kF4sMaxWaves * 16];
  const int NW = nw;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane & 15;
  const int q = lane >> 4;
  const int b = blockIdx.x;
  const int ntl = tpw + (b < textra ? 1 : 0);
  int nonfinite = 0;
  const uint32_t m0 = sgpr_const(0x11111111u), m1 = sgpr_const(0x22222222u);
  const uint32_t m2 = sgpr_const(0x44444444u), m3 = sgpr_const(0x88888888u);
  const uint32_t b0 = vgpr_const(0x66666666u), b1 = vgpr_const(0x44444444u);
  const uint32_t b3 = vgpr_const(0x22222222u);
  const v2i16 zero = {0, 0};

  for (int g0 = 0; g0 < G; g0 += slab_groups) {
    const int sg = min(slab_groups, G - g0);
    const int gq = min(kF4GroupsPerWave * wave + q, sg - 1);
    const int vs = (gq * K * kRowBlock + r) * 16;
    const int va = (gq * K * kRowBlock + r) * (int)sizeof(AT);
    auto load = [&](int t, F4Loads<K, AT>& L) {
      int tb = b + t * grid;
      asm volatile("" : "+s"(tb));
      const int i0 = tile16_of(tb, tiles) * 16;
      const int rb = i0 / kRowBlock, r0 = i0 % kRowBlock;
      const int64_t c0 = ((int64_t)rb * G + g0) * K * kRowBlock + r0;
      const i32x4_t rs = buffer_rsrc(bits + c0, t < ntl);
      const i32x4_t ra = buffer_rsrc(scales + c0, t < ntl);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        L.s[k] = as_uint4(raw_buffer_load_b128(rs, vs + k * kRowBlock * 16, 0, kAuxNt));
        L.a[k] = load_scale<AT>(ra, va + k * kRowBlock * (int)sizeof(AT));
      }
    };
    // thread xt: 8 columns of group gl (wavefront w converts its own groups)
    const int xt = threadIdx.x;
    const bool has_x = xt < sg * 16;
    const int64_t col = (int64_t)g0 * kGroup + 8 * (has_x ? xt : 0);
    float xv[8], sv[K][8];
    load8_x<XF>(x, col, xv);
#pragma unroll
    for (int k = 0; k < K; ++k) load8_f32<AT>(s_in + (int64_t)k * n + col, sv[k]);
    F4Loads<K, AT> Lb[kF4Ahead + 1];
    if (EARLY) {
      load(0, Lb[0]);
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      load(0, Lb[0]);
    }
    float corr[K];
    {
      const int gl = xt >> 4, word = (xt >> 2) & 3, sub = xt & 3;
      const bool odd = (sub & 1) != 0;
      const float c_lo = odd ? 1.f : 5.f, c_hi = odd ? 0.f : 3.f;
      const bool h = (sub >> 1) != 0;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        float v[8];
        uint32_t mx = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // class 3 (columns e >= 4 of an odd thread) negated; its c is 0
          const float p = has_x ? sv[k][e] * xv[e] : 0.f;
          v[e] = (e >= 4 && odd) ? -p : p;
          mx = max(mx, __float_as_uint(p) & 0x7fffffffu);
        }
        mx = max(mx, dpp_u32<kQuadXor1>(mx));
        mx = max(mx, dpp_u32<kQuadXor2>(mx));
        const int eb = (int)(mx >> 23);
        if (eb == 0xff) nonfinite = 1;
        const int code = mx == 0 ? kE8M0One : (eb > 7 ? eb - 7 : 0);
        if (sub == 0 && has_x) codes[(k * kF4sMaxSlab + gl) * 4 + word] = (uint8_t)code;
        float cs = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) cs = fmaf(e < 4 ? c_lo : c_hi, v[e], cs);
        uint8_t* base = ops + (k * kF4sMaxSlab + gl) * kF4sOpBytes + word * 32 + 16 * (sub & 1) +
                        8 * (int)h;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float sc = __builtin_ldexpf(1.f, part_code(code, p) - kE8M0One);
          uint32_t P[4];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const v2i16 c8 =
                __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(zero, v[2 * d], v[2 * d + 1], sc, false);
            P[d] = (uint32_t)__builtin_bit_cast(int, c8);
            if (p < 3) {
              // what this part leaves (exact: the part holds the leading bits)
              const auto back = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)P[d], sc, false);
              v[2 * d] -= back[0];
              v[2 * d + 1] -= back[1];
            }
          }
          if (has_x) *reinterpret_cast<uint2*>(base + p * kGroup) = pair_terms(P, h);
        }
        cs = cs + __uint_as_float(dpp_u32<kQuadXor1>(__float_as_uint(cs)));
        cs = cs + __uint_as_float(dpp_u32<kQuadXor2>(__float_as_uint(cs)));
        cs = cs + __uint_as_float(dpp_u32<kRowHalfMirror>(__float_as_uint(cs)));
        cs = cs + __uint_as_float(dpp_u32<kRowMirror>(__float_as_uint(cs)));
        corr[k] = cs;
      }
    }
#pragma unroll
    for (int j = 1; j < kF4Ahead; ++j)
      if (j < NT) load(j, Lb[j]);
    wave_lds_sync();
    // A operands of kernel k, word i: lane 16c + rho holds A row rho =
    // 4 qa + p (part p of group qa), nonzero only in K-block qa (lane blocks
    // 2 (qa & 1), 2 (qa & 1) + 1, bytes 16 (qa >> 1) ..)
    v8i_t A[K][4];
    int ascale[K][4];
    {
      const int qa = r >> 2, part = r & 3;
      const int gl = kF4GroupsPerWave * wave + qa;
      const bool live = gl < sg && (qa & 1) == (q >> 1);
      const int glc = min(gl, sg - 1);
      const bool upper = (qa >> 1) != 0;
      const uint32_t keep = live ? ~0u : 0u;
      const uint32_t klo = upper ? 0u : keep, khi = upper ? keep : 0u;
      const int sq = min(kF4GroupsPerWave * wave + q, sg - 1);
      const bool srow = (r >> 2) == q && kF4GroupsPerWave * wave + q < sg;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const uint8_t* base = ops + (k * kF4sMaxSlab + glc) * kF4sOpBytes + part * kGroup +
                              16 * (q & 1);
        uint4 dd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dd[i] = *reinterpret_cast<const uint4*>(base + 32 * i);
        const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + (k * kF4sMaxSlab + sq) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          A[k][i] = v8i_t{(int)(dd[i].x & klo), (int)(dd[i].y & klo), (int)(dd[i].z & klo),
                          (int)(dd[i].w & klo), (int)(dd[i].x & khi), (int)(dd[i].y & khi),
                          (int)(dd[i].z & khi), (int)(dd[i].w & khi)};
          asm volatile("" : "+v"(A[k][i]));
          const int code = (int)((cw >> (8 * i)) & 0xffu);
          ascale[k][i] = srow ? part_code(code, part) : kE8M0One;
        }
      }
    }

    auto mul = [&](F4Loads<K, AT>& L, float a) {
      v4f_t d[K];
#pragma unroll
      for (int k = 0; k < K; ++k) d[k] = v4f_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const uint32_t w = i == 0 ? L.s[k].x : i == 1 ? L.s[k].y : i == 2 ? L.s[k].z : L.s[k].w;
          v8i_t B;
          B[0] = (int)((w & m0) | b0);
          B[1] = (int)((w & m1) | b1);
          B[2] = (int)(w & m2);
          B[3] = (int)((w & m3) | b3);
          B[4] = B[5] = B[6] = B[7] = 0;
          d[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[k][i], B, d[k], 0, 4, 0,
                                                                  ascale[k][i], 0, kE8M0One);
        }
      }
#pragma unroll
      for (int k = 0; k < K; ++k)
        a = fmaf(alpha_to_f32<AT>(L.a[k]), ((d[k][0] + d[k][1]) + (d[k][2] + d[k][3])) - corr[k],
                 a);
      return a;
    };
    auto step = [&](int t, F4Loads<K, AT>& L) {
      float uu = mul(L, 0.f);
      {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(uu), __float_as_uint(uu),
                                                        false, false);
        uu = __uint_as_float(a[0]) + __uint_as_float(a[1]);
        const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(uu), __float_as_uint(uu),
                                                        false, false);
        uu = __uint_as_float(c[0]) + __uint_as_float(c[1]);
      }
      if (q == 0) {
        float* dst = red + (t * NW + wave) * 16 + r;
        *dst = g0 == 0 ? uu : *dst + uu;
      }
    };
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntl) break;
      if (t + kF4Ahead < NT) load(t + kF4Ahead, Lb[(t + kF4Ahead) % (kF4Ahead + 1)]);
      step(t, Lb[t % (kF4Ahead + 1)]);
    }
  }

  const bool bad = __syncthreads_or(nonfinite) != 0;
  for (int idx = threadIdx.x; idx < ntl * 16; idx += NW * kWave) {
    const int t = idx >> 4, rr = idx & 15;
    float uu = red[(t * NW) * 16 + rr];
    for (int w = 1; w < NW; ++w) uu += red[(t * NW + w) * 16 + rr];
    const int i = tile16_of(b + t * grid, tiles) * 16 + rr;
    if (i < m) y[i] = bad ? __builtin_nanf("") : uu;
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
  // the kernel has one tile slot per tile of its fullest workgroup
  const int slots = (tiles + grid - 1) / grid;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(NW * kWave), 0, stream,
                       reinterpret_cast<const uint4*>(packed),
                       reinterpret_cast<const uint16_t*>(x), geo.G, tiles, slab, grid, NW,
                       tiles / grid, tiles % grid, y, geo.m);
  };
  // the first tile's signs go out behind the activations unless one tile
  // per workgroup meets a single column slab
  switch (slots) {
    case 1:
      if (nslabs > 1)
        go(gemv_f4_kernel<AT, K, 1, true>);
      else
        go(gemv_f4_kernel<AT, K, 1, false>);
      break;
    case 2: go(gemv_f4_kernel<AT, K, 2, true>); break;
    case 3: go(gemv_f4_kernel<AT, K, 3, true>); break;
    case 4: go(gemv_f4_kernel<AT, K, 4, true>); break;
    case 5: go(gemv_f4_kernel<AT, K, 5, true>); break;
    case 6: go(gemv_f4_kernel<AT, K, 6, true>); break;
    case 7: go(gemv_f4_kernel<AT, K, 7, true>); break;
    default: go(gemv_f4_kernel<AT, K, 8, true>); break;
  }
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

// 2..4 tokens: the shape rules of launch_f4_k with the few-token kernel's
// wavefront budget
template <typename AT, int K, int TT>
int launch_f4_tokens_k(const Geom& geo, const void* packed, const void* X, int ldx, float* Y,
                       int ldy, hipStream_t stream) {
  const int max_slab = kF4GroupsPerWave * f4_max_waves(K, TT);
  const int nslabs = (geo.G + max_slab - 1) / max_slab;
  const int slab = (geo.G + nslabs - 1) / nslabs;
  const int NW = (slab + kF4GroupsPerWave - 1) / kF4GroupsPerWave;
  const int tiles = geo.RB * (kRowBlock / 16);
  int grid = tiles < 256 ? tiles : 256;
  if (grid * kF4J < tiles) grid = (tiles + kF4J - 1) / kF4J;
  const int slots = (tiles + grid - 1) / grid;
  auto go = [&](auto slot_count, auto early) {
    constexpr int S = decltype(slot_count)::value;
    constexpr bool E = decltype(early)::value;
    hipLaunchKernelGGL((gemm_f4_kernel<AT, K, S, TT, E>), dim3(grid), dim3(NW * kWave), 0, stream,
                       reinterpret_cast<const uint4*>(packed),
                       reinterpret_cast<const uint16_t*>(X), geo.G, tiles, slab, grid, NW,
                       tiles / grid, tiles % grid, Y, geo.m, ldx, ldy);
  };
  switch (slots) {
    case 1: go(std::integral_constant<int, 1>{}, std::false_type{}); break;
    case 2: go(std::integral_constant<int, 2>{}, std::true_type{}); break;
    case 3: go(std::integral_constant<int, 3>{}, std::true_type{}); break;
    case 4: go(std::integral_constant<int, 4>{}, std::true_type{}); break;
    case 5: go(std::integral_constant<int, 5>{}, std::true_type{}); break;
    case 6: go(std::integral_constant<int, 6>{}, std::true_type{}); break;
    case 7: go(std::integral_constant<int, 7>{}, std::true_type{}); break;
    default: go(std::integral_constant<int, 8>{}, std::true_type{}); break;
  }
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

template <typename AT, int TT>
int launch_f4_tokens_t(const Geom& geo, const void* packed, const void* X, int ldx, float* Y,
                       int ldy, hipStream_t stream) {
  switch (geo.K) {
    case 1: return launch_f4_tokens_k<AT, 1, TT>(geo, packed, X, ldx, Y, ldy, stream);
    case 2: return launch_f4_tokens_k<AT, 2, TT>(geo, packed, X, ldx, Y, ldy, stream);
    case 3: return launch_f4_tokens_k<AT, 3, TT>(geo, packed, X, ldx, Y, ldy, stream);
    case 4: return launch_f4_tokens_k<AT, 4, TT>(geo, packed, X, ldx, Y, ldy, stream);
  }
  return MBOK_ERR_UNSUPPORTED;
}

// Several tokens, one product per group: the shape rules of launch_f4_k
template <typename AT, int K, int NO>
int launch_f4g_k(const Geom& geo, const void* packed, const void* X, int T, int ldx, float* Y,
                 int ldy, hipStream_t stream) {
  const int max_slab = kF4GroupsPerWave * f4g_waves(NO);
  const int nslabs = (geo.G + max_slab - 1) / max_slab;
  const int slab = (geo.G + nslabs - 1) / nslabs;
  const int NW = (slab + kF4GroupsPerWave - 1) / kF4GroupsPerWave;
  const int tiles = geo.RB * (kRowBlock / 16);
  int grid = tiles < 256 ? tiles : 256;
  if (grid * kF4J < tiles) grid = (tiles + kF4J - 1) / kF4J;
  const int slots = (tiles + grid - 1) / grid;
  auto go = [&](auto slot_count, auto early) {
    constexpr int S = decltype(slot_count)::value;
    constexpr bool E = decltype(early)::value;
    hipLaunchKernelGGL((gemm_f4g_kernel<AT, K, S, NO, E>), dim3(grid), dim3(NW * kWave), 0, stream,
                       reinterpret_cast<const uint4*>(packed),
                       reinterpret_cast<const uint16_t*>(X), geo.G, tiles, slab, grid, NW,
                       tiles / grid, tiles % grid, Y, geo.m, T, ldx, ldy);
  };
  switch (slots) {
    case 1: go(std::integral_constant<int, 1>{}, std::false_type{}); break;
    case 2: go(std::integral_constant<int, 2>{}, std::true_type{}); break;
    case 3: go(std::integral_constant<int, 3>{}, std::true_type{}); break;
    case 4: go(std::integral_constant<int, 4>{}, std::true_type{}); break;
    case 5: go(std::integral_constant<int, 5>{}, std::true_type{}); break;
    case 6: go(std::integral_constant<int, 6>{}, std::true_type{}); break;
    case 7: go(std::integral_constant<int, 7>{}, std::true_type{}); break;
    default: go(std::integral_constant<int, 8>{}, std::true_type{}); break;
  }
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

template <typename AT, int NO>
int launch_f4g_t(const Geom& geo, const void* packed, const void* X, int T, int ldx, float* Y,
                 int ldy, hipStream_t stream) {
  switch (geo.K) {
    case 1: return launch_f4g_k<AT, 1, NO>(geo, packed, X, T, ldx, Y, ldy, stream);
    case 2: return launch_f4g_k<AT, 2, NO>(geo, packed, X, T, ldx, Y, ldy, stream);
    case 3: return launch_f4g_k<AT, 3, NO>(geo, packed, X, T, ldx, Y, ldy, stream);
    case 4: return launch_f4g_k<AT, 4, NO>(geo, packed, X, T, ldx, Y, ldy, stream);
  }
  return MBOK_ERR_UNSUPPORTED;
}

template <typename AT>
int launch_f4_tokens(const Geom& geo, const void* packed, const void* X, int T, int ldx,
                     float* Y, int ldy, hipStream_t stream) {
  switch (T) {
    case 2: return launch_f4_tokens_t<AT, 2>(geo, packed, X, ldx, Y, ldy, stream);
    case 3: return launch_f4_tokens_t<AT, 3>(geo, packed, X, ldx, Y, ldy, stream);
    case 4: return launch_f4_tokens_t<AT, 4>(geo, packed, X, ldx, Y, ldy, stream);
  }
  return MBOK_ERR_SHAPE;
}

template <typename AT, int K, bool XF>
int launch_f4_svid_k(const Geom& geo, const void* packed, const void* x, const AT* s_in,
                     float* y, hipStream_t stream) {
  const int nslabs = (geo.G + kF4sMaxSlab - 1) / kF4sMaxSlab;
  const int slab = (geo.G + nslabs - 1) / nslabs;
  const int NW = (slab + kF4GroupsPerWave - 1) / kF4GroupsPerWave;
  const int tiles = geo.RB * (kRowBlock / 16);
  int grid = tiles < 256 ? tiles : 256;
  if (grid * kF4J < tiles) grid = (tiles + kF4J - 1) / kF4J;
  const int slots = (tiles + grid - 1) / grid;
  auto go = [&](auto slot_count, auto early) {
    constexpr int S = decltype(slot_count)::value;
    constexpr bool E = decltype(early)::value;
    hipLaunchKernelGGL((gemv_f4_svid_kernel<AT, K, S, XF, E>), dim3(grid), dim3(NW * kWave), 0,
                       stream, reinterpret_cast<const uint4*>(packed), x, s_in, geo.G, tiles,
                       slab, grid, NW, tiles / grid, tiles % grid, y, geo.m);
  };
  switch (slots) {
    case 1: go(std::integral_constant<int, 1>{}, std::false_type{}); break;
    case 2: go(std::integral_constant<int, 2>{}, std::true_type{}); break;
    case 3: go(std::integral_constant<int, 3>{}, std::true_type{}); break;
    case 4: go(std::integral_constant<int, 4>{}, std::true_type{}); break;
    case 5: go(std::integral_constant<int, 5>{}, std::true_type{}); break;
    case 6: go(std::integral_constant<int, 6>{}, std::true_type{}); break;
    case 7: go(std::integral_constant<int, 7>{}, std::true_type{}); break;
    default: go(std::integral_constant<int, 8>{}, std::true_type{}); break;
  }
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

template <typename AT, bool XF>
int launch_f4_svid_t(const Geom& geo, const void* packed, const void* x, const void* s_in,
                     float* y, hipStream_t stream) {
  const AT* si = reinterpret_cast<const AT*>(s_in);
  switch (geo.K) {
    case 1: return launch_f4_svid_k<AT, 1, XF>(geo, packed, x, si, y, stream);
    case 2: return launch_f4_svid_k<AT, 2, XF>(geo, packed, x, si, y, stream);
    case 3: return launch_f4_svid_k<AT, 3, XF>(geo, packed, x, si, y, stream);
    case 4: return launch_f4_svid_k<AT, 4, XF>(geo, packed, x, si, y, stream);
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

int gemm_f4_max_tokens() { return kF4MaxTokens; }
int gemm_f4g_max_tokens() { return kF4gMaxTokens; }

int launch_gemm_f4g(const mbok_desc* d, const void* packed, const void* X, int64_t T,
                    int64_t ldx, float* Y, int64_t ldy, hipStream_t stream) {
  if (T < 1 || T > kF4gMaxTokens) return MBOK_ERR_SHAPE;
  if ((T - 1) * ldx + d->n > INT32_MAX || (T - 1) * ldy + d->m > INT32_MAX)
    return MBOK_ERR_UNSUPPORTED;
  const Geom geo = make_geom(d);
  const bool two = T > kF4gTokens;
  if (d->alpha_dtype == MBOK_F16)
    return two ? launch_f4g_t<uint16_t, 2>(geo, packed, X, (int)T, (int)ldx, Y, (int)ldy, stream)
               : launch_f4g_t<uint16_t, 1>(geo, packed, X, (int)T, (int)ldx, Y, (int)ldy, stream);
  return two ? launch_f4g_t<float, 2>(geo, packed, X, (int)T, (int)ldx, Y, (int)ldy, stream)
             : launch_f4g_t<float, 1>(geo, packed, X, (int)T, (int)ldx, Y, (int)ldy, stream);
}

int launch_gemm_f4(const mbok_desc* d, const void* packed, const void* X, int64_t T,
                   int64_t ldx, float* Y, int64_t ldy, hipStream_t stream) {
  if (T < 2 || T > kF4MaxTokens) return MBOK_ERR_SHAPE;
  // token offsets are formed in 32 bits
  if ((T - 1) * ldx + d->n > INT32_MAX || (T - 1) * ldy + d->m > INT32_MAX)
    return MBOK_ERR_UNSUPPORTED;
  const Geom geo = make_geom(d);
  return d->alpha_dtype == MBOK_F16
             ? launch_f4_tokens<uint16_t>(geo, packed, X, (int)T, (int)ldx, Y, (int)ldy, stream)
             : launch_f4_tokens<float>(geo, packed, X, (int)T, (int)ldx, Y, (int)ldy, stream);
}

int launch_svid_f4(const mbok_desc* d, const void* packed, const void* x, int32_t x_dtype,
                   const void* s_in, float* y, hipStream_t stream) {
  const Geom geo = make_geom(d);
  const bool xf = x_dtype == MBOK_F32;
  if (d->alpha_dtype == MBOK_F16)
    return xf ? launch_f4_svid_t<uint16_t, true>(geo, packed, x, s_in, y, stream)
              : launch_f4_svid_t<uint16_t, false>(geo, packed, x, s_in, y, stream);
  return xf ? launch_f4_svid_t<float, true>(geo, packed, x, s_in, y, stream)
            : launch_f4_svid_t<float, false>(geo, packed, x, s_in, y, stream);
}

}  // namespace mbok
