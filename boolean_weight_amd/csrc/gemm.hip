// Multi-token product Y = X . W_hat^T on the matrix cores (gfx950).
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// Paper-Notes reading note, 关键设计: W ~ sum_k alpha_k B_k with group-wise
// scales; with many tokens the product is a dense contraction, so each tile
// of W_hat = sum_k alpha_k (.) B_k is formed once per workgroup, rounded to
// bf16 and contracted with the bf16 activations by MFMA with fp32
// accumulation.
//
// Workgroup tile: 256 tokens x 256 output rows, 4 wavefronts of 128 x 128
// (4 x 4 blocks of v_mfma_f32_32x32x16_bf16, 256 accumulator registers per
// lane).  The contraction runs in steps of 64 input columns (half a scale
// group); X and W_hat tiles of a step live in LDS as bf16 rows padded to 144
// bytes (conflict-free 16-byte fragment reads and writes), double-buffered so
// that the next step's loads and unpacking overlap this step's MFMAs.
//
// Unpacking (one thread per output row): for each (row, group) the 2^K level
// values sum_k (+-alpha_k) are formed in fp32 and rounded to bf16 once; their
// low and high bytes are kept "byte-planar" in two registers each (K <= 3).
// In the L64 word order the K sign bits of 4 consecutive columns 4q..4q+3 sit
// at bit q of the word's 4 bytes, so the per-byte level indices of a quad are
// ((W1 >> q) & 0x01010101) | ((W2 >> q) & ..) << 1 | ((W3 >> q) & ..) << 2, and
// v_perm_b32 turns that selector into 4 low bytes and 4 high bytes of bf16
// weights at once; two more perms interleave them into natural column order.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "mbok_device.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
// a native vector type keeps the activation staging in registers (a uint4
// struct member went through scratch memory)
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int BT = 256;         // tokens per workgroup tile
constexpr int BN = 256;         // output rows per workgroup tile
constexpr int BK = 64;          // input columns per step
constexpr int LDS_STRIDE = 72;  // bf16 elements per LDS row (64 + 8 padding)
constexpr int TILE_ELEMS = 256 * LDS_STRIDE;
constexpr int GEMM_THREADS = 256;

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;  // nearest-even
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Byte-planar bf16 levels of one (row, group): lo_a/hi_a hold the low/high
// bytes of levels 0..3, lo_b/hi_b of levels 4..7.  Level index bit k-1 is the
// sign bit of kernel k (1 = +alpha_k).
struct Levels {
  uint32_t lo_a, lo_b, hi_a, hi_b;
};

// What is left of an fp32 value after its rounding to bf16.  The difference
// is exact in fp32 (it is v's own low significand bits) and at most half a
// bf16 ulp of v, so hi + bf16(lo) carries 16 significant bits of v.
__device__ __forceinline__ float bf16_residue(float v) { return v - (float)(__bf16)v; }

// LO = false: the levels rounded to bf16 (the default product).  LO = true:
// the bf16 rounding of each level's residue, for the second pass of the
// two-pass product (hi + lo levels, ~2^-16 relative error per weight).
template <int K, bool LO = false>
__device__ __forceinline__ Levels make_levels(const float* a) {
  float l[8];
#pragma unroll
  for (int idx = 0; idx < 8; ++idx) {
    float v = (idx & 1) ? a[0] : -a[0];
    if (K >= 2) v += (idx & 2) ? a[1] : -a[1];
    if (K >= 3) v += (idx & 4) ? a[2] : -a[2];
    l[idx] = LO ? bf16_residue(v) : v;
  }
  const uint32_t p01 = bf16_pair(l[0], l[1]), p23 = bf16_pair(l[2], l[3]);
  const uint32_t p45 = bf16_pair(l[4], l[5]), p67 = bf16_pair(l[6], l[7]);
  Levels L;
  // v_perm_b32(s0, s1, sel): selector byte 0..3 picks s1 bytes, 4..7 s0 bytes
  L.lo_a = __builtin_amdgcn_perm(p23, p01, 0x06040200u);
  L.hi_a = __builtin_amdgcn_perm(p23, p01, 0x07050301u);
  L.lo_b = __builtin_amdgcn_perm(p67, p45, 0x06040200u);
  L.hi_b = __builtin_amdgcn_perm(p67, p45, 0x07050301u);
  return L;
}

// Unpack one 32-column sign word per kernel (w[k]) into 32 bf16 weights in
// natural column order: out[2q], out[2q+1] hold columns 4q..4q+3.
template <int K>
__device__ __forceinline__ void unpack_word(const uint32_t* w, const Levels& L, uint32_t* out) {
  constexpr uint32_t M = 0x11111111u;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // nibble j = 2e + a of V holds the level index of quad q = 4a + b, element e
    uint32_t V = (w[0] >> b) & M;
    if (K >= 2) V |= ((w[1] >> b) & M) << 1;
    if (K >= 3) V |= ((w[2] >> b) & M) << 2;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int q = 4 * a + b;
      const uint32_t sel = (a ? (V >> 4) : V) & 0x0f0f0f0fu;
      const uint32_t lo = __builtin_amdgcn_perm(L.lo_b, L.lo_a, sel);
      const uint32_t hi = __builtin_amdgcn_perm(L.hi_b, L.hi_a, sel);
      out[2 * q] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
      out[2 * q + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    }
  }
}

// K = 4 (16 levels): direct fp32 sums, then bf16 (LO: their residues).
template <bool LO = false>
__device__ __forceinline__ void unpack_word_k4(const uint32_t* w, const float* a, uint32_t* out) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) s += ((w[k] >> (8 * e + q)) & 1u) ? a[k] : -a[k];
      v[e] = LO ? bf16_residue(s) : s;
    }
    out[2 * q] = bf16_pair(v[0], v[1]);
    out[2 * q + 1] = bf16_pair(v[2], v[3]);
  }
}

// Selector words of one 32-column sign word per kernel: V[b] nibble 2e + a is
// the level index of quad q = 4a + b, element e (see unpack_word).
template <int K>
__device__ __forceinline__ void word_selectors(const uint32_t* w, uint32_t* V) {
  constexpr uint32_t M = 0x11111111u;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t v = (w[0] >> b) & M;
    if (K >= 2) v |= ((w[1] >> b) & M) << 1;
    if (K >= 3) v |= ((w[2] >> b) & M) << 2;
    V[b] = v;
  }
}

// Quads 4a .. 4a+3 of a word (16 columns 16a .. 16a+15) as 8 bf16 pairs.
__device__ __forceinline__ void unpack_quads(const uint32_t* V, int a, const Levels& L,
                                             uint32_t* out) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t sel = (a ? (V[b] >> 4) : V[b]) & 0x0f0f0f0fu;
    const uint32_t lo = __builtin_amdgcn_perm(L.lo_b, L.lo_a, sel);
    const uint32_t hi = __builtin_amdgcn_perm(L.hi_b, L.hi_a, sel);
    out[2 * b] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    out[2 * b + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
}

// Output element of a tile: the first pass (or the one-pass product) stores
// its sum; the residue pass adds its sum to what the first pass stored.
template <bool LO>
__device__ __forceinline__ void store_out(float* y, float v) {
  *y = LO ? *y + v : v;
}

template <typename AT, int K, bool LO>
__global__ void __launch_bounds__(GEMM_THREADS) gemm_mfma_kernel(
    const uint2* __restrict__ bits, const AT* __restrict__ scales, const uint16_t* __restrict__ X,
    int64_t ldx, float* __restrict__ Y, int64_t ldy, int T, int m, int m_pad, int G) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  // buffer b: activations at smem + 2b * TILE_ELEMS, weights right after

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wt = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.y * BT;
  const int n0 = blockIdx.x * BN;
  const int S = G * 2;  // steps of 64 columns

  // unpack role: thread = output row n0 + tid; rows past m_pad read row
  // m_pad - 1 and are zeroed (branch-free)
  const int row = n0 + tid;
  const bool row_ok = row < m_pad;
  const int rowc = row_ok ? row : m_pad - 1;
  const int rb = rowc / kRowBlock, rr = rowc % kRowBlock;
  const uint2* bits_row = bits + 2 * ((int64_t)rb * G * K * kRowBlock + rr);
  const AT* scales_row = scales + (int64_t)rb * G * K * kRowBlock + rr;

  // X copy role: segment j of a step = token tid/8 + 32j, 8 columns (tid%8)*8
  const int xpart = tid & 7;
  const uint16_t* xrow[8];
  bool xok[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = t0 + (tid >> 3) + 32 * j;
    xok[j] = t < T;
    xrow[j] = X + (int64_t)(xok[j] ? t : T - 1) * ldx + xpart * 8;
  }

  struct StepRegs {
    uint4 x[8];
    uint2 w[K];
    float a[K];
  };
  StepRegs R0, R1;

  auto load_step = [&](int s, StepRegs& R) {
    const int g = s >> 1, half = s & 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) R.x[j] = *reinterpret_cast<const uint4*>(xrow[j] + s * BK);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t c = (uint32_t)(g * K + k) * kRowBlock;
      R.w[k] = bits_row[2 * c + half];
      R.a[k] = alpha_to_f32<AT>(scales_row[c]);
    }
  };
  // zero what lies outside the problem (tokens >= T, rows >= m_pad)
  auto mask_step = [&](StepRegs& R) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (!xok[j]) R.x[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      R.w[k] = row_ok ? R.w[k] : make_uint2(0u, 0u);
      R.a[k] = row_ok ? R.a[k] : 0.f;
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  Levels L;

  // One step: MFMAs on buffer cb while the registers R (step sn) are written
  // to buffer 1-cb, a quarter per 16-column sub-step.  EVEN: sn starts a group
  // (new levels).
  auto step = [&](int cb, StepRegs& R, bool even) {
    mask_step(R);
    if (K <= 3 && even) L = make_levels<K, LO>(R.a);
    const uint16_t* xs = smem + 2 * cb * TILE_ELEMS + (wt * 128 + lrow) * LDS_STRIDE + lk;
    const uint16_t* ws = smem + (2 * cb + 1) * TILE_ELEMS + (wn * 128 + lrow) * LDS_STRIDE + lk;
    uint16_t* xd = smem + 2 * (cb ^ 1) * TILE_ELEMS + (tid >> 3) * LDS_STRIDE + xpart * 8;
    uint4* wd = reinterpret_cast<uint4*>(smem + (2 * (cb ^ 1) + 1) * TILE_ELEMS + tid * LDS_STRIDE);
    uint32_t V[4];
    // fragments of sub-step kk + 1 are read while the MFMAs of kk run
    bf16x8 av[2][4], bv[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) av[0][i] = *reinterpret_cast<const bf16x8*>(xs + i * 32 * LDS_STRIDE);
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[0][j] = *reinterpret_cast<const bf16x8*>(ws + j * 32 * LDS_STRIDE);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
      if (kk < 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[cur ^ 1][i] =
              *reinterpret_cast<const bf16x8*>(xs + i * 32 * LDS_STRIDE + 16 * (kk + 1));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bv[cur ^ 1][j] =
              *reinterpret_cast<const bf16x8*>(ws + j * 32 * LDS_STRIDE + 16 * (kk + 1));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cur][i], bv[cur][j], acc[i][j], 0, 0, 0);
      // a quarter of the next step: 2 activation segments, 16 weight columns
      *reinterpret_cast<uint4*>(xd + (2 * kk) * 32 * LDS_STRIDE) = R.x[2 * kk];
      *reinterpret_cast<uint4*>(xd + (2 * kk + 1) * 32 * LDS_STRIDE) = R.x[2 * kk + 1];
      uint32_t out[8];
      if (K <= 3) {
        if ((kk & 1) == 0) {
          uint32_t w[K];
#pragma unroll
          for (int k = 0; k < K; ++k) w[k] = (kk >> 1) ? R.w[k].y : R.w[k].x;
          word_selectors<K>(w, V);
        }
        unpack_quads(V, kk & 1, L, out);
      } else {
        uint32_t w[K], o32[16];
#pragma unroll
        for (int k = 0; k < K; ++k) w[k] = (kk >> 1) ? R.w[k].y : R.w[k].x;
        unpack_word_k4<LO>(w, R.a, o32);
#pragma unroll
        for (int q = 0; q < 8; ++q) out[q] = o32[8 * (kk & 1) + q];
      }
      wd[2 * kk] = make_uint4(out[0], out[1], out[2], out[3]);
      wd[2 * kk + 1] = make_uint4(out[4], out[5], out[6], out[7]);
      // interleave: each MFMA followed by a few vector / LDS instructions
      // (the next sub-step's 8 fragment reads go in between the first MFMAs)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (q < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
      }
    }
  };

  // prologue: step 0 into buffer 0
  load_step(0, R0);
  load_step(1, R1);
  mask_step(R0);
  {
    if (K <= 3) L = make_levels<K, LO>(R0.a);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4*>(smem + (tid >> 3) * LDS_STRIDE + xpart * 8 + j * 32 * LDS_STRIDE) =
          R0.x[j];
    uint4* wd = reinterpret_cast<uint4*>(smem + TILE_ELEMS + tid * LDS_STRIDE);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w[K], out[16];
#pragma unroll
      for (int k = 0; k < K; ++k) w[k] = h ? R0.w[k].y : R0.w[k].x;
      if (K <= 3)
        unpack_word<K>(w, L, out);
      else
        unpack_word_k4<LO>(w, R0.a, out);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wd[4 * h + j] = make_uint4(out[4 * j], out[4 * j + 1], out[4 * j + 2], out[4 * j + 3]);
    }
  }
  __syncthreads();
  // steady state, two steps per iteration; loads run two steps ahead (the
  // step index is clamped at the end, the extra loads are never used)
  for (int s = 0; s < S; s += 2) {
    load_step(min(s + 2, S - 1), R0);
    step(0, R1, false);  // compute step s, store step s+1 (odd)
    __syncthreads();
    load_step(min(s + 3, S - 1), R1);
    step(1, R0, true);  // compute step s+1, store step s+2 (even)
    __syncthreads();
  }

  // C layout: lane l, register r -> token 8(r/4) + 4(l/32) + r%4, row l%32
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 128 + j * 32 + lrow;
      if (n >= m) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + wt * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t < T) store_out<LO>(Y + (int64_t)t * ldy + n, acc[i][j][r]);
      }
    }
}

// Two wavefronts per SIMD.  With one wavefront per SIMD the unpacking and
// LDS traffic of a step sit between its MFMAs (hardware counters: MFMA busy
// + VALU + LDS + waits add up to the whole wave lifetime), so this variant
// splits the 256 x 256 tile over 8 wavefronts of 128 tokens x 64 rows
// (2 x 4 ... 4 x 2 blocks of 32 x 32, 128 accumulator registers): while one
// wavefront of a SIMD runs MFMAs the other unpacks, copies and reads
// fragments.  Two threads share a row in the unpack (32 columns each, a
// quarter of them per 16-column sub-step); each thread copies 4 activation
// segments per step.
//
// Tiles are numbered token tile major (tile = ty * ntx + tx).  The last
// `ntiles mod #CU` tiles would run as a partial final round, so they are
// split into two 128-row halves (blocks nfull + 2r + h): each wavefront then
// covers 32 rows, and the final round takes about half as long.
constexpr int GEMM8_THREADS = 512;

__device__ __forceinline__ void unpack_two_quads(const uint32_t* V, int a, int b0, const Levels& L,
                                                 uint32_t* out) {
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int b = b0 + bb;
    const uint32_t sel = (a ? (V[b] >> 4) : V[b]) & 0x0f0f0f0fu;
    const uint32_t lo = __builtin_amdgcn_perm(L.lo_b, L.lo_a, sel);
    const uint32_t hi = __builtin_amdgcn_perm(L.hi_b, L.hi_a, sel);
    out[2 * bb] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    out[2 * bb + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
}

// The body of one workgroup: JB = 2 for a whole 256-row tile, 1 for one
// 128-row half of a tile of the partial final round (a compile-time constant,
// so the loop has no branches on it).
template <typename AT, int K, int JB, bool LO>
__device__ __forceinline__ void mfma8_tile(const uint32_t* __restrict__ bits,
                                           const AT* __restrict__ scales,
                                           const uint16_t* __restrict__ X, int64_t ldx,
                                           float* __restrict__ Y, int64_t ldy, int T, int m,
                                           int m_pad, int G, int ntx, int tile, int half,
                                           uint16_t* smem) {
  // buffer b: activations at smem + 2b * TILE_ELEMS, weights right after
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int tile_rows = JB == 2 ? BN : BN / 2;
  // wavefront tile: TI blocks of 32 tokens x TJ blocks of 32 rows; a whole
  // tile takes 2 x 4 wavefronts of 128 x 64, a half tile 4 x 2 of 64 x 64
  // (4 fragment reads per 4 MFMAs instead of 5 for 128 x 32)
  constexpr int TI = JB == 2 ? 4 : 2, TJ = 2;
  const int wt = JB == 2 ? (wave & 1) : (wave & 3);    // token block of the wavefront
  const int wn = JB == 2 ? (wave >> 1) : (wave >> 2);  // row block of the wavefront
  const int t0 = (tile / ntx) * BT;
  const int n0 = (tile % ntx) * BN + half * (BN / 2);
  const int S = G * 2;  // steps of 64 columns

  // unpack role: TPR threads per row, each 64 / TPR columns of a step (a
  // whole tile: row n0 + tid/2, columns 32 (tid % 2) ..; a half tile: row
  // n0 + tid/4, columns 16 (tid % 4) .., so that every wavefront unpacks)
  constexpr int TPR = JB == 2 ? 2 : 4;
  static_assert(GEMM8_THREADS / TPR == tile_rows, "one row per TPR threads");
  const int urow = tid / TPR, upart = tid % TPR;
  const int uword = JB == 2 ? upart : upart >> 1;  // 32-column word of the step
  const int row = n0 + urow;
  const int rowc = row < m_pad ? row : m_pad - 1;
  const uint32_t row_chunk = (uint32_t)(rowc / kRowBlock) * (uint32_t)(G * K * kRowBlock) +
                             (uint32_t)(rowc % kRowBlock);

  // X copy role: segment j = token tid/8 + 64 j, columns 8 (tid % 8) .. + 7.
  // Tokens past T read token T - 1 and rows past the padded row count read
  // the last padded row: every load stays inside the buffers, and the
  // products of those tokens and rows are never stored (each output element
  // depends only on its own token and row), so nothing needs masking.
  const int xpart = tid & 7;
  uint32_t xoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + (tid >> 3) + 64 * j;
    xoff[j] = (uint32_t)((int64_t)(t < T ? t : T - 1) * ldx) + xpart * 8;
  }

  struct StepRegs {
    u32x4 x[4];
    uint32_t w[K];
    AT a[K];  // raw scales: converted where they are used, so that nothing
              // waits on these loads in the step that issues them
  };
  auto scales_f32 = [](const StepRegs& R, float* f) {
#pragma unroll
    for (int k = 0; k < K; ++k) f[k] = alpha_to_f32<AT>(R.a[k]);
  };
  StepRegs R0, R1;
  auto load_step = [&](int s, StepRegs& R) {
    const int g = s >> 1;
    const uint32_t word = 2 * (s & 1) + uword;
#pragma unroll
    for (int j = 0; j < 4; ++j) R.x[j] = *reinterpret_cast<const u32x4*>(X + xoff[j] + s * BK);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t ch = row_chunk + (uint32_t)(g * K + k) * kRowBlock;
      R.w[k] = bits[ch * 4u + word];
      R.a[k] = scales[ch];
    }
  };
  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  Levels L;

  // compute step from buffer cb, store the next step (registers R) into cb^1
  auto step = [&](int cb, StepRegs& R, bool even) {
    if (K <= 3 && even) {
      float af[K];
      scales_f32(R, af);
      L = make_levels<K, LO>(af);
    }
    const uint16_t* xs =
        smem + 2 * cb * TILE_ELEMS + (wt * 32 * TI + lrow) * LDS_STRIDE + lk;
    const uint16_t* ws =
        smem + (2 * cb + 1) * TILE_ELEMS + (wn * 32 * TJ + lrow) * LDS_STRIDE + lk;
    uint16_t* xd = smem + 2 * (cb ^ 1) * TILE_ELEMS + (tid >> 3) * LDS_STRIDE + xpart * 8;
    uint4* wd = reinterpret_cast<uint4*>(smem + (2 * (cb ^ 1) + 1) * TILE_ELEMS +
                                         urow * LDS_STRIDE + upart * (64 / TPR));
    uint32_t V[4];
    if (K <= 3) word_selectors<K>(R.w, V);
    // fragments of sub-step kk + 1 are read while the MFMAs of kk run
    bf16x8 pa[2][TI], pb[2][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
      pa[0][i] = *reinterpret_cast<const bf16x8*>(xs + i * 32 * LDS_STRIDE);
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      pb[0][j] = *reinterpret_cast<const bf16x8*>(ws + j * 32 * LDS_STRIDE);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) {
        const int nb = (kk + 1) & 1;
#pragma unroll
        for (int i = 0; i < TI; ++i)
          pa[nb][i] = *reinterpret_cast<const bf16x8*>(xs + i * 32 * LDS_STRIDE + 16 * (kk + 1));
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          pb[nb][j] = *reinterpret_cast<const bf16x8*>(ws + j * 32 * LDS_STRIDE + 16 * (kk + 1));
      }
      const bf16x8* av = pa[kk & 1];
      const bf16x8* bv = pb[kk & 1];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int i = 0; i < TI; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
      // a quarter of the next step: one activation segment, 8 weight columns
      *reinterpret_cast<u32x4*>(xd + kk * 64 * LDS_STRIDE) = R.x[kk];
      // 8 weight columns per sub-step (a half tile: in the first two only).
      // The thread's 8-column piece of its word is kk (a whole tile), or
      // 2 h + kk with h = upart % 2 (a half tile); piece q is quads 2q, 2q+1.
      // Register arrays are indexed with constants only (h selects).
      if (JB == 2 || kk < 2) {
        const bool h = (upart & 1) != 0;
        uint32_t out[4];
        if (K <= 3) {
          if (JB == 2)
            unpack_two_quads(V, kk >> 1, 2 * (kk & 1), L, out);
          else
            unpack_two_quads(V, h, 2 * kk, L, out);
        } else {
          uint32_t o32[16];
          float af[K];
          scales_f32(R, af);
          unpack_word_k4<LO>(R.w, af, o32);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            out[e] = JB == 2 ? o32[4 * kk + e] : (h ? o32[8 + 4 * kk + e] : o32[4 * kk + e]);
        }
        wd[kk] = make_uint4(out[0], out[1], out[2], out[3]);
      }
    }
  };

  // prologue: step 0 into buffer 0
  load_step(0, R0);
  load_step(1, R1);
  {
    float af0[K];
    scales_f32(R0, af0);
    if (K <= 3) L = make_levels<K, LO>(af0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(smem + (tid >> 3) * LDS_STRIDE + xpart * 8 + j * 64 * LDS_STRIDE) =
          R0.x[j];
    {
      uint4* wd = reinterpret_cast<uint4*>(smem + TILE_ELEMS + urow * LDS_STRIDE +
                                           upart * (64 / TPR));
      uint32_t out[16];
      if (K <= 3)
        unpack_word<K>(R0.w, L, out);
      else
        unpack_word_k4<LO>(R0.w, af0, out);
      // out[4 p .. 4 p + 3]: 8-column piece p of the word (a half tile's
      // thread takes pieces 2 h, 2 h + 1; constant indices, h selects)
      constexpr int NP = 4 / (TPR / 2);  // pieces per thread: 4 or 2
      const bool h = (upart & 1) != 0;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = JB == 2 ? out[4 * j + e] : (h ? out[8 + 4 * j + e] : out[4 * j + e]);
        wd[j] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
  __syncthreads();
  // (Pinning these loads to the top of the step with a scheduling barrier
  // was measured slower: it also keeps the first fragment reads below them.)
  for (int s = 0; s < S; s += 2) {
    load_step(min(s + 2, S - 1), R0);
    step(0, R1, false);  // compute step s, store step s+1 (odd)
    __syncthreads();
    load_step(min(s + 3, S - 1), R1);
    step(1, R0, true);  // compute step s+1, store step s+2 (even)
    __syncthreads();
  }

  // C layout: lane l, register r -> token 8(r/4) + 4(l/32) + r%4, row l%32
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int n = n0 + wn * 32 * TJ + j * 32 + lrow;
      if (n >= m) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + wt * 32 * TI + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t < T) store_out<LO>(Y + (int64_t)t * ldy + n, acc[i][j][r]);
      }
    }
}

// Tile at position p of the XCD-blocked order: pairs of token tiles, sweeping
// the row tiles (p -> token tile 2q + d, row tile tx), the last token tile
// alone when their count is odd.  Workgroup b runs on XCD b % 8, so giving
// XCD x the positions x * nfull / 8 .. of the full round puts ~16 row tiles
// x 2 token tiles on each XCD: its L2 holds those activations and weights
// instead of every XCD streaming every token tile.
__device__ __forceinline__ int tile_at(int p, int ntx, int nty) {
  const int q = p / (2 * ntx);
  const int rem = p - q * 2 * ntx;
  if (2 * q + 1 < nty) return (2 * q + (rem & 1)) * ntx + (rem >> 1);
  return 2 * q * ntx + rem;
}

template <typename AT, int K, bool LO>
__global__ void __launch_bounds__(GEMM8_THREADS) gemm_mfma8_kernel(
    const uint32_t* __restrict__ bits, const AT* __restrict__ scales,
    const uint16_t* __restrict__ X, int64_t ldx, float* __restrict__ Y, int64_t ldy, int T, int m,
    int m_pad, int G, int ntx, int nfull, int xcd_order) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int b = blockIdx.x;
  const int nty = (T + BT - 1) / BT;
  if (b < nfull) {
    int p = b;
    if (xcd_order && (nfull & 7) == 0) p = (b & 7) * (nfull >> 3) + (b >> 3);
    const int tile = xcd_order ? tile_at(p, ntx, nty) : p;
    mfma8_tile<AT, K, 2, LO>(bits, scales, X, ldx, Y, ldy, T, m, m_pad, G, ntx, tile, 0, smem);
  } else {
    const int p = nfull + ((b - nfull) >> 1);
    const int tile = xcd_order ? tile_at(p, ntx, nty) : p;
    mfma8_tile<AT, K, 1, LO>(bits, scales, X, ldx, Y, ldy, T, m, m_pad, G, ntx, tile,
                         (b - nfull) & 1, smem);
  }
}

// Compute units of the current device (queried once per device; host
// threads that race on the first query store the same value).
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// MBOK_GEMM_ORDER=token keeps the plain token-major tile order (for
// measurements); the default is the XCD-blocked order.
int gemm_xcd_order() {
  const char* v = getenv("MBOK_GEMM_ORDER");
  return v && strcmp(v, "token") == 0 ? 0 : 1;
}

template <typename AT, int K, bool LO>
void launch_mfma8_k(const Geom& geo, const uint32_t* bits, const AT* scales, const uint16_t* Xb,
                    int64_t T, int64_t ldx, float* Y, int64_t ldy, hipStream_t stream) {
  const size_t lds = 4 * TILE_ELEMS * sizeof(uint16_t);
  const int ntx = (geo.m + BN - 1) / BN;
  const int64_t ntiles = (int64_t)ntx * ((T + BT - 1) / BT);
  // one workgroup per compute unit at a time (the tiles take 147 KB of LDS)
  const int ncu = compute_units();
  const int64_t rem = ntiles % ncu;
  const int64_t nfull = ntiles - rem;
  hipLaunchKernelGGL((gemm_mfma8_kernel<AT, K, LO>), dim3((unsigned)(nfull + 2 * rem)),
                     dim3(GEMM8_THREADS), lds, stream, bits, scales, Xb, ldx, Y, ldy, (int)T,
                     geo.m, geo.RB * kRowBlock, geo.G, ntx, (int)nfull, gemm_xcd_order());
}

template <typename AT, bool LO>
void launch_mfma8(const Geom& geo, const void* packed, const void* X, int64_t T, int64_t ldx,
                  float* Y, int64_t ldy, hipStream_t stream) {
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(packed);
  const AT* scales = reinterpret_cast<const AT*>(reinterpret_cast<const char*>(packed) +
                                                 geo.bits_bytes);
  const uint16_t* Xb = reinterpret_cast<const uint16_t*>(X);
  switch (geo.K) {
    case 1: launch_mfma8_k<AT, 1, LO>(geo, bits, scales, Xb, T, ldx, Y, ldy, stream); break;
    case 2: launch_mfma8_k<AT, 2, LO>(geo, bits, scales, Xb, T, ldx, Y, ldy, stream); break;
    case 3: launch_mfma8_k<AT, 3, LO>(geo, bits, scales, Xb, T, ldx, Y, ldy, stream); break;
    default: launch_mfma8_k<AT, 4, LO>(geo, bits, scales, Xb, T, ldx, Y, ldy, stream); break;
  }
}

bool use_mfma8() {
  const char* v = getenv("MBOK_GEMM_WAVES");
  return !(v && atoi(v) == 4);
}

template <typename AT, bool LO>
void launch_mfma4(const Geom& geo, const void* packed, const void* X, int64_t T, int64_t ldx,
                  float* Y, int64_t ldy, hipStream_t stream) {
  const uint2* bits = reinterpret_cast<const uint2*>(packed);
  const AT* scales = reinterpret_cast<const AT*>(reinterpret_cast<const char*>(packed) +
                                                 geo.bits_bytes);
  const size_t lds = 4 * TILE_ELEMS * sizeof(uint16_t);
  dim3 grid((geo.m + BN - 1) / BN, (unsigned)((T + BT - 1) / BT));
  const int m_pad = geo.RB * kRowBlock;
  const uint16_t* Xb = reinterpret_cast<const uint16_t*>(X);
  switch (geo.K) {
    case 1:
      hipLaunchKernelGGL((gemm_mfma_kernel<AT, 1, LO>), grid, dim3(GEMM_THREADS), lds, stream,
                         bits, scales, Xb, ldx, Y, ldy, (int)T, geo.m, m_pad, geo.G);
      break;
    case 2:
      hipLaunchKernelGGL((gemm_mfma_kernel<AT, 2, LO>), grid, dim3(GEMM_THREADS), lds, stream,
                         bits, scales, Xb, ldx, Y, ldy, (int)T, geo.m, m_pad, geo.G);
      break;
    case 3:
      hipLaunchKernelGGL((gemm_mfma_kernel<AT, 3, LO>), grid, dim3(GEMM_THREADS), lds, stream,
                         bits, scales, Xb, ldx, Y, ldy, (int)T, geo.m, m_pad, geo.G);
      break;
    default:
      hipLaunchKernelGGL((gemm_mfma_kernel<AT, 4, LO>), grid, dim3(GEMM_THREADS), lds, stream,
                         bits, scales, Xb, ldx, Y, ldy, (int)T, geo.m, m_pad, geo.G);
      break;
  }
}

// passes = 1: one product with the levels rounded to bf16.  passes = 2: that
// product, then on the same stream a second one with the bf16 residues of the
// levels, added into Y (the stream orders the two launches).
template <typename AT>
int launch_mfma(const Geom& geo, const void* packed, const void* X, int64_t T, int64_t ldx,
                float* Y, int64_t ldy, int passes, hipStream_t stream) {
  // the 8-wavefront kernel indexes signs and activations with 32-bit offsets
  const bool fits32 = geo.bits_bytes / 4 < (int64_t(1) << 32) && T * ldx < (int64_t(1) << 32);
  if (fits32 && use_mfma8()) {
    launch_mfma8<AT, false>(geo, packed, X, T, ldx, Y, ldy, stream);
    if (passes == 2) launch_mfma8<AT, true>(geo, packed, X, T, ldx, Y, ldy, stream);
  } else {
    launch_mfma4<AT, false>(geo, packed, X, T, ldx, Y, ldy, stream);
    if (passes == 2) launch_mfma4<AT, true>(geo, packed, X, T, ldx, Y, ldy, stream);
  }
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

}  // namespace

// Few-token kernel by token count and layer size, from measurements on
// MI355X (HIP graph of the calls, cold weights; LLaMA-7B MLP step = gate and
// up 11008x4096 plus down 4096x11008, K = 3; us per step):
//
//   tokens                       2     3     4     6     8
//   fp4 x fp8, two tokens per
//     one-token product (f4)    22.9  30.2  33.8   -     -
//   fp4 x fp8, one product per
//     group, 8 tokens (f4g)     25.4  26.9  29.2  34.4  39.2
//   bf16 +-1 (skinny.hip)       35.5  35.8  36.1  36.3  37.9
//
// and on 4096x4096, K = 2: f4 4.68, f4g 4.89, bf16 +-1 5.05 us at 2 tokens;
// f4g 5.30 / 5.77 / 6.85 against 5.15 / 5.17 / 5.24 us at 3 / 4 / 6.  The
// fp4 x fp8 kernels turn signs into operands with 4 vector instructions per
// 128 signs whatever the token count, but every workgroup converts every
// token's activations to fp8 parts before its first product, so they lose
// to the bf16 +-1 kernels on small layers and beyond 6 tokens.
// MBOK_SKINNY_VARIANT=f4|f4g|stream|blocks forces a kernel; any other value
// (e.g. =skinny) takes the bf16 +-1 kernels with their own choice by shape.
enum TokenKernel { kTokSkinny = 0, kTokF4 = 1, kTokF4g = 2 };

TokenKernel token_kernel(const mbok_desc* d, int64_t T) {
  const char* v = getenv("MBOK_SKINNY_VARIANT");
  if (v && *v) {
    if (strcmp(v, "f4") == 0 && T >= 2 && T <= gemm_f4_max_tokens()) return kTokF4;
    if (strcmp(v, "f4g") == 0 && T >= 2 && T <= gemm_f4g_max_tokens()) return kTokF4g;
    return kTokSkinny;
  }
  if (T == 2) return kTokF4;
  const int64_t work = (int64_t)d->K * d->m * d->n;
  if (T <= 6 && work >= (int64_t(1) << 26)) return kTokF4g;
  return kTokSkinny;
}

int launch_gemm(const mbok_desc* d, const void* packed, const void* X, int64_t T, int64_t ldx,
                float* Y, int64_t ldy, int passes, hipStream_t stream) {
  const Geom geo = make_geom(d);
  if (T == 1) return launch_gemv(d, packed, X, MBOK_BF16, Y, nullptr, stream);
  // the two-term product keeps the bf16 +-1 kernels' exact fp32 scaling
  if (passes == 1 && T <= skinny_max_tokens() && (T - 1) * ldx + d->n <= INT32_MAX &&
      (T - 1) * ldy + d->m <= INT32_MAX) {
    const TokenKernel tk = token_kernel(d, T);
    if (tk == kTokF4) return launch_gemm_f4(d, packed, X, T, ldx, Y, ldy, stream);
    if (tk == kTokF4g) return launch_gemm_f4g(d, packed, X, T, ldx, Y, ldy, stream);
  }
  if (T <= skinny_max_tokens()) return launch_skinny(d, packed, X, T, ldx, Y, ldy, stream);
  if (T > 65535LL * BT) return MBOK_ERR_SHAPE;
  if (d->alpha_dtype == MBOK_F16)
    return launch_mfma<uint16_t>(geo, packed, X, T, ldx, Y, ldy, passes, stream);
  return launch_mfma<float>(geo, packed, X, T, ldx, Y, ldy, passes, stream);
}

}  // namespace mbok
