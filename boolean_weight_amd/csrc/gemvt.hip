// Transposed decode product dx = W_hat^T g for one gradient vector g: the
// activation gradient through the Boolean weights.
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures":
// the gist.science summaries' Boolean-domain training propagates gradients
// through the Boolean weights; the Paper-Notes reading note, 关键设计, splits
// the product into K Boolean products of signs.  Here
//     dx[j] = sum_i sum_k (alpha_k[i, g(j)] * g[i]) * b_k[i, j],
// i.e. per (row, kernel) the scaled gradient c = alpha * g (fp32) is added to
// or subtracted from every column of the row's group.
//
// Table form, transposed from the decode kernels: the signs of one byte
// position (8 columns spaced 4 apart) in 4 consecutive rows form a 4 x 8 bit
// block; a two-step delta-swap transpose turns it into 8 nibbles, one per
// column, whose bit t is row t.  A 16-entry table of the signed sums of the 4
// rows' c values (entry p = sum_t (bit t of p ? c_t : -c_t)) then gives each
// column's contribution with one lookup.
//
// Work split: each wavefront takes one column group g and one slice of its
// row blocks, stages each (row block, group, kernel) plane (64 rows x 16
// bytes) in its own LDS region and walks it in 4 steps of 16 rows: lane
// 16 rq + p takes byte position p of rows 4 rq .. 4 rq + 3 of the step, and
// keeps 8 column sums across all its planes.  The lane of row r builds a
// quarter of its row quad's table from the quad's four c values (quad
// permutations), so a plane's 16 tables and its bits reach LDS together.  The
// 4 row-quad lanes of a byte position are added at the end, then the 4
// wavefronts (slices) of a workgroup in order; with several workgroups per
// column group each writes its 128 partial sums to the workspace and a
// second kernel adds them in order.
#include <mutex>

#include "mbok_exact.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

constexpr int kTargetWaves = 2048;    // ~8 wavefronts per compute unit
constexpr int kSlicesPerBlock = 4;    // wavefronts (row-block slices) per workgroup
constexpr int kMaxBlocksY = 16;       // workgroups along the rows of a column group
constexpr int kMaxSlices = kSlicesPerBlock * kMaxBlocksY;

template <typename GT>
__device__ __forceinline__ float load_grad(const GT* g, int64_t i);
template <>
__device__ __forceinline__ float load_grad<float>(const float* g, int64_t i) { return g[i]; }
template <>
__device__ __forceinline__ float load_grad<uint16_t>(const uint16_t* g, int64_t i) {
  return bf16_bits_to_f32(g[i]);
}

// 4 x 8 bit transpose inside a word.  In: bit 8t + q = (row t, column q).
// Out: column q < 4 at bits 8q .. 8q+3, column 4 + c at bits 8c+4 .. 8c+7,
// bit t of each nibble = row t.  Two delta swaps: the off-diagonal 2 x 2
// blocks of each 4 x 4 half (distance 14), then the off-diagonal entries of
// each 2 x 2 block (distance 7).
__device__ __forceinline__ uint32_t transpose4x8(uint32_t x) {
  uint32_t t = ((x >> 14) ^ x) & 0x0000cccc;
  x ^= t ^ (t << 14);
  t = ((x >> 7) ^ x) & 0x00aa00aa;
  x ^= t ^ (t << 7);
  return x;
}

__device__ __forceinline__ int nibble_shift(int q) { return 8 * (q & 3) + 4 * (q >> 2); }

// Each wavefront's LDS region is its own, and a wavefront's LDS operations
// complete in order: waiting for them (and keeping the compiler from moving
// memory accesses across) is all the ordering needed.  A workgroup barrier
// would also wait for the next plane's global loads, meant to stay in flight.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <typename GT, typename AT, int K>
__global__ void __launch_bounds__(kSlicesPerBlock * kWave) gemvt_kernel(
    const uint4* __restrict__ bits, const AT* __restrict__ scales, const GT* __restrict__ grad,
    float* __restrict__ out, int m, int G, int RB, int rbs, int64_t slice_stride) {
  __shared__ uint4 plane[kSlicesPerBlock][2][kRowBlock];
  // the 16 tables of a plane (one per row quad), 16 entries each
  __shared__ float4 tab[kSlicesPerBlock][2][kRowBlock];
  __shared__ float red[kSlicesPerBlock][kGroup];
  const int g = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int slice = blockIdx.y * kSlicesPerBlock + wave;
  const int rq = lane >> 4, p = lane & 15;
  const int u = lane & 3;  // this lane's quarter of its own row quad's table
  const int rb0 = slice * rbs;
  const int rb1 = min(rb0 + rbs, RB);
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;

  const int np = (rb1 > rb0 ? rb1 - rb0 : 0) * K;  // planes of this slice
  auto chunk = [&](int t) -> int64_t {
    const int rb = rb0 + t / K, k = t % K;
    return ((int64_t)(rb * G + g) * K + k) * kRowBlock + lane;
  };
  uint4 nb = make_uint4(0, 0, 0, 0);
  AT na = AT(0);
  if (np > 0) {
    nb = bits[chunk(0)];
    na = scales[chunk(0)];
  }
  float gv = 0.f;
  const int w = p >> 2, e = p & 3;
  // v_perm selector: byte e of the low word, byte e of the high word
  const uint32_t sel = (uint32_t)e | ((uint32_t)(4 + e) << 8) | 0x0c0c0000u;
  for (int t = 0; t < np; ++t) {
    const uint4 cb = nb;
    const AT ca = na;
    if (t % K == 0) {
      const int64_t row = (int64_t)(rb0 + t / K) * kRowBlock + lane;
      gv = row < m ? load_grad<GT>(grad, row) : 0.f;
    }
    if (t + 1 < np) {
      nb = bits[chunk(t + 1)];
      na = scales[chunk(t + 1)];
    }
    // c of this lane's row (padding rows: alpha = 0 and g = 0), then the c of
    // all four rows of the lane's row quad by quad permutations
    const float c = alpha_to_f32(ca) * gv;
    const float c0 = __int_as_float(quad_perm_i<0x00>(__float_as_int(c)));
    const float c1 = __int_as_float(quad_perm_i<0x55>(__float_as_int(c)));
    const float c2 = __int_as_float(quad_perm_i<0xaa>(__float_as_int(c)));
    const float c3 = __int_as_float(quad_perm_i<0xff>(__float_as_int(c)));
    // entries 4u + v, v = 0..3: bits 0, 1 of the entry come from v, bits 2, 3
    // from u; entry = (+-c0 +-c1) + (+-c2 +-c3)
    const float hiq = ((u & 1) ? c2 : -c2) + ((u & 2) ? c3 : -c3);
    float4 ent;
    ent.x = (-c0 - c1) + hiq;
    ent.y = (c0 - c1) + hiq;
    ent.z = (-c0 + c1) + hiq;
    ent.w = (c0 + c1) + hiq;
    const int pb = t & 1;
    plane[wave][pb][lane] = cb;
    tab[wave][pb][lane] = ent;  // row quad lane / 4, entries 4u .. 4u+3
    lds_sync();
    const uint32_t* pl = reinterpret_cast<const uint32_t*>(plane[wave][pb]);
    const float* tb = reinterpret_cast<const float*>(tab[wave][pb]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r0 = 16 * s + 4 * rq;
      // byte p of rows r0 .. r0+3 -> one word, row t in byte t
      const uint32_t d0 = pl[4 * r0 + w], d1 = pl[4 * (r0 + 1) + w];
      const uint32_t d2 = pl[4 * (r0 + 2) + w], d3 = pl[4 * (r0 + 3) + w];
      const uint32_t lo = __builtin_amdgcn_perm(d1, d0, sel);  // bytes: b0, b1, 0, 0
      const uint32_t hi = __builtin_amdgcn_perm(d3, d2, sel);  // bytes: b2, b3, 0, 0
      const uint32_t X = transpose4x8(lo | (hi << 16));
      const float* tq = tb + 16 * (r0 >> 2);  // table of row quad r0 / 4
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += tq[(X >> nibble_shift(q)) & 0xfu];
    }
  }
  // the four row-quad lanes of a byte position hold the same columns
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    acc[q] += __shfl_xor(acc[q], 16, kWave);
    acc[q] += __shfl_xor(acc[q], 32, kWave);
  }
  if (rq == 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) red[wave][32 * w + 4 * q + e] = acc[q];
  }
  __syncthreads();
  // the workgroup's slices, added in order
  if (threadIdx.x < kGroup) {
    float v = red[0][threadIdx.x];
#pragma unroll
    for (int sv = 1; sv < kSlicesPerBlock; ++sv) v += red[sv][threadIdx.x];
    out[blockIdx.y * slice_stride + (int64_t)g * kGroup + threadIdx.x] = v;
  }
}

// dx[j] = the sum over slice groups s of partial[s * n + j], in order, all
// loads of a thread issued together.
__global__ void __launch_bounds__(256) gemvt_reduce_kernel(const float* __restrict__ partial,
                                                           int S, int n, float* __restrict__ dx) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  float buf[kMaxBlocksY];
#pragma unroll
  for (int s = 0; s < kMaxBlocksY; ++s) buf[s] = s < S ? partial[(int64_t)s * n + j] : 0.f;
  float v = buf[0];
#pragma unroll
  for (int s = 1; s < kMaxBlocksY; ++s) v += buf[s];
  dx[j] = v;
}

// Row-block slices per column group: enough wavefronts to fill the chip,
// kSlicesPerBlock per workgroup, at most kMaxBlocksY workgroups per group
// (SY).  Without a workspace SY = 1.
void slicing(const Geom& geo, bool have_ws, int& SY, int& rbs) {
  int want = (kTargetWaves + geo.G - 1) / geo.G;  // wavefront slices
  want = want < 1 ? 1 : (want > kMaxSlices ? kMaxSlices : want);
  if (!have_ws && want > kSlicesPerBlock) want = kSlicesPerBlock;
  if (want > geo.RB) want = geo.RB;
  rbs = (geo.RB + want - 1) / want;
  const int S = (geo.RB + rbs - 1) / rbs;
  SY = (S + kSlicesPerBlock - 1) / kSlicesPerBlock;
}

template <typename GT, typename AT>
int launch_t(const Geom& geo, const void* packed, const void* grad, float* dx, void* ws,
             hipStream_t stream) {
  const uint4* bits = reinterpret_cast<const uint4*>(packed);
  const AT* scales =
      reinterpret_cast<const AT*>(reinterpret_cast<const char*>(packed) + geo.bits_bytes);
  int SY, rbs;
  slicing(geo, ws != nullptr, SY, rbs);
  float* out = SY > 1 ? reinterpret_cast<float*>(ws) : dx;
  const GT* gr = reinterpret_cast<const GT*>(grad);
  dim3 grid((unsigned)geo.G, (unsigned)SY), block(kSlicesPerBlock * kWave);
  switch (geo.K) {
    case 1:
      hipLaunchKernelGGL((gemvt_kernel<GT, AT, 1>), grid, block, 0, stream, bits, scales, gr, out,
                         geo.m, geo.G, geo.RB, rbs, (int64_t)geo.n);
      break;
    case 2:
      hipLaunchKernelGGL((gemvt_kernel<GT, AT, 2>), grid, block, 0, stream, bits, scales, gr, out,
                         geo.m, geo.G, geo.RB, rbs, (int64_t)geo.n);
      break;
    case 3:
      hipLaunchKernelGGL((gemvt_kernel<GT, AT, 3>), grid, block, 0, stream, bits, scales, gr, out,
                         geo.m, geo.G, geo.RB, rbs, (int64_t)geo.n);
      break;
    case 4:
      hipLaunchKernelGGL((gemvt_kernel<GT, AT, 4>), grid, block, 0, stream, bits, scales, gr, out,
                         geo.m, geo.G, geo.RB, rbs, (int64_t)geo.n);
      break;
    default:
      return MBOK_ERR_UNSUPPORTED;
  }
  if (hipGetLastError() != hipSuccess) return MBOK_ERR_HIP;
  if (SY > 1) {
    hipLaunchKernelGGL(gemvt_reduce_kernel, dim3((geo.n + 255) / 256), dim3(256), 0, stream, out,
                       SY, geo.n, dx);
    if (hipGetLastError() != hipSuccess) return MBOK_ERR_HIP;
  }
  return MBOK_OK;
}

// Scratch of mbok_gemvt_noalloc: the slices' partial column sums, in a
// file-scope device array instead of a caller workspace.  Every shape the
// descriptor accepts needs at most 523,264 bytes here (n = 65408: 2 slice
// groups x 65408 columns x 4 bytes), so 512 KiB covers all of them.  Each
// device holds its own copy until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(512) << 10;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MBOK_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MBOK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MBOK_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MBOK_OK;
}

}  // namespace

size_t gemvt_scratch_bytes() { return kScratchBytes; }

int launch_gemvt_noalloc(const mbok_desc* d, const void* packed, const void* grad,
                         int32_t g_dtype, float* dx, hipStream_t stream) {
  if (gemvt_workspace_bytes(d) > kScratchBytes) return MBOK_ERR_SCRATCH;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != MBOK_OK) return st;
  return launch_gemvt(d, packed, grad, g_dtype, dx, ws, stream);
}

size_t gemvt_workspace_bytes(const mbok_desc* d) {
  const Geom geo = make_geom(d);
  int SY, rbs;
  slicing(geo, true, SY, rbs);
  return SY > 1 ? (size_t)SY * (size_t)geo.n * sizeof(float) : 0;
}

int launch_gemvt(const mbok_desc* d, const void* packed, const void* grad, int32_t g_dtype,
                 float* dx, void* ws, hipStream_t stream) {
  const Geom geo = make_geom(d);
  const bool f16a = d->alpha_dtype == MBOK_F16;
  if (g_dtype == MBOK_BF16)
    return f16a ? launch_t<uint16_t, uint16_t>(geo, packed, grad, dx, ws, stream)
                : launch_t<uint16_t, float>(geo, packed, grad, dx, ws, stream);
  return f16a ? launch_t<float, uint16_t>(geo, packed, grad, dx, ws, stream)
              : launch_t<float, float>(geo, packed, grad, dx, ws, stream);
}

}  // namespace mbok
