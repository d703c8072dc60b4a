// Ceiling microbenchmarks of the part (gfx950), built as libmbok_ceilings.so
// beside the MBOK library.  Not part of the product path: bench.py times
// them to report each kernel against what this part can reach as well as
// against its nameplate figures.
//
//  * empty:  a kernel that does nothing, launched with a given grid; its
//            back-to-back interval in a HIP graph is the launch floor of any
//            kernel of that shape.
//  * spin:   one workgroup per compute unit doing fp32 arithmetic for a
//            given time (the 100 MHz real-time counter), to keep the chip busy
//            while the host enqueues a timed region behind it.
//  * read:   every byte of a buffer read once with nontemporal 16-byte loads,
//            a contiguous chunk per workgroup: the read bandwidth a streaming
//            kernel can reach.
//  * mfma:   independent matrix-core products per wavefront (four
//            accumulator chains), bf16 v_mfma_f32_32x32x16_bf16 or the scaled
//            fp4 x fp8 v_mfma_scale_f32_16x16x128_f8f6f4 with the scale
//            operands constant or different in every lane.  Results are
//            written only when an impossible value appears, so nothing is
//            stored but nothing is dead either.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mbok_ceilings.h"

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef short v8s_t __attribute__((ext_vector_type(8)));

__global__ void empty_kernel() {}
// The same, under its own name: bench.py brackets each timed region with it,
// so that a kernel trace can find the region's dispatches (the launch-floor
// measurement runs empty_kernel thousands of times).
__global__ void region_marker_kernel() {}

// Busy for `ticks` of the 100 MHz real-time counter, then ends: it keeps the
// stream (and, with one workgroup per compute unit doing fp32 arithmetic,
// the whole chip) busy while the host enqueues the work that follows it.  The
// loop ends because the counter only advances.
__global__ void spin_kernel(uint64_t ticks, float* out) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  float v = (float)threadIdx.x;
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) {
#pragma unroll
    for (int i = 0; i < 64; ++i) v = fmaf(v, 0.999f, 0.001f);
  }
  if (v == -1.f) out[0] = v;  // never true: v stays in (0, threadIdx.x]
}

constexpr int kReadUnroll = 8;  // loads in flight per thread

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Workgroup b reads the b-th contiguous chunk of the buffer, 8 nontemporal
// 16-byte loads in flight per thread (the fastest of the read patterns
// measured on this part: grid-stride or chunked, 4/8/16 loads in flight,
// temporal or nontemporal).  Nothing is stored unless an impossible value
// appears, so the loads stay live and the kernel ends without a reduction.
__global__ void __launch_bounds__(1024) read_kernel(const uint4* __restrict__ buf, int64_t n16,
                                                    float* __restrict__ out) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += (int64_t)kReadUnroll * blockDim.x) {
    u32x4_t v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t k = i + (int64_t)u * blockDim.x;
      v[u] = k < b1 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(buf + k))
                    : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) out[blockIdx.x] = 1.f;
}

__global__ void __launch_bounds__(1024) mfma_bf16_kernel(float* out, int iters) {
  v8s_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (short)(0x3f80 + ((threadIdx.x + i) & 7));
    b[i] = (short)(0x3f80 + ((threadIdx.x * 3 + i) & 7));
  }
  v16f_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const float s = c0[0] + c1[1] + c2[2] + c3[3];
  if (s == -1.2345f) out[blockIdx.x] = s;
}

template <bool VSCALE>
__global__ void __launch_bounds__(1024) mfma_f4f8_kernel(float* out, int iters) {
  v8i_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = i < 4 ? (int)(0x22222222u ^ ((threadIdx.x * 0x01010101u) & 0x88888888u)) : 0;
    b[i] = (int)(0x38383838u + i);
  }
  // per-lane scale codes near 1.0 (127 +- 3), or the constant 127
  const int sa = VSCALE ? 124 + (int)(threadIdx.x % 7) : 127;
  const int sb = VSCALE ? 124 + (int)((threadIdx.x / 7) % 7) : 127;
  v4f_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c0, 4, 0, 0, sa, 0, sb);
    c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c1, 4, 0, 0, sa, 0, sb);
    c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c2, 4, 0, 0, sa, 0, sb);
    c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c3, 4, 0, 0, sa, 0, sb);
  }
  const float s = c0[0] + c1[1] + c2[2] + c3[3];
  if (s == -1.2345f) out[blockIdx.x] = s;
}

bool shape_ok(int grid, int block) {
  return grid >= 1 && grid <= (1 << 20) && block >= 64 && block <= 1024 && block % 64 == 0;
}

}  // namespace

extern "C" {

int mbok_ceiling_marker(void* stream) {
  hipLaunchKernelGGL(region_marker_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
int mbok_ceiling_empty(int grid, int block, void* stream) {
  if (!shape_ok(grid, block)) return -1;
  hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(block), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int mbok_ceiling_spin(int microseconds, float* out, void* stream) {
  if (microseconds < 1 || microseconds > 100000 || !out) return -1;
  hipLaunchKernelGGL(spin_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream,
                     (uint64_t)microseconds * 100, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int mbok_ceiling_read(const void* buf, size_t bytes, float* out, int grid, int block,
                      void* stream) {
  if (!buf || !out || !shape_ok(grid, block) || bytes % 16 != 0 ||
      ((uintptr_t)buf & 15) != 0)
    return -1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(block), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(buf), (int64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int mbok_ceiling_mfma(int kind, float* out, int iters, int grid, int block, void* stream) {
  if (!out || !shape_ok(grid, block) || iters < 1) return -1;
  hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case MBOK_CEILING_MFMA_BF16:
      hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(block), 0, s, out, iters);
      break;
    case MBOK_CEILING_MFMA_F4F8:
      hipLaunchKernelGGL(mfma_f4f8_kernel<false>, dim3(grid), dim3(block), 0, s, out, iters);
      break;
    case MBOK_CEILING_MFMA_F4F8_LANE_SCALES:
      hipLaunchKernelGGL(mfma_f4f8_kernel<true>, dim3(grid), dim3(block), 0, s, out, iters);
      break;
    default:
      return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
