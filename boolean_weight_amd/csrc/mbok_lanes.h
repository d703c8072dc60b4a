// Lane exchanges across the four 16-lane blocks of a wavefront (gfx950
// v_permlane16_swap / v_permlane32_swap, no LDS round trip).  Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbok {

// Swap the upper 32 lanes of a with the lower 32 lanes of b.
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// Swap the odd 16-lane rows of a with the even 16-lane rows of b.
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

// Broadcast of one value per 16-lane block: afterwards r[j] in every block is
// the value v held in block j.
__device__ __forceinline__ void spread4(uint32_t v, uint32_t (&r)[4]) {
  uint32_t lo = v, hi = v;
  swap32(lo, hi);  // blocks: lo = [v0 v1 v0 v1], hi = [v2 v3 v2 v3]
  r[0] = lo, r[1] = lo, r[2] = hi, r[3] = hi;
  swap16(r[0], r[1]);
  swap16(r[2], r[3]);
}

}  // namespace mbok
