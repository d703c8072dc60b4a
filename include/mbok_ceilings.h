/*
 * mbok_ceilings.h -- microbenchmarks of the part's own ceilings, for
 * measurement only (libmbok_ceilings.so, built beside libmbok.so).  Not part
 * of the MBOK product path: bench.py runs them so that every kernel can be
 * reported against what this GPU reaches as well as against its nameplate
 * figures (8 TB/s HBM, 2.5 PFLOP/s dense bf16).
 *
 * Every call enqueues one kernel on `stream` (a hipStream_t; NULL = the
 * default stream) and returns 0, -1 for a bad argument (nothing launched) or
 * -5 when the launch fails.  Shapes: 1 <= grid <= 2^20 workgroups of
 * `block` threads, a multiple of 64 from 64 to 1024.  Pointers are device
 * memory owned by the caller.
 */
#ifndef MBOK_CEILINGS_H
#define MBOK_CEILINGS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A kernel that does nothing: timed back to back in a HIP graph, the launch
 * floor of a kernel with this grid. */
int mbok_ceiling_empty(int grid, int block, void* stream);

/* One workgroup of region_marker_kernel, an empty kernel with a name of its
 * own: launched just before and just after a timed region, it lets a kernel
 * trace pick out the region's dispatches. */
int mbok_ceiling_marker(void* stream);

/* One workgroup per compute unit doing fp32 arithmetic for `microseconds`
 * (1 .. 100000) of the 100 MHz real-time counter, then done: enqueued before
 * a timed region, it keeps the chip busy while the host enqueues the region's
 * work.  out (one float) is written only if an impossible value appears. */
int mbok_ceiling_spin(int microseconds, float* out, void* stream);

/* Reads bytes (a multiple of 16) of buf (16-byte aligned) once with
 * nontemporal 16-byte loads, one contiguous chunk per workgroup; out[grid] is
 * written only if an impossible value appears. */
int mbok_ceiling_read(const void* buf, size_t bytes, float* out, int grid, int block,
                      void* stream);

/* Matrix-core issue rate: each wavefront runs `iters` rounds of four
 * independent products of the given kind.  out[grid] is written only if an
 * impossible value appears (so normally never). */
enum {
  MBOK_CEILING_MFMA_BF16 = 0,             /* v_mfma_f32_32x32x16_bf16 */
  MBOK_CEILING_MFMA_F4F8 = 1,             /* scaled 16x16x128, fp4 A, fp8 B, constant scales */
  MBOK_CEILING_MFMA_F4F8_LANE_SCALES = 2  /* the same with a different scale in every lane */
};
int mbok_ceiling_mfma(int kind, float* out, int iters, int grid, int block, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MBOK_CEILINGS_H */
