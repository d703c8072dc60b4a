// Packs int8 +-1 sign planes and natural-order scales into the L64 layout
// described in include/mbok.h: one thread per 16-byte chunk (row, group,
// kernel); chunk c = ((rb*G + g)*K + k)*64 + r holds the group's 128 signs as
// four uint32 words, bit (8e + q) of word w being column 32w + 4q + e of the
// group, bit 1 = +1.  The scale of the chunk goes to value index c of the
// scale region.  Rows past m are written as zero bits and zero scales.
#include "mbok_device.h"
#include "mbok_launch.h"

namespace mbok {
namespace {

template <typename AT>
__global__ void __launch_bounds__(256) pack_kernel(const int8_t* __restrict__ signs,
                                                   const AT* __restrict__ alpha, int m, int n,
                                                   int K, int RB, int row_stride, int group_stride,
                                                   uint4* __restrict__ bits,
                                                   AT* __restrict__ scales) {
  const int G = n / kGroup;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)RB * G * K * kRowBlock;
  if (c >= total) return;
  const int r = (int)(c % kRowBlock);
  int64_t t = c / kRowBlock;
  const int k = (int)(t % K);
  t /= K;
  const int g = (int)(t % G);
  const int rb = (int)(t / G);
  const int i = rb * kRowBlock + r;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  AT a = AT(0);
  if (i < m) {
    const int4* src = reinterpret_cast<const int4*>(signs + ((int64_t)k * m + i) * n +
                                                    (int64_t)g * kGroup);
#pragma unroll
    for (int v = 0; v < 8; ++v) {  // 16 signs per 16-byte load
      const int4 s = src[v];
      const uint32_t parts[4] = {(uint32_t)s.x, (uint32_t)s.y, (uint32_t)s.z, (uint32_t)s.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          // byte b of part p is column 16v + 4p + b = 32w + 4q + e with
          // w = v/2, q = 4(v%2) + p, e = b; bit 1 when the int8 is >= 0
          const uint32_t bit = ((~parts[p]) >> (8 * b + 7)) & 1u;
          w[v >> 1] |= bit << (8 * b + 4 * (v & 1) + p);
        }
      }
    }
    a = alpha[((int64_t)k * m + i) * row_stride + (int64_t)g * group_stride];
  }
  bits[c] = make_uint4(w[0], w[1], w[2], w[3]);
  scales[c] = a;
}

// alpha[(k m + i) * row_stride + g * group_stride] is the scale of chunk
// (row i, group g, kernel k): (G, 1) for per-group scales, (1, 0) for one
// scale per row (the SVID s_out).
int pack_strided(const mbok_desc* d, const int8_t* signs, const void* alpha, void* packed,
                 int row_stride, int group_stride, hipStream_t stream) {
  const Geom geo = make_geom(d);
  const int64_t total = (int64_t)geo.RB * geo.G * geo.K * kRowBlock;
  const int block = 256;
  const int64_t blocks = (total + block - 1) / block;
  if (blocks > 0x7fffffff) return MBOK_ERR_SHAPE;
  uint4* bits = reinterpret_cast<uint4*>(packed);
  char* scales = reinterpret_cast<char*>(packed) + geo.bits_bytes;
  if (d->alpha_dtype == MBOK_F16)
    hipLaunchKernelGGL(pack_kernel<uint16_t>, dim3((unsigned)blocks), dim3(block), 0, stream,
                       signs, reinterpret_cast<const uint16_t*>(alpha), geo.m, geo.n, geo.K,
                       geo.RB, row_stride, group_stride, bits,
                       reinterpret_cast<uint16_t*>(scales));
  else
    hipLaunchKernelGGL(pack_kernel<float>, dim3((unsigned)blocks), dim3(block), 0, stream,
                       signs, reinterpret_cast<const float*>(alpha), geo.m, geo.n, geo.K,
                       geo.RB, row_stride, group_stride, bits, reinterpret_cast<float*>(scales));
  return hipGetLastError() == hipSuccess ? MBOK_OK : MBOK_ERR_HIP;
}

}  // namespace

int launch_pack(const mbok_desc* d, const int8_t* signs, const void* alpha, void* packed,
                hipStream_t stream) {
  return pack_strided(d, signs, alpha, packed, d->n / kGroup, 1, stream);
}

int launch_svid_pack(const mbok_desc* d, const int8_t* signs, const void* s_out, void* packed,
                     hipStream_t stream) {
  return pack_strided(d, signs, s_out, packed, 1, 0, stream);
}

}  // namespace mbok
