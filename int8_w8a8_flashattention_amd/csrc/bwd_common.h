// bwd_common.h - device helpers shared by the backward's kernels (bwd_kernels.hip,
// bwd_dq_kernels.hip).
#pragma once

#include "i8a_device.h"

namespace i8a {
namespace bwd {

__device__ __forceinline__ float bmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return bmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Token of slot jv for lane half hv in a 16-token group (the row order of a 32x32 MFMA
// result's registers).
__device__ __forceinline__ int ckey(int hv, int jv) { return 4 * hv + (jv & 3) + 8 * (jv >> 2); }

__device__ __forceinline__ v16f mfma16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ----------------------------------------------------------------------------------
// Copy of one 32-token operand tile (64 * D contiguous bytes) into LDS by the four waves
// of a workgroup with direct-to-LDS loads: wave w's lanes move the 16-byte chunks
// 256 r + 64 w + lane.
template <int D>
__device__ __forceinline__ void wg_copy_tile(const char* __restrict__ src, char* dst, int tid) {
  constexpr int NCH = 64 * D / 16;
  const int w = tid >> 6;
  const uint32_t base = lds_addr(dst);
#pragma unroll
  for (int r = 0; r * 256 < NCH; ++r) {
    if (r * 256 + w * 64 < NCH) {  // wave-uniform
      const int chunk = r * 256 + tid;
      if (chunk < NCH) lds_dma16(src + (int64_t)chunk * 16, base + (r * 256 + w * 64) * 16);
    }
  }
}

// Number of 16-byte copies that wave w issues per tile in wg_copy_tile<D>.
template <int D>
__host__ __device__ constexpr int tile_dma_count(int w) {
  int n = 0;
  for (int r = 0; r * 256 < 4 * D; ++r)
    if (r * 256 + w * 64 < 4 * D) ++n;
  return n;
}

}  // namespace bwd
}  // namespace i8a
