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

// Bytes of a wave's LDS staging area for store_rows_f32<EC>.
template <int EC>
constexpr int staging_bytes() {
  return 32 * (4 * EC + 16);
}

// A wave's 32 rows of fp32 results (32 x 32 MFMA accumulators: lane (m, hh) holds
// channels 32 db + 8 J + 4 hh .. + 3 of row m), times mul, stored to rows row0 + r * D
// for r < nvalid.  Direct stores would write 16 bytes in each of 32 rows per
// instruction; instead EC channels at a time go through the wave's LDS area (rows
// padded to 4 EC + 16 bytes) and come back as 16 bytes of one row per lane, EC / 4 lanes
// per row, so that every store writes whole 128-byte lines or more.
template <int D, int EC>
__device__ __forceinline__ void store_rows_f32(const v16f (&acc)[D / 32], float mul, char* area,
                                               float* __restrict__ row0, int nvalid, int lane) {
  constexpr int EPITCH = 4 * EC + 16;
  constexpr int LPR = EC / 4;    // lanes per row of a pass
  constexpr int RPI = 64 / LPR;  // rows per read and store
  static_assert(D % EC == 0 && EC % 32 == 0 && RPI >= 1, "whole 32-channel blocks per pass");
  const int m = lane & 31, hh = lane >> 5;
  const int rr = lane / LPR, cc = lane % LPR;
#pragma unroll
  for (int p = 0; p < D / EC; ++p) {
#pragma unroll
    for (int db = 0; db < EC / 32; ++db)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        v4f x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = acc[p * (EC / 32) + db][4 * J + r] * mul;
        *reinterpret_cast<v4f*>(area + m * EPITCH + 4 * (32 * db + 8 * J + 4 * hh)) = x;
      }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = RPI * i + rr;
      const v4f x = *reinterpret_cast<const v4f*>(area + row * EPITCH + 16 * cc);
      if (row < nvalid) *reinterpret_cast<v4f*>(row0 + (int64_t)row * D + p * EC + 4 * cc) = x;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ----------------------------------------------------------------------------------
// Copy of one 32-token operand tile (64 * D contiguous bytes) into LDS by the four waves
// of a workgroup with direct-to-LDS loads: wave w's lanes move the 16-byte chunks
// 256 r + 64 w + lane.
// Direct-to-LDS copy of 16 bytes per lane from the wave-uniform address sbase plus the
// lane's 32-bit byte offset voff (the instruction's scalar-base form), into LDS at the
// wave-uniform address lds_base (+ 16 x lane).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Copy of one 32-token operand tile (64 * D contiguous bytes) into LDS by the NT threads
// of a workgroup: wave w's lanes move the 16-byte chunks NT r + 64 w + lane.  The
// lanes' offsets are computed once; a copy is then a scalar base, an m0 write and the
// load.  The chunk count 4 D is a multiple of 64, so a wave copies whole rows of 64
// chunks or none.
template <int D, int NT = 256>
struct TileCopy {
  static constexpr int NCH = 64 * D / 16;
  static constexpr int R = (NCH + NT - 1) / NT;
  uint32_t voff[R];
  int w;
  __device__ __forceinline__ explicit TileCopy(int tid)
      : w(__builtin_amdgcn_readfirstlane(tid >> 6)) {
#pragma unroll
    for (int r = 0; r < R; ++r) voff[r] = (uint32_t)(r * NT + tid) * 16;
  }
  __device__ __forceinline__ void operator()(const char* src, char* dst) const {
    const uint32_t base = lds_addr(dst);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (NCH % NT == 0 || r * NT + w * 64 < NCH)  // wave-uniform
        lds_dma16_s(src, voff[r], base + (uint32_t)(r * NT + w * 64) * 16);
  }
};

// Number of 16-byte copies that wave w issues per tile with TileCopy<D>.
template <int D>
__host__ __device__ constexpr int tile_dma_count(int w) {
  int n = 0;
  for (int r = 0; r * 256 < 4 * D; ++r)
    if (r * 256 + w * 64 < 4 * D) ++n;
  return n;
}

}  // namespace bwd
}  // namespace i8a
