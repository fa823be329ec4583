// attn_kernels.hip - the INT8 W8A8 FlashAttention-2 forward on gfx950.
//
// Each wave owns 32 query rows of one head and keeps, per lane, one query's running
// max, sum and 32 x D output accumulator column.  Per 64-key tile:
//   S^T = K . Q^T     v_mfma_i32_32x32x32_i8   (exact int32)
//   t   = f32(S^T) * c_j - M                   (c_j = sk_j * qsc: the key scale times the
//   p   = exp2(t)                               query's scale and softmax scale)
//   O^T += V^T . P^T  v_mfma_f32_32x32x16_f16  (P rounded to fp16, V exact in fp16)
//   l   += sum of the same fp16 P values
// so the normalized output is a weighted mean with identical weights in numerator
// and denominator.  The running max M is only raised (with a rescale of O and l)
// when a tile's max exceeds it by more than TAU in log2 units, which bounds every
// p by 2^TAU and skips most rescales.
//
// K (int8) and the exact fp16 V come from the workspace in MFMA fragment order, and
// so does Q where the kernel does not quantize it itself; the K/V tile copy into LDS
// is linear, so every LDS operand read is a conflict-free 16-byte read.
//
// One kernel, attn_pipe_kernel, software-pipelined over two tiles: 8 waves and 256
// query rows per workgroup at D = 128; 4 waves and 128 rows at D <= 64 (three
// workgroups per CU) and at D = 256 (one wave per SIMD, whose 512 registers hold the
// accumulators and both tiles' state).
#include <float.h>

#include <type_traits>

#include "i8a_device.h"
#include "i8a_launch.h"

namespace i8a {

typedef float v32f __attribute__((ext_vector_type(32)));

#ifndef PIPE_TAU
#define PIPE_TAU 12.0f
#endif
constexpr float TAU = PIPE_TAU;  // lazy-rescale threshold, log2 units

template <int D, bool QO = false>
struct Lay {
  static constexpr int NKB = D / 32;             // 32-wide blocks of the head dim
  static constexpr int KB = TK * D;              // bytes of the int8 K codes
  static constexpr int VB = TK * D * 2;          // bytes of the fp16 V
  static constexpr int KO = tile_bytes(D);       // offset of the outlier channels' K
  static constexpr int STAGE = tile_bytes(D, QO);  // one pipeline stage = one tile block
  static constexpr int NCH = STAGE / 16;         // 16-byte chunks per tile
  static constexpr int ROUNDS = (NCH + 255) / 256;
  static_assert(STAGE % 16 == 0, "tiles are copied in 16-byte chunks");
};

// Max of two scores.  The IEEE-754-2019 maximum (v_maximum3_f32) needs no quieting
// of its inputs, unlike fmaxf (maxNum) after a select or a lane exchange; the scores
// are never NaN, where the two agree.
__device__ __forceinline__ float smax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Value of the lane 32 apart (the other half of the wave), through v_permlane32_swap
// (a VALU exchange, no LDS round trip): with v in both operands the swap leaves the
// low half's values in one result and the high half's in the other.
__device__ __forceinline__ float other_half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return smax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float other_half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until this wave's outstanding vector-memory operations (the direct-to-LDS
// tile copies) have completed: vmcnt = 0, lgkmcnt and expcnt left unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Copy one prepared tile block (global) into an LDS stage with direct-to-LDS loads:
// every lane moves one 16-byte chunk, a wave fills 1 KB of consecutive LDS.
template <int D>
__device__ __forceinline__ void copy_tile_async(const char* __restrict__ src, char* stage,
                                                int tid) {
  using LY = Lay<D>;
  const int w = tid >> 6;
#pragma unroll
  for (int r = 0; r < LY::ROUNDS; ++r) {
    const int chunk = r * 256 + tid;
    if (r * 256 + w * 64 < LY::NCH) {  // wave-uniform: this wave has chunks left
      char* lbase = stage + (r * 256 + w * 64) * 16;
      if (chunk < LY::NCH)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + (int64_t)chunk * 16),
                                         (__attribute__((address_space(3))) void*)(lbase), 16, 0,
                                         0);
    }
  }
}

// Work item of a workgroup: a query-tile slot, a sequence and a head.  Slots are the
// slowest-varying index, and under the causal mask slot 0 is the last (longest) query
// tile, so the heaviest workgroups are dispatched first and the short ones fill the
// tail.  With xcd_map the heads of one kv group land on blocks with the same id mod 8,
// i.e. on one XCD (blocks are dispatched round-robin over the 8 XCDs), so that group's
// K/V stays in that XCD's L2.
__device__ __forceinline__ void decode_work(int bid, int nseq, int Hq, int Hkv, int xcd_map,
                                            int& slot, int& s, int& h) {
  const int nbh = nseq * Hq;
  slot = bid / nbh;
  const int r = bid % nbh;
  if (xcd_map) {
    const int G = Hq / Hkv;
    const int x = r & 7, kk = r >> 3;
    const int grp = x + 8 * (kk / G);
    s = grp / Hkv;
    h = (grp % Hkv) * G + kk % G;
  } else {
    s = r / Hq;
    h = r % Hq;
  }
}

// The epilogue of both kernels: a wave's 32 rows of O / l in fp16.  Lane (m, hh) holds
// channels 32 db + 8 J + 4 hh .. + 3 of row m, so direct stores would write 8 bytes in
// each of 32 rows per instruction.  Instead EC channels at a time go to the wave's LDS
// area (rows padded to 2 EC + 16 bytes) and come back as 16 bytes of one row per lane,
// EC / 8 lanes per row, so that every store writes whole rows of EC channels (128-byte
// lines and more).  `inv` is 1 / l (0 for rows past the sequence end, which are not
// stored).  The area holds 32 (2 EC + 16) bytes and is this wave's alone.
template <int D, int EC>
__device__ __forceinline__ void store_rows(const v16f (&o)[D / 32], float inv, char* area,
                                           _Float16* __restrict__ out, const Act& aq,
                                           int64_t start, int h, int qw0, int L, int lane) {
  constexpr int EPITCH = 2 * EC + 16;
  constexpr int LPR = EC / 8;    // lanes per row of a pass
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
        v4h o4;
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = (_Float16)(o[p * (EC / 32) + db][4 * J + r] * inv);
        *reinterpret_cast<v4h*>(area + m * EPITCH + 2 * (32 * db + 8 * J + 4 * hh)) = o4;
      }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = RPI * i + rr;
      const v8h v8 = *reinterpret_cast<const v8h*>(area + row * EPITCH + 16 * cc);
      if (qw0 + row < L)
        *reinterpret_cast<v8h*>(out + aq.off(start, h, qw0 + row) + p * EC + 8 * cc) = v8;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// The matrix products of the forward.  With ASM (D = 256, one wave per SIMD, where the
// compiler would put every product's result in accumulation registers and copy the
// scores and key-scale products back one register at a time for the softmax) they are
// issued from inline assembly, so that each result lives in the register file its
// readers want: the P.V and row-sum accumulators in accumulation registers (AGPRs;
// only the rare rescale and the epilogue read them), the scores and key-scale products
// in vector registers.  The compiler does not see the assembly as matrix instructions
// and counts no wait states for it, so the hardware's required wait states between a
// product and a vector instruction that reads its result are the caller's: settle()
// (a result read: 21 wait states, more than the 16-pass products need) and the NOP
// variants (an operand written by the instruction just before: 2).
template <bool ASM>
struct Mm {
  // S = A.B for one 32x32 block of scores (int8, exact int32), a fresh accumulator.
  static __device__ __forceinline__ v16i qk0(v4i a, v4i b) {
    if constexpr (ASM) {
      v16i c;
      asm volatile("v_mfma_i32_32x32x32_i8 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
      return c;
    } else {
      v16i z;
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0;
      return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, z, 0, 0, 0);
    }
  }
  static __device__ __forceinline__ void qk(v16i& c, v4i a, v4i b) {
    if constexpr (ASM)
      asm volatile("v_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
    else
      c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
  // o += A.B (fp16 inputs, fp32 accumulation).
  template <bool NOP = false>
  static __device__ __forceinline__ void pv(v16f& o, v8h a, v8h b) {
    if constexpr (ASM) {
      if constexpr (NOP)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
      else
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
    } else {
      o = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, o, 0, 0, 0);
    }
  }
  template <bool NOP = false>
  static __device__ __forceinline__ void rowsum(v4f& l, v8h a, v8h b) {
    if constexpr (ASM) {
      if constexpr (NOP)
        asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(l) : "v"(a), "v"(b));
      else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(l) : "v"(a), "v"(b));
    } else {
      l = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, l, 0, 0, 0);
    }
  }
  // A.B with a fresh accumulator (the Q outlier products, D <= 128: always the builtin).
  static __device__ __forceinline__ v16f f16_0(v8h a, v8h b) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, v16f{}, 0, 0, 0);
  }
  // The outer product a_l . b_l over the two 32-lane blocks (v_mfma_f32_32x32x1_2b_f32).
  static __device__ __forceinline__ v32f outer(float a, float b) {
    if constexpr (ASM) {
      v32f c;
      asm volatile("v_mfma_f32_32x32x1_2b_f32 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
      return c;
    } else {
      v32f z;
#pragma unroll
      for (int i = 0; i < 32; ++i) z[i] = 0.0f;
      return __builtin_amdgcn_mfma_f32_32x32x1f32(a, b, z, 0, 0, 0);
    }
  }
  // 21 wait states before x is read; x passes through so its readers stay after them.
  template <typename T>
  static __device__ __forceinline__ void settle_v(T& x) {
    if constexpr (ASM) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(x));
  }
  static __device__ __forceinline__ void settle_v3(v32f& x, v16i& y, v16i& z) {
    if constexpr (ASM) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(x), "+v"(y), "+v"(z));
  }
  template <int N>
  static __device__ __forceinline__ void settle_acc(v16f (&o)[N], v4f& l) {
    if constexpr (ASM) {
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+a"(l));
#pragma unroll
      for (int i = 0; i < N; ++i) asm volatile("" : "+a"(o[i]));
    }
  }
};

// Unnormalized fast Walsh-Hadamard transform of a D-channel query row in the operand
// layout of the forward's Q: lane (m, hh) holds channels 32 kb + 16 hh + i (i < 16) as
// x[16 kb + i].  The stages run in the order s = 0, 1, ..., log2(D) - 1, and stage s
// replaces the pair (x_c, x_{c + 2^s}) with bit s of c clear by (x_c + x_{c + 2^s},
// x_c - x_{c + 2^s}), the same fp32 operations as the preparation's fwht_row, so the
// rows are bit-identical: stages 0-3 pair values inside a 16-channel chunk, stage 4 the
// two half-rows of lanes m and m + 32 (v_permlane32_swap gives every lane both), the
// later ones chunks kb and kb + 2^(s-5) of the lane.
template <int D>
__device__ __forceinline__ void fwht_qrow(float (&x)[D / 2], int hh) {
  constexpr int N = D / 2;
#pragma unroll
  for (int h = 1; h < 16; h *= 2)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (!(i & h)) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[i]), __float_as_uint(x[i]),
                                                    false, false);
    const float lo = __uint_as_float(r[0]), hi = __uint_as_float(r[1]);
    x[i] = hh ? lo - hi : lo + hi;
  }
#pragma unroll
  for (int h = 16; h < N; h *= 2)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (!(i & h)) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
}

// The forward's own Q quantization (the kernels' FQ path): lane (m, hh) holds channels
// 32 kb + 16 hh + j (j < 16) of query row qi, exactly its B-operand fragment positions, so
// the codes are made in place with the preparation's row rule (row_scale, RowQ), bit
// for bit.  The row's absolute maximum combines the two half-rows of lanes m and
// m + 32 (a max is exact in any order); with qmode bit 0, the wave's maximum (its 32
// rows are one block).  With qmode bit 1 the rows are Hadamard-rotated first
// (fwht_qrow).  Rows past the sequence end get zero codes and scale 0.  QO: the kv
// group's outlier channels (oc, QO_MAX entries, -1 padded) are zeroed first, and the
// row's values at the outlier slots 8 hh .. 8 hh + 7 go to qo.  Returns the row scale
// (QO: 2^-60 where the int8 part is all zero).
template <int D, bool QO>
__device__ __forceinline__ float quantize_own_q(const _Float16* __restrict__ qin, const Act& aq,
                                                int64_t start, int h, int qi, int L, int hh,
                                                int qmode, const int32_t* __restrict__ oc,
                                                v4i (&qf)[D / 32], v8h& qo) {
  const bool qblk = (qmode & 1) != 0;
  constexpr int NKB = D / 32;
  const bool real = qi < L;
  v8h xr[NKB][2];
  if (real) {
    const _Float16* row = qin + aq.off(start, h, qi) + 16 * hh;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 2; ++e) xr[kb][e] = *reinterpret_cast<const v8h*>(row + 32 * kb + 8 * e);
  }
  // QO: bit 16 kb + c % 16 of omask marks outlier channel c = 32 kb + 16 hh + c % 16
  // among this lane's channels.
  uint64_t omask = 0;
  if constexpr (QO) {
#pragma unroll
    for (int o = 0; o < QO_MAX; ++o) {
      const int c = oc[o];
      if (c >= 0 && ((c >> 4) & 1) == hh) omask |= 1ull << (16 * (c >> 5) + (c & 15));
    }
    const _Float16* row = qin + aq.off(start, h, qi);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = oc[8 * hh + j];
      qo[j] = (real && c >= 0) ? row[c] : (_Float16)0.0f;
    }
  }
  if (!QO && (qmode & 2)) {
    // Rotated rows: the transform in fp32, then the row rule on its results.
    float x[D / 2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int j = 0; j < 8; ++j) x[16 * kb + 8 * e + j] = real ? (float)xr[kb][e][j] : 0.0f;
    fwht_qrow<D>(x, hh);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < D / 2; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    if (qblk) amax = group_max<64>(amax);
    const RowQ rq(real ? row_scale(amax, 24) : 0.0f);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float lo8[8], hi8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lo8[j] = x[16 * kb + j];
        hi8[j] = x[16 * kb + 8 + j];
      }
      const uint2 lo = real ? rq.pack8(lo8) : make_uint2(0u, 0u);
      const uint2 hi = real ? rq.pack8(hi8) : make_uint2(0u, 0u);
      qf[kb] = v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
    }
    return rq.s;
  } else if constexpr (!QO) {
    // The fp16 values go into the arithmetic as they are: the absolute maximum from
    // their bit patterns, the codes from fp16 operands (exact conversions).
    uint32_t mb = 0;
    if (real) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 2; ++e) mb = absmax_bits8(xr[kb][e], mb);
    }
    float amax = absmax_of_bits(mb);
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    if (qblk) amax = group_max<64>(amax);
    const RowQ rq(real ? row_scale(amax, 24) : 0.0f);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint2 lo = real ? rq.pack8h(xr[kb][0]) : make_uint2(0u, 0u);
      const uint2 hi = real ? rq.pack8h(xr[kb][1]) : make_uint2(0u, 0u);
      qf[kb] = v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
    }
    return rq.s;
  } else {
    float xf[NKB][2][8];
    float amax = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool keep = ((omask >> (16 * kb + 8 * e + j)) & 1) == 0;
          xf[kb][e][j] = (real && keep) ? (float)xr[kb][e][j] : 0.0f;
          amax = fmaxf(amax, fabsf(xf[kb][e][j]));
        }
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    if (qblk) amax = group_max<64>(amax);
    const RowQ rq(real ? row_scale(amax, 24) : 0.0f);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint2 lo = real ? rq.pack8(xf[kb][0]) : make_uint2(0u, 0u);
      const uint2 hi = real ? rq.pack8(xf[kb][1]) : make_uint2(0u, 0u);
      qf[kb] = v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
    }
    return rq.s == 0.0f ? 0x1p-60f : rq.s;
  }
}

// ----------------------------------------------------------------------------------
// Software-pipelined forward for D <= 128: at D = 128 one workgroup of 8 waves (256
// query rows) per CU with a four-stage LDS ring; at D <= 64 workgroups of 4 waves (128
// rows), three per CU, with three stages.  The row sum on the MFMA.
//
// A 32 x 64 wave-tile needs 24 MFMAs (8 int8 for the scores, 16 fp16 for P.V) and
// about 160 vector instructions of softmax (per score: conversion, key scale,
// exponent FMA, exponential, half a pack, a share of the max).  A wave issues vector
// instructions at one per four cycles or so, and only about six fit under one 32-cycle
// MFMA, so every phase of a tile needs MFMAs to run beside its vector work.  The tiles
// therefore run as a pipeline over two tiles: with tile j's scores converted
// (t = f32(S) * sk) and its max folded into M, iteration j issues the score MFMAs of
// tile j+1 and the P.V MFMAs of tile j, one per slot, and spreads over the same slots
// the exponentials of tile j, the conversion (and mask) of tile j+1's scores, its
// row max and the rescale decision (pipe_step).  M is raised after the slots if a row
// needs it (rare: the rescale of O and l waits for tile j's P.V).  The row sum l is
// one more fp16 MFMA per 16 keys, a 16x16x32 one (half the matrix-unit cycles of a
// P.V product) whose 0/1 A operand sums the same fp16 P values the P.V product
// consumes (register 0 is read at the end), which keeps the vector unit free of the
// sum; dot-product instructions stall behind a running MFMA.
//
// The ring holds tiles j (V for P.V), j+1 (K and scales), j+2 (landed) and j+3 (in
// flight): every wave copies its share of tile j+3 into the stage tile j-1 left, one
// instruction every few slots of iteration j, and waits for its share of tile j+2 at
// the end of it, before the one barrier of the iteration.
//
// Under the causal mask a wave stops computing after its diagonal tile and from then
// on only copies and passes the barriers; the two waves of each SIMD take the row
// blocks b and 7 - b of the tile, so every SIMD gets the same number of tiles.

// Copy one prepared tile block into an LDS stage with direct-to-LDS loads that the
// compiler does not track: the waits are explicit (vm_wait), so no compiler-inserted
// wait makes a tile's work wait for the next tile's copy.  Every round moves 4 KB: the
// global base and the LDS base (M0) are scalars, the lane's byte offset 16 * tid is the
// one vector operand of every round.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16_sbase(const char* sbase, uint32_t voff,
                                                uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// The same for the lanes in `lanes` only (a wave-wide mask), with EXEC narrowed and
// restored inside the one statement, so the caller gets no branch.  With no lane set
// the load runs with EXEC = 0 and moves nothing.
__device__ __forceinline__ void lds_dma16_sbase_lanes(const char* sbase, uint32_t voff,
                                                      uint32_t lds_base, uint64_t lanes) {
  uint64_t saved;
  asm volatile(
      "s_and_saveexec_b64 %0, %4\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\ts_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base)), "s"(lanes)
      : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// A tile is copied in rounds of NW * 1 KB.  In every round but the last, wave w moves
// the 1 KB at 1 KB * w of the round.  The last round may be partial; there each wave
// moves R consecutive 16-byte chunks (the last wave possibly fewer, never none), so
// every wave issues exactly ROUNDS copy instructions per tile and one constant wait
// covers any wave's copies.
template <int D, int NW, bool QO = false>
struct Dma {
  static constexpr int NT = 64 * NW;  // threads
  static constexpr int NCH = Lay<D, QO>::NCH;
  static constexpr int ROUNDS = (NCH + NT - 1) / NT;
  static constexpr int REM = NCH - (ROUNDS - 1) * NT;  // chunks of the last round
  static constexpr int R = (REM + NW - 1) / NW;         // a wave's chunks in it
  static_assert(REM > (NW - 1) * R, "every wave copies part of the last round");
};

// Round r of a tile copy for this wave.  In a partial last round the wave's lanes past
// its R chunks are masked off, with no wave-uniform branch, so an unrolled caller stays
// one basic block.  The lane's byte offset 16 * tid stays the one vector operand; the
// scalar base is moved back by the wave's 1 KB so that lane l reads chunk cb + l.
template <int D, int NW, bool QO>
__device__ __forceinline__ void copy_tile_round(const char* __restrict__ src, char* stage, int tid,
                                                int w, int r) {
  using DM = Dma<D, NW, QO>;
  const uint32_t lds0 = lds_addr(stage);
  if (r + 1 < DM::ROUNDS || DM::REM == DM::NT) {
    lds_dma16_sbase(src + r * DM::NT * 16, 16u * (uint32_t)tid,
                    lds0 + (uint32_t)(r * DM::NT * 16 + w * 1024));
  } else {
    const int cb = r * DM::NT + w * DM::R;  // the wave's first chunk (uniform)
    const int n = DM::REM - w * DM::R < DM::R ? DM::REM - w * DM::R : DM::R;
    lds_dma16_sbase_lanes(src + 16 * (cb - 64 * w), 16u * (uint32_t)tid, lds0 + 16u * (uint32_t)cb,
                          n >= 64 ? ~0ull : (1ull << n) - 1);
  }
}

// All rounds of a tile copy for this wave.
template <int D, int NW, bool QO>
__device__ __forceinline__ void copy_tile_dma(const char* __restrict__ src, char* stage, int tid,
                                              int w) {
#pragma unroll
  for (int r = 0; r < Dma<D, NW, QO>::ROUNDS; ++r) copy_tile_round<D, NW, QO>(src, stage, tid, w, r);
}

// Workgroups per CU the kernel is built for (its register and LDS budget): one at D = 128
// (eight waves) and D = 256; three at D <= 64 (four waves each), where the per-score
// vector work outweighs the matrix work and a third wave per SIMD hides more of its
// latencies; two with Q outlier detection, whose registers would spill at three.  (Four
// at D = 32 spill inside the loop and measured 14 % slower.)
constexpr int wg_per_cu(int D, int NW, bool QO) {
  return (NW >= 8 || D > 128) ? 1 : QO ? 2 : 3;
}

// FQ: the kernel quantizes its Q rows itself from the fp16 input qin (layout aq, the
// output's), with the Q/K row rule, with qmode bit 0 one scale per 32-row block counted
// from the sequence start, with bit 1 after the Hadamard rotation; otherwise it reads
// the prepared fragments q8 and scales qs.
// QO (with FQ): Q outlier channels.  The kv group's channels (ochan) are left out of
// the int8 Q rows, and their fp16 products come from one 32x32x16 fp16 MFMA per
// 32-key block with the tile's fp16 K values of those channels:
//   t = f32(S^T) * c_j + So^T * qk_log2 - M,   c_j = sk_j * qsc
// (qsc = sq * qk_log2, with sq replaced by 2^-60 where the int8 part is all zero: its
// scores are 0 there).
template <int D, bool CAUSAL, int NW, bool FQ, bool QO = false>
__global__ __launch_bounds__(64 * NW, wg_per_cu(D, NW, QO)) void attn_pipe_kernel(
    const int8_t* __restrict__ q8, const float* __restrict__ qs, int64_t Qpad,
    const _Float16* __restrict__ qin, int qmode, _Float16* __restrict__ out, Act aq, Seqs seqs,
    int Hq, int Hkv, int nseq, int xcd_map, float qk_log2, const char* __restrict__ tiles,
    int64_t Ppad, const int32_t* __restrict__ ochan) {
  static_assert(!QO || FQ, "the outlier channels' Q values come from the fused Q path");
  using LY = Lay<D, QO>;
  using DM = Dma<D, NW, QO>;
  using MM = Mm<(D > 128)>;             // products from assembly at D = 256
  constexpr int NKB = LY::NKB;
  constexpr int BMW = 32 * NW;          // query rows per workgroup
  constexpr int NS = NW >= 8 ? 4 : 3;   // ring stages
  static_assert(BQ % BMW == 0, "query tiles stay inside a sequence's padded Q slots");
  // The output goes through a per-wave LDS area after the ring (store_rows): EC channels
  // of the wave's 32 rows at a time, rows padded to EPITCH bytes.
  constexpr int EC = D < 64 ? D : 64;
  constexpr int EPITCH = 2 * EC + 16;
  // Where the ring and the staging areas of the workgroups of a CU would not fit the 160
  // KB of LDS together (D = 256, and D = 64 at three workgroups per CU), the output is
  // staged in the ring once no tile uses it any more.
  constexpr int WGPC = wg_per_cu(D, NW, QO);
  constexpr bool EPI_IN_RING = (NS * LY::STAGE + NW * 32 * EPITCH) * WGPC > 160 * 1024;
  static_assert(!EPI_IN_RING || NW * 32 * EPITCH <= NS * LY::STAGE, "staging fits the ring");
  __shared__ __attribute__((aligned(16)))
  char smem[NS * LY::STAGE + (EPI_IN_RING ? 0 : NW * 32 * EPITCH)];

  int slot, s, h;
  decode_work(blockIdx.x, nseq, Hq, Hkv, xcd_map, slot, s, h);
  int64_t start;
  int L;
  seqs.bounds(s, start, L);
  const int nqt_s = (L + BMW - 1) / BMW;
  if (slot >= nqt_s) return;
  const int qt = CAUSAL ? nqt_s - 1 - slot : slot;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t pbase = Seqs::pstart(s, start);
  const char* tsrc = tiles + ((int64_t)g * (Ppad / TK) + pbase / TK) * LY::STAGE;

  // Waves w and w + 4 share a SIMD; with 8 waves they take the 32-row blocks w and
  // 7 - w of the query tile, so that under the causal mask every SIMD gets the same
  // number of visible tiles.
  const int blk = NW == 8 ? (w < 4 ? w : 11 - w) : w;
  const int q0 = qt * BMW;
  const int qw0 = q0 + 32 * blk;
  const int qi = qw0 + m;
  const int ntile_seq = (L + TK - 1) / TK;
  const int nt = CAUSAL ? min(ntile_seq, (min(q0 + BMW, L) - 1) / TK + 1) : ntile_seq;
  // The wave's last tile with a visible key (its causal diagonal): later tiles of the
  // workgroup it only helps to copy.
  const int jv = CAUSAL ? min(nt - 1, qw0 / TK) : nt - 1;
  // Tile j needs a mask for this wave when some of its keys lie above the wave's
  // causal diagonal or past the sequence end; `last` is then the lane's last visible
  // key relative to the tile's first key plus 4 hh (its register offsets are relative
  // to that).
  const int last_key = CAUSAL ? min(qi, L - 1) : L - 1;
  auto needs_mask = [&](int jj) {
    return (CAUSAL && jj * TK + TK - 1 > qw0) || jj * TK + TK > L;
  };

  // Prologue: tiles 0 .. NS-2 stream into their stages while the wave's Q rows load.
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < nt)
      copy_tile_dma<D, NW, QO>(tsrc + (int64_t)i * LY::STAGE, smem + i * LY::STAGE, tid, w);
  v4i qf[NKB];
  float qsc;
  v8h qo;  // QO: the row's values at the outlier slots 8 hh .. 8 hh + 7
  if constexpr (FQ) {
    const float sq = quantize_own_q<D, QO>(qin, aq, start, h, qi, L, hh, qmode,
                                           ochan + ((int64_t)s * Hkv + g) * QO_MAX, qf, qo);
    qsc = QO ? sq * qk_log2 : fmaxf(sq * qk_log2, FLT_MIN);
  } else {
    const int64_t qslot = (int64_t)h * Qpad + Seqs::qpstart(s, start) + qw0;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      qf[kb] = reinterpret_cast<const v4i*>(q8 + qslot * D)[kb * 64 + lane];
    qsc = fmaxf(qs[qslot + m] * qk_log2, FLT_MIN);
  }
  vm_wait<0>();
  __syncthreads();

  v16f o[NKB];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int db = 0; db < NKB; ++db) o[db][i] = 0.0f;
  // The row sum l: one 16x16x32 fp16 MFMA per key group kg, with pk[kg] as its B
  // operand.  Read that way, lane b's 8 values are k-slice b / 16 of column b % 16, and
  // they belong to query b % 32 (keys 8 (b / 32) ..): k-slices 0 and 2 hold columns
  // 0..15's own queries, slices 1 and 3 the queries 16 higher.  The A operand `sel` is 1
  // where row i's k-slice matches (i / 4) % 2, else 0, so result row i sums the 16 keys of
  // query n + 16 ((i / 4) % 2) in column n; a lane l holds rows 4 (l / 16) .. + 3 of
  // column l % 16, so all four of its registers are the sum of its own query l % 32.
  // The products 1 * p and 0 * p are exact and the sum is fp32, as in P.V.
  v4f lacc = {0.0f, 0.0f, 0.0f, 0.0f};
  v8h sel;
  {
    const _Float16 one = (((lane >> 4) ^ (lane >> 2)) & 1) ? (_Float16)0.0f : (_Float16)1.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = one;
  }
  // The tile's exponent arguments t = f32(S) * c - M (log2 units), with c = sk_j * qsc
  // from one fp32 MFMA per tile (cscale) in the S^T register layout, M the running
  // maximum.  With QO the outlier products add So * qk_log2.
  float mrun = -INFINITY;
  float t[32];  // the current tile's exponent arguments (key j: see key_off())
  v8h pk[4];    // its probabilities, fp16, the P^T operand of P.V per key group
  // c_j = sk_j * qsc for the tile's 64 keys: v_mfma_f32_32x32x1_2b_f32 with lane l giving
  // the scale of key l (block l / 32, row l % 32) and its query's qsc (column l % 32), so
  // register 16 nb + i holds key 32 nb + 8 (i/4) + 4 hh + i%4, as the scores do.
  auto cscale = [&](float sk_lane) -> v32f { return MM::outer(sk_lane, qsc); };

  // Register i of the S^T block nb holds key 32 nb + 8 (i/4) + 4 hh + i%4 of the tile;
  // off(i) is that key relative to the tile's first key + 4 hh.
  auto key_off = [](int i) { return 32 * (i >> 4) + 8 * ((i >> 2) & 3) + (i & 3); };
  // M is raised (with a rescale of O and l, and the arguments t shifted) only where the
  // tile's largest argument mrel exceeds TAU.  Only register 0 of the row-sum
  // accumulator is read, so only it is rescaled.
  auto raise = [&](float mrel) {
    const bool upd = mrel > TAU;
    if (__any(upd)) {
      const float d = upd ? mrel : 0.0f;
      const float alpha = __builtin_amdgcn_exp2f(-d);
      mrun += d;
      lacc[0] *= alpha;
#pragma unroll
      for (int db = 0; db < NKB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) t[i] -= d;
    }
  };
  // p = 2^t rounded to fp16 for the 16 keys of group kg (P^T operand).
  auto expo = [&](int kg) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      v2f pp;
      pp[0] = __builtin_amdgcn_exp2f(t[8 * kg + e]);
      pp[1] = __builtin_amdgcn_exp2f(t[8 * kg + e + 1]);
      const v2h ph = __builtin_convertvector(pp, v2h);
      pk[kg][e] = ph[0];
      pk[kg][e + 1] = ph[1];
    }
  };
  // Row sum and P.V of key group kg.
  auto pv = [&](const char* st, int kg) {
    const v4i* vl = reinterpret_cast<const v4i*>(st + LY::KB);
    MM::template rowsum<true>(lacc, sel, pk[kg]);
#pragma unroll
    for (int db = 0; db < NKB; ++db) {
      const v4i va = vl[(kg * NKB + db) * 64 + lane];
      MM::template pv<true>(o[db], __builtin_bit_cast(v8h, va), pk[kg]);
    }
  };

  // One iteration as a fixed schedule of slots, one MFMA each, fenced with scheduling
  // barriers so the compiler keeps the order:
  //   MFMAs: the 2 NKB score products of the next tile (with QO its two outlier
  //          products), its key-scale product, then per key group kg the row sum and
  //          the NKB P.V products of this tile;
  //   LDS:   every MFMA operand is read PF slots ahead of its MFMA (a ring of PF + 1
  //          fragments), the next tile's key scales two slots ahead of their first use;
  //   VMEM:  this wave's share of the copy of a later tile, one instruction every few
  //          slots;
  //   VALU:  the exponentials of this tile (item i: FMA and exp2 of score i, the fp16
  //          pack after every odd i) over the slots before the third row-sum MFMA that
  //          needs them, the conversion of the next tile's scores (item i: cvt and one
  //          FMA against the key-scale product and the running max, with QO one more
  //          for the outlier product, with MASK the causal/tail select, a max3 after
  //          every odd i) from the slot its scores and the key-scale product are ready,
  //          and the row max exchange and rescale decision in the last slot.
  // Returns the next tile's row max in log2 units; upd_any: some row needs a rescale.
  auto pipe_step = [&](const char* cur, const char* nxt, const char* dsrc, char* dstage,
                       auto MASK, int last, bool& upd_any) -> float {
    constexpr bool masked = decltype(MASK)::value;
    constexpr int NQK = 2 * NKB;                // int8 score MFMAs
    constexpr int NSC = NQK + (QO ? 2 : 0);     // score MFMAs (QO: the outlier products)
    constexpr int XC = NSC;                     // the key-scale product c = sk * qsc
    constexpr int NPV = NSC + 1;                // first row-sum / P.V slot
    constexpr int NM = NPV + 4 * (NKB + 1);     // all MFMAs of the iteration
    constexpr int PF = 3;                       // operand prefetch distance, in MFMAs
    constexpr int E_END = NPV + 2 * (NKB + 1);  // exponentials end before row sum 2
    constexpr int C_BEG = NPV + 2;              // conversions start once c is in
    constexpr int C_END = NM - 2;               // the last two slots: the row max exchange
    constexpr int NC = C_END - C_BEG;
    const v4i* kl = reinterpret_cast<const v4i*>(nxt);
    const v4i* kol = reinterpret_cast<const v4i*>(nxt + LY::KO);
    const v4i* vl = reinterpret_cast<const v4i*>(cur + LY::KB);
    const float* skl = reinterpret_cast<const float*>(nxt + LY::KB + LY::VB);
    // Operand of MFMA slot x (the key-scale and row-sum MFMAs take none): K fragment
    // (nb, kb) for the score products, the outlier channels' K fragment of block nb, V
    // fragment (kg, db) for P.V.
    auto operand = [&](int x) -> v4i {
      if (x < NQK) return kl[((x / NKB) * NKB + x % NKB) * 64 + lane];
      if (x < NSC) return kol[(x - NQK) * 64 + lane];
      const int y = x - NPV, kg = y / (NKB + 1), db = y % (NKB + 1) - 1;
      return vl[(kg * NKB + db) * 64 + lane];
    };
    auto has_operand = [&](int x) {
      return x < NSC || (x >= NPV && (x - NPV) % (NKB + 1) != 0);
    };
    v16i sn[2];
    v16f so[2];
    v32f cn;          // c = sk * qsc of the next tile
    float skn = 0.0f;  // the next tile's key scale of key `lane`
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sn[nb][i] = 0;
    v4i fr[PF + 1];
    float p_even = 0.0f, cm0 = -INFINITY, cm1 = -INFINITY, mc_next = 0.0f;
#pragma unroll
    for (int x = 0; x < PF; ++x)
      if (has_operand(x)) fr[x % (PF + 1)] = operand(x);
#pragma clang loop unroll(full)
    for (int x = 0; x < NM; ++x) {
      // the MFMA of slot x
      if (x < NQK) {
        const int nb = x / NKB, kb = x % NKB;
        if (kb == 0)
          sn[nb] = MM::qk0(fr[x % (PF + 1)], qf[kb]);
        else
          MM::qk(sn[nb], fr[x % (PF + 1)], qf[kb]);
      } else if (x < NSC) {
        so[x - NQK] = MM::f16_0(__builtin_bit_cast(v8h, fr[x % (PF + 1)]), qo);
      } else if (x == XC) {
        cn = cscale(skn);
      } else {
        const int y = x - NPV, kg = y / (NKB + 1), db = y % (NKB + 1) - 1;
        if (db < 0)
          MM::rowsum(lacc, sel, pk[kg]);
        else
          MM::pv(o[db], __builtin_bit_cast(v8h, fr[x % (PF + 1)]), pk[kg]);
      }
      // operand PF slots ahead
      if (x + PF < NM && has_operand(x + PF)) fr[(x + PF) % (PF + 1)] = operand(x + PF);
      // the next tile's key scale of key `lane`, for its key-scale product
      if (x == (XC >= PF ? XC - PF : 0)) skn = skl[lane];
      // this wave's rounds of the copy: round r at slot 2 + r (NM - 4) / R
#pragma unroll
      for (int r = 0; r < DM::ROUNDS; ++r)
        if (x == 2 + (r * (NM - 4)) / DM::ROUNDS)
          copy_tile_round<D, NW, QO>(dsrc, dstage, tid, w, r);
      // exponentials of this tile: items [E(x), E(x + 1))
      if (x < E_END) {
        const int i0 = (32 * x) / E_END, i1 = (32 * (x + 1)) / E_END;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (i < i0 || i >= i1) continue;
          const float pi = __builtin_amdgcn_exp2f(t[i]);
          if (i & 1) {
            const v2f pp = {p_even, pi};
            const v2h ph = __builtin_convertvector(pp, v2h);
            pk[i >> 3][(i & 7) - 1] = ph[0];
            pk[i >> 3][i & 7] = ph[1];
          } else {
            p_even = pi;
          }
        }
      }
      if (x >= C_BEG && x < C_END) {
        // conversion of the next tile's scores: items [C(x), C(x + 1)); with products from
        // assembly, the key-scale product's and the scores' wait states first
        if (x == C_BEG) MM::settle_v3(cn, sn[0], sn[1]);
        const int c = x - C_BEG;
        const int i0 = (32 * c) / NC, i1 = (32 * (c + 1)) / NC;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (i < i0 || i >= i1) continue;
          const int nb = i >> 4;
          if constexpr (QO)
            t[i] = __builtin_fmaf((float)sn[nb][i & 15], cn[i],
                                  __builtin_fmaf(so[nb][i & 15], qk_log2, -mrun));
          else
            t[i] = __builtin_fmaf((float)sn[nb][i & 15], cn[i], -mrun);
          if (masked && key_off(i) > last) t[i] = -INFINITY;
          if (i & 1) {
            if (i & 2) cm1 = smax(smax(cm1, t[i - 1]), t[i]);
            else cm0 = smax(smax(cm0, t[i - 1]), t[i]);
          }
        }
      }
      // the row max of the next tile and the rescale decision, under the last MFMAs
      if (x == NM - 1) {
        mc_next = other_half_max(smax(cm0, cm1));
        upd_any = __any(mc_next > TAU);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return mc_next;
  };

  // Tile 0: its scores, converted and masked where needed, set M (key 0 is visible to
  // every row, so M is finite) and make the arguments relative to it.
  {
    const v4i* kl = reinterpret_cast<const v4i*>(smem);
    const float* skl = reinterpret_cast<const float*>(smem + LY::KB + LY::VB);
    v16i sc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      sc[nb] = MM::qk0(kl[(nb * NKB) * 64 + lane], qf[0]);
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb) MM::qk(sc[nb], kl[(nb * NKB + kb) * 64 + lane], qf[kb]);
    }
    v16f so0[2];
    if constexpr (QO) {
      const v4i* kol = reinterpret_cast<const v4i*>(smem + LY::KO);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        so0[nb] = MM::f16_0(__builtin_bit_cast(v8h, kol[nb * 64 + lane]), qo);
    }
    v32f c0 = cscale(skl[lane]);
    MM::settle_v3(c0, sc[0], sc[1]);
    const bool msk0 = needs_mask(0);
    const int last0 = last_key - 4 * hh;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float base = QO ? so0[i >> 4][i & 15] * qk_log2 : 0.0f;
      t[i] = __builtin_fmaf((float)sc[i >> 4][i & 15], c0[i], base);
      if (msk0 && key_off(i) > last0) t[i] = -INFINITY;
    }
    float m0 = smax(t[0], t[1]), m1 = smax(t[2], t[3]);
#pragma unroll
    for (int i = 4; i < 32; i += 4) {
      m0 = smax(smax(m0, t[i]), t[i + 1]);
      m1 = smax(smax(m1, t[i + 2]), t[i + 3]);
    }
    mrun = other_half_max(smax(m0, m1));
#pragma unroll
    for (int i = 0; i < 32; ++i) t[i] -= mrun;
  }

  // Tiles 0 .. nt-2: tile j's exponentials and P.V beside tile j+1's scores.  The copy
  // of tile j + NS - 1 goes into the stage tile j - 1 left; without such a tile the
  // step copies tile j again into that stage, which no later tile uses (the remaining
  // ones need fewer than NS stages), so the step has no branch.  A wave whose
  // remaining rows see none of tile j+1 (the causal diagonal of the rows below it)
  // masks all of its scores, and its probabilities are 0.
  int scur = 0;  // stage of tile j
  int j = 0;
  // One iteration; the two loops below differ only in the mask of the next tile's
  // scores (a wave's masked tiles all come after its unmasked ones).  Every wave runs
  // nt - 1 iterations, each ending with the one barrier.
  auto iterate = [&](auto MASK) {
    const int snxt = scur == NS - 1 ? 0 : scur + 1;
    const char* cur = smem + scur * LY::STAGE;
    const char* nxt = smem + snxt * LY::STAGE;
    const char* dsrc = tsrc + (int64_t)(j + NS - 1 < nt ? j + NS - 1 : j) * LY::STAGE;
    char* dst = smem + (scur == 0 ? NS - 1 : scur - 1) * LY::STAGE;
    bool upd_any;
    const float mc = pipe_step(cur, nxt, dsrc, dst, MASK, last_key - (j + 1) * TK - 4 * hh, upd_any);
    // With products from assembly: the wait states of the step's last P.V products before
    // anything (the rescale, or a register copy the compiler places between the loops)
    // reads the accumulators.
    MM::settle_acc(o, lacc);
    if (upd_any) raise(mc);
    // Tile j + 2 must have landed; the copy issued in this step may run on when it is
    // for a later tile.
    vm_wait<NS >= 4 ? DM::ROUNDS : 0>();
    __syncthreads();
    scur = snxt;
  };
  for (; j < jv && !needs_mask(j + 1); ++j) iterate(std::false_type{});
  for (; j < jv; ++j) iterate(std::true_type{});
  // The wave's last visible tile: its exponentials and P.V.
  {
    const char* cur = smem + scur * LY::STAGE;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) expo(kg);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) pv(cur, kg);
  }
  // Tiles past the wave's diagonal (causal): only its share of the copies and the
  // barriers, so the other waves of the workgroup get their tiles.
  for (; j + 1 < nt; ++j) {
    if (j + NS - 1 < nt) {
      const int st = scur == 0 ? NS - 1 : scur - 1;
      copy_tile_dma<D, NW, QO>(tsrc + (int64_t)(j + NS - 1) * LY::STAGE, smem + st * LY::STAGE, tid,
                           w);
    }
    vm_wait<0>();
    __syncthreads();
    scur = scur == NS - 1 ? 0 : scur + 1;
  }
  // No copy outlives the workgroup (the last steps' copies go to stages no tile uses).
  vm_wait<0>();

  char* area;
  if constexpr (EPI_IN_RING) {
    // Every wave's copies have landed (the wait above) and, past this barrier, every
    // wave's P.V is done, so no stage is read any more; each wave takes its part of it.
    __syncthreads();
    area = smem + w * 32 * EPITCH;
  } else {
    area = smem + NS * LY::STAGE + w * 32 * EPITCH;
  }
  MM::settle_acc(o, lacc);
  store_rows<D, EC>(o, qi < L ? 1.0f / lacc[0] : 0.0f, area, out, aq, start, h, qw0, L, lane);
}

// ----------------------------------------------------------------------------------
// Debug: the int32 score tile from the forward's own prepared Q and K fragments
// (read straight from the workspace), one wave per aligned 32x32 block of sequence s
// and query head h, with the scales, the K mean and the prepared V rows of the same
// rows and keys.  Entries past the sequence's length are not written.
template <int D>
__global__ __launch_bounds__(64) void debug_qk_kernel(
    const int8_t* __restrict__ q8, const float* __restrict__ qs, int64_t Qpad, Seqs seqs,
    int Hq, int Hkv, int s, int h, int row0, int rows, int col0, int cols,
    const char* __restrict__ tiles, const float* __restrict__ sv_ws,
    const float* __restrict__ svc_ws, const float* __restrict__ kmean_ws, int64_t Ppad,
    int tstride, const int32_t* __restrict__ ochan_ws, DebugOut o) {
  constexpr int NKB = D / 32;
  const int lane = threadIdx.x, m = lane & 31, hh = lane >> 5;
  const int qbase = (row0 & ~31) + 32 * blockIdx.x;
  const int kbase = (col0 & ~31) + 32 * blockIdx.y;
  int64_t start;
  int L;
  seqs.bounds(s, start, L);
  // A block wholly past the sequence's end reads nothing (its slots may belong to the
  // next sequence or lie past the workspace's Q rows).
  if (qbase >= L || kbase >= L) return;
  const int g = h / (Hq / Hkv);
  const int64_t pbase = Seqs::pstart(s, start);
  const int64_t qslot = (int64_t)h * Qpad + Seqs::qpstart(s, start) + qbase;

  v4i qf[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) qf[kb] = reinterpret_cast<const v4i*>(q8 + qslot * D)[kb * 64 + lane];

  const int tile0 = kbase - kbase % TK, nb = (kbase % TK) / 32;
  const char* tb = tiles + ((int64_t)g * (Ppad / TK) + (pbase + tile0) / TK) * tstride;
  const v4i* kt = reinterpret_cast<const v4i*>(tb);
  v16i acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kt[(nb * NKB + kb) * 64 + lane], qf[kb], acc, 0,
                                                0, 0);
  const int qrow = qbase + m;
  const bool qin = qrow >= row0 && qrow < row0 + rows && qrow < L;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int n = kbase + 8 * (i >> 2) + 4 * hh + (i & 3);
    if (qin && n >= col0 && n < col0 + cols && n < L)
      o.s32[(int64_t)(qrow - row0) * o.cols + (n - col0)] = acc[i];
  }
  if (o.qscale && blockIdx.y == 0 && hh == 0 && qin) o.qscale[qrow - row0] = qs[qslot + m];
  const int n = kbase + m;
  const bool kin = n >= col0 && n < col0 + cols && n < L;
  if (blockIdx.x == 0 && hh == 0 && kin) {
    if (o.kscale) o.kscale[n - col0] = reinterpret_cast<const float*>(tb + 3 * TK * D)[n - tile0];
    if (o.vscale) o.vscale[n - col0] = sv_ws[(int64_t)g * Ppad + pbase + n];
  }
  // The prepared V rows of this block's keys, from the tile's V fragments.
  if (o.vhat && blockIdx.x == 0) {
    const _Float16* vt = reinterpret_cast<const _Float16*>(tb + TK * D);
    for (int idx = lane; idx < 32 * D; idx += 64) {
      const int nl = idx / D, d = idx % D, nk = kbase + nl;
      if (nk >= col0 && nk < col0 + cols && nk < L)
        o.vhat[(int64_t)(nk - col0) * D + d] = vt[vtile_off(nk - tile0, d, D)];
    }
  }
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int d = lane; d < D; d += 64) {
      if (o.kmean) o.kmean[d] = kmean_ws[((int64_t)s * Hkv + g) * D + d];
      if (o.vchan) o.vchan[d] = svc_ws[((int64_t)s * Hkv + g) * D + d];
    }
    if (o.ochan && lane < QO_MAX) o.ochan[lane] = ochan_ws[((int64_t)s * Hkv + g) * QO_MAX + lane];
  }
}

// ----------------------------------------------------------------------------------
static Act act_of(const FwdGeom& g, int H) {
  Act a;
  a.seq_unit = (int64_t)H * g.D;
  if (g.cu) {
    a.head_stride = g.D;
    a.tok_stride = (int64_t)H * g.D;
  } else {
    a.head_stride = (int64_t)g.S * g.D;
    a.tok_stride = g.D;
  }
  return a;
}

template <int D, bool C>
static hipError_t attn_d(const FwdGeom& g, const WsPlan& p, const void* ws, hipStream_t stream) {
  const char* w = static_cast<const char*>(ws);
  // Waves per workgroup of the pipelined kernel.  At D <= 64 a step has little MFMA work
  // beside the fixed cost of its barrier and copy wait, and a wave's registers leave room
  // for three workgroups of four waves per CU, which hide each other's barriers
  // (B4 H16 S2048 non-causal: D = 32 64.8 -> 57.5 us, D = 64 76.6 -> 75.2 us against
  // eight waves; D = 64 74.6 against 77.5 us at three workgroups per CU against two).  At D = 128 eight waves in one workgroup share every tile copy and LDS
  // stage.  At D = 256 a wave needs more than half of a SIMD's registers (the 128
  // accumulator registers of O and both tiles' state), so four waves, one per SIMD.
  constexpr int NW = (D <= 64 || D > 128) ? 4 : 8;
  const int bm = 32 * NW;
  const int nqt = (g.max_len + bm - 1) / bm;
  const int64_t blocks = (int64_t)nqt * g.nseq * g.Hq;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int ngroups = g.nseq * g.Hkv;
  const int xcd_map = ((g.nseq * g.Hq) % 8 == 0 && ngroups % 8 == 0) ? 1 : 0;
  // Rotated Q and K rows carry H H^T = D I: an extra exact factor 1/D on the logits.
  const float qk_log2 = g.softmax_scale * 1.4426950408889634f * (g.rot ? 1.0f / g.D : 1.0f);
  Seqs sq{g.cu, g.S, g.max_len, g.T};
  using Kern = decltype(&attn_pipe_kernel<D, C, NW, false, false>);
  Kern kern;
  if constexpr (D <= 128) {
    if (g.qout && !g.fuse_q) return hipErrorInvalidValue;
    kern = g.qout     ? attn_pipe_kernel<D, C, NW, true, true>
           : g.fuse_q ? attn_pipe_kernel<D, C, NW, true, false>
                      : attn_pipe_kernel<D, C, NW, false, false>;
  } else {
    if (g.qout) return hipErrorInvalidValue;
    kern = g.fuse_q ? attn_pipe_kernel<D, C, NW, true, false> : attn_pipe_kernel<D, C, NW, false, false>;
  }
  kern<<<dim3((unsigned)blocks), dim3(64 * NW), 0, stream>>>(
      reinterpret_cast<const int8_t*>(w + p.off_q8), reinterpret_cast<const float*>(w + p.off_qs),
      p.Qpad, static_cast<const _Float16*>(g.q), g.qblk | (g.rot ? 2 : 0),
      static_cast<_Float16*>(g.out),
      act_of(g, g.Hq), sq, g.Hq, g.Hkv, g.nseq, xcd_map, qk_log2, w + p.off_tiles, p.Ppad,
      reinterpret_cast<const int32_t*>(w + p.off_ochan));
  return hipGetLastError();
}

hipError_t launch_attn(const FwdGeom& g, const WsPlan& p, const void* ws, hipStream_t stream) {
#define I8A_ATT(DD)                                            \
  case DD:                                                     \
    return g.causal ? attn_d<DD, true>(g, p, ws, stream)       \
                    : attn_d<DD, false>(g, p, ws, stream);
  switch (g.D) {
    I8A_ATT(32) I8A_ATT(64) I8A_ATT(128) I8A_ATT(256)
    default:
      return hipErrorInvalidValue;
  }
#undef I8A_ATT
}

template <int D>
static hipError_t debug_d(const FwdGeom& g, const WsPlan& p, const void* ws, int s, int h,
                          int row0, int rows, int col0, int cols, const DebugOut& o,
                          hipStream_t stream) {
  const char* w = static_cast<const char*>(ws);
  const int rb = ((row0 + rows - 1) >> 5) - (row0 >> 5) + 1;
  const int cb = ((col0 + cols - 1) >> 5) - (col0 >> 5) + 1;
  Seqs sq{g.cu, g.S, g.max_len, g.T};
  debug_qk_kernel<D><<<dim3(rb, cb), dim3(64), 0, stream>>>(
      reinterpret_cast<const int8_t*>(w + p.off_q8), reinterpret_cast<const float*>(w + p.off_qs),
      p.Qpad, sq, g.Hq, g.Hkv, s, h, row0, rows, col0, cols, w + p.off_tiles,
      reinterpret_cast<const float*>(w + p.off_sv), reinterpret_cast<const float*>(w + p.off_svc),
      reinterpret_cast<const float*>(w + p.off_kmean), p.Ppad, tile_bytes(D, g.qout != 0),
      reinterpret_cast<const int32_t*>(w + p.off_ochan), o);
  return hipGetLastError();
}

hipError_t launch_debug_qk(const FwdGeom& g, const WsPlan& p, const void* ws, int32_t s,
                           int32_t h, int32_t row0, int32_t rows, int32_t col0, int32_t cols,
                           const DebugOut& o, hipStream_t stream) {
  switch (g.D) {
    case 32: return debug_d<32>(g, p, ws, s, h, row0, rows, col0, cols, o, stream);
    case 64: return debug_d<64>(g, p, ws, s, h, row0, rows, col0, cols, o, stream);
    case 128: return debug_d<128>(g, p, ws, s, h, row0, rows, col0, cols, o, stream);
    case 256: return debug_d<256>(g, p, ws, s, h, row0, rows, col0, cols, o, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace i8a
