// i8a_device.h - device-side types, layouts and quantization steps shared by the
// kernels of the INT8 W8A8 attention forward (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "i8a_launch.h"

namespace i8a {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));


// Where the tokens of sequence s live.  Dense batches are the special case
// cu == nullptr, start(s) = s * S, len(s) = S.  Sequences whose bounds are not
// inside [0, T] or exceed max_len read as empty, so a malformed cu_seqlens can
// never send a kernel out of bounds.
struct Seqs {
  const int32_t* cu;
  int32_t S;        // dense length
  int32_t max_len;  // longest sequence allowed
  int64_t T;        // total tokens
  __device__ __forceinline__ void bounds(int s, int64_t& start, int& len) const {
    if (!cu) {
      start = (int64_t)s * S;
      len = S;
      return;
    }
    const int64_t a = cu[s], b = cu[s + 1];
    if (a < 0 || b < a || b > T || b - a > max_len) {
      start = 0;
      len = 0;
      return;
    }
    start = a;
    len = (int)(b - a);
  }
  // First padded workspace slot of sequence s: sequences are laid out back to back,
  // each starting on a TK boundary, in Hkv * Ppad slots per tensor.
  static __device__ __forceinline__ int64_t pstart(int s, int64_t start) {
    return (int64_t)TK * (start / TK + s);
  }
  // The same for the Q slots, padded to BQ rows: the BQ-row query tiles of one
  // sequence never reach into the next one's slots.
  static __device__ __forceinline__ int64_t qpstart(int s, int64_t start) {
    return (int64_t)BQ * (start / BQ + s);
  }
};

// Element offset of token t of head h of sequence s in an fp16 activation tensor:
// dense [B, H, S, D] has head_stride = S*D, tok_stride = D; packed [T, H, D] has
// head_stride = D, tok_stride = H*D; in both the sequence starts at start*H*D.
struct Act {
  int64_t head_stride, tok_stride, seq_unit;  // seq_unit = H * D
  __device__ __forceinline__ int64_t off(int64_t start, int h, int64_t t) const {
    return start * seq_unit + (int64_t)h * head_stride + t * tok_stride;
  }
};

// ---------------------------------------------------------------------------------
// Direct-to-LDS copies.
//
// One 16-byte-per-lane load from global memory straight into LDS: lane l's 16 bytes at
// gptr land at LDS byte lds_base + 16 l (lds_base is made wave-uniform; it goes to M0,
// and one wait state separates the M0 write from the load).  It is issued through
// inline assembly so that the compiler does not track it: the compiler's own
// bookkeeping of direct-to-LDS loads makes every later LDS read wait until all of them
// have landed, which would stall each tile's compute on the prefetch of the next one.
// Callers wait for their copies themselves with vm_wait<N>.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}
// M0 is a reserved register to the compiler; nothing else in these kernels uses it
// (their code reads M0 only in these loads), so clobbering it here is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
#pragma clang diagnostic pop
// Wait until at most N vector-memory loads of this wave are outstanding (they complete
// in issue order).  The memory clobber keeps every LDS read of the copied data after it.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// ---------------------------------------------------------------------------------
// Quantization steps (the row rule of the Quantization table's "Per-row int8" row).

// Scale of a row with absolute maximum `amax`: fp32(amax / 127), and for V rows that
// value rounded up to a `bits`-bit significand (bits < 24).  amax / 127.0f is the
// correctly rounded IEEE division (HIP's default for fp32 '/').
__device__ __forceinline__ float row_scale(float amax, int bits) {
  float t = amax / 127.0f;
  if (bits < 24) {
    const uint32_t drop = 24u - (uint32_t)bits;
    const uint32_t lo = (1u << drop) - 1u;
    t = __uint_as_float((__float_as_uint(t) + lo) & ~lo);
  }
  return t;
}

// Symmetric int8 code of x for a row scale s: rint(x / s), with the correctly rounded
// fp32 quotient and round-half-to-even; a zero scale gives 0.  No clamp is needed:
// the scale is RN(amax / 127) (or that rounded up), so |x| / s <= 127 (1 + 2^-23) and
// the rounded quotient never reaches 127.5.
// `y` is the row's correctly rounded reciprocal RN(1/s) (0 when s == 0): with it the
// quotient RN(x/s) is q0 = RN(x*y) corrected once by the exact remainder
// r = x - s*q0 (an FMA), q = RN(q0 + r*y) -- the FMA division step of Markstein,
// exact for every quotient here (no overflow or underflow occurs in it).
struct RowQ {
  float s, y;
  __device__ __forceinline__ explicit RowQ(float scale)
      : s(scale), y(scale == 0.0f ? 0.0f : 1.0f / scale) {}
  // The corrected quotient RN(x/s) (before rounding to an integer).
  __device__ __forceinline__ float quot(float x) const {
    const float q0 = __fmul_rn(x, y);
    const float r = __builtin_fmaf(-q0, s, x);
    return __builtin_fmaf(r, y, q0);
  }
  __device__ __forceinline__ float code(float x) const { return __builtin_rintf(quot(x)); }
  // The code as the low byte of a float's bits: q + 1.5 * 2^23 is rounded to an integer
  // by the add itself (round to nearest, ties to even, as rint) for |q| < 2^22, and its
  // bits are 0x4B400000 plus that integer, whose low byte is the code's two's
  // complement byte.
  static __device__ __forceinline__ uint32_t code_bits(float q) {
    return __float_as_uint(q + 12582912.0f);
  }
  // Four codes' low bytes packed little-endian into one dword (v_perm_b32: selector
  // bytes 0-3 pick the second source's bytes, 4-7 the first's, 0x0c a zero byte).
  static __device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2,
                                                   uint32_t b3) {
    const uint32_t p01 = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
  }
  // Eight codes packed little-endian into two dwords (two's complement bytes).
  __device__ __forceinline__ uint2 pack8(const float (&x)[8]) const {
    uint32_t b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = code_bits(quot(x[j]));
    return make_uint2(pack4(b[0], b[1], b[2], b[3]), pack4(b[4], b[5], b[6], b[7]));
  }
  // The same from fp16 values (converted exactly to fp32 inside the arithmetic).
  __device__ __forceinline__ uint2 pack8h(const v8h& x) const {
    uint32_t b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = code_bits(quot((float)x[j]));
    return make_uint2(pack4(b[0], b[1], b[2], b[3]), pack4(b[4], b[5], b[6], b[7]));
  }
};

// Largest |x| of eight fp16 values, as fp32: with the sign bits cleared, fp16 bit
// patterns order like their values (finite inputs), so a packed unsigned max of the
// 16-bit halves finds it.
__device__ __forceinline__ uint32_t absmax_bits8(const v8h& x, uint32_t acc) {
  typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
  const uint4 w = __builtin_bit_cast(uint4, x);
  v2u16 m = __builtin_bit_cast(v2u16, acc);
  m = __builtin_elementwise_max(m, __builtin_bit_cast(v2u16, w.x & 0x7fff7fffu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(v2u16, w.y & 0x7fff7fffu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(v2u16, w.z & 0x7fff7fffu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(v2u16, w.w & 0x7fff7fffu));
  return __builtin_bit_cast(uint32_t, m);
}
__device__ __forceinline__ float absmax_of_bits(uint32_t acc) {
  const uint32_t lo = acc & 0xffffu, hi = acc >> 16;
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(lo > hi ? lo : hi));
}

// A lane permutation through DPP (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_perm(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over groups of G consecutive lanes (G a power of two <= 64), all lanes active.
// Within 16-lane rows DPP does it: quad_perm [1,0,3,2] and [2,3,0,1] leave the quad
// max in every lane of a quad; row_half_mirror (lane i <- 7 - i) then pairs the two
// quads of each 8 lanes, and row_mirror (lane i <- 15 - i) the two halves of a row.
// Wider groups finish with cross-row shuffles.
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (G >= 2) v = fmaxf(v, dpp_perm<0xB1>(v));
  if constexpr (G >= 4) v = fmaxf(v, dpp_perm<0x4E>(v));
  if constexpr (G >= 8) v = fmaxf(v, dpp_perm<0x141>(v));
  if constexpr (G >= 16) v = fmaxf(v, dpp_perm<0x140>(v));
  if constexpr (G >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if constexpr (G >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Unnormalized fast Walsh-Hadamard transform of one D-channel row (the Quantization
// table's Hadamard rotation) held by G = D/8 consecutive lanes, lane lc holding
// channels 8 lc .. 8 lc + 7, in fp32, with the stages in the order s = 0, 1, ...,
// log2(D) - 1: the pair (x[i], x[i + 2^s]) with bit s of i clear becomes
// (x[i] + x[i + 2^s], x[i] - x[i + 2^s]).  Stages 0-2 pair values inside a lane, the
// later ones lane lc with lane lc ^ 2^(s-3).  Every lane of the group takes part.
template <int G>
__device__ __forceinline__ void fwht_row(float (&x)[8], int lc) {
#pragma unroll
  for (int h = 1; h < 8; h *= 2)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (!(j & h)) {
        const float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
#pragma unroll
  for (int m = 1; m < G; m *= 2) {
    const bool hi = (lc & m) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __shfl_xor(x[j], m, 64);
      x[j] = hi ? p - x[j] : x[j] + p;
    }
  }
}

// fp16 load of 8 consecutive values as fp32.
__device__ __forceinline__ void load8_f32(const _Float16* p, float (&x)[8]) {
  const v8h h = *reinterpret_cast<const v8h*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)h[j];
}

// An exact sum of at most 8 fp16 values (a double) times 2^24 as an integer.  Every fp16
// number is a multiple of 2^-24 below 2^16 in magnitude, so such a sum, accumulated in
// fp64 in any order, is exact (it needs at most 43 of the 53 significand bits), and
// y = sum * 2^24 is an integer with |y| < 2^43: it is split as floor(y / 2^32) (a small
// signed integer) and the remainder in [0, 2^32), both converted exactly.
__device__ __forceinline__ int64_t fixed24_of_sum8(double sum) {
  const double y = sum * 0x1p24;
  const double hi = __builtin_floor(y * 0x1p-32);
  const double lo = y - hi * 0x1p32;
  return (int64_t)((uint64_t)(int64_t)(int32_t)hi << 32) + (int64_t)(uint32_t)lo;
}

// The K-smoothing mean of one (sequence, kv head) from its np <= MAX_PARTS launch-1
// partial sums pp[np][D] (int64, units of 2^-24): the integer total divided in fp64 by
// L * 2^24 and rounded to fp32 (integer sums, so every workgroup that reduces them gets
// the same mean), written to mean (shared) and, if given, kmean_out.  Every thread
// issues all its loads of the partials at once, 16 bytes (two channels) each, so the
// reduction costs about one memory latency rather than one per few partials.  red is
// 512 int64 of shared memory; all 256 threads of the workgroup must call it.
template <int D>
__device__ __forceinline__ void reduce_kmean(const int64_t* __restrict__ pp, int np, int L,
                                             int64_t* red, float* mean,
                                             float* __restrict__ kmean_out) {
  typedef long long v2l __attribute__((ext_vector_type(2)));
  constexpr int NPAIR = D / 2;                       // channel pairs
  constexpr int TPP = 256 / NPAIR;                   // threads per pair
  constexpr int MAXK = (MAX_PARTS + TPP - 1) / TPP;  // partials per thread, at most
  constexpr int CH = MAXK < 16 ? MAXK : 16;          // loads in flight per round
  const int cp = threadIdx.x % NPAIR, r = threadIdx.x / NPAIR;
  const v2l* src = reinterpret_cast<const v2l*>(pp) + cp;
  v2l acc = {0, 0};
#pragma unroll
  for (int k0 = 0; k0 < MAXK; k0 += CH) {
    v2l v[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int i = r + (k0 + k) * TPP;
      v[k] = i < np ? src[(int64_t)i * NPAIR] : v2l{0, 0};
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) acc += v[k];
  }
  red[2 * threadIdx.x] = acc.x;
  red[2 * threadIdx.x + 1] = acc.y;
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    int64_t tot = 0;
    for (int k = 0; k < TPP; ++k) tot += red[2 * (k * NPAIR + d / 2) + (d & 1)];
    const float mu = (float)((double)tot / ((double)L * 16777216.0));
    mean[d] = mu;
    if (kmean_out) kmean_out[d] = mu;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------
// MFMA operand layouts (v_mfma_i32_32x32x32_i8 and v_mfma_f32_32x32x16_f16).
//
// For a 32x32 MFMA, lane l supplies row (l % 32) of A and column (l % 32) of B for
// the k-slice numbered l / 32; the result lane l holds column l % 32 and rows
// 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.  The kernels compute the transposed
// products S^T = K . Q^T and O^T = V^T . P^T so that a lane's result registers all
// belong to one query (column l % 32): the row statistics of the softmax stay in
// the lane, and the S^T registers become the P^T operand of the next MFMA as they
// are.
//
// K tile (TK keys x D int8), A operand of S^T: 16-byte fragments ordered
//   [key block nb = n/32][d block kb = d/32][lane = n%32 + 32*((d%32)/16)][d%16].
// V tile (TK keys x D fp16), A operand of O^T: 16-byte fragments ordered
//   [key group kg = n/16][d block db = d/32][lane = d%32 + 32*hv][jv]
// where a key n (nl = n % 16) sits at hv = (nl % 8) / 4, jv = 4*(nl / 8) + nl % 4,
// the order in which the S^T result registers hold keys.
// Q (B operand of S^T): lane l holds query l % 32, bytes d = 32*kb + 16*(l/32) + j.

__device__ __forceinline__ int ktile_off(int n, int d, int D) {  // byte offset in tile
  const int nb = n >> 5, nl = n & 31, kb = d >> 5, hh = (d & 31) >> 4, j = d & 15;
  return ((nb * (D >> 5) + kb) * 64 + nl + 32 * hh) * 16 + j;
}

__device__ __forceinline__ int vtile_off(int n, int d, int D) {  // element offset in tile
  const int kg = n >> 4, nl = n & 15, hv = (nl & 7) >> 2, jv = ((nl >> 3) << 2) + (nl & 3);
  const int db = d >> 5, dl = d & 31;
  return ((kg * (D >> 5) + db) * 64 + dl + 32 * hv) * 8 + jv;
}

__device__ __forceinline__ int qfrag_off(int m, int d) {  // byte offset, 32 rows
  const int kb = d >> 5, hh = (d & 31) >> 4, j = d & 15;
  return (kb * 64 + m + 32 * hh) * 16 + j;
}

}  // namespace i8a
