// quant_kernels.hip - row quantization and the K/V preparation of the forward.
//
// All three kernels are HBM-bound streaming passes: rows are read once with 16-byte
// coalesced loads, one row per group of D/8 lanes, and the row absolute maximum is a
// butterfly reduction inside that lane group.
#include "i8a_device.h"
#include "i8a_launch.h"

namespace i8a {

// ----------------------------------------------------------------------------------
// Public row quantizer (Supporting kernels table, row quant_rowwise).  G lanes per row
// (G = next power of two >= d/8); lanes beyond d/8 only join the reduction.
template <int G>
__global__ __launch_bounds__(256) void quant_rowwise_kernel(
    const _Float16* __restrict__ x, int64_t rows, int d, const float* __restrict__ sub_mean,
    int64_t rows_per_group, int scale_bits, int8_t* __restrict__ codes,
    float* __restrict__ scales) {
  constexpr int RPB = 256 / G;  // rows per block pass
  const int c = threadIdx.x % G;
  const int rsub = threadIdx.x / G;
  const bool active = c * 8 < d;
  for (int64_t r = (int64_t)blockIdx.x * RPB + rsub; r - rsub < rows;
       r += (int64_t)gridDim.x * RPB) {
    const bool live = active && r < rows;
    float v[8];
    float amax = 0.0f;
    if (live) {
      load8_f32(x + r * d + c * 8, v);
      if (sub_mean) {
        const float* m = sub_mean + (r / rows_per_group) * d + c * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = v[j] - m[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    }
    amax = group_max<G>(amax);
    const float s = row_scale(amax, scale_bits);
    if (live) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) lo |= ((uint32_t)quant_code(v[j], s) & 255u) << (8 * j);
#pragma unroll
      for (int j = 0; j < 4; ++j) hi |= ((uint32_t)quant_code(v[4 + j], s) & 255u) << (8 * j);
      *reinterpret_cast<uint2*>(codes + r * d + c * 8) = make_uint2(lo, hi);
      if (c == 0) scales[r] = s;
    }
  }
}

// ----------------------------------------------------------------------------------
// Stage 1 of the preparation, one workgroup per (chunk of CH tokens, kv head,
// sequence): exact per-channel partial sums of K over the chunk's tokens (the
// K-smoothing statistic), and V quantized per token with its 4-bit scale, written as
// the exact fp16 values sv * code in the V tile layout.  Slots between the sequence
// end and its last tile boundary get V = 0 and sv = 0.
template <int D>
__global__ __launch_bounds__(256) void prep_stage1_kernel(
    const _Float16* __restrict__ k, const _Float16* __restrict__ v, Act act, Seqs seqs, int Hkv,
    int nch, int64_t Ppad, int64_t* __restrict__ kpart, float* __restrict__ sv_ws,
    _Float16* __restrict__ vh_ws) {
  constexpr int G = D / 8;       // lanes per row
  constexpr int RPP = 256 / G;   // rows per pass
  __shared__ int64_t red[RPP * D];
  __shared__ __attribute__((aligned(16))) _Float16 vt[TK * D];

  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  int64_t start;
  int L;
  seqs.bounds(s, start, L);
  const int t0 = c * CH;
  if (t0 >= L) return;
  const int t_real = min(L, t0 + CH);
  const int t_pad = min(((L + TK - 1) / TK) * TK, t0 + CH);
  const int64_t pbase = Seqs::pstart(s, start);
  const int lc = threadIdx.x % G, rsub = threadIdx.x / G;

  // K partial sums over this chunk (exact int64 fixed point).
  int64_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0;
  for (int t = t0 + rsub; t < t_real; t += RPP) {
    const v8h kv = *reinterpret_cast<const v8h*>(k + act.off(start, g, t) + lc * 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += fp16_fixed24(kv[j]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rsub * D + lc * 8 + j] = acc[j];
  __syncthreads();
  if (threadIdx.x < D) {
    int64_t tot = 0;
    for (int r = 0; r < RPP; ++r) tot += red[r * D + threadIdx.x];
    kpart[(((int64_t)s * Hkv + g) * nch + c) * D + threadIdx.x] = tot;
  }

  // V rows, one TK-token tile at a time through LDS into the fragment layout.
  for (int tt = t0; tt < t_pad; tt += TK) {
    for (int n = rsub; n < TK; n += RPP) {
      const int t = tt + n;
      float x[8];
      float amax = 0.0f;
      const bool real = t < L;
      if (real) {
        load8_f32(v + act.off(start, g, t) + lc * 8, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
      }
      amax = group_max<G>(amax);
      const float sv = real ? row_scale(amax, 4) : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // sv has a 4-bit significand and |code| <= 127, so the product is exact in
        // fp32 and in fp16.
        const float vh = real ? sv * (float)quant_code(x[j], sv) : 0.0f;
        vt[vtile_off(n, lc * 8 + j, D)] = (_Float16)vh;
      }
      if (lc == 0) sv_ws[(int64_t)g * Ppad + pbase + t] = sv;
    }
    __syncthreads();
    _Float16* dst = vh_ws + ((int64_t)g * Ppad + pbase + tt) * D;
    for (int i = threadIdx.x; i < TK * D / 8; i += 256)
      reinterpret_cast<v8h*>(dst)[i] = reinterpret_cast<const v8h*>(vt)[i];
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------------
// Stage 2, same grid: the K mean of the sequence (sum of the stage-1 partials, fp64
// divide, fp32), then K rows quantized from fp32(k) - mean into the K tile layout.
template <int D>
__global__ __launch_bounds__(256) void prep_stage2_kernel(
    const _Float16* __restrict__ k, Act act, Seqs seqs, int Hkv, int nch, int64_t Ppad,
    const int64_t* __restrict__ kpart, float* __restrict__ kmean_ws, float* __restrict__ sk_ws,
    int8_t* __restrict__ k8_ws) {
  constexpr int G = D / 8;
  constexpr int RPP = 256 / G;
  __shared__ float mean[D];

  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  int64_t start;
  int L;
  seqs.bounds(s, start, L);
  const int t0 = c * CH;
  if (t0 >= L) return;
  const int t_pad = min(((L + TK - 1) / TK) * TK, t0 + CH);
  const int64_t pbase = Seqs::pstart(s, start);
  const int lc = threadIdx.x % G, rsub = threadIdx.x / G;

  if (threadIdx.x < D) {
    const int nc = (L + CH - 1) / CH;
    const int64_t* pp = kpart + ((int64_t)s * Hkv + g) * nch * D + threadIdx.x;
    int64_t tot = 0;
    for (int i = 0; i < nc; ++i) tot += pp[(int64_t)i * D];
    const float m = (float)((double)tot / ((double)L * 16777216.0));
    mean[threadIdx.x] = m;
    if (c == 0) kmean_ws[((int64_t)s * Hkv + g) * D + threadIdx.x] = m;
  }
  __syncthreads();

  float mu[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mu[j] = mean[lc * 8 + j];
  for (int t = t0 + rsub; t < t_pad; t += RPP) {
    const bool real = t < L;
    float x[8];
    float amax = 0.0f;
    if (real) {
      load8_f32(k + act.off(start, g, t) + lc * 8, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = x[j] - mu[j];
        amax = fmaxf(amax, fabsf(x[j]));
      }
    }
    amax = group_max<G>(amax);
    const float sk = real ? row_scale(amax, 24) : 0.0f;
    uint32_t lo = 0, hi = 0;
    if (real) {
#pragma unroll
      for (int j = 0; j < 4; ++j) lo |= ((uint32_t)quant_code(x[j], sk) & 255u) << (8 * j);
#pragma unroll
      for (int j = 0; j < 4; ++j) hi |= ((uint32_t)quant_code(x[4 + j], sk) & 255u) << (8 * j);
    }
    const int n = t % TK;
    int8_t* tile = k8_ws + ((int64_t)g * Ppad + pbase + (t - n)) * D;
    *reinterpret_cast<uint2*>(tile + ktile_off(n, lc * 8, D)) = make_uint2(lo, hi);
    if (lc == 0) sk_ws[(int64_t)g * Ppad + pbase + t] = sk;
  }
}

// ----------------------------------------------------------------------------------
hipError_t launch_quant_rowwise(const void* x, int64_t rows, int32_t d, const float* sub_mean,
                                int64_t rows_per_group, int32_t scale_bits, int8_t* codes,
                                float* scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  int g = 1;
  while (g * 8 < d) g *= 2;
  const int rpb = 256 / g;
  int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks > 65536) blocks = 65536;
  const _Float16* xp = static_cast<const _Float16*>(x);
#define I8A_QR(GG)                                                                       \
  case GG:                                                                               \
    quant_rowwise_kernel<GG><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(          \
        xp, rows, d, sub_mean, rows_per_group, scale_bits, codes, scales);               \
    break;
  switch (g) {
    I8A_QR(1) I8A_QR(2) I8A_QR(4) I8A_QR(8) I8A_QR(16) I8A_QR(32) I8A_QR(64)
    default:
      return hipErrorInvalidValue;
  }
#undef I8A_QR
  return hipGetLastError();
}

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

template <int D>
static hipError_t prep_d(const FwdGeom& g, const WsPlan& p, void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  const Act ak = act_of(g, g.Hkv);
  Seqs sq{g.cu, g.S, g.max_len, g.T};
  const dim3 grid(p.nch, g.Hkv, g.nseq);
  prep_stage1_kernel<D><<<grid, 256, 0, stream>>>(
      static_cast<const _Float16*>(g.k), static_cast<const _Float16*>(g.v), ak, sq, g.Hkv,
      p.nch, p.Ppad, reinterpret_cast<int64_t*>(w + p.off_kpart),
      reinterpret_cast<float*>(w + p.off_sv), reinterpret_cast<_Float16*>(w + p.off_vh));
  prep_stage2_kernel<D><<<grid, 256, 0, stream>>>(
      static_cast<const _Float16*>(g.k), ak, sq, g.Hkv, p.nch, p.Ppad,
      reinterpret_cast<const int64_t*>(w + p.off_kpart),
      reinterpret_cast<float*>(w + p.off_kmean), reinterpret_cast<float*>(w + p.off_sk),
      reinterpret_cast<int8_t*>(w + p.off_k8));
  return hipGetLastError();
}

hipError_t launch_prep(const FwdGeom& g, const WsPlan& p, void* ws, hipStream_t stream) {
  if (p.nch == 0) return hipSuccess;  // every sequence is empty
  switch (g.D) {
    case 32: return prep_d<32>(g, p, ws, stream);
    case 64: return prep_d<64>(g, p, ws, stream);
    case 128: return prep_d<128>(g, p, ws, stream);
    case 256: return prep_d<256>(g, p, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace i8a
