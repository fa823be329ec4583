// decode_kernels.hip - split-KV decode over an int8 K/V cache on gfx950: one new query
// token per sequence attends every cached token (the Attention kernels table's
// attn_decode row, in its int8-V and fp16-V variants).
//
// Cache fill, two launches: the exact per-channel K sums (the forward's first
// launch), then one grid whose first half quantizes K (K-smoothing mean subtracted)
// and second half V into 32-token tiles in MFMA fragment order (dtile_bytes).
//
// Decode: a workgroup of NW waves takes one chunk of the tiles of one (batch, kv
// head) and up to 32 of that kv head's query heads.  The query heads of the group are
// the 32 columns of the forward's transposed products
//   S^T = K . Q^T     v_mfma_i32_32x32x32_i8   (exact int32)
//   O^T = V^T . P^T   v_mfma_f32_32x32x16_f16  (P rounded to fp16, fp32 accumulation)
// so one pass over a tile serves every query head of the group, and a lane keeps one
// query's running max, sum and output column, as in the forward.  Each wave streams
// its own tiles (every NW-th tile of the chunk) through a private ring of NST LDS
// stages filled with direct-to-LDS loads, so no barrier is needed inside the loop.
// At the end the waves' states are merged in LDS into the chunk's partial result (or
// straight into the output when the chunk is the whole cache), and a second kernel
// merges the chunks' partials.
//
// The int8 V codes are turned into fp16 in registers: a byte permute places each
// biased code (code + 128) in the low mantissa byte of 1024.0 (fp16 0x6400), one
// packed subtraction of 1152 leaves the code exactly, and one packed multiply by the
// key's V scale (stored in fp16) gives the fp16 value sv * code, exact whenever that
// product is a normal fp16 number (sv has a 4-bit significand, |code| <= 127).
#include <float.h>

#include "i8a_device.h"
#include "i8a_launch.h"

namespace i8a {

namespace {

constexpr float DTAU = 8.0f;  // lazy-rescale threshold, log2 units (the forward uses 12)

// Launch shape, per V format: up to max_stages LDS stages per wave (max_stages - 1
// tiles in flight while one is computed) and up to max_waves waves per workgroup,
// within lds_budget bytes of LDS per workgroup.  Measured on the batched serving
// shape: the int8 tiles want more waves (their dequantization is VALU work), the
// larger fp16 tiles more copies in flight.
constexpr int max_stages(int vf) { return vf == VF_INT8 ? 2 : 3; }
constexpr int max_waves(int vf) { return vf == VF_INT8 ? 4 : 1; }
constexpr int lds_budget(int vf) { return vf == VF_INT8 ? 72 * 1024 : 54 * 1024; }

constexpr int dtile_rounds(int D, int vf) { return (dtile_bytes(D, vf) / 16 + 63) / 64; }
// Stages per wave: the most, up to max_stages, whose copies in flight vmcnt can count
// and whose ring for one wave fits the budget.
constexpr int dec_stages(int D, int vf) {
  int n = max_stages(vf);
  while (n > 2 &&
         ((n - 1) * dtile_rounds(D, vf) >= 64 || n * dtile_bytes(D, vf) > lds_budget(vf)))
    --n;
  return n;
}
// Waves per workgroup: as many as keep the workgroup's rings within the budget.
constexpr int dec_waves(int D, int vf) {
  int w = max_waves(vf);
  while (w > 1 && w * dec_stages(D, vf) * dtile_bytes(D, vf) > lds_budget(vf)) w /= 2;
  return w;
}

template <int D, int VF>
struct DLay {
  static constexpr int NKB = D / 32;
  static constexpr int VOFF = TKD * D;                                           // V block
  static constexpr int SKOFF = VOFF + (VF == VF_INT8 ? TKD * D : 2 * TKD * D);  // K scales
  static constexpr int SVOFF = SKOFF + TKD * 4;                                  // V scales
  static constexpr int BYTES = dtile_bytes(D, VF);
  static constexpr int NCH = BYTES / 16;              // 16-byte chunks per tile
  static constexpr int ROUNDS = dtile_rounds(D, VF);  // one-wave copy instructions per tile
  static constexpr int NST = dec_stages(D, VF);
  static constexpr int NW = dec_waves(D, VF);
  static_assert(BYTES % 16 == 0, "tiles are copied in 16-byte chunks");
  static_assert((NST - 1) * ROUNDS < 64, "vmcnt holds at most 63 outstanding loads");
  static_assert(NW * NST * BYTES <= 160 * 1024, "the rings fit in LDS");
};

__device__ __forceinline__ float smax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
// Max / sum with the lane 32 apart (v_permlane32_swap, no LDS round trip).
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

// Copy one cache tile into a wave-private LDS stage: lane l moves 16-byte chunks
// 64 r + l, one direct-to-LDS load per round (every round has an active lane, so each
// copy is exactly ROUNDS load instructions).
template <int D, int VF>
__device__ __forceinline__ void copy_dtile(const char* __restrict__ src, char* dst, int lane) {
  using LY = DLay<D, VF>;
  const uint32_t base = lds_addr(dst);
#pragma unroll
  for (int r = 0; r < LY::ROUNDS; ++r) {
    const int chunk = r * 64 + lane;
    if (r + 1 < LY::ROUNDS || chunk < LY::NCH) lds_dma16(src + (int64_t)chunk * 16, base + r * 1024);
  }
}

// Wait until at most `ahead` tile copies (R load instructions each) are outstanding,
// ahead in [0, A]; vmcnt takes an immediate, hence the unrolled choice.
template <int R, int A>
__device__ __forceinline__ void wait_copies(int ahead) {
  if constexpr (A == 0) {
    vm_wait<0>();
  } else {
    if (ahead >= A)
      vm_wait<A * R>();
    else
      wait_copies<R, A - 1>(ahead);
  }
}

// Key of V fragment slot jv for lane half hv within a 16-key group (the order in which
// the S^T result registers hold keys).
__device__ __forceinline__ int vkey(int hv, int jv) { return 4 * hv + (jv & 3) + 8 * (jv >> 2); }

// Eight biased int8 codes (two dwords, byte j = slot j) times the slots' fp16 scales.
__device__ __forceinline__ v8h dequant8(uint32_t lo, uint32_t hi, v8h sv) {
  const uint32_t K = 0x64646464u;
  v4i u;
  u[0] = (int)__builtin_amdgcn_perm(K, lo, 0x05010400u);
  u[1] = (int)__builtin_amdgcn_perm(K, lo, 0x07030602u);
  u[2] = (int)__builtin_amdgcn_perm(K, hi, 0x05010400u);
  u[3] = (int)__builtin_amdgcn_perm(K, hi, 0x07030602u);
  const v8h x = __builtin_bit_cast(v8h, u);
  const _Float16 bias = (_Float16)1152.0f;
  return (x - bias) * sv;
}

}  // namespace

// ----------------------------------------------------------------------------------
// Cache fill, launch 2.  Workgroups [0, nk) quantize K, [nk, 2 nk) V; each takes tpw
// TK-token slabs (two cache tiles each) of one (batch, kv head).  Rows past S are
// zero in both (codes, scales, values), so a masked key multiplies finite numbers.
template <int D>
struct FillKShared {
  int64_t red[512];
  float mean[D];
};
template <int D>
struct FillVShared {
  __attribute__((aligned(16))) _Float16 vraw[TK * D];
  float2 rsy[TK];
};
template <int D>
union FillShared {
  FillKShared<D> k;
  FillVShared<D> v;
};

template <int D, int VF>
__device__ __forceinline__ void fill_k(const _Float16* __restrict__ k, int S, int npart, int tpw,
                                       int ntd, const int64_t* __restrict__ kpart,
                                       float* __restrict__ kmean, char* __restrict__ tiles,
                                       int c, int64_t bg, FillKShared<D>& sh) {
  using LY = DLay<D, VF>;
  constexpr int G = D / 8, RPP = 256 / G, NP = TK / RPP;
  const int nt = (S + TK - 1) / TK;
  const int tlo = c * tpw;
  if (tlo >= nt) return;
  const int thi = min(nt, tlo + tpw);
  const int lc = threadIdx.x % G, rsub = threadIdx.x / G;
  const _Float16* kb = k + bg * S * D;
  v8h kr[NP];
  auto load_rows = [&](int t0) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = t0 + i * RPP + rsub;
      if (t < S) kr[i] = *reinterpret_cast<const v8h*>(kb + (int64_t)t * D + lc * 8);
    }
  };
  load_rows(tlo * TK);  // in flight during the mean reduction
  reduce_kmean<D>(kpart + bg * npart * D, (nt + tpw - 1) / tpw, S, sh.red, sh.mean,
                  c == 0 ? kmean + bg * D : nullptr);
  float mu[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mu[j] = sh.mean[lc * 8 + j];

  for (int tt = tlo; tt < thi; ++tt) {
    if (tt > tlo) load_rows(tt * TK);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = tt * TK + i * RPP + rsub;
      const bool real = t < S;
      float x[8];
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = real ? (float)kr[i][j] - mu[j] : 0.0f;
        amax = fmaxf(amax, fabsf(x[j]));
      }
      amax = group_max<G>(amax);
      const RowQ rq(real ? row_scale(amax, 24) : 0.0f);
      const uint2 codes = real ? rq.pack8(x) : make_uint2(0u, 0u);
      const int dt = t / TKD;
      if (dt < ntd) {
        char* tile = tiles + (bg * ntd + dt) * LY::BYTES;
        *reinterpret_cast<uint2*>(tile + ktile_off(t % TKD, lc * 8, D)) = codes;
        if (lc == 0) reinterpret_cast<float*>(tile + LY::SKOFF)[t % TKD] = rq.s;
      }
    }
  }
}

template <int D, int VF>
__device__ __forceinline__ void fill_v(const _Float16* __restrict__ v, int S, int tpw, int ntd,
                                       char* __restrict__ tiles, int c, int64_t bg,
                                       FillVShared<D>& sh) {
  using LY = DLay<D, VF>;
  constexpr int G = D / 8, RPP = 256 / G, NP = TK / RPP, NKB = D / 32;
  const int nt = (S + TK - 1) / TK;
  const int tlo = c * tpw;
  if (tlo >= nt) return;
  const int thi = min(nt, tlo + tpw);
  const int lc = threadIdx.x % G, rsub = threadIdx.x / G;
  const _Float16* vb = v + bg * S * D;

  for (int tt = tlo; tt < thi; ++tt) {
    const int t0 = tt * TK;
    v8h vr[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = t0 + i * RPP + rsub;
      if (t < S) {
        vr[i] = *reinterpret_cast<const v8h*>(vb + (int64_t)t * D + lc * 8);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) vr[i][j] = (_Float16)0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int n = i * RPP + rsub;
      *reinterpret_cast<v8h*>(sh.vraw + n * D + lc * 8) = vr[i];
      if constexpr (VF == VF_INT8) {
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)vr[i][j]));
        amax = group_max<G>(amax);
        if (lc == 0) {
          const RowQ rq(t0 + n < S ? row_scale(amax, 4) : 0.0f);
          sh.rsy[n] = make_float2(rq.s, rq.y);
        }
      }
    }
    __syncthreads();
    // Fragment f = (dsub * NKB + db) * 64 + lane' of the slab's tiles 2 tt + dsub.
    for (int f = threadIdx.x; f < 2 * NKB * 64; f += 256) {
      const int lanep = f & 63, db = (f >> 6) % NKB, dsub = (f >> 6) / NKB;
      const int dt = 2 * tt + dsub;
      if (dt >= ntd) continue;
      const int d = 32 * db + (lanep & 31), hv = lanep >> 5;
      char* tile = tiles + (bg * ntd + dt) * LY::BYTES;
      if constexpr (VF == VF_INT8) {
        uint32_t wd[4];
#pragma unroll
        for (int kg = 0; kg < 2; ++kg)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            uint32_t acc = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int n = 32 * dsub + 16 * kg + vkey(hv, 4 * half + j);
              const float2 sy = sh.rsy[n];
              RowQ rq(0.0f);
              rq.s = sy.x;
              rq.y = sy.y;
              acc = __builtin_amdgcn_cvt_pk_u8_f32(rq.code((float)sh.vraw[n * D + d]) + 128.0f, j,
                                                   acc);
            }
            wd[2 * kg + half] = acc;
          }
        *reinterpret_cast<uint4*>(tile + LY::VOFF + (db * 64 + lanep) * 16) =
            make_uint4(wd[0], wd[1], wd[2], wd[3]);
      } else {
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
          v8h fr;
#pragma unroll
          for (int jv = 0; jv < 8; ++jv) fr[jv] = sh.vraw[(32 * dsub + 16 * kg + vkey(hv, jv)) * D + d];
          *reinterpret_cast<v8h*>(tile + LY::VOFF + ((kg * NKB + db) * 64 + lanep) * 16) = fr;
        }
      }
    }
    if constexpr (VF == VF_INT8) {
      // V scales in fp16, ordered [hv][key group][jv] within a tile.
      if (threadIdx.x < 2 * TKD) {
        const int dsub = threadIdx.x / TKD, e = threadIdx.x % TKD;
        const int dt = 2 * tt + dsub;
        if (dt < ntd) {
          const int hv = e >> 4, kg = (e >> 3) & 1, jv = e & 7;
          const int n = 32 * dsub + 16 * kg + vkey(hv, jv);
          char* tile = tiles + (bg * ntd + dt) * LY::BYTES;
          reinterpret_cast<_Float16*>(tile + LY::SVOFF)[e] = (_Float16)sh.rsy[n].x;
        }
      }
    }
    __syncthreads();
  }
}

template <int D, int VF>
__global__ __launch_bounds__(256) void kvc_fill_kernel(const _Float16* __restrict__ k,
                                                       const _Float16* __restrict__ v, int S,
                                                       int npart, int tpw, int ntd,
                                                       const int64_t* __restrict__ kpart,
                                                       float* __restrict__ kmean,
                                                       char* __restrict__ tiles, int nk) {
  __shared__ FillShared<D> sh;
  int b = blockIdx.x;
  const bool is_v = b >= nk;
  if (is_v) b -= nk;
  const int c = b % npart;
  const int64_t bg = b / npart;
  if (is_v)
    fill_v<D, VF>(v, S, tpw, ntd, tiles, c, bg, sh.v);
  else
    fill_k<D, VF>(k, S, npart, tpw, ntd, kpart, kmean, tiles, c, bg, sh.k);
}

// Zeroes of the tiles a prefix fill leaves to appends: for every (batch, kv head), the
// per_bg-byte tile area from byte `first` on, in 16-byte stores (a grid-stride loop
// over all of them).  Slots that no append has written then hold zero codes, scales and
// values, so a decode whose last tile reaches past its sequence's last appended token
// multiplies finite numbers by the masked keys' zero weights.
__global__ __launch_bounds__(256) void kvc_zero_kernel(char* __restrict__ tiles, int64_t per_bg,
                                                       int64_t first, int64_t n16, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t bg = i / n16, j = i % n16;
    reinterpret_cast<uint4*>(tiles + bg * per_bg + first)[j] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// ----------------------------------------------------------------------------------
// Append: n new tokens of each (batch, kv head) (workgroup bg = b * Hkv + g) into the
// cache slots pos[b], pos[b] + 1, ...; a token whose slot falls outside [0, S) is not
// written.  K rows are quantized against the stored K-smoothing mean of the kv head,
// V rows per token (int8 V) or copied (fp16 V), each value into the place the fill
// gives it: K codes at ktile_off, V codes in the fragment slot of its key (the
// inverse of vkey), scales in key order (K) or [hv][key group][jv] order (V).  A row is
// handled by D / 8 lanes, 8 channels each.
template <int D, int VF>
__global__ __launch_bounds__(256) void kvc_append_kernel(const _Float16* __restrict__ k,
                                                         const _Float16* __restrict__ v, int n,
                                                         const int32_t* __restrict__ pos,
                                                         int Hkv, int S, int ntd,
                                                         const float* __restrict__ kmean,
                                                         char* __restrict__ tiles) {
  using LY = DLay<D, VF>;
  constexpr int G = D / 8, RPP = 256 / G, NKB = D / 32;
  const int64_t bg = blockIdx.x;
  const int b = (int)(bg / Hkv);
  const int p0 = pos[b];
  const int lc = threadIdx.x % G, rsub = threadIdx.x / G;
  float mu[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mu[j] = kmean[bg * D + lc * 8 + j];
  for (int i0 = 0; i0 < n; i0 += RPP) {
    const int i = i0 + rsub;
    const int64_t slot = (int64_t)p0 + i;
    const bool live = i < n && slot >= 0 && slot < S;
    // The rows are loaded whatever their slot (their loads do not wait for pos).
    v8h kr, vr;
#pragma unroll
    for (int j = 0; j < 8; ++j) kr[j] = vr[j] = (_Float16)0.0f;
    if (i < n) {
      kr = *reinterpret_cast<const v8h*>(k + (bg * n + i) * D + lc * 8);
      vr = *reinterpret_cast<const v8h*>(v + (bg * n + i) * D + lc * 8);
    }
    float x[8];
    float amax = 0.0f, vmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = (float)kr[j] - mu[j];
      amax = fmaxf(amax, fabsf(x[j]));
      vmax = fmaxf(vmax, fabsf((float)vr[j]));
    }
    amax = group_max<G>(amax);
    vmax = group_max<G>(vmax);
    if (!live) continue;
    const int t = (int)(slot % TKD);
    char* tile = tiles + (bg * ntd + slot / TKD) * LY::BYTES;
    const RowQ rq(row_scale(amax, 24));
    *reinterpret_cast<uint2*>(tile + ktile_off(t, lc * 8, D)) = rq.pack8(x);
    if (lc == 0) reinterpret_cast<float*>(tile + LY::SKOFF)[t] = rq.s;
    // The key's place among the fragment slots: key group kg, lane half hv, slot jv.
    const int kg = t >> 4, r = t & 15, hv = (r >> 2) & 1, jv = (r & 3) + 4 * (r >> 3);
    if constexpr (VF == VF_INT8) {
      const RowQ rv(row_scale(vmax, 4));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = lc * 8 + j, db = d >> 5, lanep = 32 * hv + (d & 31);
        const int code = (int)rv.code((float)vr[j]);
        tile[LY::VOFF + (db * 64 + lanep) * 16 + (2 * kg + (jv >> 2)) * 4 + (jv & 3)] =
            (char)(uint8_t)(code + 128);
      }
      if (lc == 0)
        reinterpret_cast<_Float16*>(tile + LY::SVOFF)[16 * hv + 8 * kg + jv] = (_Float16)rv.s;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = lc * 8 + j, db = d >> 5, lanep = 32 * hv + (d & 31);
        reinterpret_cast<_Float16*>(tile + LY::VOFF + ((kg * NKB + db) * 64 + lanep) * 16)[jv] =
            vr[j];
      }
    }
  }
}

// ----------------------------------------------------------------------------------
// Decode.  Workgroup id = ((b * Hkv + g) * nqb + qb) * nchunk + c.
template <int D, int VF>
__global__ __launch_bounds__(64 * dec_waves(D, VF)) void decode_kernel(
    const _Float16* __restrict__ q, _Float16* __restrict__ out, const char* __restrict__ tiles,
    int Hq, int Hkv, int S, int ntd, int nqb, int tpc, int nchunk, float qk_log2,
    float* __restrict__ part_o, float* __restrict__ part_ml, const int32_t* __restrict__ lens) {
  using LY = DLay<D, VF>;
  constexpr int NKB = LY::NKB, SB = LY::BYTES, NW = LY::NW, NST = LY::NST;
  constexpr int MROW = D + 1;               // merge row stride in floats (odd: no conflicts)
  constexpr int MWAVE = 32 * MROW + 64;     // per wave: 32 output rows, then 32 (m, l)
  constexpr int RING = NW * NST * SB;
  constexpr int MERGE = NW * MWAVE * 4;
  __shared__ __attribute__((aligned(16))) char smem[RING > MERGE ? RING : MERGE];

  int r = blockIdx.x;
  const int c = r % nchunk;
  r /= nchunk;
  const int qb = r % nqb;
  r /= nqb;
  const int g = r % Hkv, b = r / Hkv;
  const int G = Hq / Hkv;
  const int h0 = g * G + 32 * qb;           // first query head of this workgroup
  const int gv = min(32, G - 32 * qb);      // query heads in it
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  char* ring = smem + w * NST * SB;
  const int64_t bg = (int64_t)b * Hkv + g;
  const char* tsrc = tiles + bg * ntd * SB;
  // The sequence's cached tokens: all S, or its first lens[b] (clamped to [0, S]).
  const int Sb = lens ? min(max(lens[b], 0), S) : S;
  const int ntb = (Sb + TKD - 1) / TKD;
  const int t_lo = c * tpc, t_hi = min(ntb, t_lo + tpc);
  const int nmine = t_lo + w < t_hi ? (t_hi - t_lo - w + NW - 1) / NW : 0;

#pragma unroll
  for (int s = 0; s + 1 < NST; ++s)
    if (s < nmine) copy_dtile<D, VF>(tsrc + (int64_t)(t_lo + w + NW * s) * SB, ring + s * SB, lane);

  // The query rows, quantized as the forward quantizes Q rows: lane (m, hh) holds
  // bytes 32 kb + 16 hh + j of row m (the B-operand layout), and the row absmax joins
  // the two lane halves.  Lanes past the group's heads hold zero codes.
  v4i qf[NKB];
  float qsc;
  {
    const bool live = m < gv;
    float x[NKB][2][8];
    float amax = 0.0f;
    const _Float16* qrow = q + ((int64_t)b * Hq + h0 + m) * D + 16 * hh;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        v8h a;
        if (live) {
          a = *reinterpret_cast<const v8h*>(qrow + 32 * kb + 8 * e);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) a[j] = (_Float16)0.0f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[kb][e][j] = (float)a[j];
          amax = fmaxf(amax, fabsf(x[kb][e][j]));
        }
      }
    amax = other_half_max(amax);
    const RowQ rq(row_scale(amax, 24));
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint2 lo = rq.pack8(x[kb][0]), hi = rq.pack8(x[kb][1]);
      qf[kb] = v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
    }
    // An all-zero row has scale 0: FLT_MIN stands in (its scores are 0 either way), so
    // a masked score of -inf still gives p = 0.
    qsc = fmaxf(rq.s * qk_log2, FLT_MIN);
  }

  v16f o[NKB];
#pragma unroll
  for (int db = 0; db < NKB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  float mrun = -INFINITY, lsum = 0.0f;
  const bool ragged = Sb % TKD != 0;

  // One 32-key tile, as in the forward: scores, lazy max, fp16 P, row sum, P.V.
  auto step = [&](const char* st, int t) {
    const v4i* kl = reinterpret_cast<const v4i*>(st);
    v16i acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kl[kb * 64 + lane], qf[kb], acc, 0, 0, 0);
    // Register i holds key 8*(i/4) + 4*hh + i%4 of the tile.
    const float* skl = reinterpret_cast<const float*>(st + LY::SKOFF);
    float tv[16];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const v4f skv = *reinterpret_cast<const v4f*>(skl + 8 * J + 4 * hh);
#pragma unroll
      for (int i = 0; i < 4; ++i) tv[4 * J + i] = (float)acc[4 * J + i] * skv[i];
    }
    if (ragged && t == ntb - 1) {  // keys past the sequence's last in its last tile
      const int last = Sb - 1 - t * TKD - 4 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) > last) tv[i] = -INFINITY;
    }
    float m0 = smax(tv[0], tv[1]), m1 = smax(tv[2], tv[3]);
#pragma unroll
    for (int i = 4; i < 16; i += 4) {
      m0 = smax(smax(m0, tv[i]), tv[i + 1]);
      m1 = smax(smax(m1, tv[i + 2]), tv[i + 3]);
    }
    const float mc = other_half_max(smax(m0, m1)) * qsc;
    const bool upd = mc > mrun + DTAU;
    if (__any(upd)) {
      const float mnew = upd ? mc : mrun;
      const float alpha = upd ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.0f;
      mrun = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NKB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    const float muse = mrun == -INFINITY ? 0.0f : mrun;
    v8h pk[2];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      v2f pp;
      pp[0] = __builtin_amdgcn_exp2f(__builtin_fmaf(tv[i], qsc, -muse));
      pp[1] = __builtin_amdgcn_exp2f(__builtin_fmaf(tv[i + 1], qsc, -muse));
      const v2h ph = __builtin_convertvector(pp, v2h);
      pk[i >> 3][i & 7] = ph[0];
      pk[i >> 3][(i & 7) + 1] = ph[1];
    }
    const v2h ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const v2h pr = {pk[kg][e], pk[kg][e + 1]};
        lsum = __builtin_amdgcn_fdot2(pr, ones, lsum, false);
      }
    if constexpr (VF == VF_INT8) {
      const v8h* svl = reinterpret_cast<const v8h*>(st + LY::SVOFF);
      const v8h sv0 = svl[2 * hh], sv1 = svl[2 * hh + 1];
      const uint4* vl = reinterpret_cast<const uint4*>(st + LY::VOFF);
#pragma unroll
      for (int db = 0; db < NKB; ++db) {
        const uint4 cw = vl[db * 64 + lane];
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(dequant8(cw.x, cw.y, sv0), pk[0], o[db],
                                                        0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(dequant8(cw.z, cw.w, sv1), pk[1], o[db],
                                                        0, 0, 0);
      }
    } else {
      const v4i* vl = reinterpret_cast<const v4i*>(st + LY::VOFF);
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int db = 0; db < NKB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(v8h, vl[(kg * NKB + db) * 64 + lane]), pk[kg], o[db], 0, 0, 0);
    }
  };

  for (int i = 0; i < nmine; ++i) {
    const int nx = i + NST - 1;
    if (nx < nmine)
      copy_dtile<D, VF>(tsrc + (int64_t)(t_lo + w + NW * nx) * SB, ring + (nx % NST) * SB, lane);
    // Tile i has landed once at most the copies issued after it are outstanding.
    wait_copies<LY::ROUNDS, NST - 1>(min(NST - 1, nmine - 1 - i));
    step(ring + (i % NST) * SB, t_lo + w + NW * i);
  }

  // Merge of the waves' states.  A wave without tiles has m = -inf, l = 0, o = 0 and
  // weighs 0.  A chunk past the sequence's tokens has no tile at all: its common max is
  // -inf and its sum 0 (a zero output row when it is the whole cache).
  lsum = other_half_sum(lsum);
  __syncthreads();  // every wave is done with its ring
  {
    float* mo = reinterpret_cast<float*>(smem) + w * MWAVE;
    if (m < gv) {
#pragma unroll
      for (int db = 0; db < NKB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          mo[m * MROW + 32 * db + 8 * (i >> 2) + 4 * hh + (i & 3)] = o[db][i];
      if (hh == 0) {
        mo[32 * MROW + 2 * m] = mrun;
        mo[32 * MROW + 2 * m + 1] = lsum;
      }
    }
  }
  __syncthreads();
  const float* mall = reinterpret_cast<const float*>(smem);
  for (int e = tid; e < gv * D; e += 64 * NW) {
    const int qq = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mall[ww * MWAVE + 32 * MROW + 2 * qq]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float* base = mall + ww * MWAVE;
      const float mw = base[32 * MROW + 2 * qq];
      const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      num += f * base[qq * MROW + d];
      den += f * base[32 * MROW + 2 * qq + 1];
    }
    const int64_t row = (int64_t)b * Hq + h0 + qq;
    if (nchunk == 1) {
      out[row * D + d] = (_Float16)(den > 0.0f ? num / den : 0.0f);
    } else {
      part_o[(row * nchunk + c) * D + d] = num;
      if (d == 0) {
        part_ml[(row * nchunk + c) * 2] = M;
        part_ml[(row * nchunk + c) * 2 + 1] = den;
      }
    }
  }
}

// Merge of the chunks' partials: out = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c
// for each output element (one per thread).  A chunk past its sequence's tokens holds
// m_c = -inf and l_c = 0 and weighs 0; a sequence with no token gets a zero row.  Up to
// MC chunks are loaded all at once (one memory latency); more take further passes.
constexpr int MC = 16;

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml,
                                                           int nchunk, int64_t nel,
                                                           _Float16* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= nel) return;
  const int64_t row = e / D;
  const int d = (int)(e % D);
  const float2* ml = part_ml + row * nchunk;
  const float* po = part_o + row * nchunk * D + d;
  float M = -INFINITY, num = 0.0f, den = 0.0f;
  for (int c0 = 0; c0 < nchunk; c0 += MC) {
    float2 mv[MC];
    float ov[MC];
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      if (c0 + c < nchunk) {
        mv[c] = ml[c0 + c];
        ov[c] = po[(int64_t)(c0 + c) * D];
      } else {
        mv[c] = make_float2(-INFINITY, 0.0f);
        ov[c] = 0.0f;
      }
    }
    float Mn = M;
#pragma unroll
    for (int c = 0; c < MC; ++c) Mn = fmaxf(Mn, mv[c].x);
    const float a = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    num *= a;
    den *= a;
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      const float f = mv[c].x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv[c].x - Mn);
      num += f * ov[c];
      den += f * mv[c].y;
    }
    M = Mn;
  }
  out[e] = (_Float16)(den > 0.0f ? num / den : 0.0f);
}

// ----------------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

KvcPlan plan_kvcache(int32_t B, int32_t Hkv, int32_t S, int32_t D, int32_t vf) {
  KvcPlan p;
  p.B = B;
  p.Hkv = Hkv;
  p.S = S;
  p.D = D;
  p.vf = vf;
  p.ntd = (S + TKD - 1) / TKD;
  const int nt = (S + TK - 1) / TK;
  p.tpw = (nt + MAX_PARTS - 1) / MAX_PARTS;
  if (p.tpw < 1) p.tpw = 1;
  p.npart = (nt + p.tpw - 1) / p.tpw;
  size_t off = 0;
  p.off_kpart = off;
  off = align256(off + (size_t)B * Hkv * p.npart * D * 8);
  p.off_kmean = off;
  off = align256(off + (size_t)B * Hkv * D * 4);
  p.off_tiles = off;
  off = align256(off + (size_t)B * Hkv * p.ntd * dtile_bytes(D, vf));
  p.total = off;
  return p;
}

// Target number of decode workgroups (a few per CU), and the fewest tiles a wave
// takes, so that its prologue (the query quantization) and the merge stay small.
static const int kDecTargetWG = 1024;
static const int kDecMinTilesPerWave = 8;

DecPlan plan_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D, int32_t vf) {
  DecPlan p;
  const int G = Hq / Hkv;
  const int ntd = (S + TKD - 1) / TKD;
  p.nqb = (G + 31) / 32;
  p.nw = dec_waves(D, vf);
  const int64_t units = (int64_t)B * Hkv * p.nqb;
  int64_t want = (kDecTargetWG + units - 1) / units;
  const int64_t cap = (ntd + p.nw * kDecMinTilesPerWave - 1) / (p.nw * kDecMinTilesPerWave);
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  int tpc = (int)((ntd + want - 1) / want);
  tpc = (tpc + p.nw - 1) / p.nw * p.nw;
  p.tpc = tpc;
  p.nchunk = (ntd + tpc - 1) / tpc;
  p.off_po = p.off_pml = p.total = 0;
  if (p.nchunk > 1) {
    size_t off = align256((size_t)B * Hq * p.nchunk * D * 4);
    p.off_pml = off;
    p.total = align256(off + (size_t)B * Hq * p.nchunk * 8);
  }
  return p;
}

// The fill of the first n_fill <= S tokens (k, v [B, Hkv, n_fill, D]): the K sums and
// the mean over those tokens, their K and V tiles; later tiles are zeroed for appends.
template <int D, int VF>
static hipError_t fill_d(const void* k, const void* v, const KvcPlan& p, int32_t n_fill,
                         char* cache, hipStream_t stream) {
  const int nt = (n_fill + TK - 1) / TK;
  int tpw = (nt + MAX_PARTS - 1) / MAX_PARTS;
  if (tpw < 1) tpw = 1;
  const int npart = (nt + tpw - 1) / tpw;  // at most p.npart: the plan's for S >= n_fill
  const int64_t nk = (int64_t)npart * p.B * p.Hkv;
  if (2 * nk > 0x7fffffff) return hipErrorInvalidValue;
  int64_t* kpart = reinterpret_cast<int64_t*>(cache + p.off_kpart);
  hipError_t e = launch_ksum_dense(k, p.B, p.Hkv, n_fill, D, npart, tpw, kpart, stream);
  if (e != hipSuccess) return e;
  kvc_fill_kernel<D, VF><<<dim3((unsigned)(2 * nk)), 256, 0, stream>>>(
      static_cast<const _Float16*>(k), static_cast<const _Float16*>(v), n_fill, npart, tpw,
      p.ntd, kpart, reinterpret_cast<float*>(cache + p.off_kmean), cache + p.off_tiles, (int)nk);
  e = hipGetLastError();
  // The fill writes whole TK-token slabs (two tiles each); the tiles after them are
  // zeroed for the appends.
  const int filled = 2 * nt < p.ntd ? 2 * nt : p.ntd;
  if (e != hipSuccess || filled == p.ntd) return e;
  using LY = DLay<D, VF>;
  const int64_t n16 = (int64_t)(p.ntd - filled) * LY::BYTES / 16;
  const int64_t total = n16 * p.B * p.Hkv;
  const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
  kvc_zero_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(
      cache + p.off_tiles, (int64_t)p.ntd * LY::BYTES, (int64_t)filled * LY::BYTES, n16, total);
  return hipGetLastError();
}

hipError_t launch_kvcache_fill(const void* k, const void* v, const KvcPlan& p, int32_t n_fill,
                               void* cache, hipStream_t stream) {
  char* c = static_cast<char*>(cache);
#define I8A_FILL(DD)                                                                    \
  case DD:                                                                              \
    return p.vf == VF_INT8 ? fill_d<DD, VF_INT8>(k, v, p, n_fill, c, stream)            \
                           : fill_d<DD, VF_FP16>(k, v, p, n_fill, c, stream);
  switch (p.D) {
    I8A_FILL(32) I8A_FILL(64) I8A_FILL(128) I8A_FILL(256)
    default:
      return hipErrorInvalidValue;
  }
#undef I8A_FILL
}

template <int D, int VF>
static hipError_t decode_d(const void* q, void* out, int Hq, float softmax_scale,
                           const KvcPlan& p, const DecPlan& dp, const char* cache, char* ws,
                           const int32_t* lens, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.B * p.Hkv * dp.nqb * dp.nchunk;
  if (blocks > 0x7fffffff || (int64_t)p.B * Hq > 0x7fffffff) return hipErrorInvalidValue;
  const float qk_log2 = softmax_scale * 1.4426950408889634f;
  float* po = dp.nchunk > 1 ? reinterpret_cast<float*>(ws + dp.off_po) : nullptr;
  float* pml = dp.nchunk > 1 ? reinterpret_cast<float*>(ws + dp.off_pml) : nullptr;
  decode_kernel<D, VF><<<dim3((unsigned)blocks), dim3(64 * dec_waves(D, VF)), 0, stream>>>(
      static_cast<const _Float16*>(q), static_cast<_Float16*>(out), cache + p.off_tiles, Hq,
      p.Hkv, p.S, p.ntd, dp.nqb, dp.tpc, dp.nchunk, qk_log2, po, pml, lens);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || dp.nchunk == 1) return e;
  const int64_t nel = (int64_t)p.B * Hq * D;
  decode_merge_kernel<D><<<dim3((unsigned)((nel + 255) / 256)), 256, 0, stream>>>(
      po, reinterpret_cast<const float2*>(pml), dp.nchunk, nel, static_cast<_Float16*>(out));
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, void* out, int32_t Hq, float softmax_scale,
                         const KvcPlan& p, const DecPlan& dp, const void* cache, void* ws,
                         const int32_t* lens, hipStream_t stream) {
  const char* c = static_cast<const char*>(cache);
  char* w = static_cast<char*>(ws);
#define I8A_DEC(DD)                                                                        \
  case DD:                                                                                 \
    return p.vf == VF_INT8 ? decode_d<DD, VF_INT8>(q, out, Hq, softmax_scale, p, dp, c, w, \
                                                   lens, stream)                           \
                           : decode_d<DD, VF_FP16>(q, out, Hq, softmax_scale, p, dp, c, w, \
                                                   lens, stream);
  switch (p.D) {
    I8A_DEC(32) I8A_DEC(64) I8A_DEC(128) I8A_DEC(256)
    default:
      return hipErrorInvalidValue;
  }
#undef I8A_DEC
}

template <int D, int VF>
static hipError_t append_d(const void* k, const void* v, int32_t n, const int32_t* pos,
                           const KvcPlan& p, char* cache, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.B * p.Hkv;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  kvc_append_kernel<D, VF><<<dim3((unsigned)blocks), 256, 0, stream>>>(
      static_cast<const _Float16*>(k), static_cast<const _Float16*>(v), n, pos, p.Hkv, p.S,
      p.ntd, reinterpret_cast<const float*>(cache + p.off_kmean), cache + p.off_tiles);
  return hipGetLastError();
}

hipError_t launch_kvcache_append(const void* k, const void* v, int32_t n, const int32_t* pos,
                                 const KvcPlan& p, void* cache, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  char* c = static_cast<char*>(cache);
#define I8A_APP(DD)                                                                   \
  case DD:                                                                            \
    return p.vf == VF_INT8 ? append_d<DD, VF_INT8>(k, v, n, pos, p, c, stream)        \
                           : append_d<DD, VF_FP16>(k, v, n, pos, p, c, stream);
  switch (p.D) {
    I8A_APP(32) I8A_APP(64) I8A_APP(128) I8A_APP(256)
    default:
      return hipErrorInvalidValue;
  }
#undef I8A_APP
}

}  // namespace i8a
