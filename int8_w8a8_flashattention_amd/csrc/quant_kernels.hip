// quant_kernels.hip - row quantization and the Q, K and V preparation of the forward.
//
// All of these kernels are HBM-bound streaming passes: rows are read once with 16-byte
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
    const RowQ rq(row_scale(amax, scale_bits));
    if (live) {
      *reinterpret_cast<uint2*>(codes + r * d + c * 8) = rq.pack8(v);
      if (c == 0) scales[r] = rq.s;
    }
  }
}

// ----------------------------------------------------------------------------------
// K/V preparation over the TK-token tiles of every (sequence, kv head).  A tile's
// block in the workspace (tile_bytes) holds its int8 K codes, its exact fp16
// dequantized V and its fp32 K scales, in the order the attention kernel copies them
// to LDS.  Slots between a sequence's end and its last tile boundary are zero (codes,
// V and scales), so a masked key still multiplies finite numbers.
//
// Launch 1 computes only the exact per-channel K sums (the K-smoothing statistic);
// launch 2 runs everything that reads them (the K quantization) together with the
// work that does not (V tiles, Q rows), so the one dependent step of the preparation
// costs a short pass over K and the rest streams in one grid.

// Launch 1 (workgroup = tpw consecutive tiles of one sequence and kv head): the exact
// per-channel sums of the tiles' K rows as one int64 partial, in units of 2^-24 (every
// fp16 value is an integer multiple of 2^-24; each thread sums its values of a tile in
// fp64, exactly, and adds that sum to its integer partial).  With VCH (V quantized per
// channel), also the per-channel maxima of |v| over the same tokens as one fp32
// partial; with QO (Q outlier detection), the per-channel maxima of |q| over the same
// tokens and the kv head's Gq query heads.
template <int D, bool VCH, bool QO = false>
__global__ __launch_bounds__(256) void prep_ksum_kernel(const _Float16* __restrict__ k,
                                                        const _Float16* __restrict__ v,
                                                        Act act, Seqs seqs, int Hkv, int npart,
                                                        int tpw, int64_t* __restrict__ kpart,
                                                        float* __restrict__ vpart,
                                                        const _Float16* __restrict__ q = nullptr,
                                                        Act aq = Act{}, int Gq = 1,
                                                        float* __restrict__ qopart = nullptr) {
  constexpr int G = D / 8;      // lanes per row
  constexpr int RPP = 256 / G;  // rows per pass
  constexpr int NP = TK / RPP;  // rows per thread and tile
  __shared__ int64_t red[RPP * D];
  __shared__ float redv[VCH ? RPP * D : 1];
  __shared__ float redq[QO ? RPP * D : 1];
  int b = blockIdx.x;
  const int c = b % npart;
  b /= npart;
  const int g = b % Hkv, s = b / Hkv;
  int64_t start;
  int L;
  seqs.bounds(s, start, L);
  const int nt = (L + TK - 1) / TK;
  const int tile_lo = c * tpw;
  if (tile_lo >= nt) return;
  const int tile_hi = min(nt, tile_lo + tpw);
  const int lc = threadIdx.x % G, rsub = threadIdx.x / G;

  int64_t acc[8];
  float vmx[8], qmx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc[j] = 0;
    vmx[j] = 0.0f;
    qmx[j] = 0.0f;
  }
  for (int tt = tile_lo; tt < tile_hi; ++tt) {
    const int t0 = tt * TK;
    v8h kr[NP], vr[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = t0 + i * RPP + rsub;
      if (t < L) {
        kr[i] = *reinterpret_cast<const v8h*>(k + act.off(start, g, t) + lc * 8);
        if constexpr (VCH) vr[i] = *reinterpret_cast<const v8h*>(v + act.off(start, g, t) + lc * 8);
      }
    }
    // The tile's NP <= 8 values per channel summed exactly in fp64, then added to the
    // integer partial.
    static_assert(NP <= 8, "fixed24_of_sum8 takes sums of at most 8 values");
    double ts[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ts[j] = 0.0;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (t0 + i * RPP + rsub < L) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          ts[j] += (double)(float)kr[i][j];
          if constexpr (VCH) vmx[j] = fmaxf(vmx[j], fabsf((float)vr[i][j]));
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += fixed24_of_sum8(ts[j]);
    if constexpr (QO) {
      // The group's query heads four at a time, all of their row loads issued before any
      // maximum is taken.
      constexpr int HU = 4;
      for (int hq0 = g * Gq; hq0 < (g + 1) * Gq; hq0 += HU) {
        v8h qr[HU][NP];
#pragma unroll
        for (int u = 0; u < HU; ++u)
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            const int t = t0 + i * RPP + rsub;
            if (hq0 + u < (g + 1) * Gq && t < L)
              qr[u][i] = *reinterpret_cast<const v8h*>(q + aq.off(start, hq0 + u, t) + lc * 8);
          }
#pragma unroll
        for (int u = 0; u < HU; ++u)
#pragma unroll
          for (int i = 0; i < NP; ++i)
            if (hq0 + u < (g + 1) * Gq && t0 + i * RPP + rsub < L) {
#pragma unroll
              for (int j = 0; j < 8; ++j) qmx[j] = fmaxf(qmx[j], fabsf((float)qr[u][i][j]));
            }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    red[rsub * D + lc * 8 + j] = acc[j];
    if constexpr (VCH) redv[rsub * D + lc * 8 + j] = vmx[j];
    if constexpr (QO) redq[rsub * D + lc * 8 + j] = qmx[j];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    int64_t tot = 0;
    float mx = 0.0f, mq = 0.0f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) {
      tot += red[r * D + threadIdx.x];
      if constexpr (VCH) mx = fmaxf(mx, redv[r * D + threadIdx.x]);
      if constexpr (QO) mq = fmaxf(mq, redq[r * D + threadIdx.x]);
    }
    const int64_t o = (((int64_t)s * Hkv + g) * npart + c) * D + threadIdx.x;
    kpart[o] = tot;
    if constexpr (VCH) vpart[o] = mx;
    if constexpr (QO) qopart[o] = mq;
  }
}

// ----------------------------------------------------------------------------------
// The Q outlier channels of one (sequence, kv head) from the launch-1 channel maxima
// (a max is exact in any order): channel d is an outlier when its maximum exceeds
// QO_THRESHOLD; of more than QO_MAX candidates the largest maxima are kept, ties to
// the lower channel.  Leaves in sh.slot[d] the channel's position in the increasing
// list of kept channels (-1 if not kept) and, if ochan_out is given, writes the list
// padded with -1.  Every thread of the 256-thread workgroup must call it.
// This thread's maximum over the partials r, r + 256/D, ... (< np <= MAX_PARTS) of
// channel d (pp points at the partials' channel d, rows D apart): every load issued at
// once, CH at a time, so the reduction costs a few memory latencies rather than one per
// partial.
template <int D>
__device__ __forceinline__ float partial_max(const float* __restrict__ pp, int np, int r) {
  constexpr int TPC = 256 / D;  // threads per channel
  constexpr int MAXK = (MAX_PARTS + TPC - 1) / TPC;
  constexpr int CH = MAXK < 16 ? MAXK : 16;
  float mx = 0.0f;
#pragma unroll
  for (int k0 = 0; k0 < MAXK; k0 += CH) {
    float v[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int i = r + (k0 + k) * TPC;
      v[k] = i < np ? pp[(int64_t)i * D] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) mx = fmaxf(mx, v[k]);
  }
  return mx;
}

template <int D>
struct QoShared {
  float amax[D];
  int keep[D];
  int slot[D];
  int chan[QO_MAX + 1];  // the kept channels, then their count
  float red[256];
  int wkeep[4];          // kept channels per wave of the first D threads
};

template <int D>
__device__ __forceinline__ void select_outliers(const float* __restrict__ pp, int np,
                                                QoShared<D>& sh, int32_t* __restrict__ ochan_out) {
  constexpr int TPC = 256 / D;  // threads per channel
  const int d = threadIdx.x % D, r = threadIdx.x / D;
  float mx = partial_max<D>(pp + d, np, r);
  sh.red[threadIdx.x] = mx;
  __syncthreads();
  if (r == 0) {
    for (int k2 = 1; k2 < TPC; ++k2) mx = fmaxf(mx, sh.red[k2 * D + d]);
    sh.amax[d] = mx;
  }
  __syncthreads();
  if (r == 0) {
    const float a = sh.amax[d];
    int rank = 0;
    for (int e = 0; e < D; ++e) {
      const float b = sh.amax[e];
      rank += (b > QO_THRESHOLD && (b > a || (b == a && e < d))) ? 1 : 0;
    }
    sh.keep[d] = (a > QO_THRESHOLD && rank < QO_MAX) ? 1 : 0;
  }
  __syncthreads();
  // Positions by prefix counts: channel d = threadIdx.x (r == 0) is in wave d / 64 at lane
  // d % 64; a ballot counts the kept channels below it in its wave, the per-wave totals
  // those of the waves before.
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const bool kd = r == 0 && sh.keep[d] != 0;
  const uint64_t kmask = __ballot(kd);
  if (r == 0 && lane == 0) sh.wkeep[wv] = __popcll(kmask);
  __syncthreads();
  if (r == 0) {
    int pos = __popcll(kmask & ((1ull << lane) - 1ull));
    for (int x = 0; x < wv; ++x) pos += sh.wkeep[x];
    sh.slot[d] = kd ? pos : -1;
    if (kd) sh.chan[pos] = d;
    if (d == D - 1) sh.chan[QO_MAX] = pos + (kd ? 1 : 0);
  }
  __syncthreads();
  if (ochan_out && threadIdx.x < QO_MAX)
    ochan_out[threadIdx.x] = (int)threadIdx.x < sh.chan[QO_MAX] ? sh.chan[threadIdx.x] : -1;
}

// Launch 2, V part (workgroup = tpw consecutive tiles of one sequence and kv head): V
// quantized with the 4-bit scale rule, per token or (VCH) per channel with the scales
// from the launch-1 maxima, written as the exact fp16 values scale * code in the V
// fragment layout.
//   Phase A: coalesced loads of the tile's V rows; each row's scale and reciprocal
//            (per token); the raw rows into LDS.
//   Phase B: each thread assembles whole 16-byte V fragments (8 keys of one channel)
//            from LDS and stores them with coalesced writes.
template <int D>
struct PrepVShared {
  __attribute__((aligned(16))) _Float16 vraw[TK * D];
  float2 rsy[TK];
  float2 csy[D];
  float red[256];
};

template <int D, bool VCH>
__device__ __forceinline__ void prep_v_body(const _Float16* __restrict__ v, const Act& act,
                                            const Seqs& seqs, int Hkv, int npart, int tpw,
                                            int64_t Ppad, const float* __restrict__ vpart,
                                            float* __restrict__ svc_ws,
                                            float* __restrict__ sv_ws, char* __restrict__ tiles,
                                            int tstride, int c, int g, int s,
                                            PrepVShared<D>& sh) {
  constexpr int G = D / 8;       // lanes per row
  constexpr int RPP = 256 / G;   // rows per pass
  constexpr int NP = TK / RPP;   // rows per thread and tile
  constexpr int NF = TK * D / 8 / 256;  // V fragments per thread and tile
  _Float16* vraw = sh.vraw;
  float2* rsy = sh.rsy;

  int64_t start;
  int L;
  seqs.bounds(s, start, L);
  const int nt = (L + TK - 1) / TK;
  const int tile_lo = c * tpw;
  if (tile_lo >= nt) return;
  const int tile_hi = min(nt, tile_lo + tpw);
  const int64_t pbase = Seqs::pstart(s, start);
  const int lc = threadIdx.x % G, rsub = threadIdx.x / G;

  // A tile's V rows (zero past the sequence end).  The first tile's are requested before
  // the channel maxima are reduced (they do not depend on them), so the two memory
  // latencies overlap.
  auto load_rows = [&](int t0, v8h (&vr)[NP]) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = t0 + i * RPP + rsub;
      if (t < L) {
        vr[i] = *reinterpret_cast<const v8h*>(v + act.off(start, g, t) + lc * 8);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) vr[i][j] = (_Float16)0.0f;
      }
    }
  };
  v8h vr[NP];
  load_rows(tile_lo * TK, vr);

  if constexpr (VCH) {
    // The channel maxima of the whole sequence from the launch-1 partials (a max is
    // exact in any order), then each channel's scale and reciprocal.
    constexpr int TPC = 256 / D;
    const int d = threadIdx.x % D, r = threadIdx.x / D;
    const int np = (nt + tpw - 1) / tpw;
    float mx = partial_max<D>(vpart + ((int64_t)s * Hkv + g) * npart * D + d, np, r);
    sh.red[threadIdx.x] = mx;
    __syncthreads();
    if (r == 0) {
      for (int k2 = 1; k2 < TPC; ++k2) mx = fmaxf(mx, sh.red[k2 * D + d]);
      const RowQ rq(row_scale(mx, 4));
      sh.csy[d] = make_float2(rq.s, rq.y);
      if (c == 0) svc_ws[((int64_t)s * Hkv + g) * D + d] = rq.s;
    }
    __syncthreads();
  }

  for (int tt = tile_lo; tt < tile_hi; ++tt) {
    const int t0 = tt * TK;
    if (tt > tile_lo) load_rows(t0, vr);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int n = i * RPP + rsub, t = t0 + n;
      *reinterpret_cast<v8h*>(vraw + n * D + lc * 8) = vr[i];
      if constexpr (!VCH) {
        const bool real = t < L;
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)vr[i][j]));
        amax = group_max<G>(amax);
        if (lc == 0) {
          const RowQ rq(real ? row_scale(amax, 4) : 0.0f);
          rsy[n] = make_float2(rq.s, rq.y);
          if (real) sv_ws[(int64_t)g * Ppad + pbase + t] = rq.s;
        }
      }
    }
    __syncthreads();
    v8h* dst = reinterpret_cast<v8h*>(tiles + ((int64_t)g * (Ppad / TK) + (pbase + t0) / TK) *
                                                  tstride + TK * D);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      // fragment f = (kg * D/32 + db) * 64 + lane', lane' = dl + 32 * hv
      const int f = i * 256 + threadIdx.x;
      const int lanep = f & 63, kgdb = f >> 6;
      const int db = kgdb % (D / 32), kg = kgdb / (D / 32);
      const int d = 32 * db + (lanep & 31), hv = lanep >> 5;
      v8h frag;
#pragma unroll
      for (int jv = 0; jv < 8; ++jv) {
        const int n = 16 * kg + (jv < 4 ? 4 * hv + jv : 8 + 4 * hv + (jv - 4));
        const float2 sy = VCH ? sh.csy[d] : rsy[n];
        RowQ rq(0.0f);
        rq.s = sy.x;
        rq.y = sy.y;
        // The scale has a 4-bit significand and |code| <= 127: the product is exact
        // in fp16.  (Rows past the sequence end are zero and give 0.)
        frag[jv] = (_Float16)(rq.s * rq.code((float)vraw[n * D + d]));
      }
      dst[f] = frag;
    }
    __syncthreads();
  }
}

// Launch 2, K part (workgroup = tpw consecutive tiles of one sequence and kv head): the
// K-smoothing mean of the sequence, reduced by every workgroup from
// the launch-1 partials (at most MAX_PARTS of them; integer sums, so every workgroup
// gets the same value), divided in fp64 and rounded to fp32; then the K rows of the
// workgroup's tiles quantized from fp32(k) - mean into the K fragment layout, with
// the K scales after the V block.  With QO the Q outlier channels are selected from
// the launch-1 maxima, left out of the K rows (zero before the row's maximum is
// taken) and stored as the fp16 K values themselves after the scales: per 32-key
// block, lane n % 32 + 32 (o / 8) holds slot o % 8 of key n (the A operand of a
// 32x32x16 fp16 MFMA over the QO_MAX slots; empty slots hold 0).
template <int D>
struct PrepKShared {
  int64_t red[512];
  float mean[D];
  QoShared<D> qo;
};

template <int D, bool ROT, bool QO>
__device__ __forceinline__ void prep_k_body(const _Float16* __restrict__ k, const Act& act,
                                            const Seqs& seqs, int Hkv, int npart, int tpw,
                                            int64_t Ppad, const int64_t* __restrict__ kpart,
                                            float* __restrict__ kmean_ws,
                                            const float* __restrict__ qopart,
                                            int32_t* __restrict__ ochan_ws,
                                            char* __restrict__ tiles, int tstride, int c, int g,
                                            int s, PrepKShared<D>& sh) {
  constexpr int G = D / 8;
  constexpr int RPP = 256 / G;
  constexpr int NP = TK / RPP;
  int64_t* red = sh.red;
  float* mean = sh.mean;
  int64_t start;
  int L;
  seqs.bounds(s, start, L);
  const int nt = (L + TK - 1) / TK;
  const int tile_lo = c * tpw;
  if (tile_lo >= nt) return;
  const int tile_hi = min(nt, tile_lo + tpw);
  const int64_t pbase = Seqs::pstart(s, start);
  const int lc = threadIdx.x % G, rsub = threadIdx.x / G;

  // The first tile's K rows are requested before the mean reduction (they do not
  // depend on it), so the two memory latencies overlap.
  auto load_rows = [&](int t0, v8h (&kr)[NP]) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = t0 + i * RPP + rsub;
      if (t < L) kr[i] = *reinterpret_cast<const v8h*>(k + act.off(start, g, t) + lc * 8);
    }
  };
  v8h kr[NP];
  load_rows(tile_lo * TK, kr);

  reduce_kmean<D>(kpart + ((int64_t)s * Hkv + g) * npart * D, (nt + tpw - 1) / tpw, L, red, mean,
                  c == 0 ? kmean_ws + ((int64_t)s * Hkv + g) * D : nullptr);
  float mu[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mu[j] = mean[lc * 8 + j];
  bool out_ch[8] = {};
  if constexpr (QO) {
    select_outliers<D>(qopart + ((int64_t)s * Hkv + g) * npart * D, (nt + tpw - 1) / tpw, sh.qo,
                       c == 0 ? ochan_ws + ((int64_t)s * Hkv + g) * QO_MAX : nullptr);
#pragma unroll
    for (int j = 0; j < 8; ++j) out_ch[j] = sh.qo.slot[lc * 8 + j] >= 0;
  }

  for (int tt = tile_lo; tt < tile_hi; ++tt) {
    const int t0 = tt * TK;
    char* tile = tiles + ((int64_t)g * (Ppad / TK) + (pbase + t0) / TK) * tstride;
    float* sk_tile = reinterpret_cast<float*>(tile + 3 * TK * D);
    if (tt > tile_lo) load_rows(t0, kr);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int n = i * RPP + rsub, t = t0 + n;
      const bool real = t < L;
      float x[8];
      float amax = 0.0f;
      if constexpr (ROT) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = real ? (float)kr[i][j] - mu[j] : 0.0f;
        fwht_row<G>(x, lc);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
      } else if (real) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[j] = out_ch[j] ? 0.0f : (float)kr[i][j] - mu[j];
          amax = fmaxf(amax, fabsf(x[j]));
        }
      }
      amax = group_max<G>(amax);
      const RowQ rq(real ? row_scale(amax, 24) : 0.0f);
      const uint2 codes = real ? rq.pack8(x) : make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(tile + ktile_off(n, lc * 8, D)) = codes;
      if (lc == 0) sk_tile[n] = rq.s;
      if constexpr (QO) {
        // The outlier slots of this key, QO_MAX / G of them per lane.
        _Float16* ko = reinterpret_cast<_Float16*>(tile + tile_bytes(D));
#pragma unroll
        for (int o = lc; o < QO_MAX; o += G) {
          const int ch = o < sh.qo.chan[QO_MAX] ? sh.qo.chan[o] : -1;
          const _Float16 kv = (real && ch >= 0) ? k[act.off(start, g, t) + ch] : (_Float16)0.0f;
          ko[((n >> 5) * 64 + (n & 31) + 32 * (o >> 3)) * 8 + (o & 7)] = kv;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------------
// Q preparation (workgroup = QCH query rows of one sequence and query head): the rows
// quantized with the Q/K row rule into the B-operand fragment order of 32-row blocks
// (the attention kernel loads a block straight into registers), and the row scales.
// Rows past the sequence end get zero codes and scale 0.  The fragments are assembled
// in LDS and written with coalesced 16-byte stores.
// Query rows per Q preparation workgroup: small work items, so that many more
// workgroups than fit at once stream through and their loads, quantization and stores
// overlap.
constexpr int QCH = 64;
static_assert(BQ % QCH == 0 && QCH % 32 == 0, "Q chunks hold whole 32-row blocks");

// qblk: one scale per block of 32 rows (counted from the sequence start) instead of one
// per row: the block's largest row absolute maximum sets the scale of all its rows.
// QO: the outlier channels of the head's kv group (from the launch-1 maxima) are set
// to zero before the rows are quantized.
template <int D, bool ROT, bool QO>
__device__ __forceinline__ void prep_q_body(const _Float16* __restrict__ q, const Act& act,
                                            const Seqs& seqs, int64_t Qpad,
                                            int8_t* __restrict__ q8, float* __restrict__ qs,
                                            int c, int h, int s, int8_t* frag, int qblk,
                                            const float* __restrict__ qopart, int Hkv, int Gq,
                                            int npart, int tpw, QoShared<D>& qsh) {
  __shared__ float rowmax[QCH];
  constexpr int G = D / 8;       // lanes per row
  constexpr int RPP = 256 / G;   // rows per pass
  constexpr int NP = QCH / RPP;  // rows per thread
  int64_t start;
  int L;
  seqs.bounds(s, start, L);
  const int r0 = c * QCH;
  // Chunks up to the end of the sequence's last BQ-row query tile: rows past the
  // sequence end within that tile are written too (zero codes, scale 0).
  if (r0 >= (L + BQ - 1) / BQ * BQ) return;
  const int lc = threadIdx.x % G, rsub = threadIdx.x / G;
  const int64_t slot = (int64_t)h * Qpad + Seqs::qpstart(s, start) + r0;
  bool out_ch[8] = {};
  if constexpr (QO) {
    const int nt = (L + TK - 1) / TK;
    select_outliers<D>(qopart + ((int64_t)s * Hkv + h / Gq) * npart * D, (nt + tpw - 1) / tpw,
                       qsh, nullptr);
#pragma unroll
    for (int j = 0; j < 8; ++j) out_ch[j] = qsh.slot[lc * 8 + j] >= 0;
  }

  v8h xr[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = r0 + i * RPP + rsub;
    if (t < L) xr[i] = *reinterpret_cast<const v8h*>(q + act.off(start, h, t) + lc * 8);
  }
  float x[NP][8], amax[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int n = i * RPP + rsub;
    const bool real = r0 + n < L;
    amax[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[i][j] = (real && !out_ch[j]) ? (float)xr[i][j] : 0.0f;
    if constexpr (ROT) fwht_row<G>(x[i], lc);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax[i] = fmaxf(amax[i], fabsf(x[i][j]));
    amax[i] = group_max<G>(amax[i]);
  }
  if (qblk) {
    // The block maxima through LDS (a max is exact in any order).
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (lc == 0) rowmax[i * RPP + rsub] = amax[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int b0 = (i * RPP + rsub) & ~31;
      float m = 0.0f;
      for (int r = 0; r < 32; ++r) m = fmaxf(m, rowmax[b0 + r]);
      amax[i] = m;
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int n = i * RPP + rsub;
    const bool real = r0 + n < L;
    const RowQ rq(real ? row_scale(amax[i], 24) : 0.0f);
    const uint2 codes = real ? rq.pack8(x[i]) : make_uint2(0u, 0u);
    *reinterpret_cast<uint2*>(frag + (n >> 5) * 32 * D + qfrag_off(n & 31, lc * 8)) = codes;
    if (lc == 0) qs[slot + n] = rq.s;
  }
  __syncthreads();
  const v4i* src = reinterpret_cast<const v4i*>(frag);
  v4i* dst = reinterpret_cast<v4i*>(q8 + slot * D);
  for (int k = threadIdx.x; k < QCH * D / 16; k += 256) dst[k] = src[k];
}

// Launch 2: blocks [0, nk) quantize K, blocks [nk, 2 nk) prepare V (both over (part,
// kv head, sequence)) and the remaining blocks prepare the Q rows (over (row chunk,
// query head, sequence)).  The K workgroups come first: each reduces the partial sums
// to the mean before it streams its rows, and the V and Q streams fill the machine
// meanwhile.
template <int D>
union PrepShared {
  PrepKShared<D> k;
  PrepVShared<D> v;
  struct {
    __attribute__((aligned(16))) int8_t frag[QCH * D];
    QoShared<D> qo;
  } q;
};

template <int D, bool ROT, bool VCH, bool QO>
__global__ __launch_bounds__(256) void prep_kvq_kernel(
    const _Float16* __restrict__ q, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, Act aq, Act akv, Seqs seqs, int Hq, int Hkv, int npart,
    int tpw, int64_t Ppad, int64_t Qpad, int nqc, const int64_t* __restrict__ kpart,
    const float* __restrict__ vpart, float* __restrict__ kmean_ws, float* __restrict__ svc_ws,
    float* __restrict__ sv_ws, char* __restrict__ tiles, int8_t* __restrict__ q8,
    float* __restrict__ qs, int nk, int qblk, const float* __restrict__ qopart,
    int32_t* __restrict__ ochan_ws) {
  __shared__ PrepShared<D> sh;
  constexpr int tstride = tile_bytes(D, QO);
  int b = blockIdx.x;
  if (b < 2 * nk) {
    const bool is_v = b >= nk;
    if (is_v) b -= nk;
    const int c = b % npart;
    b /= npart;
    if (is_v)
      prep_v_body<D, VCH>(v, akv, seqs, Hkv, npart, tpw, Ppad, vpart, svc_ws, sv_ws, tiles,
                          tstride, c, b % Hkv, b / Hkv, sh.v);
    else
      prep_k_body<D, ROT, QO>(k, akv, seqs, Hkv, npart, tpw, Ppad, kpart, kmean_ws, qopart,
                              ochan_ws, tiles, tstride, c, b % Hkv, b / Hkv, sh.k);
  } else {
    b -= 2 * nk;
    const int c = b % nqc;
    b /= nqc;
    prep_q_body<D, ROT, QO>(q, aq, seqs, Qpad, q8, qs, c, b % Hq, b / Hq, sh.q.frag, qblk, qopart,
                            Hkv, Hq / Hkv, npart, tpw, sh.q.qo);
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

// Launches of the preparation.  With k/v (PH_KV): launch 1 sums K (and with VCH takes
// the V channel maxima), launch 2 quantizes K and prepares V; with q (PH_Q) the Q rows
// ride in launch 2.  ROT: the K and Q rows are Hadamard-rotated before they are
// quantized.
template <int D, bool ROT, bool VCH, bool QO>
static hipError_t prep_d(const FwdGeom& g, const WsPlan& p, void* ws, bool kv, bool qq,
                         hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  const Act akv = act_of(g, g.Hkv), aq = act_of(g, g.Hq);
  Seqs sq{g.cu, g.S, g.max_len, g.T};
  const int64_t nk = kv ? (int64_t)p.npart * g.Hkv * g.nseq : 0;
  const int nqc = (g.max_len + BQ - 1) / BQ * (BQ / QCH);
  const int64_t nq = qq ? (int64_t)nqc * g.Hq * g.nseq : 0;
  if (2 * nk + nq > 0x7fffffff) return hipErrorInvalidValue;
  const _Float16* kp = static_cast<const _Float16*>(g.k);
  const _Float16* vp = static_cast<const _Float16*>(g.v);
  float* vpart = reinterpret_cast<float*>(w + p.off_vpart);
  float* qopart = reinterpret_cast<float*>(w + p.off_qopart);
  const _Float16* qp = static_cast<const _Float16*>(g.q);
  if (kv)
    prep_ksum_kernel<D, VCH, QO><<<dim3((unsigned)nk), 256, 0, stream>>>(
        kp, vp, akv, sq, g.Hkv, p.npart, p.tpw, reinterpret_cast<int64_t*>(w + p.off_kpart),
        vpart, qp, aq, g.Hq / g.Hkv, qopart);
  if (2 * nk + nq > 0)
    prep_kvq_kernel<D, ROT, VCH, QO><<<dim3((unsigned)(2 * nk + nq)), 256, 0, stream>>>(
        static_cast<const _Float16*>(g.q), kp, vp, aq, akv, sq, g.Hq, g.Hkv, p.npart, p.tpw,
        p.Ppad, p.Qpad, nqc, reinterpret_cast<const int64_t*>(w + p.off_kpart), vpart,
        reinterpret_cast<float*>(w + p.off_kmean), reinterpret_cast<float*>(w + p.off_svc),
        reinterpret_cast<float*>(w + p.off_sv), w + p.off_tiles,
        reinterpret_cast<int8_t*>(w + p.off_q8), reinterpret_cast<float*>(w + p.off_qs),
        (int)nk, g.qblk, qopart, reinterpret_cast<int32_t*>(w + p.off_ochan));
  return hipGetLastError();
}

// The variants of one head dim.  Q outlier detection comes without the rotation and
// for D <= 128 only (the caller checks).
template <int D>
static hipError_t prep_dispatch(const FwdGeom& g, const WsPlan& p, void* ws, bool kv, bool qq,
                                hipStream_t stream) {
  if (g.qout) {
    if constexpr (D <= 128) {
      if (g.rot) return hipErrorInvalidValue;
      return g.vch ? prep_d<D, false, true, true>(g, p, ws, kv, qq, stream)
                   : prep_d<D, false, false, true>(g, p, ws, kv, qq, stream);
    }
    return hipErrorInvalidValue;
  }
  if (g.vch)
    return g.rot ? prep_d<D, true, true, false>(g, p, ws, kv, qq, stream)
                 : prep_d<D, false, true, false>(g, p, ws, kv, qq, stream);
  return g.rot ? prep_d<D, true, false, false>(g, p, ws, kv, qq, stream)
               : prep_d<D, false, false, false>(g, p, ws, kv, qq, stream);
}

hipError_t launch_prep(const FwdGeom& g, const WsPlan& p, void* ws, bool kv, bool qq,
                       hipStream_t stream) {
  if (g.max_len == 0) return hipSuccess;  // every sequence is empty
  switch (g.D) {
#define I8A_PREP(DD)                                                              \
  case DD:                                                                        \
    return prep_dispatch<DD>(g, p, ws, kv, qq, stream);
    I8A_PREP(32) I8A_PREP(64) I8A_PREP(128) I8A_PREP(256)
#undef I8A_PREP
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_ksum_dense(const void* k, int32_t B, int32_t Hkv, int32_t S, int32_t D,
                             int32_t npart, int32_t tpw, int64_t* kpart, hipStream_t stream) {
  Act a;
  a.seq_unit = (int64_t)Hkv * D;
  a.head_stride = (int64_t)S * D;
  a.tok_stride = D;
  Seqs sq{nullptr, S, S, (int64_t)B * S};
  const int64_t nb = (int64_t)npart * Hkv * B;
  if (nb == 0) return hipSuccess;
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  const _Float16* kp = static_cast<const _Float16*>(k);
  switch (D) {
#define I8A_KS(DD)                                                                      \
  case DD:                                                                              \
    prep_ksum_kernel<DD, false><<<dim3((unsigned)nb), 256, 0, stream>>>(             \
        kp, nullptr, a, sq, Hkv, npart, tpw, kpart, nullptr);                           \
    break;
    I8A_KS(32) I8A_KS(64) I8A_KS(128) I8A_KS(256)
#undef I8A_KS
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace i8a
