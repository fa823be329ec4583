// attn_kernels.hip - the INT8 W8A8 FlashAttention-2 forward on gfx950.
//
// One workgroup = 4 waves = 128 query rows of one head.  Each wave owns 32 rows and
// keeps, per lane, one query's running max, sum and 32 x D output accumulator
// column.  Per 64-key tile:
//   S^T = K . Q^T     v_mfma_i32_32x32x32_i8   (exact int32)
//   t   = f32(S^T) * sk_j                      (the query scale and softmax scale are
//   p   = exp2(t * qsc - M)                     one per-lane factor qsc)
//   O^T += V^T . P^T  v_mfma_f32_32x32x16_f16  (P rounded to fp16, V exact in fp16)
//   l   += sum of the same fp16 P values      (v_dot2_f32_f16)
// so the normalized output is a weighted mean with identical weights in numerator
// and denominator.  The running max M is only raised (with a rescale of O and l)
// when a tile's max exceeds it by more than TAU in log2 units, which bounds every
// p by 2^TAU and skips most rescales.
//
// Q, K (int8) and the exact fp16 V come from the workspace in MFMA fragment order:
// the Q fragments go straight to registers with coalesced 16-byte loads, and the K/V
// tile copy into LDS is linear, so every LDS operand read is a conflict-free 16-byte
// read.
#include <float.h>

#include "i8a_device.h"
#include "i8a_launch.h"

namespace i8a {

constexpr int BM = BQ;       // query rows per workgroup
constexpr float TAU = 8.0f;  // lazy-rescale threshold, log2 units

template <int D>
struct Lay {
  static constexpr int NKB = D / 32;             // 32-wide blocks of the head dim
  static constexpr int KB = TK * D;              // bytes of the int8 K codes
  static constexpr int VB = TK * D * 2;          // bytes of the fp16 V
  static constexpr int STAGE = tile_bytes(D);    // one pipeline stage = one tile block
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const int8_t* __restrict__ q8, const float* __restrict__ qs, int64_t Qpad,
    _Float16* __restrict__ out, Act aq, Seqs seqs, int Hq, int Hkv, int nseq, int xcd_map,
    float qk_log2, const char* __restrict__ tiles, int64_t Ppad) {
  using LY = Lay<D>;
  constexpr int NKB = LY::NKB;
  __shared__ __attribute__((aligned(16))) char smem[2 * LY::STAGE];

  int slot, s, h;
  decode_work(blockIdx.x, nseq, Hq, Hkv, xcd_map, slot, s, h);
  int64_t start;
  int L;
  seqs.bounds(s, start, L);
  const int nqt_s = (L + BM - 1) / BM;  // query tiles of this sequence
  if (slot >= nqt_s) return;
  const int qt = CAUSAL ? nqt_s - 1 - slot : slot;
  const int g = h / (Hq / Hkv);
  // The wave index is wave-uniform: readfirstlane lets the compiler see that, so the
  // per-wave tile conditions below become scalar branches.
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t pbase = Seqs::pstart(s, start);
  const char* tsrc = tiles + ((int64_t)g * (Ppad / TK) + pbase / TK) * LY::STAGE;

  const int q0 = qt * BM;
  const int qw0 = q0 + 32 * w;
  const int ntile_seq = (L + TK - 1) / TK;
  const int nt = CAUSAL ? min(ntile_seq, (min(q0 + BM, L) - 1) / TK + 1) : ntile_seq;

  // Prologue: tile 0 streams into stage 0 while the wave's 32 prepared Q rows (int8
  // fragments, one 16-byte load per lane and d block) go to registers.
  copy_tile_async<D>(tsrc, smem, tid);
  const int64_t qslot = (int64_t)h * Qpad + Seqs::qpstart(s, start) + qw0;
  v4i qf[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
    qf[kb] = reinterpret_cast<const v4i*>(q8 + qslot * D)[kb * 64 + lane];
  const float qsc = fmaxf(qs[qslot + m] * qk_log2, FLT_MIN);
  wait_vmem();
  __syncthreads();

  v16f o[NKB];
#pragma unroll
  for (int db = 0; db < NKB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  float mrun = -INFINITY, lsum = 0.0f;
  const int qi = qw0 + m;

  // One 64-key tile.  `masked`: some key of the tile lies above this wave's diagonal
  // or past the sequence end; only those tiles pay for the mask, in a uniform branch
  // of its own.  qsc > 0 (an all-zero query row has scale 0; FLT_MIN stands in for
  // it, its scores are 0 either way), so a masked score of -inf gives p = 0 and a
  // fully masked tile gives a row max of -inf without special cases.
  auto tile_step = [&](const char* st, int kt0, bool masked) {
    const v4i* kl = reinterpret_cast<const v4i*>(st);
    const v4i* vl = reinterpret_cast<const v4i*>(st + LY::KB);
    const float* skl = reinterpret_cast<const float*>(st + LY::KB + LY::VB);

    v16i acc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][i] = 0;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        acc[nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kl[(nb * NKB + kb) * 64 + lane], qf[kb],
                                                        acc[nb], 0, 0, 0);
    }
    // Register i of block nb holds key 32*nb + 8*(i/4) + 4*hh + i%4 of the tile.
    float tv[32];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const v4f skv = *reinterpret_cast<const v4f*>(skl + 32 * nb + 8 * J + 4 * hh);
#pragma unroll
        for (int r = 0; r < 4; ++r) tv[16 * nb + 4 * J + r] = (float)acc[nb][4 * J + r] * skv[r];
      }
    if (masked) {
      // Key kt0 + 4*hh + off_i is masked when off_i exceeds one per-lane bound (the
      // last visible key, causal diagonal or sequence end, relative to kt0 + 4*hh):
      // one compare and one select per score.
      const int last = (CAUSAL ? min(qi, L - 1) : L - 1) - kt0 - 4 * hh;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int off = 32 * (i >> 4) + 8 * ((i >> 2) & 3) + (i & 3);
        if (off > last) tv[i] = -INFINITY;
      }
    }

    // M is raised (with a rescale of O and l) only where the tile's max exceeds it by
    // more than TAU.  The lane max runs as two chains of v_maximum3.
    float m0 = smax(tv[0], tv[1]), m1 = smax(tv[2], tv[3]);
#pragma unroll
    for (int i = 4; i < 32; i += 4) {
      m0 = smax(smax(m0, tv[i]), tv[i + 1]);
      m1 = smax(smax(m1, tv[i + 2]), tv[i + 3]);
    }
    const float mc = other_half_max(smax(m0, m1)) * qsc;
    const bool upd = mc > mrun + TAU;
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
    // A row whose keys were all masked so far keeps M = -inf and takes its
    // probabilities against 0 (all of them are 0).
    const float muse = mrun == -INFINITY ? 0.0f : mrun;

    // p = 2^(t * qsc - M), rounded to fp16: the P^T operand of the P.V product and the
    // terms of the row sum (one v_dot2 chain).
    v8h pk[4];
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      v2f pp;
      pp[0] = __builtin_amdgcn_exp2f(__builtin_fmaf(tv[i], qsc, -muse));
      pp[1] = __builtin_amdgcn_exp2f(__builtin_fmaf(tv[i + 1], qsc, -muse));
      const v2h ph = __builtin_convertvector(pp, v2h);
      pk[i >> 3][i & 7] = ph[0];
      pk[i >> 3][(i & 7) + 1] = ph[1];
    }
    const v2h ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const v2h pr = {pk[kg][e], pk[kg][e + 1]};
        lsum = __builtin_amdgcn_fdot2(pr, ones, lsum, false);
      }

#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int db = 0; db < NKB; ++db) {
        const v4i va = vl[(kg * NKB + db) * 64 + lane];
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, va), pk[kg], o[db],
                                                        0, 0, 0);
      }
  };

  for (int j = 0; j < nt; ++j) {
    if (j + 1 < nt)
      copy_tile_async<D>(tsrc + (int64_t)(j + 1) * LY::STAGE, smem + ((j + 1) & 1) * LY::STAGE,
                         tid);
    const int kt0 = j * TK;
    if (!CAUSAL || kt0 <= qw0 + 31)
      tile_step(smem + (j & 1) * LY::STAGE, kt0,
                (CAUSAL && kt0 + TK - 1 > qw0) || kt0 + TK > L);
    wait_vmem();
    __syncthreads();
  }

  lsum = other_half_sum(lsum);
  if (qi < L) {
    const float inv = 1.0f / lsum;
    _Float16* orow = out + aq.off(start, h, qi);
#pragma unroll
    for (int db = 0; db < NKB; ++db)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        v4h o4;
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = (_Float16)(o[db][4 * J + r] * inv);
        *reinterpret_cast<v4h*>(orow + 32 * db + 8 * J + 4 * hh) = o4;
      }
  }
}

// ----------------------------------------------------------------------------------
// Debug: the int32 score tile from the forward's own prepared Q and K fragments
// (read straight from the workspace), one wave per aligned 32x32 block.
template <int D>
__global__ __launch_bounds__(64) void debug_qk_kernel(
    const int8_t* __restrict__ q8, const float* __restrict__ qs, int64_t Qpad, int S, int Hq,
    int Hkv, int b, int h, int row0, int rows, int col0, int cols,
    const char* __restrict__ tiles, const float* __restrict__ sv_ws,
    const float* __restrict__ kmean_ws, int64_t Ppad, int32_t* __restrict__ s32,
    float* __restrict__ qscale, float* __restrict__ kscale, float* __restrict__ vscale,
    float* __restrict__ kmean_out) {
  constexpr int NKB = D / 32;
  const int lane = threadIdx.x, m = lane & 31, hh = lane >> 5;
  const int qbase = (row0 & ~31) + 32 * blockIdx.x;
  const int kbase = (col0 & ~31) + 32 * blockIdx.y;
  const int64_t start = (int64_t)b * S;
  const int g = h / (Hq / Hkv);
  const int64_t pbase = Seqs::pstart(b, start);
  const int64_t qslot = (int64_t)h * Qpad + Seqs::qpstart(b, start) + qbase;

  v4i qf[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) qf[kb] = reinterpret_cast<const v4i*>(q8 + qslot * D)[kb * 64 + lane];

  const int tile0 = kbase - kbase % TK, nb = (kbase % TK) / 32;
  const char* tb = tiles + ((int64_t)g * (Ppad / TK) + (pbase + tile0) / TK) * tile_bytes(D);
  const v4i* kt = reinterpret_cast<const v4i*>(tb);
  v16i acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kt[(nb * NKB + kb) * 64 + lane], qf[kb], acc, 0,
                                                0, 0);
  const int qrow = qbase + m;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int n = kbase + 8 * (i >> 2) + 4 * hh + (i & 3);
    if (qrow >= row0 && qrow < row0 + rows && n >= col0 && n < col0 + cols)
      s32[(int64_t)(qrow - row0) * cols + (n - col0)] = acc[i];
  }
  if (qscale && blockIdx.y == 0 && hh == 0 && qrow >= row0 && qrow < row0 + rows)
    qscale[qrow - row0] = qs[qslot + m];
  const int n = kbase + m;
  if (blockIdx.x == 0 && hh == 0 && n >= col0 && n < col0 + cols) {
    if (kscale) kscale[n - col0] = reinterpret_cast<const float*>(tb + 3 * TK * D)[n - tile0];
    if (vscale) vscale[n - col0] = sv_ws[(int64_t)g * Ppad + pbase + n];
  }
  if (kmean_out && blockIdx.x == 0 && blockIdx.y == 0)
    for (int d = lane; d < D; d += 64) kmean_out[d] = kmean_ws[((int64_t)b * Hkv + g) * D + d];
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
  const int nqt = (g.max_len + BM - 1) / BM;
  const int64_t blocks = (int64_t)nqt * g.nseq * g.Hq;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int ngroups = g.nseq * g.Hkv;
  const int xcd_map = ((g.nseq * g.Hq) % 8 == 0 && ngroups % 8 == 0) ? 1 : 0;
  // Rotated Q and K rows carry H H^T = D I: an extra exact factor 1/D on the logits.
  const float qk_log2 = g.softmax_scale * 1.4426950408889634f * (g.rot ? 1.0f / g.D : 1.0f);
  Seqs sq{g.cu, g.S, g.max_len, g.T};
  attn_fwd_kernel<D, C><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      reinterpret_cast<const int8_t*>(w + p.off_q8), reinterpret_cast<const float*>(w + p.off_qs),
      p.Qpad, static_cast<_Float16*>(g.out), act_of(g, g.Hq), sq, g.Hq, g.Hkv, g.nseq, xcd_map,
      qk_log2, w + p.off_tiles, p.Ppad);
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
static hipError_t debug_d(const FwdGeom& g, const WsPlan& p, const void* ws, int b, int h,
                          int row0, int rows, int col0, int cols, int32_t* s32, float* qscale,
                          float* kscale, float* vscale, float* kmean, hipStream_t stream) {
  const char* w = static_cast<const char*>(ws);
  const int rb = ((row0 + rows - 1) >> 5) - (row0 >> 5) + 1;
  const int cb = ((col0 + cols - 1) >> 5) - (col0 >> 5) + 1;
  debug_qk_kernel<D><<<dim3(rb, cb), dim3(64), 0, stream>>>(
      reinterpret_cast<const int8_t*>(w + p.off_q8), reinterpret_cast<const float*>(w + p.off_qs),
      p.Qpad, g.S, g.Hq, g.Hkv, b, h, row0, rows, col0, cols, w + p.off_tiles,
      reinterpret_cast<const float*>(w + p.off_sv),
      reinterpret_cast<const float*>(w + p.off_kmean), p.Ppad, s32, qscale, kscale, vscale,
      kmean);
  return hipGetLastError();
}

hipError_t launch_debug_qk(const FwdGeom& g, const WsPlan& p, const void* ws, int32_t b,
                           int32_t h, int32_t row0, int32_t rows, int32_t col0, int32_t cols,
                           int32_t* s32, float* qscale, float* kscale, float* vscale,
                           float* kmean, hipStream_t stream) {
  switch (g.D) {
    case 32: return debug_d<32>(g, p, ws, b, h, row0, rows, col0, cols, s32, qscale, kscale, vscale, kmean, stream);
    case 64: return debug_d<64>(g, p, ws, b, h, row0, rows, col0, cols, s32, qscale, kscale, vscale, kmean, stream);
    case 128: return debug_d<128>(g, p, ws, b, h, row0, rows, col0, cols, s32, qscale, kscale, vscale, kmean, stream);
    case 256: return debug_d<256>(g, p, ws, b, h, row0, rows, col0, cols, s32, qscale, kscale, vscale, kmean, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace i8a
