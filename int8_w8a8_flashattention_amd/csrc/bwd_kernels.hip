// bwd_kernels.hip - backward of the differentiable int8 attention on gfx950 (the
// Attention kernels table's attn_bwd row: a gradient-checked backward on full fp16
// state).  The quantization of the forward is taken as the identity, so this is the
// gradient of exact attention at the fp16 inputs:
//   P = softmax(s Q K^T + mask),  dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
//   dS = P * (dP - D),  dQ = s dS K,  dK = s dS^T Q      (GQA: dK, dV summed over the
//                                                         group's query heads)
// in O(S) memory: P is recomputed tile by tile, FlashAttention-2 style, from its
// row log-sum-exp.  Every product runs on v_mfma_f32_32x32x16_f16 (fp16 operands, fp32
// accumulation); P and dS are rounded to fp16 as MFMA operands.
//
// Launch 1 (bwd_prep_kernel) writes Q, K, V and dO into the workspace in two operand
// orders for 32-token blocks:
//   row fragments (R): lane l holds token l % 32, channels 16 kd + 8 (l / 32) + 0..7 of
//     a 16-channel slice kd: the A or B operand of a product contracting over d;
//   column fragments (C): lane l holds channel 32 db + l % 32 of the 8 tokens
//     16 tg + vkey(l / 32, 0..7) of a 16-token group tg: the A operand of a product
//     contracting over tokens, in the order in which a 32x32 MFMA result holds its
//     rows, so that a result (P or dS) is the B operand of the next product as it is.
// Launch 2 (bwd_dq_kernel, lane = query): sweep 1 over the keys gives each row's
//   log-sum-exp and D; sweep 2 recomputes P and dS and accumulates dQ^T = K^T dS^T.
// Launch 3 (bwd_dkdv_kernel, lane = key): four waves take the group's query heads in
//   turn for the same 32 keys and accumulate dV^T = dO^T P and dK^T = Q^T dS; the
//   waves' sums are added in LDS.
#include <float.h>

#include "i8a_device.h"
#include "i8a_launch.h"

namespace i8a {

namespace {

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

}  // namespace

// ----------------------------------------------------------------------------------
// Launch 1: one workgroup per 32-token block of one (batch, head) of one tensor.
// Tensor t: 0 = Q, 1 = dO (Hq heads), 2 = K, 3 = V (Hkv heads).  R fragments for all
// four, C fragments for Q, dO and K.  Tokens past S are zero.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const _Float16* __restrict__ q,
                                                       const _Float16* __restrict__ dout,
                                                       const _Float16* __restrict__ k,
                                                       const _Float16* __restrict__ v, int B,
                                                       int Hq, int Hkv, int S, int nrb,
                                                       _Float16* __restrict__ qr,
                                                       _Float16* __restrict__ qc,
                                                       _Float16* __restrict__ dor,
                                                       _Float16* __restrict__ doc,
                                                       _Float16* __restrict__ kr,
                                                       _Float16* __restrict__ kc,
                                                       _Float16* __restrict__ vr) {
  __shared__ __attribute__((aligned(16))) _Float16 blk[32 * (D + 8)];
  constexpr int LD = D + 8;  // padded row (halves)
  int id = blockIdx.x;
  const int rb = id % nrb;
  id /= nrb;
  const int nq = B * Hq;
  int t, bh;
  if (id < 2 * nq) {
    t = id / nq;
    bh = id % nq;
  } else {
    id -= 2 * nq;
    t = 2 + id / (B * Hkv);
    bh = id % (B * Hkv);
  }
  const _Float16* src = t == 0 ? q : t == 1 ? dout : t == 2 ? k : v;
  _Float16* rdst = t == 0 ? qr : t == 1 ? dor : t == 2 ? kr : vr;
  _Float16* cdst = t == 0 ? qc : t == 1 ? doc : t == 2 ? kc : nullptr;
  const int64_t Sp = (int64_t)nrb * 32;
  src += (int64_t)bh * S * D;
  rdst += ((int64_t)bh * Sp + (int64_t)rb * 32) * D;
  if (cdst) cdst += ((int64_t)bh * Sp + (int64_t)rb * 32) * D;

  // The block's rows into LDS (16-byte chunks), zero past S.
  for (int c = threadIdx.x; c < 32 * D / 8; c += 256) {
    const int r = c / (D / 8), d0 = (c % (D / 8)) * 8;
    const int tok = rb * 32 + r;
    v8h x;
    if (tok < S) {
      x = *reinterpret_cast<const v8h*>(src + (int64_t)tok * D + d0);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = (_Float16)0.0f;
    }
    *reinterpret_cast<v8h*>(blk + r * LD + d0) = x;
  }
  __syncthreads();
  // R fragments: chunk c = kd * 64 + lane.
  for (int c = threadIdx.x; c < 32 * D / 8; c += 256) {
    const int kd = c >> 6, lane = c & 63;
    const int r = lane & 31, d0 = 16 * kd + 8 * (lane >> 5);
    reinterpret_cast<v8h*>(rdst)[c] = *reinterpret_cast<const v8h*>(blk + r * LD + d0);
  }
  // C fragments: chunk c = (tgl * D/32 + db) * 64 + lane.
  if (cdst) {
    for (int c = threadIdx.x; c < 32 * D / 8; c += 256) {
      const int lane = c & 63, db = (c >> 6) % (D / 32), tgl = (c >> 6) / (D / 32);
      const int d = 32 * db + (lane & 31), hv = lane >> 5;
      v8h x;
#pragma unroll
      for (int jv = 0; jv < 8; ++jv) x[jv] = blk[(16 * tgl + ckey(hv, jv)) * LD + d];
      reinterpret_cast<v8h*>(cdst)[c] = x;
    }
  }
}

// ----------------------------------------------------------------------------------
// Launch 2: dQ.  Workgroup = 4 waves = 128 queries of one (batch, query head); wave w
// owns queries q0 = 128 * blockIdx.x + 32 w .. +31, lane l query q0 + l % 32.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_kernel(
    const _Float16* __restrict__ qr, const _Float16* __restrict__ dor,
    const _Float16* __restrict__ kr, const _Float16* __restrict__ kc,
    const _Float16* __restrict__ vr, float* __restrict__ lse2, float* __restrict__ dvec,
    float* __restrict__ dq, int Hq, int Hkv, int S, int nrb, float c_log2, float scale) {
  constexpr int NKD = D / 16, NDB = D / 32;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, m = lane & 31, hh = lane >> 5;
  const int q0 = 128 * blockIdx.x + 32 * w;
  if (q0 >= nrb * 32) return;  // a wave entirely in the padding of the last block
  const int64_t Sp = (int64_t)nrb * 32;
  const int64_t qbase = ((int64_t)b * Hq + h) * Sp;
  const int64_t kbase = ((int64_t)b * Hkv + g) * Sp;
  const v8h* qf_src = reinterpret_cast<const v8h*>(qr + (qbase + q0) * D);
  const v8h* df_src = reinterpret_cast<const v8h*>(dor + (qbase + q0) * D);
  v8h qf[NKD], df[NKD];
#pragma unroll
  for (int kd = 0; kd < NKD; ++kd) {
    qf[kd] = qf_src[kd * 64 + lane];
    df[kd] = df_src[kd * 64 + lane];
  }
  const int qi = q0 + m;
  const int nkb = CAUSAL ? q0 / 32 + 1 : nrb;

  // S^T (keys x queries) and dP^T of key block kb, scaled and masked scores in t.
  auto scores = [&](int kb, float (&t)[16], v16f& dp) {
    const v8h* ka = reinterpret_cast<const v8h*>(kr + (kbase + 32 * kb) * D);
    const v8h* va = reinterpret_cast<const v8h*>(vr + (kbase + 32 * kb) * D);
    v16f sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.0f;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      sc = mfma16(ka[kd * 64 + lane], qf[kd], sc);
      dp = mfma16(va[kd * 64 + lane], df[kd], dp);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
      const bool dead = key >= S || (CAUSAL && key > qi);
      t[i] = dead ? -INFINITY : sc[i] * c_log2;
    }
  };

  // Sweep 1: running max, sum and sum of p * dP (log2 units).
  float mr = -INFINITY, l = 0.0f, a = 0.0f;
  for (int kb = 0; kb < nkb; ++kb) {
    float t[16];
    v16f dp;
    scores(kb, t, dp);
    float mt = t[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = bmax(mt, t[i]);
    const float mn = bmax(mr, half_max(mt));
    const float al = mr == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mr - mn);
    const float mu = mn == -INFINITY ? 0.0f : mn;
    l *= al;
    a *= al;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(t[i] - mu);
      l += p;
      a = __builtin_fmaf(p, dp[i], a);
    }
    mr = mn;
  }
  l = half_sum(l);
  a = half_sum(a);
  // Every row has a visible key (key 0), so l > 0 and mr is finite.
  const float lse = mr + log2f(l);
  const float Dv = a / l;
  if (hh == 0) {
    lse2[qbase + qi] = lse;
    dvec[qbase + qi] = Dv;
  }

  // Sweep 2: P, dS and dQ^T = K^T dS^T.
  v16f acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
  for (int kb = 0; kb < nkb; ++kb) {
    float t[16];
    v16f dp;
    scores(kb, t, dp);
    v8h ds[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(t[i] - lse);
      ds[i >> 3][i & 7] = (_Float16)(p * (dp[i] - Dv));
    }
    const v8h* kca = reinterpret_cast<const v8h*>(kc + (kbase + 32 * kb) * D);
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = mfma16(kca[(gg * NDB + db) * 64 + lane], ds[gg], acc[db]);
  }
  if (qi < S) {
    float* orow = dq + (((int64_t)b * Hq + h) * S + qi) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        v4f o4;
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = acc[db][4 * J + r] * scale;
        *reinterpret_cast<v4f*>(orow + 32 * db + 8 * J + 4 * hh) = o4;
      }
  }
}

// ----------------------------------------------------------------------------------
// Launch 3: dK and dV.  Workgroup = 4 waves on the 32 keys k0 = 32 * blockIdx.x .. +31
// of one (batch, kv head); wave w takes the group's query heads w, w + 4, ...; lane l
// holds key k0 + l % 32.  The waves' partial dK^T, dV^T are added in LDS at the end.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    const _Float16* __restrict__ qr, const _Float16* __restrict__ qc,
    const _Float16* __restrict__ dor, const _Float16* __restrict__ doc,
    const _Float16* __restrict__ kr, const _Float16* __restrict__ vr,
    const float* __restrict__ lse2, const float* __restrict__ dvec, float* __restrict__ dk,
    float* __restrict__ dv, int Hq, int Hkv, int S, int nrb, float c_log2, float scale) {
  constexpr int NKD = D / 16, NDB = D / 32;
  __shared__ float red[32 * D];
  const int g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, m = lane & 31, hh = lane >> 5;
  const int k0 = 32 * blockIdx.x;
  const int64_t Sp = (int64_t)nrb * 32;
  const int64_t kbase = ((int64_t)b * Hkv + g) * Sp;
  const v8h* kf_src = reinterpret_cast<const v8h*>(kr + (kbase + k0) * D);
  const v8h* vf_src = reinterpret_cast<const v8h*>(vr + (kbase + k0) * D);
  v8h kf[NKD], vf[NKD];
#pragma unroll
  for (int kd = 0; kd < NKD; ++kd) {
    kf[kd] = kf_src[kd * 64 + lane];
    vf[kd] = vf_src[kd * 64 + lane];
  }
  const int kj = k0 + m;
  v16f accv[NDB], acck[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) accv[db][i] = acck[db][i] = 0.0f;

  const int qb0 = CAUSAL ? k0 / 32 : 0;
  for (int hg = w; hg < G; hg += 4) {
    const int h = g * G + hg;
    const int64_t qbase = ((int64_t)b * Hq + h) * Sp;
    for (int qb = qb0; qb < nrb; ++qb) {
      const v8h* qa = reinterpret_cast<const v8h*>(qr + (qbase + 32 * qb) * D);
      const v8h* da = reinterpret_cast<const v8h*>(dor + (qbase + 32 * qb) * D);
      v16f sc, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.0f;
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) {
        sc = mfma16(qa[kd * 64 + lane], kf[kd], sc);
        dp = mfma16(da[kd * 64 + lane], vf[kd], dp);
      }
      // Register i holds query 32 qb + 8 (i / 4) + 4 hh + i % 4.
      v8h p16[2], ds16[2];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const int qrow = 32 * qb + 8 * J + 4 * hh;
        const v4f lv = *reinterpret_cast<const v4f*>(lse2 + qbase + qrow);
        const v4f dv4 = *reinterpret_cast<const v4f*>(dvec + qbase + qrow);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * J + r;
          const bool dead = CAUSAL && kj > qrow + r;
          const float p = dead ? 0.0f : __builtin_amdgcn_exp2f(sc[i] * c_log2 - lv[r]);
          p16[i >> 3][i & 7] = (_Float16)p;
          ds16[i >> 3][i & 7] = (_Float16)(p * (dp[i] - dv4[r]));
        }
      }
      const v8h* dca = reinterpret_cast<const v8h*>(doc + (qbase + 32 * qb) * D);
      const v8h* qca = reinterpret_cast<const v8h*>(qc + (qbase + 32 * qb) * D);
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          accv[db] = mfma16(dca[(gg * NDB + db) * 64 + lane], p16[gg], accv[db]);
          acck[db] = mfma16(qca[(gg * NDB + db) * 64 + lane], ds16[gg], acck[db]);
        }
    }
  }

  // Sum of the four waves: dV^T, then dK^T, through red[key][d] (wave 0 stores, the
  // others add in turn).
  auto reduce_store = [&](v16f (&acc)[NDB], float* out, float mul) {
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      if (w == ww) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int d = 32 * db + 8 * (i >> 2) + 4 * hh + (i & 3);
            float* cell = red + m * D + d;
            *cell = ww == 0 ? acc[db][i] : *cell + acc[db][i];
          }
      }
      __syncthreads();
    }
    for (int e = threadIdx.x; e < 32 * D; e += 256) {
      const int key = k0 + e / D;
      if (key < S) out[(((int64_t)b * Hkv + g) * S + key) * D + e % D] = red[e] * mul;
    }
    __syncthreads();
  };
  reduce_store(accv, dv, 1.0f);
  reduce_store(acck, dk, scale);
}

// ----------------------------------------------------------------------------------
static size_t align256b(size_t x) { return (x + 255) & ~(size_t)255; }

BwdPlan plan_bwd(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D) {
  BwdPlan p;
  p.nrb = (S + 31) / 32;
  const int64_t Sp = (int64_t)p.nrb * 32;
  const int64_t S128 = (int64_t)((S + 127) / 128) * 128;
  const size_t qbytes = (size_t)B * Hq * Sp * D * 2, kbytes = (size_t)B * Hkv * Sp * D * 2;
  size_t off = 0;
  p.off_qr = off; off = align256b(off + qbytes);
  p.off_qc = off; off = align256b(off + qbytes);
  p.off_dor = off; off = align256b(off + qbytes);
  p.off_doc = off; off = align256b(off + qbytes);
  p.off_kr = off; off = align256b(off + kbytes);
  p.off_kc = off; off = align256b(off + kbytes);
  p.off_vr = off; off = align256b(off + kbytes);
  p.off_lse = off; off = align256b(off + (size_t)B * Hq * S128 * 4);
  p.off_dvec = off; off = align256b(off + (size_t)B * Hq * S128 * 4);
  p.total = off;
  return p;
}

template <int D, bool C>
static hipError_t bwd_d(const BwdArgs& a, const BwdPlan& p, char* ws, hipStream_t stream) {
  const int64_t nprep = (int64_t)p.nrb * (2 * a.B * a.Hq + 2 * a.B * a.Hkv);
  if (nprep > 0x7fffffff) return hipErrorInvalidValue;
  auto H = [&](size_t off) { return reinterpret_cast<_Float16*>(ws + off); };
  bwd_prep_kernel<D><<<dim3((unsigned)nprep), 256, 0, stream>>>(
      static_cast<const _Float16*>(a.q), static_cast<const _Float16*>(a.dout),
      static_cast<const _Float16*>(a.k), static_cast<const _Float16*>(a.v), a.B, a.Hq, a.Hkv,
      a.S, p.nrb, H(p.off_qr), H(p.off_qc), H(p.off_dor), H(p.off_doc), H(p.off_kr),
      H(p.off_kc), H(p.off_vr));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float c_log2 = a.softmax_scale * 1.4426950408889634f;
  float* lse = reinterpret_cast<float*>(ws + p.off_lse);
  float* dvec = reinterpret_cast<float*>(ws + p.off_dvec);
  bwd_dq_kernel<D, C><<<dim3((unsigned)((a.S + 127) / 128), a.Hq, a.B), 256, 0, stream>>>(
      H(p.off_qr), H(p.off_dor), H(p.off_kr), H(p.off_kc), H(p.off_vr), lse, dvec, a.dq, a.Hq,
      a.Hkv, a.S, p.nrb, c_log2, a.softmax_scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_dkdv_kernel<D, C><<<dim3((unsigned)p.nrb, a.Hkv, a.B), 256, 0, stream>>>(
      H(p.off_qr), H(p.off_qc), H(p.off_dor), H(p.off_doc), H(p.off_kr), H(p.off_vr), lse,
      dvec, a.dk, a.dv, a.Hq, a.Hkv, a.S, p.nrb, c_log2, a.softmax_scale);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& p, void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
#define I8A_BWD(DD)                                                  \
  case DD:                                                           \
    return a.causal ? bwd_d<DD, true>(a, p, w, stream)               \
                    : bwd_d<DD, false>(a, p, w, stream);
  switch (a.D) {
    I8A_BWD(32) I8A_BWD(64) I8A_BWD(128)
    default:
      return hipErrorInvalidValue;
  }
#undef I8A_BWD
}

}  // namespace i8a
