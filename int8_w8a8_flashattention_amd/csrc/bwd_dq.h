// bwd_dq.h - the backward's dQ kernel (launch 2 of attn_bwd), instantiated in
// bwd_dq_kernels.hip (D <= 128, products' results in vector registers) and in
// bwd_dq256_kernels.hip (D = 256, whose operands and accumulators exceed the vector
// registers, so its results stay in the accumulation registers).
#pragma once

#include <float.h>

#include "bwd_common.h"
#include "i8a_launch.h"

namespace i8a {
namespace bwd {

// Waves per dQ workgroup (32 queries each); the key blocks' tiles in LDS serve them all.
// At D = 256 a wave needs more than half of a SIMD's registers, so four.
template <int D>
constexpr int dq_waves() {
  return D <= 128 ? 8 : 4;
}

// ----------------------------------------------------------------------------------
// Launch 2: dQ.  Workgroup = dq_waves<D>() waves of 32 queries of one (batch, query
// head); wave w owns queries q0 = qblk0 + 32 w .. +31, lane l query q0 + l % 32.  The key
// blocks' operand tiles (K and V in row order, K in column order) stream through a
// two-stage LDS ring shared by the workgroup's waves, one block ahead.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * dq_waves<D>()) void bwd_dq_kernel(
    const _Float16* __restrict__ qr, const _Float16* __restrict__ dor,
    const _Float16* __restrict__ kr, const _Float16* __restrict__ kc,
    const _Float16* __restrict__ vr, float* __restrict__ lse2, float* __restrict__ dvec,
    float* __restrict__ dq, int B, int Hq, int Hkv, int S, int nrb, float c_log2, float scale) {
  constexpr int NKD = D / 16, NDB = D / 32, TB = 64 * D;  // TB: bytes of a 32-token tile
  // The key blocks' tiles (two stages of K rows, V rows and K columns); afterwards the
  // waves' output staging areas.
  constexpr int EQ = 32;  // channels per output pass
  constexpr int SMEM = 2 * 3 * TB > dq_waves<D>() * staging_bytes<EQ>()
                           ? 2 * 3 * TB
                           : dq_waves<D>() * staging_bytes<EQ>();
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  // blockIdx.x = ((group of 32 dq_waves<D>() queries, from the last) x B + batch) x Hq
  // + head: under the causal mask the heaviest groups of every head are dispatched first.
  const int h = blockIdx.x % Hq, b = (blockIdx.x / Hq) % B;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, m = lane & 31, hh = lane >> 5;
  const int qblk0 =
      32 * dq_waves<D>() * ((nrb + dq_waves<D>() - 1) / dq_waves<D>() - 1 - (int)(blockIdx.x / Hq / B));
  const int q0 = qblk0 + 32 * w;
  const bool active = q0 < nrb * 32;  // waves past the padded length only copy
  const int64_t Sp = (int64_t)nrb * 32;
  const int64_t qbase = ((int64_t)b * Hq + h) * Sp;
  const int64_t kbase = ((int64_t)b * Hkv + g) * Sp;
  const char* krb = reinterpret_cast<const char*>(kr + kbase * D);
  const char* vrb = reinterpret_cast<const char*>(vr + kbase * D);
  const char* kcb = reinterpret_cast<const char*>(kc + kbase * D);
  const int nkb_wg = CAUSAL ? min(nrb, qblk0 / 32 + dq_waves<D>()) : nrb;  // the group's key blocks
  const int nkb = CAUSAL ? q0 / 32 + 1 : nrb;                  // this wave's
  const int qi = q0 + m;

  v8h qf[NKD], df[NKD];
  if (active) {
    const v8h* qs = reinterpret_cast<const v8h*>(qr + (qbase + q0) * D);
    const v8h* ds = reinterpret_cast<const v8h*>(dor + (qbase + q0) * D);
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      qf[kd] = qs[kd * 64 + lane];
      df[kd] = ds[kd * 64 + lane];
    }
  } else {
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[kd][j] = df[kd][j] = (_Float16)0.0f;
  }
  // Consumed here, so that the compiler waits for these loads before the loops (a wait
  // at their first use inside a loop would also wait for the tile copies).
#pragma unroll
  for (int kd = 0; kd < NKD; ++kd) asm volatile("" : : "v"(qf[kd]), "v"(df[kd]));

  const TileCopy<D, 64 * dq_waves<D>()> copy(tid);
  auto issue = [&](int kb, int st, bool with_kc) {
    copy(krb + (int64_t)kb * TB, smem + (st * 3 + 0) * TB);
    copy(vrb + (int64_t)kb * TB, smem + (st * 3 + 1) * TB);
    if (with_kc) copy(kcb + (int64_t)kb * TB, smem + (st * 3 + 2) * TB);
  };
  // S^T (keys x queries) and dP^T of key block kb from LDS stage st.
  auto scores = [&](int st, v16f& sc, v16f& dp) {
    const v8h* ka = reinterpret_cast<const v8h*>(smem + (st * 3 + 0) * TB);
    const v8h* va = reinterpret_cast<const v8h*>(smem + (st * 3 + 1) * TB);
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.0f;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      sc = mfma16(ka[kd * 64 + lane], qf[kd], sc);
      dp = mfma16(va[kd * 64 + lane], df[kd], dp);
    }
  };
  // Masked scores to -inf.  Only a block that reaches past this wave's first query
  // (causal) or past the sequence holds masked pairs, so the others skip the compares
  // (a wave-uniform branch).  The scale c_log2 > 0 is applied later, inside the
  // exponent's argument, which keeps -inf.
  auto mask = [&](int kb, v16f& sc) {
    if ((CAUSAL && 32 * kb + 31 > q0) || 32 * kb + 32 > S) {
      // Keeps this path a branch: without a statement that cannot be executed
      // speculatively, the compiler turns it into selects that every block executes.
      asm volatile("");
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (key >= S || (CAUSAL && key > qi)) sc[i] = -INFINITY;
      }
    }
  };

  // Sweep 1: running max, sum and sum of p * dP (log2 units).
  float mr = -INFINITY, l = 0.0f, a = 0.0f;
  issue(0, 0, false);
  vm_wait<0>();
  __syncthreads();
  for (int kb = 0; kb < nkb_wg; ++kb) {
    if (kb + 1 < nkb_wg) issue(kb + 1, (kb + 1) & 1, false);
    if (active && kb < nkb) {
      v16f sc, dp;
      scores(kb & 1, sc, dp);
      mask(kb, sc);
      float mt = sc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = bmax(mt, sc[i]);
      // Every block of this wave holds a visible key for each of its rows, so mn is
      // finite from the first block on.
      const float mn = bmax(mr, half_max(mt) * c_log2);
      const float al = mr == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mr - mn);
      l *= al;
      a *= al;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c_log2, -mn));
        l += p;
        a = __builtin_fmaf(p, dp[i], a);
      }
      mr = mn;
    }
    vm_wait<0>();
    __syncthreads();
  }
  l = half_sum(l);
  a = half_sum(a);
  // Every row has a visible key (key 0), so l > 0 and mr is finite.
  const float lse = active ? mr + log2f(l) : 0.0f;
  const float Dv = active ? a / l : 0.0f;
  if (active && hh == 0) {
    lse2[qbase + qi] = lse;
    dvec[qbase + qi] = Dv;
  }

  // Sweep 2: P, dS and dQ^T = K^T dS^T.
  v16f acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
  issue(0, 0, true);
  vm_wait<0>();
  __syncthreads();
  for (int kb = 0; kb < nkb_wg; ++kb) {
    if (kb + 1 < nkb_wg) issue(kb + 1, (kb + 1) & 1, true);
    // Unconditional, as in the dK/dV kernel: past this wave's last key block every score
    // is masked and dS is zero (a wave past the padded length has zero operands, lse = 0
    // and D = 0, so dS is zero too).
    {
      v16f sc, dp;
      scores(kb & 1, sc, dp);
      mask(kb, sc);
      v8h ds[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c_log2, -lse));
        ds[i >> 3][i & 7] = (_Float16)(p * (dp[i] - Dv));
      }
      const v8h* kca = reinterpret_cast<const v8h*>(smem + ((kb & 1) * 3 + 2) * TB);
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = mfma16(kca[(gg * NDB + db) * 64 + lane], ds[gg], acc[db]);
    }
    vm_wait<0>();
    __syncthreads();
  }
  // The loop's last barrier leaves the tile stages unused: they stage the output.
  store_rows_f32<D, EQ>(acc, scale, smem + w * staging_bytes<EQ>(),
                        dq + (((int64_t)b * Hq + h) * S + q0) * D, active ? min(32, S - q0) : 0,
                        lane);
}


template <int D, bool C>
static hipError_t dq_d(const BwdArgs& a, const BwdPlan& p, char* ws, hipStream_t stream) {
  const int64_t ngrp = (p.nrb + dq_waves<D>() - 1) / dq_waves<D>();
  if (ngrp * a.B * a.Hq > 0x7fffffff) return hipErrorInvalidValue;
  auto H = [&](size_t off) { return reinterpret_cast<_Float16*>(ws + off); };
  bwd_dq_kernel<D, C><<<dim3((unsigned)(ngrp * a.B * a.Hq)), 64 * dq_waves<D>(), 0, stream>>>(
      H(p.off_qr), H(p.off_dor), H(p.off_kr), H(p.off_kc), H(p.off_vr),
      reinterpret_cast<float*>(ws + p.off_lse), reinterpret_cast<float*>(ws + p.off_dvec), a.dq,
      a.B, a.Hq, a.Hkv, a.S, p.nrb, a.softmax_scale * 1.4426950408889634f, a.softmax_scale);
  return hipGetLastError();
}

}  // namespace bwd
}  // namespace i8a
