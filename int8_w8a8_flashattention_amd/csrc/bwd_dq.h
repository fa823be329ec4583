// bwd_dq.h - the backward's dQ kernel (launch 2 of attn_bwd), instantiated in
// bwd_dq_kernels.hip (D <= 128, products' results in vector registers) and in
// bwd_dq256_kernels.hip (D = 256, whose operands and accumulators exceed the vector
// registers, so its results stay in the accumulation registers).
#pragma once

#include <float.h>

#include <type_traits>

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
// blocks' operand tiles (K and V in row order, K in column order) stream through an LDS
// ring shared by the workgroup's waves.
//   Two waves per SIMD (D <= 128): each block's products, then its vector arithmetic;
//   the two waves of a SIMD overlap one's products with the other's arithmetic (two
//   stages, the next block landing).
//   One wave per SIMD (D = 256, PIPE): both sweeps are software-pipelined over two key
//   blocks.  The step of block kb runs the score products (S^T and dP^T) of block kb + 1,
//   one per slot, beside block kb's vector arithmetic (and, in sweep 2, block kb's dQ
//   products), while block kb + 2 lands in a third stage.  With two waves per SIMD this
//   schedule measured slower: a wave that mixes products and arithmetic overlaps less
//   with its neighbour than two waves that alternate them.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * dq_waves<D>()) void bwd_dq_kernel(
    const _Float16* __restrict__ qr, const _Float16* __restrict__ dor,
    const _Float16* __restrict__ kr, const _Float16* __restrict__ kc,
    const _Float16* __restrict__ vr, float* __restrict__ lse2, float* __restrict__ dvec,
    float* __restrict__ dq, int B, int Hq, int Hkv, int S, int nrb, float c_log2, float scale) {
  constexpr int NKD = D / 16, NDB = D / 32, TB = 64 * D;  // TB: bytes of a 32-token tile
  // Stages of a key block's tiles (K rows, V rows, K columns); afterwards the waves'
  // output staging areas.
  constexpr bool PIPE = dq_waves<D>() < 8;
  constexpr int NST = PIPE ? 3 : 2, STG = 3 * TB;
  constexpr int EQ = 32;  // channels per output pass
  constexpr int SMEM = NST * STG > dq_waves<D>() * staging_bytes<EQ>()
                           ? NST * STG
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
  // Copy of key block kb into stage st.
  auto issue = [&](int kb, int st, bool with_kc) {
    copy(krb + (int64_t)kb * TB, smem + st * STG);
    copy(vrb + (int64_t)kb * TB, smem + st * STG + TB);
    if (with_kc) copy(kcb + (int64_t)kb * TB, smem + st * STG + 2 * TB);
  };
  auto next_stage = [&](int st) { return st == NST - 1 ? 0 : st + 1; };
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
  // S^T (keys x queries) and dP^T of the block in stage st, all at once.
  auto scores = [&](const char* st, v16f& sc, v16f& dp) {
    const v8h* ka = reinterpret_cast<const v8h*>(st);
    const v8h* va = reinterpret_cast<const v8h*>(st + TB);
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.0f;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      sc = mfma16(ka[kd * 64 + lane], qf[kd], sc);
      dp = mfma16(va[kd * 64 + lane], df[kd], dp);
    }
  };

  // One step as a fixed schedule of slots, one product each, fenced so the compiler
  // keeps the order: slots 0 .. NSD-1 the score products of the next block (S^T and dP^T
  // alternating over the channel slices), in sweep 2 then the NQ dQ products of the
  // current block; every product's operand is read from LDS PF slots ahead.  work(x) is
  // the slot's share of the current block's vector arithmetic.
  constexpr int NSD = 2 * NKD, NQ = 2 * NDB, PF = 2;
  auto step = [&](int stn, int stc, v16f& sc, v16f& dp, v16f (&acc)[NDB], const v8h (&ds)[2],
                  auto SWEEP2, auto work) {
    constexpr bool two = decltype(SWEEP2)::value;
    constexpr int NM = NSD + (two ? NQ : 0);
    const v8h* ka = reinterpret_cast<const v8h*>(smem + stn * STG);
    const v8h* va = reinterpret_cast<const v8h*>(smem + stn * STG + TB);
    const v8h* kca = reinterpret_cast<const v8h*>(smem + stc * STG + 2 * TB);
    auto operand = [&](int x) -> v8h {
      if (x < NSD) return ((x & 1) ? va : ka)[(x >> 1) * 64 + lane];
      return kca[(x - NSD) * 64 + lane];  // (gg NDB + db) = x - NSD
    };
    v8h fr[PF + 1];
#pragma unroll
    for (int x = 0; x < PF; ++x) fr[x] = operand(x);
    v16f sn, dn;
#pragma clang loop unroll(full)
    for (int x = 0; x < NM; ++x) {
      const v8h op = fr[x % (PF + 1)];
      if (x + PF < NM) fr[(x + PF) % (PF + 1)] = operand(x + PF);
      if (x < NSD) {
        if (x & 1)
          dn = mfma16(op, df[x >> 1], x == 1 ? v16f{} : dn);
        else
          sn = mfma16(op, qf[x >> 1], x == 0 ? v16f{} : sn);
      } else if constexpr (two) {
        const int y = x - NSD;
        acc[y % NDB] = mfma16(op, ds[y / NDB], acc[y % NDB]);
      }
      work(x);
      __builtin_amdgcn_sched_barrier(0);
    }
    sc = sn;
    dp = dn;
  };

  // Sweep 1: running max, sum and sum of p * dP (log2 units).  Block 0 holds a visible
  // key (key 0) for every row, so the max is finite from the first block on.
  float mr = -INFINITY, l = 0.0f, a = 0.0f;
  int st0 = 0;  // stage of block kb
  if constexpr (!PIPE) {
    issue(0, 0, false);
    vm_wait<0>();
    __syncthreads();
    for (int kb = 0; kb < nkb_wg; ++kb) {
      if (kb + 1 < nkb_wg) issue(kb + 1, (kb + 1) & 1, false);
      if (active && kb < nkb) {
        v16f sc, dp;
        scores(smem + (kb & 1) * STG, sc, dp);
        mask(kb, sc);
        float mt = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = bmax(mt, sc[i]);
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
  } else {
    // Every wave runs every block of the group; a block past its causal diagonal is
    // all masked and adds nothing (its max is -inf and its p are 0).
    issue(0, st0, false);
    if (nkb_wg > 1) issue(1, next_stage(st0), false);
    vm_wait<0>();
    __syncthreads();
    v16f sc, dp;
    scores(smem + st0 * STG, sc, dp);
    mask(0, sc);
    v16f acc_none[NDB];
    const v8h ds_none[2] = {};
    for (int kb = 0; kb < nkb_wg; ++kb) {
      const int st1 = next_stage(st0);
      if (kb + 2 < nkb_wg) issue(kb + 2, next_stage(st1), false);
      float mn = 0.0f;
      // Slot work: the block's max (slot 0), the new running max and the rescale
      // (slot 1), then the 16 exponentials with their sums over slots 2 .. NSD-1.
      auto work = [&](int x) {
        if (x == 0) {
          float mt = sc[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mt = bmax(mt, sc[i]);
          mn = mt;
        } else if (x == 1) {
          mn = bmax(mr, half_max(mn) * c_log2);
          const float al = mr == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mr - mn);
          l *= al;
          a *= al;
          mr = mn;
        } else if (x < NSD) {
          const int i0 = 16 * (x - 2) / (NSD - 2), i1 = 16 * (x - 1) / (NSD - 2);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (i < i0 || i >= i1) continue;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c_log2, -mn));
            l += p;
            a = __builtin_fmaf(p, dp[i], a);
          }
        }
      };
      step(st1, st0, sc, dp, acc_none, ds_none, std::false_type{}, work);
      mask(kb + 1, sc);
      vm_wait<0>();
      __syncthreads();
      st0 = st1;
    }
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

  // Sweep 2: P, dS and dQ^T = K^T dS^T.  Unconditional, as in the dK/dV kernel: past
  // this wave's last key block every score is masked and dS is zero (a wave past the
  // padded length has zero operands, lse = 0 and D = 0, so dS is zero too).
  v16f acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
  st0 = 0;
  if constexpr (!PIPE) {
    issue(0, 0, true);
    vm_wait<0>();
    __syncthreads();
    for (int kb = 0; kb < nkb_wg; ++kb) {
      if (kb + 1 < nkb_wg) issue(kb + 1, (kb + 1) & 1, true);
      const char* st = smem + (kb & 1) * STG;
      v16f sc, dp;
      scores(st, sc, dp);
      mask(kb, sc);
      v8h ds[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c_log2, -lse));
        ds[i >> 3][i & 7] = (_Float16)(p * (dp[i] - Dv));
      }
      const v8h* kca = reinterpret_cast<const v8h*>(st + 2 * TB);
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = mfma16(kca[(gg * NDB + db) * 64 + lane], ds[gg], acc[db]);
      vm_wait<0>();
      __syncthreads();
    }
  } else {
    issue(0, st0, true);
    if (nkb_wg > 1) issue(1, next_stage(st0), true);
    vm_wait<0>();
    __syncthreads();
    v16f sc, dp;
    scores(smem + st0 * STG, sc, dp);
    mask(0, sc);
    for (int kb = 0; kb < nkb_wg; ++kb) {
      const int st1 = next_stage(st0);
      if (kb + 2 < nkb_wg) issue(kb + 2, next_stage(st1), true);
      v8h ds[2];
      // Slot work: the block's 16 elements p = 2^(s c - lse), dS = p (dP - D) over the
      // score slots, before the dQ products that take them.
      auto work = [&](int x) {
        if (x < NSD) {
          const int i0 = 16 * x / NSD, i1 = 16 * (x + 1) / NSD;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (i < i0 || i >= i1) continue;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c_log2, -lse));
            ds[i >> 3][i & 7] = (_Float16)(p * (dp[i] - Dv));
          }
        }
      };
      step(st1, st0, sc, dp, acc, ds, std::true_type{}, work);
      mask(kb + 1, sc);
      vm_wait<0>();
      __syncthreads();
      st0 = st1;
    }
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
