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
// Launch 3 (bwd_dkdv_kernel, lane = key): each wave owns 32 keys and accumulates
//   dV^T = dO^T P and dK^T = Q^T dS over the query blocks of the query heads of its kv
//   head; under the causal mask each group of 128 keys is split over two workgroups.
// Launch 4 (bwd_combine_kernel, causal only): adds the second workgroup's partial sums.
// Both main kernels stream their operand tiles through LDS rings shared by the four
// waves of a workgroup (direct-to-LDS copies ahead of use).  No atomics are used: the
// results do not depend on the order in which workgroups run.
#include <float.h>

#include <type_traits>

#include "bwd_common.h"
#include "i8a_launch.h"

namespace i8a {

using namespace bwd;

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
// Launch 3: dK and dV.  Workgroup = 4 waves on a group of 128 keys of one (batch, kv
// head); wave w owns keys k0 = kblk0 + 32 w .. +31, lane l key k0 + l % 32, and sums the
// contributions of the group's query heads itself.  The work items are (query head,
// query block) pairs; under the causal mask the group's items are dealt alternately to
// two workgroups (part 0 writes dK and dV, part 1 partial sums that the combine kernel
// adds).  The items' operand tiles (Q and dO in row and column order, with the rows'
// statistics) stream through LDS rings shared by the four waves, three items ahead, and
// each step is software-pipelined (see the loop).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    const _Float16* __restrict__ qr, const _Float16* __restrict__ qc,
    const _Float16* __restrict__ dor, const _Float16* __restrict__ doc,
    const _Float16* __restrict__ kr, const _Float16* __restrict__ vr,
    const float* __restrict__ lse2, const float* __restrict__ dvec, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ pk, float* __restrict__ pv, int B, int Hq,
    int Hkv, int S, int nrb, int nsplit, float c_log2, float scale) {
  constexpr int NKD = D / 16, NDB = D / 32, TB = 64 * D;
  // Two rings: row stages (Q and dO in row order), read one step before their item's
  // step, and column stages (Q and dO in column order, then the block's 32 row
  // log-sum-exps and 32 D values), read at their item's step and the next.
  // D <= 128: the software-pipelined loop (rings of 4 and 5 stages); D = 256: a plain
  // loop one item ahead (2 and 2 stages, 128.5 KB), since the pipeline's rings would not
  // fit the 160 KB of LDS.
  constexpr bool PIPE = D <= 128;
  constexpr int NR = PIPE ? 4 : 2, NC = PIPE ? 5 : 2, RB = 2 * TB, CB = 2 * TB + 256;
  constexpr int EK = D < 128 ? D : 128;  // channels per output pass
  static_assert(4 * staging_bytes<EK>() <= NR * RB + NC * CB, "the staging areas fit the rings");
  __shared__ __attribute__((aligned(16))) char smem[NR * RB + NC * CB];
  char* const rring = smem;
  char* const cring = smem + NR * RB;
  // blockIdx.x = ((key group of 128 x nsplit + part) x B + batch) x Hkv + kv head: the
  // heaviest groups under the causal mask are dispatched first.
  const int g = blockIdx.x % Hkv, b = (blockIdx.x / Hkv) % B;
  const int part = (blockIdx.x / Hkv / B) % nsplit;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, m = lane & 31, hh = lane >> 5;
  const int kblk0 = 128 * (int)(blockIdx.x / Hkv / B / nsplit);
  const int k0 = kblk0 + 32 * w;
  const bool active = k0 < nrb * 32;
  const int64_t Sp = (int64_t)nrb * 32;
  const int64_t kbase = ((int64_t)b * Hkv + g) * Sp;
  const int kj = k0 + m;

  v8h kf[NKD], vf[NKD];
  if (active) {
    const v8h* ks = reinterpret_cast<const v8h*>(kr + (kbase + k0) * D);
    const v8h* vs = reinterpret_cast<const v8h*>(vr + (kbase + k0) * D);
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      kf[kd] = ks[kd * 64 + lane];
      vf[kd] = vs[kd * 64 + lane];
    }
  } else {
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd)
#pragma unroll
      for (int j = 0; j < 8; ++j) kf[kd][j] = vf[kd][j] = (_Float16)0.0f;
  }
#pragma unroll
  for (int kd = 0; kd < NKD; ++kd) asm volatile("" : : "v"(kf[kd]), "v"(vf[kd]));

  v16f accv[NDB], acck[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) accv[db][i] = acck[db][i] = 0.0f;

  // Work items of the group: (query head, query block) pairs, query blocks from the
  // first one that reaches the group's first key (causal) to the end.
  const int qb0 = CAUSAL ? kblk0 / 32 : 0;
  const int nqb = nrb - qb0;
  // Items in the order j = 0, 1, ...: query blocks from the last one down, the group's
  // query heads inside, so that the workgroups of a kv head, which all start at the last
  // block, read the same tiles at about the same time and share them in L2.  Part p of
  // nsplit takes the items j = p (mod nsplit).
  const int nitem = (G * nqb - part + nsplit - 1) / nsplit;
  // A part can have no items (G = 1 and a group with one query block): it still writes
  // its partial rows below (zeros), since the combine kernel adds every row.
  // Under the causal mask only items with a query block at or below the group's last
  // wave's first key block (qb <= kblk0 / 32 + 3: the last 4 G of the order, j >=
  // G (nqb - 4)) can hold masked pairs; items before it_m skip the mask.
  int it_m = nitem;
  if (CAUSAL) {
    const int jm = G * (nqb - 4) - part;
    it_m = jm <= 0 ? 0 : min(nitem, (jm + nsplit - 1) / nsplit);
  }
  // Copies of the items into their row and column stages, in item order (0, 1, 2, ...;
  // each once), following a cursor over (query block, head) instead of dividing by G.
  // Every wave issues 4 tile_dma_count<D>(w) + 1 copies per item (the statistics: 4
  // lanes of each wave, waves 0-1 the log-sum-exps, waves 2-3 the D values).
  const TileCopy<D> copy(tid);
  const uint32_t stat_off = 16u * (4u * (uint32_t)(w & 1) + (uint32_t)lane);
  int cur_hg = part % G, cur_qb = nrb - 1 - part / G, cur_cs = 0, cur_it = 0;
  auto issue = [&]() {
    const int64_t qbase = ((int64_t)b * Hq + g * G + cur_hg) * Sp;
    const int64_t off = (qbase + 32 * (int64_t)cur_qb) * D * 2;
    char* rs = rring + (cur_it & (NR - 1)) * RB;
    char* cs = cring + cur_cs * CB;
    copy(reinterpret_cast<const char*>(qr) + off, rs);
    copy(reinterpret_cast<const char*>(dor) + off, rs + TB);
    copy(reinterpret_cast<const char*>(qc) + off, cs);
    copy(reinterpret_cast<const char*>(doc) + off, cs + TB);
    // The row statistics ride in the column stage, so the loop holds no load the
    // compiler tracks: a wait it placed for one would also wait for later copies.
    if (lane < 4)
      lds_dma16_s((w < 2 ? lse2 : dvec) + qbase + 32 * cur_qb, stat_off,
                  lds_addr(cs + 2 * TB + 64 * w));
    ++cur_it;
    cur_cs = cur_cs + 1 == NC ? 0 : cur_cs + 1;
    cur_hg += nsplit;
    while (cur_hg >= G) {
      cur_hg -= G;
      --cur_qb;
    }
  };
  // Wait for every copy but, if `one_ahead`, the last item's: its four tiles and the
  // statistics, with this wave's own number of copy instructions per tile (at D = 32
  // waves 2 and 3 copy nothing).
  auto wait_copies = [&](bool one_ahead) {
    if (!one_ahead) {
      vm_wait<0>();
      return;
    }
    switch (w) {
      case 0: vm_wait<4 * tile_dma_count<D>(0) + 1>(); break;
      case 1: vm_wait<4 * tile_dma_count<D>(1) + 1>(); break;
      case 2: vm_wait<4 * tile_dma_count<D>(2) + 1>(); break;
      default: vm_wait<4 * tile_dma_count<D>(3) + 1>(); break;
    }
  };

  // Block it's S^T and dP^T (keys x queries) from its Q and dO row tiles.
  auto scores = [&](int it, v16f& sc, v16f& dp) {
    const char* stg = rring + (it & (NR - 1)) * RB;
    const v8h* qa = reinterpret_cast<const v8h*>(stg);
    const v8h* da = reinterpret_cast<const v8h*>(stg + TB);
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.0f;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      sc = mfma16(qa[kd * 64 + lane], kf[kd], sc);
      dp = mfma16(da[kd * 64 + lane], vf[kd], dp);
    }
  };
  // Element e (register e: query 32 qb + 8 (e / 4) + 4 hh + e % 4) of block it's P^T
  // and dS^T, from its score, its dP and its row's statistics (lv, dv4 from the stage).
  auto prob = [&](int e, int qb, float s, float d, const v4f (&lv)[4], const v4f (&dv4)[4],
                  v8h (&p16)[2], v8h (&ds16)[2], auto masked) {
    const int J = e >> 2, r = e & 3;
    // Empty statements that take the inputs and give the results at this point of the
    // step: the arithmetic stays in the slot where the fences put it.
    asm volatile("" : "+v"(s), "+v"(d));
    float p = __builtin_amdgcn_exp2f(s * c_log2 - lv[J][r]);
    if constexpr (decltype(masked)::value) p = kj > 32 * qb + 8 * J + 4 * hh + r ? 0.0f : p;
    const float ds = p * (d - dv4[J][r]);
    asm volatile("" : : "v"(p), "v"(ds));
    p16[e >> 3][e & 7] = (_Float16)p;
    ds16[e >> 3][e & 7] = (_Float16)ds;
  };
  auto stats = [&](int it, v4f (&lv)[4], v4f (&dv4)[4]) {
    const float* lrow = reinterpret_cast<const float*>(cring + (it % NC) * CB + 2 * TB);
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      lv[J] = *reinterpret_cast<const v4f*>(lrow + 8 * J + 4 * hh);
      dv4[J] = *reinterpret_cast<const v4f*>(lrow + 32 + 8 * J + 4 * hh);
    }
  };
  // The query block of the next item whose softmax is computed (called in item order).
  int st_hg = part % G, st_qb = nrb - 1 - part / G;
  auto next_item_qb = [&]() {
    const int q = st_qb;
    st_hg += nsplit;
    while (st_hg >= G) {
      st_hg -= G;
      --st_qb;
    }
    return q;
  };
  // dV^T += dO^T P^T and dK^T += Q^T dS^T for block it, from its column tiles.
  auto accumulate = [&](int it, const v8h (&p16)[2], const v8h (&ds16)[2]) {
    const char* stg = cring + (it % NC) * CB;
    const v8h* dca = reinterpret_cast<const v8h*>(stg + TB);
    const v8h* qca = reinterpret_cast<const v8h*>(stg);
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        accv[db] = mfma16(dca[(gg * NDB + db) * 64 + lane], p16[gg], accv[db]);
        acck[db] = mfma16(qca[(gg * NDB + db) * 64 + lane], ds16[gg], acck[db]);
      }
  };

  if constexpr (!PIPE) {
    if (nitem > 0) {
      // Plain loop: the copy of item it + 1 runs while item it is computed, into the
      // stages that item it - 1 left at the previous step.
      issue();
      vm_wait<0>();
      __syncthreads();
      for (int it = 0; it < nitem; ++it) {
        if (it + 1 < nitem) issue();
        v16f sc, dp;
        scores(it, sc, dp);
        v4f lv[4], dv4[4];
        stats(it, lv, dv4);
        const int qb = next_item_qb();
        v8h p16[2], ds16[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (it >= it_m)
            prob(e, qb, sc[e], dp[e], lv, dv4, p16, ds16, std::true_type{});
          else
            prob(e, qb, sc[e], dp[e], lv, dv4, p16, ds16, std::false_type{});
        }
        accumulate(it, p16, ds16);
        vm_wait<0>();
        __syncthreads();
      }
    }
  } else if (nitem > 0) {
    // Software pipeline over the work items: step it runs the dV/dK products of item
    // it - 1, the score products of item it + 1 and the softmax arithmetic of item it, none
    // of which waits for another.  The copy of item it + 3 starts at step it and has two
    // steps to land: into the row stage that item it - 1 left at step it - 2 and the column
    // stage that item it - 2 left at step it - 1.  Every block is processed by every wave
    // (a block the causal mask empties adds exact zeros; a wave past the padded length is
    // never written): skipping one would give each accumulator two incoming values at the
    // loop's join, which the register allocator resolves with copies of all of them.
    issue();
    if (nitem > 1) issue();
    if (nitem > 2) issue();
    wait_copies(nitem > 2);
    __syncthreads();
    if (nitem > 3) issue();
    v16f sc, dp;
    scores(0, sc, dp);
    v8h p16[2], ds16[2];
    {
      v16f sn, dn;
      scores(min(1, nitem - 1), sn, dn);
      v4f lv[4], dv4[4];
      stats(0, lv, dv4);
      const int qb = next_item_qb();  // item 0
  #pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (it_m == 0)
          prob(e, qb, sc[e], dp[e], lv, dv4, p16, ds16, std::true_type{});
        else
          prob(e, qb, sc[e], dp[e], lv, dv4, p16, ds16, std::false_type{});
      }
      sc = sn;
      dp = dn;
    }
    wait_copies(nitem > 3);
    __syncthreads();
    constexpr int NP = D / 8;       // products of each kind per step
    auto step = [&](int it, auto masked) {
      const char* stp = cring + ((it - 1) % NC) * CB;
      const char* stn = rring + (min(it + 1, nitem - 1) & (NR - 1)) * RB;
      v8h aop[NP];
  #pragma unroll
      for (int x = 0; x < NP; ++x) {
        const int gg = x / (2 * NDB), db = (x >> 1) % NDB;
        const v8h* src = reinterpret_cast<const v8h*>(stp + ((x & 1) ? 0 : 1) * TB);
        aop[x] = src[(gg * NDB + db) * 64 + lane];
      }
      v4f lv[4], dv4[4];
      stats(it, lv, dv4);
      const int qb = next_item_qb();  // item it
      float scv[16], dpv[16];
  #pragma unroll
      for (int e = 0; e < 16; ++e) {
        scv[e] = sc[e];
        dpv[e] = dp[e];
      }
      __builtin_amdgcn_sched_barrier(0);
      v8h pn[2], dsn[2], sop[NP];
      v16f sn, dn;
  #pragma unroll
      for (int x = 0; x < 2 * NP; ++x) {
        if (x < NP) {
          const int gg = x / (2 * NDB), db = (x >> 1) % NDB;
          if (x & 1)
            acck[db] = mfma16(aop[x], ds16[gg], acck[db]);
          else
            accv[db] = mfma16(aop[x], p16[gg], accv[db]);
          const v8h* src = reinterpret_cast<const v8h*>(stn + ((x & 1) ? 1 : 0) * TB);
          sop[x] = src[(x >> 1) * 64 + lane];
        } else {
          const int y = x - NP;
          if (y < 2) {
            if (y & 1)
              dn = mfma16(sop[y], vf[y >> 1], v16f{});
            else
              sn = mfma16(sop[y], kf[y >> 1], v16f{});
          } else {
            if (y & 1)
              dn = mfma16(sop[y], vf[y >> 1], dn);
            else
              sn = mfma16(sop[y], kf[y >> 1], sn);
          }
        }
  #pragma unroll
        for (int e = x * 16 / (2 * NP); e < (x + 1) * 16 / (2 * NP); ++e)
          prob(e, qb, scv[e], dpv[e], lv, dv4, pn, dsn, masked);
        __builtin_amdgcn_sched_barrier(0);
      }
      sc = sn;
      dp = dn;
  #pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        p16[gg] = pn[gg];
        ds16[gg] = dsn[gg];
      }
    };
    // Steps with a copy to start (its wait leaves that copy in flight), then the last three;
    // each without the mask's compares up to the first item that can hold a masked pair.
    const int n_issue = nitem - 3;
    int it = 1;
    for (; it < n_issue && it < it_m; ++it) {
      issue();  // item it + 3
      step(it, std::false_type{});
      wait_copies(true);
      __syncthreads();
    }
    for (; it < n_issue; ++it) {
      issue();
      step(it, std::true_type{});
      wait_copies(true);
      __syncthreads();
    }
    for (; it < nitem && it < it_m; ++it) {
      step(it, std::false_type{});
      vm_wait<0>();
      __syncthreads();
    }
    for (; it < nitem; ++it) {
      step(it, std::true_type{});
      vm_wait<0>();
      __syncthreads();
    }
    accumulate(nitem - 1, p16, ds16);
  }

  // Part 0 writes the outputs, part 1 its partial sums (added by bwd_combine_kernel),
  // through the rings, unused once every wave is past its last block.
  __syncthreads();
  {
    const int64_t o0 = (((int64_t)b * Hkv + g) * S + k0) * D;
    const int nvalid = active ? min(32, S - k0) : 0;
    char* area = smem + w * staging_bytes<EK>();
    store_rows_f32<D, EK>(accv, 1.0f, area, (part == 0 ? dv : pv) + o0, nvalid, lane);
    store_rows_f32<D, EK>(acck, scale, area, (part == 0 ? dk : pk) + o0, nvalid, lane);
  }
}

// ----------------------------------------------------------------------------------
// Launch 4 (under the causal mask): dK += partial dK, dV += partial dV of the second
// part of every key group, in that order (n4 float4 per tensor).
__global__ __launch_bounds__(256) void bwd_combine_kernel(float* __restrict__ dk,
                                                          float* __restrict__ dv,
                                                          const float* __restrict__ pk,
                                                          const float* __restrict__ pv,
                                                          int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * n4) return;
  const bool isv = i >= n4;
  const int64_t j = isv ? i - n4 : i;
  v4f* o = reinterpret_cast<v4f*>(isv ? dv : dk) + j;
  const v4f p = reinterpret_cast<const v4f*>(isv ? pv : pk)[j];
  *o = *o + p;
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
  // Partial dK and dV of the second part of each key group (causal calls).
  const size_t obytes = (size_t)B * Hkv * S * D * 4;
  p.off_pk = off; off = align256b(off + obytes);
  p.off_pv = off; off = align256b(off + obytes);
  p.total = off;
  return p;
}

template <int D, bool C>
static hipError_t bwd_d(const BwdArgs& a, const BwdPlan& p, char* ws, hipStream_t stream) {
  // Under the causal mask each key group's items are split in two workgroups (the group
  // sizes fall linearly along the sequence; the halves let the dispatcher balance them),
  // whose sums meet in bwd_combine_kernel.
  const int nsplit = C ? 2 : 1;
  const int64_t nprep = (int64_t)p.nrb * (2 * a.B * a.Hq + 2 * a.B * a.Hkv);
  const int64_t ngrp = (p.nrb + 3) / 4;
  const int64_t n4 = (int64_t)a.B * a.Hkv * a.S * D / 4;
  if (nprep > 0x7fffffff || ngrp * a.B * a.Hq > 0x7fffffff ||
      ngrp * nsplit * a.B * a.Hkv > 0x7fffffff || (2 * n4 + 255) / 256 > 0x7fffffff)
    return hipErrorInvalidValue;
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
  float* pk = reinterpret_cast<float*>(ws + p.off_pk);
  float* pv = reinterpret_cast<float*>(ws + p.off_pv);
  e = launch_bwd_dq(a, p, ws, stream);
  if (e != hipSuccess) return e;
  bwd_dkdv_kernel<D, C><<<dim3((unsigned)(ngrp * nsplit * a.B * a.Hkv)), 256, 0, stream>>>(
      H(p.off_qr), H(p.off_qc), H(p.off_dor), H(p.off_doc), H(p.off_kr), H(p.off_vr), lse,
      dvec, a.dk, a.dv, pk, pv, a.B, a.Hq, a.Hkv, a.S, p.nrb, nsplit, c_log2,
      a.softmax_scale);
  if (nsplit == 1) return hipGetLastError();
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_combine_kernel<<<dim3((unsigned)((2 * n4 + 255) / 256)), 256, 0, stream>>>(a.dk, a.dv, pk,
                                                                                  pv, n4);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& p, void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
#define I8A_BWD(DD)                                                  \
  case DD:                                                           \
    return a.causal ? bwd_d<DD, true>(a, p, w, stream)               \
                    : bwd_d<DD, false>(a, p, w, stream);
  switch (a.D) {
    I8A_BWD(32) I8A_BWD(64) I8A_BWD(128) I8A_BWD(256)
    default:
      return hipErrorInvalidValue;
  }
#undef I8A_BWD
}

}  // namespace i8a
