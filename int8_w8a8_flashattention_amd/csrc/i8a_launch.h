// i8a_launch.h - host-side launchers of the HIP kernels, called by the C ABI layer.
// Arguments are validated by the caller; these only enqueue work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace i8a {

// Keys per workspace tile and per attention pipeline stage.
constexpr int TK = 64;
// Tokens per workgroup of the K/V preparation kernels (a multiple of TK).
constexpr int CH = 256;
static_assert(CH % TK == 0, "a prep chunk holds whole tiles");

// Q outlier channels (the outlier-aware variant): at most QO_MAX per (sequence, kv
// head), detected where max |q| exceeds QO_THRESHOLD.
constexpr int QO_MAX = 16;
constexpr float QO_THRESHOLD = 6.0f;
// Bytes of the fp16 K values of the outlier channels of one tile (A operand of a
// 32x32x16 fp16 MFMA per 32-key block).
constexpr int KO_BYTES = TK * QO_MAX * 2;

// Bytes of one prepared K/V tile of TK tokens: int8 K codes in MFMA fragment order,
// then the exact fp16 dequantized V in fragment order, then the fp32 K scales, and
// with outliers the fp16 K values of the outlier channels.
__host__ __device__ constexpr int tile_bytes(int D, bool outliers = false) {
  return TK * D * 3 + TK * 4 + (outliers ? KO_BYTES : 0);
}

// Workspace carve-up for one forward call.  All offsets are 256-byte aligned.
//   kpart  int64 [nseq][Hkv][npart][D]   exact K channel sums of tpw tiles (2^-24 units)
//   kmean  fp32  [nseq][Hkv][D]          K-smoothing means
//   vpart  fp32  [nseq][Hkv][npart][D]   V channel maxima of tpw tiles (V per channel)
//   svc    fp32  [nseq][Hkv][D]          V channel scales (V per channel)
//   sv     fp32  [Hkv][Ppad]             V row scales (kept for the debug dump)
//   qopart fp32  [nseq][Hkv][npart][D]   Q channel maxima of tpw tiles (Q outliers)
//   ochan  int32 [nseq][Hkv][QO_MAX]     Q outlier channels, increasing, -1 padded
//   tiles  bytes [Hkv][Ppad / TK][tile_bytes(D, outliers)] (room for the larger)
//   q8     int8  [Hq][Qpad / 32][32 * D] Q codes, 32-row blocks in MFMA fragment order
//   qs     fp32  [Hq][Qpad]              Q row scales
// K/V token slots are padded per sequence to TK rows (Seqs::pstart), Q slots to BQ
// rows (Seqs::qpstart), so every tile or query tile starts on a boundary.
// Cap on the K partial sums per (sequence, kv head): the K quantization workgroups
// each reduce all of them to get the mean.
constexpr int MAX_PARTS = 64;
// Padding of each sequence's Q slots: a multiple of the query rows of every attention
// workgroup, so that a query tile never reaches into the next sequence's slots.
constexpr int BQ = 256;

struct WsPlan {
  int32_t nseq, Hq, Hkv, D, ntile;  // ntile: TK-token tiles of the longest sequence
  int32_t tpw, npart;               // tiles per prep workgroup, partial sums per (seq, head)
  int64_t Ppad;                     // padded K/V token slots per kv head
  int64_t Qpad;                     // padded Q token slots per query head
  size_t off_kpart, off_kmean, off_vpart, off_svc, off_sv, off_qopart, off_ochan, off_tiles, off_q8,
      off_qs, total;
};

WsPlan plan_workspace(int32_t nseq, int64_t total_tokens, int32_t max_len, int32_t Hq,
                      int32_t Hkv, int32_t D);

// Geometry of one forward call: dense when cu == nullptr.
struct FwdGeom {
  const void *q, *k, *v;
  void* out;
  const int32_t* cu;
  int32_t nseq, S, max_len;
  int64_t T;
  int32_t Hq, Hkv, D;
  float softmax_scale;
  int causal;
  int rot;  // Q and K rows Hadamard-rotated before quantization (logits take 1/D)
  int vch;  // V quantized per channel over each sequence's tokens (else per token)
  int qblk = 0;  // Q quantized with one scale per 32-row block (else per row)
  int qout = 0;  // Q outlier channels detected and multiplied in fp16 (D <= 128)
  // The attention kernel quantizes (and with rot rotates) Q itself from q: no Q
  // preparation pass.
  int fuse_q = 0;
};

hipError_t launch_quant_rowwise(const void* x, int64_t rows, int32_t d, const float* sub_mean,
                                int64_t rows_per_group, int32_t scale_bits, int8_t* codes,
                                float* scales, hipStream_t stream);

// Preparation into the workspace: with kv, the K-smoothing mean and the K and V
// quantization; with qq, the Q quantization (codes in fragment order, row scales).
hipError_t launch_prep(const FwdGeom& g, const WsPlan& p, void* ws, bool kv, bool qq,
                       hipStream_t stream);

// Attention over the prepared workspace (K and V prepared; Q prepared too unless
// g.fuse_q).
hipError_t launch_attn(const FwdGeom& g, const WsPlan& p, const void* ws, hipStream_t stream);

// Outputs of the debug dump (every pointer but s32 may be null).
struct DebugOut {
  int32_t* s32;      // [rows][cols]
  int32_t cols;
  float* qscale;     // [rows]
  float* kscale;     // [cols]
  float* vscale;     // [cols]   V per token
  float* kmean;      // [D]
  _Float16* vhat;    // [cols][D] the prepared V rows
  float* vchan;      // [D]      V per channel
  int32_t* ochan;    // [QO_MAX] Q outlier channels of the query head's kv group
};

// Debug dump of S32, scales, K mean and prepared V rows for sequence s, query head h.
hipError_t launch_debug_qk(const FwdGeom& g, const WsPlan& p, const void* ws, int32_t s,
                           int32_t h, int32_t row0, int32_t rows, int32_t col0, int32_t cols,
                           const DebugOut& o, hipStream_t stream);

// ----------------------------------------------------------------------------------
// Decode KV cache: per (batch, kv head), ceil(S / TKD) tiles of TKD tokens, each a
// block of dtile_bytes(D, vf) bytes:
//   K codes   TKD*D int8 in the K fragment order (one 32-key block)
//   V         int8 format: TKD*D bytes, per (d block, lane) 16 bytes = the V fragments
//             of key groups 0 and 1 as biased codes (code + 128);
//             fp16 format: 2*TKD*D bytes, the fp16 V fragments of key groups 0 and 1
//   sk        TKD fp32 K scales, key order
//   sv        int8 format only: TKD fp16 V scales ordered [hv][key group][jv]
constexpr int TKD = 32;
enum VFormat { VF_INT8 = 1, VF_FP16 = 2 };
__host__ __device__ constexpr int dtile_bytes(int D, int vf) {
  return vf == VF_INT8 ? 2 * TKD * D + TKD * 4 + TKD * 2 : 3 * TKD * D + TKD * 4;
}

// Cache carve-up (256-byte aligned offsets):
//   kpart int64 [B][Hkv][npart][D]   exact K channel sums of tpw TK-token tiles
//   kmean fp32  [B][Hkv][D]          K-smoothing means
//   tiles bytes [B][Hkv][ntd][dtile_bytes]
struct KvcPlan {
  int32_t B, Hkv, S, D, vf, ntd, tpw, npart;
  size_t off_kpart, off_kmean, off_tiles, total;
};
KvcPlan plan_kvcache(int32_t B, int32_t Hkv, int32_t S, int32_t D, int32_t vf);

// Split of a decode call: the ntd tiles of a (batch, kv head) in nchunk chunks of tpc
// tiles; nqb blocks of up to 32 query heads per kv head.  Workspace (partials of the
// chunks, when nchunk > 1): o fp32 [B*Hq][nchunk][D], then (m, l) fp32 [B*Hq][nchunk][2].
struct DecPlan {
  int32_t nqb, tpc, nchunk, nw;
  size_t off_po, off_pml, total;
};
DecPlan plan_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D, int32_t vf);

// Exact per-channel K sums of dense k [B, Hkv, S, D] (the forward's launch 1).
hipError_t launch_ksum_dense(const void* k, int32_t B, int32_t Hkv, int32_t S, int32_t D,
                             int32_t npart, int32_t tpw, int64_t* kpart, hipStream_t stream);

// Fill of the decode cache's first n_fill <= S tokens from dense fp16 k, v
// [B, Hkv, n_fill, D] (the K-smoothing mean over those tokens).
hipError_t launch_kvcache_fill(const void* k, const void* v, const KvcPlan& p, int32_t n_fill,
                               void* cache, hipStream_t stream);

// Append of n tokens per (batch, kv head), fp16 k, v [B, Hkv, n, D], into the slots
// pos[b] .. pos[b] + n - 1 (device int32 [B]); slots outside [0, S) are skipped.
hipError_t launch_kvcache_append(const void* k, const void* v, int32_t n, const int32_t* pos,
                                 const KvcPlan& p, void* cache, hipStream_t stream);

// Decode of q [B, Hq, D] against a filled cache into out [B, Hq, D]; with lens (device
// int32 [B], or null for all S) sequence b attends its first lens[b] tokens.
hipError_t launch_decode(const void* q, void* out, int32_t Hq, float softmax_scale,
                         const KvcPlan& p, const DecPlan& dp, const void* cache, void* ws,
                         const int32_t* lens, hipStream_t stream);

// ----------------------------------------------------------------------------------
// Backward.  Workspace (256-byte aligned pieces), Sp = 32 * nrb tokens per head:
//   qr, qc, dor, doc  fp16 [B][Hq][Sp][D]   Q and dO in row and column fragment order
//   kr, kc, vr        fp16 [B][Hkv][Sp][D]  K (both orders) and V (row order)
//   lse, dvec         fp32 [B][Hq][S rounded up to 128]   row log2-sum-exp and D
struct BwdPlan {
  int32_t nrb;
  size_t off_qr, off_qc, off_dor, off_doc, off_kr, off_kc, off_vr, off_lse, off_dvec, off_pk,
      off_pv, total;
};
BwdPlan plan_bwd(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D);

struct BwdArgs {
  const void *q, *k, *v, *dout;
  float *dq, *dk, *dv;
  int32_t B, Hq, Hkv, S, D;
  float softmax_scale;
  int causal;
};
hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& p, void* ws, hipStream_t stream);
// The dQ kernel alone (launch 2 of launch_bwd; ws: the workspace of plan p).
hipError_t launch_bwd_dq(const BwdArgs& a, const BwdPlan& p, char* ws, hipStream_t stream);
// Its D = 256 instance (a source of its own, built without the vector-register form).
hipError_t launch_bwd_dq256(const BwdArgs& a, const BwdPlan& p, char* ws, hipStream_t stream);

}  // namespace i8a
