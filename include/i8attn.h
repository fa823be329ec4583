/*
 * i8attn.h - C ABI of the INT8 W8A8 FlashAttention forward for AMD MI355X (gfx950).
 *
 * The method is the one the "SuperL8" README describes for its attn_int8_fwd kernel
 * (Attention kernels table: "W8A8 ... FlashAttention-2. Causal, GQA/MQA, head dims
 * 32/64/128/256") with its attn_varlen_fwd variant (same table: ragged,
 * non-tile-multiple prefill) and its quant_rowwise helper (Supporting kernels table:
 * symmetric per-row int8).  Per the Quantization table, K is smoothed by subtracting
 * its per-channel mean over the sequence before it is quantized; V is quantized per
 * token.  Per the Quick start, the forward takes fp16 q, k, v and quantizes
 * internally.
 *
 * Arithmetic of one forward call (every step runs in HIP kernels):
 *   kmean[b,g,:]   = mean over the sequence's tokens of k[b,g,:,:] (exact sum, fp64
 *                    divide, rounded to fp32)
 *   q8,sq = quant(q)          sq = fp32(absmax/127)
 *   k8,sk = quant(k - kmean)  sk = fp32(absmax/127), x = fp32(k) - kmean in fp32
 *   v8,sv = quant(v)          sv = fp32(absmax/127) rounded up to a 4-bit significand
 *   quant(x): code = clamp(rint(fp32(x / scale)), -127, 127); all-zero row -> scale 0
 *   S32 = q8 . k8^T (int8 MFMA, exact int32)
 *   logit = S32 * sq_i * sk_j * softmax_scale, causal: key j > query i masked
 *   out = softmax(logit) . (sv * v8), online softmax in fp32, fp16 MFMA for P.V,
 *         fp32 accumulation, fp16 output
 *   GQA/MQA: query head h reads kv head h / (Hq / Hkv).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked "host".  fp16 tensors are passed as
 *     void* holding IEEE binary16 values.  All tensors are densely packed in the
 *     layout stated; base pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is enqueued on
 *     it and the call returns without synchronizing.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronizes, keeps no state between calls and is reentrant; calls that run
 *     concurrently need distinct workspaces.
 *   - Every argument check runs on the host before anything is enqueued: on an error
 *     nothing is written.  The detail of the last failure on the calling thread is
 *     available from i8a_last_error().
 *   - Inputs must be finite.  V entries must have magnitude <= 65024 (so that the
 *     dequantized V, whose scale is rounded up, stays within fp16 range).
 */
#ifndef I8ATTN_H
#define I8ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t i8a_status;

#define I8A_OK 0
#define I8A_ERR_INVALID_ARG (-1)          /* bad pointer, size, alignment or flag */
#define I8A_ERR_UNSUPPORTED_HEAD_DIM (-2) /* D not in {32, 64, 128, 256} */
#define I8A_ERR_WORKSPACE_TOO_SMALL (-3)  /* workspace_bytes below the required size */
#define I8A_ERR_HIP (-4)                  /* a HIP launch failed (see i8a_last_error) */

/* Scale rules accepted by quant_rowwise_i8 (significand bits of the row scale). */
#define I8A_SCALE_FP32 24 /* scale = fp32(absmax / 127): Q and K rows */
#define I8A_SCALE_V4 4    /* the same, rounded up to a 4-bit significand: V rows */

/*
 * quant_rowwise_i8 - symmetric per-row int8 quantization (SuperL8 README, Supporting
 * kernels table, row quant_rowwise; Quantization table, row "Per-row int8").
 *
 *   x        fp16 [rows, d], row-major.
 *   rows     number of rows, >= 0 (0 is a no-op).
 *   d        row length, a multiple of 8 in [8, 512].
 *   sub_mean nullable fp32 [ceil(rows / rows_per_group), d]: if given, row r is
 *            quantized from fp32(x[r]) - sub_mean[r / rows_per_group] (the
 *            K-smoothing subtraction); rows_per_group >= 1 then.
 *   scale_bits I8A_SCALE_FP32 or I8A_SCALE_V4.
 *   codes    int8 [rows, d] out, 8-byte aligned.   scales  fp32 [rows] out.
 */
i8a_status quant_rowwise_i8(const void* x, int64_t rows, int32_t d, const float* sub_mean,
                            int64_t rows_per_group, int32_t scale_bits, int8_t* codes,
                            float* scales, void* stream);

/*
 * attn_int8_workspace_bytes - device workspace needed by attn_int8_fwd (and by the
 * split entry points and attn_int8_debug_qk) for these sizes (0 if the sizes are
 * invalid).  The workspace holds the K partial sums and means, the K codes and scales,
 * the dequantized V, and the Q codes and scales, in private tiled layouts.  It needs no
 * initialization.
 */
size_t attn_int8_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D);

/*
 * attn_int8_fwd - dense INT8 W8A8 attention forward (SuperL8 README, Attention
 * kernels table, row attn_int8_fwd; Quick start call attn_int8_fwd(q, k, v,
 * causal=True)).
 *
 *   q    fp16 [B, Hq, S, D]      k, v  fp16 [B, Hkv, S, D]      out  fp16 [B, Hq, S, D]
 *   1 <= B <= 65535, S >= 1, B*S <= 2^30; 1 <= Hkv <= Hq <= 65535 with Hq % Hkv == 0
 *   (Hkv == 1 is MQA); D in {32, 64, 128, 256}.
 *   softmax_scale  finite and > 0 (the usual value is fp32(1/sqrt(D))); it multiplies
 *                  the dequantized logits and is not folded into Q.
 *   causal         0 or 1; causal means query i attends keys j <= i.
 *   workspace      device buffer of at least attn_int8_workspace_bytes(...) bytes,
 *                  256-byte aligned, not aliasing q, k, v or out.
 * out must not alias q, k or v.
 */
i8a_status attn_int8_fwd(const void* q, const void* k, const void* v, void* out, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t S, int32_t D, float softmax_scale,
                         int32_t causal, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_int8_fwd_noalloc - attn_int8_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is a 64 MiB device array inside the library, one per GPU,
 * held until the process ends, and the call allocates and frees nothing.  Arguments,
 * layouts and errors as for attn_int8_fwd without the workspace; sizes whose workspace
 * (attn_int8_workspace_bytes) exceeds 64 MiB fail with I8A_ERR_WORKSPACE_TOO_SMALL
 * before any work is enqueued (B=1, Hq=32, Hkv=8, S=4096, D=128 needs about 32 MiB).
 * Every call on one GPU uses that GPU's same array: calls that overlap on one GPU (on
 * different streams, or from several threads) race and give undefined output; calls
 * in order on one stream are safe.  No part of the array needs to start at zero.
 */
i8a_status attn_int8_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                                 float softmax_scale, int32_t causal, void* stream);

/*
 * Variants of the forward, as flags of attn_int8_fwd_ex / attn_int8_varlen_fwd_ex (any
 * combination; 0 is attn_int8_fwd itself):
 *
 * I8A_FWD_HADAMARD - Q and K rotated before quantization (SuperL8 README, Quantization
 *   table, row "Hadamard rotation": an incoherence rotation for outlier-heavy
 *   activations).  Each fp32 Q row, and each K row after the K-smoothing subtraction,
 *   is replaced by its unnormalized fast Walsh-Hadamard transform x H (Sylvester H,
 *   entries +-1), computed in fp32 with the butterfly stages s = 0, 1, ..., log2(D) - 1
 *   in that order (the pair (x[i], x[i + 2^s]) with bit s of i clear becomes
 *   (x[i] + x[i + 2^s], x[i] - x[i + 2^s])), and then quantized per row as usual.
 *   Since H H^T = D I the logits take an extra factor 1/D:
 *     logit = S32 * sq_i * sk_j * softmax_scale / D.
 *   V is not rotated.
 *
 * I8A_FWD_V_PER_CHANNEL - V quantized per channel instead of per token (Quantization
 *   table, row "V per-channel / per-token": configurable KV cache quantization): one
 *   scale per (sequence, kv head, channel) over the sequence's tokens,
 *   sv_d = fp32(max_t |v[t,d]| / 127) rounded up to a 4-bit significand, codes
 *   clamp(rint(fp32(v / sv_d)), -127, 127); out = softmax(logit) . (v8 * sv_d).
 */
#define I8A_FWD_HADAMARD 1
#define I8A_FWD_V_PER_CHANNEL 2
/*
 * I8A_FWD_Q_PER_BLOCK - Q quantized per warp (Attention kernels table, attn_w8a8_fwd
 *   row: W8A8 with per-warp quantization): one scale per block of 32 query rows of a
 *   head, the rows one wave owns, counted from the sequence start,
 *   sq_block = fp32(max over the block's rows of max_d |q| / 127), with the codes of
 *   each row by the usual rule against that scale.  Rows past the sequence end keep
 *   zero codes and scale 0.  Combines with the flags above (after the rotation).
 */
#define I8A_FWD_Q_PER_BLOCK 4
/*
 * I8A_FWD_Q_OUTLIERS - Q outlier detection (Quantization table, "Per-row int8" row:
 *   symmetric, K-smoothing, Q outlier detection; Attention kernels table, attn_w8a8_fwd
 *   row: outlier-aware), read as the mixed-precision decomposition of int8 products
 *   with outlier channels (LLM.int8(), Dettmers et al. 2022).  Per (sequence, kv head)
 *   channel d is an outlier when max |q[t, h, d]| over the sequence's tokens and the
 *   group's query heads exceeds 6; at most 16 are kept (largest maxima first, ties to
 *   the lower channel).  Q rows and the mean-smoothed K rows are quantized as usual
 *   with those channels set to zero, and the channels' fp16 values are multiplied
 *   exactly (fp32 sums):
 *     logit = (S32 * sq_i * sk_j + sum_{d outlier} q_id k_jd) * softmax_scale.
 *   Combines with I8A_FWD_V_PER_CHANNEL and I8A_FWD_Q_PER_BLOCK; with I8A_FWD_HADAMARD
 *   it is I8A_ERR_INVALID_ARG, and D = 256 is I8A_ERR_UNSUPPORTED_HEAD_DIM.
 */
#define I8A_FWD_Q_OUTLIERS 8

/* attn_int8_fwd with the variant flags above; arguments, workspace and errors as for
 * attn_int8_fwd (unknown flag bits are I8A_ERR_INVALID_ARG). */
i8a_status attn_int8_fwd_ex(const void* q, const void* k, const void* v, void* out, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t S, int32_t D, float softmax_scale,
                            int32_t causal, int32_t flags, void* workspace,
                            size_t workspace_bytes, void* stream);

/* attn_int8_fwd_ex with flags = I8A_FWD_HADAMARD. */
i8a_status attn_int8_fwd_hadamard(const void* q, const void* k, const void* v, void* out,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                                  float softmax_scale, int32_t causal, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * The phases of attn_int8_fwd as separate calls, for callers that reuse one prepared
 * K/V for several query batches and for timing each phase alone:
 *   attn_int8_prepare_kv   the K-smoothing mean and the K and V quantization;
 *   attn_int8_prepare_q    the Q quantization;
 *   attn_int8_attend       the attention over the prepared Q, K and V;
 *   attn_int8_fwd_prepared attn_int8_prepare_q followed by attn_int8_attend.
 * prepare_kv + prepare_q + attend computes exactly what attn_int8_fwd computes (it
 * enqueues the same kernels).  Sizes (B, Hq, Hkv, S, D) and the workspace must be the
 * same in every call of a sequence, and the workspace must not be modified in between
 * except by these calls; the other arguments are as for attn_int8_fwd.
 */
i8a_status attn_int8_prepare_kv(const void* k, const void* v, int32_t B, int32_t Hq, int32_t Hkv,
                                int32_t S, int32_t D, void* workspace, size_t workspace_bytes,
                                void* stream);
i8a_status attn_int8_prepare_q(const void* q, int32_t B, int32_t Hq, int32_t Hkv, int32_t S,
                               int32_t D, void* workspace, size_t workspace_bytes, void* stream);
i8a_status attn_int8_attend(void* out, int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                            float softmax_scale, int32_t causal, const void* workspace,
                            size_t workspace_bytes, void* stream);
i8a_status attn_int8_fwd_prepared(const void* q, void* out, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t S, int32_t D, float softmax_scale, int32_t causal,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_int8_varlen_workspace_bytes - workspace for attn_int8_varlen_fwd (0 if the
 * sizes are invalid).
 */
size_t attn_int8_varlen_workspace_bytes(int32_t nseq, int64_t total_tokens, int32_t max_seqlen,
                                        int32_t Hq, int32_t Hkv, int32_t D);

/*
 * attn_int8_varlen_fwd - the same forward over a packed batch of sequences of
 * different lengths (SuperL8 README, Attention kernels table, row attn_varlen_fwd:
 * ragged, non-tile-multiple prefill).  Each sequence is independent: its own K mean,
 * its own causal origin.
 *
 *   q    fp16 [total_tokens, Hq, D]   k, v  fp16 [total_tokens, Hkv, D]
 *   out  fp16 [total_tokens, Hq, D]
 *   cu_seqlens  int32 [nseq + 1] on the device: cu[0] = 0, non-decreasing,
 *               cu[nseq] = total_tokens; sequence i is tokens cu[i] .. cu[i+1]-1.
 *               Zero-length sequences are allowed.  The host cannot read it without a
 *               synchronization, so it is not checked here; a sequence whose bounds
 *               fall outside [0, total_tokens] or exceed max_seqlen is skipped by the
 *               kernels (its output rows are left unwritten) and never causes an
 *               out-of-bounds access.
 *   1 <= nseq <= 65535, 0 <= total_tokens <= 2^30, 0 <= max_seqlen <= total_tokens
 *   (host values).
 *   Other arguments as for attn_int8_fwd.
 */
i8a_status attn_int8_varlen_fwd(const void* q, const void* k, const void* v, void* out,
                                const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                                int64_t total_tokens, int32_t Hq, int32_t Hkv, int32_t D,
                                float softmax_scale, int32_t causal, void* workspace,
                                size_t workspace_bytes, void* stream);

/* attn_int8_varlen_fwd with the variant flags of attn_int8_fwd_ex (per sequence: its
 * own K mean and, with I8A_FWD_V_PER_CHANNEL, its own V channel scales). */
i8a_status attn_int8_varlen_fwd_ex(const void* q, const void* k, const void* v, void* out,
                                   const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                                   int64_t total_tokens, int32_t Hq, int32_t Hkv, int32_t D,
                                   float softmax_scale, int32_t causal, int32_t flags,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_int8_debug_qk - debug dump of the quantities the dense forward computes
 * internally, for one (batch b, query head h).  It runs the forward's own
 * quantization kernels and its int8 MFMA score path and writes:
 *   s32_out    int32 [rows, cols]: S32[row0 + i, col0 + j] = q8 . k8 (exact)
 *   qscale_out nullable fp32 [rows]: sq of the query rows
 *   kscale_out nullable fp32 [cols]: sk of the key rows (kv head h / (Hq/Hkv))
 *   vscale_out nullable fp32 [cols]: sv of the same rows
 *   kmean_out  nullable fp32 [D]:   the K-smoothing mean of that kv head
 * with 0 <= row0, row0 + rows <= S, 0 <= col0, col0 + cols <= S, rows, cols >= 1.
 * hadamard 0 or 1: 1 dumps the codes and scales of attn_int8_fwd_hadamard (rotated Q
 * and K rows).  Inputs, sizes and workspace as for attn_int8_fwd (causal is ignored:
 * scores are dumped unmasked).
 */
i8a_status attn_int8_debug_qk(const void* q, const void* k, const void* v, int32_t B, int32_t Hq,
                              int32_t Hkv, int32_t S, int32_t D, int32_t b, int32_t h,
                              int32_t row0, int32_t rows, int32_t col0, int32_t cols,
                              int32_t* s32_out, float* qscale_out, float* kscale_out,
                              float* vscale_out, float* kmean_out, int32_t hadamard,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_int8_debug_qk_ex - the dump of attn_int8_debug_qk for any forward call: dense
 * (cu_seqlens null; nseq = B, max_seqlen = S, total_tokens = B * S, tensors BHSD) or
 * varlen (cu_seqlens on the device as for attn_int8_varlen_fwd, tensors [T, H, D]),
 * with the variant flags of attn_int8_fwd_ex, for sequence `seq` and query head h.
 * It runs the preparation that forward runs (Attention kernels table, attn_int8_fwd,
 * attn_varlen_fwd and attn_w8a8_fwd rows; Quantization table) and writes, besides the
 * outputs of attn_int8_debug_qk:
 *   vhat_out  nullable fp16 [cols, D]: the dequantized V rows of kv head h/(Hq/Hkv) as
 *             the P.V product consumes them (scale times code, exact in fp16)
 *   vchan_out nullable fp32 [D]: the V channel scales (I8A_FWD_V_PER_CHANNEL only)
 *   ochan_out nullable int32 [16]: the Q outlier channels of kv head h/(Hq/Hkv) in
 *             increasing order, padded with -1 (I8A_FWD_Q_OUTLIERS only); with that
 *             flag s32_out, qscale_out and kscale_out are the int8 part's
 * vscale_out (V per token) must be null with I8A_FWD_V_PER_CHANNEL; with
 * I8A_FWD_Q_PER_BLOCK each qscale_out entry is its row's block scale.  Rows and columns
 * must lie in [0, max_seqlen); entries past the sequence's own length are not written.
 * The workspace is sized by attn_int8_workspace_bytes (dense) or
 * attn_int8_varlen_workspace_bytes (varlen).  Errors as for attn_int8_fwd_ex.
 */
i8a_status attn_int8_debug_qk_ex(const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                                 int64_t total_tokens, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t flags, int32_t seq, int32_t h, int32_t row0,
                                 int32_t rows, int32_t col0, int32_t cols, int32_t* s32_out,
                                 float* qscale_out, float* kscale_out, float* vscale_out,
                                 float* kmean_out, void* vhat_out, float* vchan_out,
                                 int32_t* ochan_out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Decode over an int8 KV cache (SuperL8 README, Attention kernels table, row
 * attn_decode: split-KV decode with an int8 KV cache, fp16-V and int8-V variants).
 *
 * attn_int8_kvcache_fill builds the cache of S tokens from fp16 K and V the way the
 * forward quantizes them: K minus its per-channel mean over the S tokens, per-row
 * int8; V per-token int8 with the 4-bit scale rule (I8A_VCACHE_INT8) or V kept in fp16
 * as given (I8A_VCACHE_FP16).  attn_int8_decode then attends one new query token per
 * (batch, query head) to all S cached tokens of its kv head, non-causally (every cached
 * token precedes the new one), with the query row quantized like a Q row:
 *   out[b,h,:] = softmax_j(q8 . k8_j * sq * sk_j * softmax_scale) . V_j
 * with V_j = sv_j * v8_j (int8 V) or the fp16 v_j (fp16 V), and out in fp16.  The
 * keys are split into chunks whose partial results are merged exactly (a rescaled
 * sum), so the split does not change what is computed.
 */
#define I8A_VCACHE_INT8 1 /* V as per-token int8 codes and scales */
#define I8A_VCACHE_FP16 2 /* V as the fp16 values */

/*
 * attn_int8_kvcache_bytes - bytes of a cache for these sizes (0 if they are invalid):
 * 1 <= B <= 65535, 1 <= Hkv <= 65535, S >= 1, B*S <= 2^30, D in {32, 64, 128, 256},
 * v_format I8A_VCACHE_INT8 or I8A_VCACHE_FP16.  The layout is private; the bulk is
 * B*Hkv*ceil(S/32) tiles of 64*D + 192 bytes (int8 V) or 96*D + 128 bytes (fp16 V).
 */
size_t attn_int8_kvcache_bytes(int32_t B, int32_t Hkv, int32_t S, int32_t D, int32_t v_format);

/*
 * attn_int8_kvcache_fill - quantize dense fp16 k, v [B, Hkv, S, D] into `cache` (device,
 * 256-byte aligned, at least attn_int8_kvcache_bytes(...) bytes, not aliasing k or v;
 * it needs no initialization and is fully rewritten).  k and v are 16-byte aligned.
 */
i8a_status attn_int8_kvcache_fill(const void* k, const void* v, int32_t B, int32_t Hkv,
                                  int32_t S, int32_t D, int32_t v_format, void* cache,
                                  size_t cache_bytes, void* stream);

/*
 * attn_int8_decode_workspace_bytes - scratch bytes attn_int8_decode needs for the
 * chunks' partial results (0 if the sizes are invalid or the call needs none).
 */
size_t attn_int8_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t S,
                                        int32_t D, int32_t v_format);

/*
 * attn_int8_decode - one decode step against a cache filled by attn_int8_kvcache_fill
 * with the same B, Hkv, S, D and v_format.
 *   q    fp16 [B, Hq, D]: the new token's query rows      out  fp16 [B, Hq, D]
 *   1 <= Hkv <= Hq <= 65535, Hq % Hkv == 0 (query head h reads kv head h / (Hq/Hkv)).
 *   softmax_scale  finite and > 0 (usually fp32(1/sqrt(D))).
 *   cache, cache_bytes  the filled cache (read only).
 *   workspace      device scratch of at least attn_int8_decode_workspace_bytes(...)
 *                  bytes, 256-byte aligned (may be NULL when that size is 0); calls
 *                  that run concurrently need distinct workspaces.
 * q and out are 16-byte aligned; out aliases neither q, the cache nor the workspace.
 */
i8a_status attn_int8_decode(const void* q, void* out, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t S, int32_t D, float softmax_scale, int32_t v_format,
                            const void* cache, size_t cache_bytes, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * A cache that grows (SuperL8 README, Attention kernels table, row attn_decode: decode
 * serves generation, which adds a token to every sequence at each step; the page gives
 * no rule for the K-smoothing mean of a growing cache).  The mean is taken once, over
 * the tokens a cache is filled with, and every appended K row is quantized against it;
 * the stored mean only moves int8 rounding, since subtracting any fixed vector from K
 * adds a per-query constant to the logits.  S is the cache's capacity in tokens.
 *
 * attn_int8_kvcache_fill_prefix - attn_int8_kvcache_fill of the first S_fill tokens
 * (1 <= S_fill <= S) of a cache of capacity S: k, v fp16 [B, Hkv, S_fill, D], the mean
 * over those tokens.  Slots S_fill .. S-1 hold zero codes, scales and values until
 * appended (a decode reaching them attends zero keys and values).
 * attn_int8_kvcache_fill is the case S_fill = S.
 */
i8a_status attn_int8_kvcache_fill_prefix(const void* k, const void* v, int32_t B, int32_t Hkv,
                                         int32_t S_fill, int32_t S, int32_t D, int32_t v_format,
                                         void* cache, size_t cache_bytes, void* stream);

/*
 * attn_int8_kvcache_append - write n_new tokens per (batch, kv head) into a filled cache.
 *   k, v   fp16 [B, Hkv, n_new, D] on the device, 16-byte aligned: token i of sequence b
 *          goes to slot pos[b] + i.
 *   pos    device int32 [B]: each sequence's first slot (usually its current length).
 *          A token whose slot lies outside [0, S) is not written (nothing else is
 *          touched); pos is read on the device, so the call cannot report it.
 *   0 <= n_new <= S (0: nothing is enqueued, and k, v, pos may be NULL).
 * K rows are quantized against the kv head's stored mean, V rows as the fill does
 * (per-token int8 with the 4-bit scale, or fp16); a slot that is written again is
 * overwritten.  Appends and decodes on one stream run in order; concurrent calls on
 * one cache must not write the same slots.
 */
i8a_status attn_int8_kvcache_append(const void* k, const void* v, int32_t B, int32_t Hkv,
                                    int32_t n_new, const int32_t* pos, int32_t S, int32_t D,
                                    int32_t v_format, void* cache, size_t cache_bytes,
                                    void* stream);

/*
 * attn_int8_decode_lens - attn_int8_decode where sequence b attends only its first
 * lens[b] cached tokens (slots 0 .. lens[b]-1, each filled or appended).
 *   lens   device int32 [B], 4-byte aligned; values are clamped to [0, S].  A sequence
 *          with no token gets a zero output row.
 * Every other argument as for attn_int8_decode (the same workspace size).  With every
 * lens[b] = S it computes what attn_int8_decode computes, bit for bit.
 */
i8a_status attn_int8_decode_lens(const void* q, void* out, int32_t B, int32_t Hq, int32_t Hkv,
                                 int32_t S, int32_t D, float softmax_scale, int32_t v_format,
                                 const int32_t* lens, const void* cache, size_t cache_bytes,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward (SuperL8 README, Attention kernels table, row attn_bwd: a gradient-checked
 * backward pass on full fp16 state; Infrastructure table, autograd row: int8 attention
 * made differentiable).  The quantization of the forward has zero derivative almost
 * everywhere and is taken as the identity (straight-through), so the backward is the
 * gradient of exact attention O = softmax(s Q K^T + mask) V at the fp16 inputs:
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
 *   dQ = s dS K,  dK = s dS^T Q,
 * with dK, dV of a kv head summed over the query heads that read it (GQA).  It runs in
 * O(S) memory (P is recomputed tile by tile from each row's log-sum-exp); every
 * product is an fp16 MFMA with fp32 accumulation, P and dS rounded to fp16 as operands.
 *
 * attn_bwd_workspace_bytes - workspace for attn_bwd (0 if the sizes are invalid): the
 * fp16 inputs in MFMA operand orders, two fp32 values per query row, and partial dK and
 * dV (fp32, the size of dk and dv) for the causal mask's split of the key groups.
 */
size_t attn_bwd_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D);

/*
 * attn_bwd - gradients of the attention.
 *   q, dout  fp16 [B, Hq, S, D]      k, v  fp16 [B, Hkv, S, D]   (16-byte aligned)
 *   dq       fp32 [B, Hq, S, D] out  dk, dv  fp32 [B, Hkv, S, D] out (16-byte aligned)
 *   1 <= B <= 65535, S >= 1, B*S <= 2^30, 1 <= Hkv <= Hq <= 65535, Hq % Hkv == 0,
 *   D in {32, 64, 128, 256}.
 *   softmax_scale, causal as for attn_int8_fwd; workspace of attn_bwd_workspace_bytes
 *   bytes, 256-byte aligned, needs no initialization.  Outputs alias no input.
 */
i8a_status attn_bwd(const void* q, const void* k, const void* v, const void* dout, float* dq,
                    float* dk, float* dv, int32_t B, int32_t Hq, int32_t Hkv, int32_t S,
                    int32_t D, float softmax_scale, int32_t causal, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Name of a status code (static string). */
const char* i8a_status_string(i8a_status status);

/* Detail of the last failure on the calling thread (static per-thread buffer). */
const char* i8a_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* I8ATTN_H */
