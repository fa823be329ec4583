// capi.hip - the extern "C" entry points declared in include/i8attn.h: argument
// validation (all on the host, before anything is enqueued), workspace planning and
// launch sequencing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "i8a_launch.h"
#include "i8attn.h"

namespace i8a {

static thread_local char g_last_error[512] = "";

static i8a_status fail(i8a_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

static i8a_status hip_fail(hipError_t e, const char* what) {
  return fail(I8A_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsPlan plan_workspace(int32_t nseq, int64_t total_tokens, int32_t max_len, int32_t Hq,
                      int32_t Hkv, int32_t D) {
  WsPlan p;
  p.nseq = nseq;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.ntile = (max_len + TK - 1) / TK;
  p.tpw = (p.ntile + MAX_PARTS - 1) / MAX_PARTS;
  if (p.tpw < 1) p.tpw = 1;
  p.npart = (p.ntile + p.tpw - 1) / p.tpw;
  p.Ppad = (int64_t)TK * ((total_tokens + TK - 1) / TK + nseq);
  p.Qpad = (int64_t)BQ * ((total_tokens + BQ - 1) / BQ + nseq);
  size_t off = 0;
  p.off_kpart = off;
  off = align256(off + (size_t)nseq * Hkv * p.npart * D * 8);
  p.off_kmean = off;
  off = align256(off + (size_t)nseq * Hkv * D * 4);
  p.off_vpart = off;
  off = align256(off + (size_t)nseq * Hkv * p.npart * D * 4);
  p.off_svc = off;
  off = align256(off + (size_t)nseq * Hkv * D * 4);
  p.off_sv = off;
  off = align256(off + (size_t)Hkv * p.Ppad * 4);
  p.off_qopart = off;
  off = align256(off + (size_t)nseq * Hkv * p.npart * D * 4);
  p.off_ochan = off;
  off = align256(off + (size_t)nseq * Hkv * QO_MAX * 4);
  p.off_tiles = off;
  off = align256(off + (size_t)Hkv * (p.Ppad / TK) * tile_bytes(D, true));
  p.off_q8 = off;
  off = align256(off + (size_t)Hq * p.Qpad * D);
  p.off_qs = off;
  off = align256(off + (size_t)Hq * p.Qpad * 4);
  p.total = off;
  return p;
}

static bool head_dim_ok(int32_t D) { return D == 32 || D == 64 || D == 128 || D == 256; }

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Heads and sequences index the y and z dimensions of the preparation grids.
static const int32_t kMaxGridYZ = 65535;

// Common checks of the forward entry points.  Sizes in tokens are bounded so that
// every element offset fits in int64 and every token index in int32.
static i8a_status check_common(const void* q, const void* k, const void* v, const void* out,
                               int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                               int32_t causal, const void* ws) {
  if (!q || !k || !v || !out) return fail(I8A_ERR_INVALID_ARG, "null q/k/v/out pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(I8A_ERR_INVALID_ARG, "q/k/v/out must be 16-byte aligned");
  if (!head_dim_ok(D))
    return fail(I8A_ERR_UNSUPPORTED_HEAD_DIM, "head dim %d not in {32,64,128,256}", D);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(I8A_ERR_INVALID_ARG, "need Hq >= 1, Hkv >= 1 and Hq %% Hkv == 0 (Hq=%d Hkv=%d)",
                Hq, Hkv);
  if (Hq > kMaxGridYZ) return fail(I8A_ERR_INVALID_ARG, "Hq must be <= %d", kMaxGridYZ);
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale))
    return fail(I8A_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(I8A_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!ws) return fail(I8A_ERR_INVALID_ARG, "null workspace");
  if (!aligned(ws, 256)) return fail(I8A_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return I8A_OK;
}

static const int64_t kMaxTokens = (int64_t)1 << 30;

// ---------------------------------------------------------------------------------
// Scratch memory of attn_int8_fwd_noalloc: the forward's workspace as a file-scope
// device array, so that the entry point allocates nothing.  Every GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch` is only a
// stand-in for the symbol: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept in scratch_ptr.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static void* scratch_ptr[kMaxDevices];
static std::mutex scratch_mu;

static hipError_t scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace i8a

using namespace i8a;

extern "C" {

const char* i8a_status_string(i8a_status s) {
  switch (s) {
    case I8A_OK: return "I8A_OK";
    case I8A_ERR_INVALID_ARG: return "I8A_ERR_INVALID_ARG";
    case I8A_ERR_UNSUPPORTED_HEAD_DIM: return "I8A_ERR_UNSUPPORTED_HEAD_DIM";
    case I8A_ERR_WORKSPACE_TOO_SMALL: return "I8A_ERR_WORKSPACE_TOO_SMALL";
    case I8A_ERR_HIP: return "I8A_ERR_HIP";
    default: return "I8A_UNKNOWN_STATUS";
  }
}

const char* i8a_last_error(void) { return g_last_error; }

i8a_status quant_rowwise_i8(const void* x, int64_t rows, int32_t d, const float* sub_mean,
                            int64_t rows_per_group, int32_t scale_bits, int8_t* codes,
                            float* scales, void* stream) {
  if (rows < 0) return fail(I8A_ERR_INVALID_ARG, "rows must be >= 0");
  if (d < 8 || d > 512 || d % 8 != 0)
    return fail(I8A_ERR_INVALID_ARG, "d must be a multiple of 8 in [8, 512] (got %d)", d);
  if (scale_bits != I8A_SCALE_FP32 && scale_bits != I8A_SCALE_V4)
    return fail(I8A_ERR_INVALID_ARG, "scale_bits must be 24 or 4");
  if (sub_mean && rows_per_group < 1)
    return fail(I8A_ERR_INVALID_ARG, "rows_per_group must be >= 1 with sub_mean");
  if (rows == 0) return I8A_OK;
  if (!x || !codes || !scales) return fail(I8A_ERR_INVALID_ARG, "null x/codes/scales pointer");
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(scales, 4) ||
      (sub_mean && !aligned(sub_mean, 4)))
    return fail(I8A_ERR_INVALID_ARG, "misaligned pointer (x 16 B, codes 8 B, floats 4 B)");
  hipError_t e = launch_quant_rowwise(x, rows, d, sub_mean, sub_mean ? rows_per_group : 1,
                                      scale_bits, codes, scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quant_rowwise_i8 launch");
  return I8A_OK;
}

size_t attn_int8_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D) {
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || !head_dim_ok(D)) return 0;
  if (B > kMaxGridYZ || Hq > kMaxGridYZ) return 0;
  if ((int64_t)B * S > kMaxTokens) return 0;
  return plan_workspace(B, (int64_t)B * S, S, Hq, Hkv, D).total;
}

size_t attn_int8_varlen_workspace_bytes(int32_t nseq, int64_t total_tokens, int32_t max_seqlen,
                                        int32_t Hq, int32_t Hkv, int32_t D) {
  if (nseq < 1 || total_tokens < 0 || total_tokens > kMaxTokens || max_seqlen < 0 ||
      max_seqlen > total_tokens || Hq < 1 || Hkv < 1 || Hq % Hkv || !head_dim_ok(D) ||
      nseq > kMaxGridYZ || Hq > kMaxGridYZ)
    return 0;
  return plan_workspace(nseq, total_tokens, max_seqlen, Hq, Hkv, D).total;
}

// The phases of a forward call, enqueued in order: K/V preparation, Q preparation,
// attention.
enum Phase { PH_KV = 1, PH_Q = 2, PH_ATTN = 4 };

static i8a_status run_phases(const FwdGeom& g, int phases, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  const WsPlan p = plan_workspace(g.nseq, g.T, g.max_len, g.Hq, g.Hkv, g.D);
  if (ws_bytes < p.total)
    return fail(I8A_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", p.total,
                ws_bytes);
  hipError_t e;
  // Q quantized inside the attention kernel where it supports the variant: the same
  // codes and scales as the Q preparation, without their round trip through memory.
  FwdGeom gf = g;
  if ((phases & PH_Q) && (phases & PH_ATTN)) {
    gf.fuse_q = 1;
    phases &= ~PH_Q;
  }
  if (phases & (PH_KV | PH_Q)) {
    e = launch_prep(g, p, ws, (phases & PH_KV) != 0, (phases & PH_Q) != 0, stream);
    if (e != hipSuccess) return hip_fail(e, "preparation launch");
  }
  if (!(phases & PH_ATTN)) return I8A_OK;
  e = launch_attn(gf, p, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return I8A_OK;
}

i8a_status attn_int8_fwd(const void* q, const void* k, const void* v, void* out, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t S, int32_t D, float softmax_scale,
                         int32_t causal, void* workspace, size_t workspace_bytes, void* stream) {
  i8a_status st = check_common(q, k, v, out, Hq, Hkv, D, softmax_scale, causal, workspace);
  if (st != I8A_OK) return st;
  if (B < 1 || S < 1 || B > kMaxGridYZ)
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= B <= %d and S >= 1", kMaxGridYZ);
  if ((int64_t)B * S > kMaxTokens) return fail(I8A_ERR_INVALID_ARG, "B*S too large");
  FwdGeom g{q, k, v, out, nullptr, B, S, S, (int64_t)B * S, Hq, Hkv, D, softmax_scale, causal};
  return run_phases(g, PH_KV | PH_Q | PH_ATTN, workspace, workspace_bytes, (hipStream_t)stream);
}

i8a_status attn_int8_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                                 float softmax_scale, int32_t causal, void* stream) {
  // The workspace check of attn_int8_fwd with a placeholder address, so that a size
  // beyond the scratch array is rejected before anything touches the device.
  i8a_status st = check_common(q, k, v, out, Hq, Hkv, D, softmax_scale, causal,
                               reinterpret_cast<void*>(256));
  if (st != I8A_OK) return st;
  if (B < 1 || S < 1 || B > kMaxGridYZ)
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= B <= %d and S >= 1", kMaxGridYZ);
  if ((int64_t)B * S > kMaxTokens) return fail(I8A_ERR_INVALID_ARG, "B*S too large");
  const size_t need = plan_workspace(B, (int64_t)B * S, S, Hq, Hkv, D).total;
  if (need > kScratchBytes)
    return fail(I8A_ERR_WORKSPACE_TOO_SMALL,
                "attn_int8_fwd_noalloc: these sizes need %zu bytes of workspace, more than its "
                "%zu-byte scratch; call attn_int8_fwd with a workspace",
                need, kScratchBytes);
  void* ws = nullptr;
  hipError_t e = scratch_for_current_device(&ws);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  return attn_int8_fwd(q, k, v, out, B, Hq, Hkv, S, D, softmax_scale, causal, ws, kScratchBytes,
                       stream);
}

// The variant flags of a forward call into its geometry.
static i8a_status apply_flags(FwdGeom& g, int32_t flags) {
  if (flags & ~(I8A_FWD_HADAMARD | I8A_FWD_V_PER_CHANNEL | I8A_FWD_Q_PER_BLOCK |
                I8A_FWD_Q_OUTLIERS))
    return fail(I8A_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  g.rot = (flags & I8A_FWD_HADAMARD) ? 1 : 0;
  g.vch = (flags & I8A_FWD_V_PER_CHANNEL) ? 1 : 0;
  g.qblk = (flags & I8A_FWD_Q_PER_BLOCK) ? 1 : 0;
  g.qout = (flags & I8A_FWD_Q_OUTLIERS) ? 1 : 0;
  if (g.qout && g.rot)
    return fail(I8A_ERR_INVALID_ARG, "I8A_FWD_Q_OUTLIERS does not combine with I8A_FWD_HADAMARD");
  if (g.qout && g.D > 128)
    return fail(I8A_ERR_UNSUPPORTED_HEAD_DIM, "I8A_FWD_Q_OUTLIERS needs D <= 128, got %d", g.D);
  return I8A_OK;
}

i8a_status attn_int8_fwd_ex(const void* q, const void* k, const void* v, void* out, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t S, int32_t D, float softmax_scale,
                            int32_t causal, int32_t flags, void* workspace,
                            size_t workspace_bytes, void* stream) {
  i8a_status st = check_common(q, k, v, out, Hq, Hkv, D, softmax_scale, causal, workspace);
  if (st != I8A_OK) return st;
  if (B < 1 || S < 1 || B > kMaxGridYZ)
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= B <= %d and S >= 1", kMaxGridYZ);
  if ((int64_t)B * S > kMaxTokens) return fail(I8A_ERR_INVALID_ARG, "B*S too large");
  FwdGeom g{q, k, v, out, nullptr, B, S, S, (int64_t)B * S, Hq, Hkv, D, softmax_scale, causal};
  st = apply_flags(g, flags);
  if (st != I8A_OK) return st;
  return run_phases(g, PH_KV | PH_Q | PH_ATTN, workspace, workspace_bytes, (hipStream_t)stream);
}

i8a_status attn_int8_fwd_hadamard(const void* q, const void* k, const void* v, void* out,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                                  float softmax_scale, int32_t causal, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return attn_int8_fwd_ex(q, k, v, out, B, Hq, Hkv, S, D, softmax_scale, causal,
                          I8A_FWD_HADAMARD, workspace, workspace_bytes, stream);
}

i8a_status attn_int8_prepare_kv(const void* k, const void* v, int32_t B, int32_t Hq, int32_t Hkv,
                                int32_t S, int32_t D, void* workspace, size_t workspace_bytes,
                                void* stream) {
  // q and out are not touched by this phase; k stands in for their checks.
  i8a_status st = check_common(k, k, v, k, Hq, Hkv, D, 1.0f, 0, workspace);
  if (st != I8A_OK) return st;
  if (B < 1 || S < 1 || B > kMaxGridYZ || (int64_t)B * S > kMaxTokens)
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= B <= %d, S >= 1, B*S in range", kMaxGridYZ);
  FwdGeom g{nullptr, k, v, nullptr, nullptr, B, S, S, (int64_t)B * S, Hq, Hkv, D, 1.0f, 0};
  return run_phases(g, PH_KV, workspace, workspace_bytes, (hipStream_t)stream);
}

i8a_status attn_int8_prepare_q(const void* q, int32_t B, int32_t Hq, int32_t Hkv, int32_t S,
                               int32_t D, void* workspace, size_t workspace_bytes, void* stream) {
  // k, v and out are not touched by this phase; q stands in for their checks.
  i8a_status st = check_common(q, q, q, q, Hq, Hkv, D, 1.0f, 0, workspace);
  if (st != I8A_OK) return st;
  if (B < 1 || S < 1 || B > kMaxGridYZ || (int64_t)B * S > kMaxTokens)
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= B <= %d, S >= 1, B*S in range", kMaxGridYZ);
  FwdGeom g{q, nullptr, nullptr, nullptr, nullptr, B, S, S, (int64_t)B * S, Hq, Hkv, D, 1.0f, 0};
  return run_phases(g, PH_Q, workspace, workspace_bytes, (hipStream_t)stream);
}

i8a_status attn_int8_attend(void* out, int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                            float softmax_scale, int32_t causal, const void* workspace,
                            size_t workspace_bytes, void* stream) {
  // Only out and the workspace are touched; out stands in for the q/k/v checks.
  i8a_status st = check_common(out, out, out, out, Hq, Hkv, D, softmax_scale, causal, workspace);
  if (st != I8A_OK) return st;
  if (B < 1 || S < 1 || B > kMaxGridYZ || (int64_t)B * S > kMaxTokens)
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= B <= %d, S >= 1, B*S in range", kMaxGridYZ);
  FwdGeom g{nullptr, nullptr, nullptr, out, nullptr, B, S, S, (int64_t)B * S, Hq, Hkv, D,
            softmax_scale, causal};
  return run_phases(g, PH_ATTN, const_cast<void*>(workspace), workspace_bytes,
                    (hipStream_t)stream);
}

i8a_status attn_int8_fwd_prepared(const void* q, void* out, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t S, int32_t D, float softmax_scale, int32_t causal,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  // k and v are not read by this phase; q stands in for their checks.
  i8a_status st = check_common(q, q, q, out, Hq, Hkv, D, softmax_scale, causal, workspace);
  if (st != I8A_OK) return st;
  if (B < 1 || S < 1 || B > kMaxGridYZ || (int64_t)B * S > kMaxTokens)
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= B <= %d, S >= 1, B*S in range", kMaxGridYZ);
  FwdGeom g{q, nullptr, nullptr, out, nullptr, B, S, S, (int64_t)B * S, Hq, Hkv, D,
            softmax_scale, causal};
  return run_phases(g, PH_Q | PH_ATTN, workspace, workspace_bytes, (hipStream_t)stream);
}

i8a_status attn_int8_varlen_fwd_ex(const void* q, const void* k, const void* v, void* out,
                                   const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                                   int64_t total_tokens, int32_t Hq, int32_t Hkv, int32_t D,
                                   float softmax_scale, int32_t causal, int32_t flags,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  {
    FwdGeom probe{};
    probe.D = D;
    const i8a_status fst = apply_flags(probe, flags);
    if (fst != I8A_OK) return fst;
  }
  if (!cu_seqlens) return fail(I8A_ERR_INVALID_ARG, "null cu_seqlens");
  if (!aligned(cu_seqlens, 4)) return fail(I8A_ERR_INVALID_ARG, "misaligned cu_seqlens");
  if (nseq < 1 || nseq > kMaxGridYZ)
    return fail(I8A_ERR_INVALID_ARG, "nseq must be in [1, %d]", kMaxGridYZ);
  if (total_tokens < 0 || total_tokens > kMaxTokens)
    return fail(I8A_ERR_INVALID_ARG, "total_tokens out of range");
  if (max_seqlen < 0 || max_seqlen > total_tokens)
    return fail(I8A_ERR_INVALID_ARG, "need 0 <= max_seqlen <= total_tokens");
  if (total_tokens == 0 || max_seqlen == 0) {
    // nothing to compute; still validate the rest for a consistent contract
    if (!head_dim_ok(D))
      return fail(I8A_ERR_UNSUPPORTED_HEAD_DIM, "head dim %d not in {32,64,128,256}", D);
    if (Hq < 1 || Hkv < 1 || Hq % Hkv || Hq > kMaxGridYZ)
      return fail(I8A_ERR_INVALID_ARG, "bad Hq/Hkv");
    return I8A_OK;
  }
  i8a_status st = check_common(q, k, v, out, Hq, Hkv, D, softmax_scale, causal, workspace);
  if (st != I8A_OK) return st;
  FwdGeom g{q, k, v, out, cu_seqlens, nseq, 0, max_seqlen, total_tokens, Hq, Hkv, D,
            softmax_scale, causal};
  st = apply_flags(g, flags);
  if (st != I8A_OK) return st;
  return run_phases(g, PH_KV | PH_Q | PH_ATTN, workspace, workspace_bytes, (hipStream_t)stream);
}

i8a_status attn_int8_varlen_fwd(const void* q, const void* k, const void* v, void* out,
                                const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                                int64_t total_tokens, int32_t Hq, int32_t Hkv, int32_t D,
                                float softmax_scale, int32_t causal, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return attn_int8_varlen_fwd_ex(q, k, v, out, cu_seqlens, nseq, max_seqlen, total_tokens, Hq,
                                 Hkv, D, softmax_scale, causal, 0, workspace, workspace_bytes,
                                 stream);
}

i8a_status attn_int8_debug_qk_ex(const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                                 int64_t total_tokens, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t flags, int32_t seq, int32_t h, int32_t row0,
                                 int32_t rows, int32_t col0, int32_t cols, int32_t* s32_out,
                                 float* qscale_out, float* kscale_out, float* vscale_out,
                                 float* kmean_out, void* vhat_out, float* vchan_out,
                                 int32_t* ochan_out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  // No output tensor is written by this entry; q stands in for its alignment check.
  i8a_status st = check_common(q, k, v, q, Hq, Hkv, D, 1.0f, 0, workspace);
  if (st != I8A_OK) return st;
  FwdGeom g{q, k, v, nullptr, cu_seqlens, nseq, cu_seqlens ? 0 : max_seqlen, max_seqlen,
            total_tokens, Hq, Hkv, D, 1.0f, 0};
  st = apply_flags(g, flags);
  if (st != I8A_OK) return st;
  if (nseq < 1 || nseq > kMaxGridYZ || max_seqlen < 1 || total_tokens < 1 ||
      total_tokens > kMaxTokens || max_seqlen > total_tokens)
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= nseq <= %d, 1 <= max_seqlen <= total_tokens",
                kMaxGridYZ);
  if (cu_seqlens && !aligned(cu_seqlens, 4))
    return fail(I8A_ERR_INVALID_ARG, "misaligned cu_seqlens");
  if (!cu_seqlens && total_tokens != (int64_t)nseq * max_seqlen)
    return fail(I8A_ERR_INVALID_ARG, "dense geometry needs total_tokens = nseq * max_seqlen");
  if (seq < 0 || seq >= nseq || h < 0 || h >= Hq)
    return fail(I8A_ERR_INVALID_ARG, "seq/h out of range");
  if (rows < 1 || cols < 1 || row0 < 0 || col0 < 0 || (int64_t)row0 + rows > max_seqlen ||
      (int64_t)col0 + cols > max_seqlen)
    return fail(I8A_ERR_INVALID_ARG, "tile [%d+%d, %d+%d] outside [0, %d)", row0, rows, col0,
                cols, max_seqlen);
  if (!s32_out || !aligned(s32_out, 4)) return fail(I8A_ERR_INVALID_ARG, "bad s32_out");
  if (vhat_out && !aligned(vhat_out, 2)) return fail(I8A_ERR_INVALID_ARG, "bad vhat_out");
  const bool vch = (flags & I8A_FWD_V_PER_CHANNEL) != 0;
  if (vch && vscale_out)
    return fail(I8A_ERR_INVALID_ARG, "vscale_out (V per token) with I8A_FWD_V_PER_CHANNEL");
  if (!vch && vchan_out)
    return fail(I8A_ERR_INVALID_ARG, "vchan_out needs I8A_FWD_V_PER_CHANNEL");
  if (ochan_out && !g.qout) return fail(I8A_ERR_INVALID_ARG, "ochan_out needs I8A_FWD_Q_OUTLIERS");
  if (ochan_out && !aligned(ochan_out, 4)) return fail(I8A_ERR_INVALID_ARG, "bad ochan_out");
  const WsPlan p = plan_workspace(nseq, total_tokens, max_seqlen, Hq, Hkv, D);
  i8a_status pst = run_phases(g, PH_KV | PH_Q, workspace, workspace_bytes, (hipStream_t)stream);
  if (pst != I8A_OK) return pst;
  const DebugOut o{s32_out,   cols,      qscale_out, kscale_out, vscale_out,
                   kmean_out, static_cast<_Float16*>(vhat_out), vchan_out, ochan_out};
  hipError_t e = launch_debug_qk(g, p, workspace, seq, h, row0, rows, col0, cols, o,
                                 (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "debug score launch");
  return I8A_OK;
}

i8a_status attn_int8_debug_qk(const void* q, const void* k, const void* v, int32_t B, int32_t Hq,
                              int32_t Hkv, int32_t S, int32_t D, int32_t b, int32_t h,
                              int32_t row0, int32_t rows, int32_t col0, int32_t cols,
                              int32_t* s32_out, float* qscale_out, float* kscale_out,
                              float* vscale_out, float* kmean_out, int32_t hadamard,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (hadamard != 0 && hadamard != 1) return fail(I8A_ERR_INVALID_ARG, "hadamard must be 0 or 1");
  if (B < 1 || S < 1 || B > kMaxGridYZ || (int64_t)B * S > kMaxTokens)
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= B <= %d, S >= 1, B*S in range", kMaxGridYZ);
  return attn_int8_debug_qk_ex(q, k, v, nullptr, B, S, (int64_t)B * S, Hq, Hkv, D,
                               hadamard ? I8A_FWD_HADAMARD : 0, b, h, row0, rows, col0, cols,
                               s32_out, qscale_out, kscale_out, vscale_out, kmean_out, nullptr,
                               nullptr, nullptr, workspace, workspace_bytes, stream);
}

static_assert(I8A_VCACHE_INT8 == VF_INT8 && I8A_VCACHE_FP16 == VF_FP16,
              "the C ABI v_format codes are the kernels' VFormat values");

static bool kvc_sizes_ok(int32_t B, int32_t Hkv, int32_t S, int32_t D, int32_t vf) {
  return B >= 1 && B <= kMaxGridYZ && Hkv >= 1 && Hkv <= kMaxGridYZ && S >= 1 &&
         (int64_t)B * S <= kMaxTokens && head_dim_ok(D) &&
         (vf == I8A_VCACHE_INT8 || vf == I8A_VCACHE_FP16) &&
         (int64_t)B * Hkv <= ((int64_t)1 << 24);
}

size_t attn_int8_kvcache_bytes(int32_t B, int32_t Hkv, int32_t S, int32_t D, int32_t v_format) {
  if (!kvc_sizes_ok(B, Hkv, S, D, v_format)) return 0;
  return plan_kvcache(B, Hkv, S, D, v_format).total;
}

static i8a_status kvc_check(int32_t B, int32_t Hkv, int32_t S, int32_t D, int32_t vf,
                            const void* cache, size_t cache_bytes, size_t* need) {
  if (!head_dim_ok(D))
    return fail(I8A_ERR_UNSUPPORTED_HEAD_DIM, "head dim %d not in {32,64,128,256}", D);
  if (vf != I8A_VCACHE_INT8 && vf != I8A_VCACHE_FP16)
    return fail(I8A_ERR_INVALID_ARG, "v_format must be I8A_VCACHE_INT8 or I8A_VCACHE_FP16");
  if (!kvc_sizes_ok(B, Hkv, S, D, vf))
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= B, Hkv <= %d, S >= 1, B*S <= 2^30 (B=%d Hkv=%d S=%d)",
                kMaxGridYZ, B, Hkv, S);
  if (!cache) return fail(I8A_ERR_INVALID_ARG, "null cache");
  if (!aligned(cache, 256)) return fail(I8A_ERR_INVALID_ARG, "cache must be 256-byte aligned");
  *need = plan_kvcache(B, Hkv, S, D, vf).total;
  if (cache_bytes < *need)
    return fail(I8A_ERR_WORKSPACE_TOO_SMALL, "cache needs %zu bytes, got %zu", *need, cache_bytes);
  return I8A_OK;
}

i8a_status attn_int8_kvcache_fill(const void* k, const void* v, int32_t B, int32_t Hkv,
                                  int32_t S, int32_t D, int32_t v_format, void* cache,
                                  size_t cache_bytes, void* stream) {
  if (!k || !v) return fail(I8A_ERR_INVALID_ARG, "null k/v pointer");
  if (!aligned(k, 16) || !aligned(v, 16))
    return fail(I8A_ERR_INVALID_ARG, "k/v must be 16-byte aligned");
  size_t need;
  i8a_status st = kvc_check(B, Hkv, S, D, v_format, cache, cache_bytes, &need);
  if (st != I8A_OK) return st;
  hipError_t e = launch_kvcache_fill(k, v, plan_kvcache(B, Hkv, S, D, v_format), S, cache,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cache fill launch");
  return I8A_OK;
}

i8a_status attn_int8_kvcache_fill_prefix(const void* k, const void* v, int32_t B, int32_t Hkv,
                                         int32_t S_fill, int32_t S, int32_t D, int32_t v_format,
                                         void* cache, size_t cache_bytes, void* stream) {
  if (!k || !v) return fail(I8A_ERR_INVALID_ARG, "null k/v pointer");
  if (!aligned(k, 16) || !aligned(v, 16))
    return fail(I8A_ERR_INVALID_ARG, "k/v must be 16-byte aligned");
  size_t need;
  i8a_status st = kvc_check(B, Hkv, S, D, v_format, cache, cache_bytes, &need);
  if (st != I8A_OK) return st;
  if (S_fill < 1 || S_fill > S)
    return fail(I8A_ERR_INVALID_ARG, "need 1 <= S_fill <= S (S_fill=%d S=%d)", S_fill, S);
  hipError_t e = launch_kvcache_fill(k, v, plan_kvcache(B, Hkv, S, D, v_format), S_fill, cache,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cache fill launch");
  return I8A_OK;
}

i8a_status attn_int8_kvcache_append(const void* k, const void* v, int32_t B, int32_t Hkv,
                                    int32_t n_new, const int32_t* pos, int32_t S, int32_t D,
                                    int32_t v_format, void* cache, size_t cache_bytes,
                                    void* stream) {
  size_t need;
  i8a_status st = kvc_check(B, Hkv, S, D, v_format, cache, cache_bytes, &need);
  if (st != I8A_OK) return st;
  if (n_new < 0 || n_new > S)
    return fail(I8A_ERR_INVALID_ARG, "need 0 <= n_new <= S (n_new=%d S=%d)", n_new, S);
  if (n_new == 0) return I8A_OK;
  if (!k || !v || !pos) return fail(I8A_ERR_INVALID_ARG, "null k/v/pos pointer");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(pos, 4))
    return fail(I8A_ERR_INVALID_ARG, "k/v must be 16-byte and pos 4-byte aligned");
  hipError_t e = launch_kvcache_append(k, v, n_new, pos, plan_kvcache(B, Hkv, S, D, v_format),
                                       cache, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cache append launch");
  return I8A_OK;
}

size_t attn_int8_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t S,
                                        int32_t D, int32_t v_format) {
  if (!kvc_sizes_ok(B, Hkv, S, D, v_format) || Hq < Hkv || Hq > kMaxGridYZ || Hq % Hkv)
    return 0;
  return plan_decode(B, Hq, Hkv, S, D, v_format).total;
}

static i8a_status decode_impl(const void* q, void* out, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t S, int32_t D, float softmax_scale, int32_t v_format,
                              const int32_t* lens, const void* cache, size_t cache_bytes,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !out) return fail(I8A_ERR_INVALID_ARG, "null q/out pointer");
  if (!aligned(q, 16) || !aligned(out, 16))
    return fail(I8A_ERR_INVALID_ARG, "q/out must be 16-byte aligned");
  size_t need;
  i8a_status st = kvc_check(B, Hkv, S, D, v_format, cache, cache_bytes, &need);
  if (st != I8A_OK) return st;
  if (Hq < Hkv || Hq > kMaxGridYZ || Hq % Hkv)
    return fail(I8A_ERR_INVALID_ARG, "need Hkv <= Hq <= %d and Hq %% Hkv == 0 (Hq=%d Hkv=%d)",
                kMaxGridYZ, Hq, Hkv);
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale))
    return fail(I8A_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  const DecPlan dp = plan_decode(B, Hq, Hkv, S, D, v_format);
  if (workspace_bytes < dp.total)
    return fail(I8A_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", dp.total,
                workspace_bytes);
  if (dp.total > 0 && (!workspace || !aligned(workspace, 256)))
    return fail(I8A_ERR_INVALID_ARG, "workspace must be non-null and 256-byte aligned");
  hipError_t e = launch_decode(q, out, Hq, softmax_scale, plan_kvcache(B, Hkv, S, D, v_format),
                               dp, cache, workspace, lens, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return I8A_OK;
}

i8a_status attn_int8_decode(const void* q, void* out, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t S, int32_t D, float softmax_scale, int32_t v_format,
                            const void* cache, size_t cache_bytes, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_impl(q, out, B, Hq, Hkv, S, D, softmax_scale, v_format, nullptr, cache,
                     cache_bytes, workspace, workspace_bytes, stream);
}

i8a_status attn_int8_decode_lens(const void* q, void* out, int32_t B, int32_t Hq, int32_t Hkv,
                                 int32_t S, int32_t D, float softmax_scale, int32_t v_format,
                                 const int32_t* lens, const void* cache, size_t cache_bytes,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!lens || !aligned(lens, 4))
    return fail(I8A_ERR_INVALID_ARG, "lens must be a non-null, 4-byte aligned device array");
  return decode_impl(q, out, B, Hq, Hkv, S, D, softmax_scale, v_format, lens, cache,
                     cache_bytes, workspace, workspace_bytes, stream);
}

static bool bwd_sizes_ok(int32_t B, int32_t Hq, int32_t Hkv, int32_t S) {
  return B >= 1 && B <= kMaxGridYZ && S >= 1 && (int64_t)B * S <= kMaxTokens && Hkv >= 1 &&
         Hq >= Hkv && Hq <= kMaxGridYZ && Hq % Hkv == 0;
}

size_t attn_bwd_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D) {
  if (!bwd_sizes_ok(B, Hq, Hkv, S) || (D != 32 && D != 64 && D != 128 && D != 256)) return 0;
  return plan_bwd(B, Hq, Hkv, S, D).total;
}

i8a_status attn_bwd(const void* q, const void* k, const void* v, const void* dout, float* dq,
                    float* dk, float* dv, int32_t B, int32_t Hq, int32_t Hkv, int32_t S,
                    int32_t D, float softmax_scale, int32_t causal, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv)
    return fail(I8A_ERR_INVALID_ARG, "null input or output pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(I8A_ERR_INVALID_ARG, "inputs and outputs must be 16-byte aligned");
  if (D != 32 && D != 64 && D != 128 && D != 256)
    return fail(I8A_ERR_UNSUPPORTED_HEAD_DIM, "backward head dim %d not in {32,64,128,256}", D);
  if (!bwd_sizes_ok(B, Hq, Hkv, S))
    return fail(I8A_ERR_INVALID_ARG, "bad sizes B=%d Hq=%d Hkv=%d S=%d", B, Hq, Hkv, S);
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale))
    return fail(I8A_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(I8A_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!workspace || !aligned(workspace, 256))
    return fail(I8A_ERR_INVALID_ARG, "workspace must be non-null and 256-byte aligned");
  const BwdPlan p = plan_bwd(B, Hq, Hkv, S, D);
  if (workspace_bytes < p.total)
    return fail(I8A_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", p.total,
                workspace_bytes);
  BwdArgs a{q, k, v, dout, dq, dk, dv, B, Hq, Hkv, S, D, softmax_scale, causal};
  hipError_t e = launch_bwd(a, p, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return I8A_OK;
}

}  // extern "C"
