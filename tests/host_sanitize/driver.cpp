// Host-side check of the C ABI's argument validation (include/i8attn.h), meant to be
// linked against the library's host code built with the address and undefined-behaviour
// sanitizers, or with the thread sanitizer.
//
// Every call below is rejected on the host before anything is enqueued, or has nothing
// to compute (an empty varlen batch, zero quantization rows): no HIP call and no kernel
// launch is ever reached, and the pointers passed are fake aligned addresses that host
// code never dereferences.  The calls that would otherwise pass are made to fail by a
// workspace or cache one byte short of what the matching *_bytes function reports.
//
// For each entry point the expected status is worked out from the header's contract
// (the order in which it checks pointers, head dim, sizes, flags and workspace) over
// seeded random arguments drawn from edge values (0, -1, INT32_MIN/MAX, 2^16, 2^30, ...)
// and from valid ranges, so that the size arithmetic runs at the largest sizes the
// contract admits.  It also checks that each *_bytes function returns nonzero exactly
// when its sizes are valid, that the value is a multiple of 256 where promised and no
// smaller than the bytes of the tensors the workspace holds (a wrapped size would be),
// and that i8a_last_error holds a terminated message after each failure, per thread.
//
// Usage: driver [iterations-per-thread] [threads]; exits 0 when every check holds.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <string>
#include <thread>
#include <vector>

#include "i8attn.h"

namespace {

std::atomic<long> g_fail{0};
std::atomic<long> g_calls{0};
std::atomic<long> g_by_status[5];  // calls per expected status: OK, -1, -2, -3, -4

struct Rng {  // splitmix64
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int below(int n) { return (int)(next() % (uint64_t)n); }
  bool coin(int pct) { return below(100) < pct; }
};

const int32_t kEdge[] = {INT32_MIN, -65536, -2, -1, 0, 1, 2, 3, 4, 7, 8, 16, 31, 32, 33,
                         64, 96, 127, 128, 255, 256, 512, 4096, 32768, 65535, 65536,
                         1 << 20, (1 << 30) - 1, 1 << 30, (1 << 30) + 1, INT32_MAX};
const int64_t kEdge64[] = {INT64_MIN, -1, 0, 1, 31, 32, 4095, 4096, (int64_t)1 << 29,
                           ((int64_t)1 << 30) - 1, (int64_t)1 << 30, ((int64_t)1 << 30) + 1,
                           (int64_t)INT32_MAX, (int64_t)1 << 40, INT64_MAX};
const int32_t kDims[] = {32, 64, 128, 256};
const int kMaxYZ = 65535;
const int64_t kMaxTok = (int64_t)1 << 30;
const size_t kScratch = (size_t)64 << 20;  // attn_int8_fwd_noalloc's scratch array

int32_t edge(Rng& r) { return kEdge[r.below(sizeof(kEdge) / sizeof(kEdge[0]))]; }
int64_t edge64(Rng& r) { return kEdge64[r.below(sizeof(kEdge64) / sizeof(kEdge64[0]))]; }

// A size that is valid most of the time: small, large, or at an edge.
int32_t pick_pos(Rng& r, int32_t hi) {
  switch (r.below(4)) {
    case 0: return edge(r);
    case 1: return 1 + r.below(hi < 64 ? hi : 64);
    case 2: return hi;
    default: return 1 + (int32_t)(r.next() % (uint64_t)hi);
  }
}
int32_t pick_dim(Rng& r) { return r.coin(85) ? kDims[r.below(4)] : edge(r); }
void pick_heads(Rng& r, int32_t* hq, int32_t* hkv) {
  if (r.coin(20)) {
    *hq = edge(r);
    *hkv = r.coin(50) ? edge(r) : 1 + r.below(8);
    return;
  }
  *hkv = r.coin(10) ? kMaxYZ : 1 + r.below(16);
  int32_t g = r.coin(10) ? 4096 : 1 + r.below(8);
  const int64_t prod = (int64_t)*hkv * g;
  *hq = prod > INT32_MAX ? INT32_MAX : (int32_t)prod;
}
float pick_scale(Rng& r, bool* ok) {
  static const float bad[] = {0.0f, -0.125f, NAN, INFINITY, -INFINITY, -0.0f};
  if (r.coin(15)) {
    *ok = false;
    return bad[r.below(6)];
  }
  *ok = true;
  return r.coin(50) ? 0.125f : 1e-30f;
}

void* addr(uint64_t a) { return reinterpret_cast<void*>((uintptr_t)a); }
void* const FAKE = addr(1 << 20);  // 256-byte aligned, never dereferenced on the host

bool dim_ok(int32_t D) { return D == 32 || D == 64 || D == 128 || D == 256; }
bool heads_ok(int32_t hq, int32_t hkv) {
  return hq >= 1 && hkv >= 1 && hq <= kMaxYZ && hq % hkv == 0;
}
bool dense_ok(int32_t B, int32_t S) {
  return B >= 1 && B <= kMaxYZ && S >= 1 && (int64_t)B * S <= kMaxTok;
}

void check(bool cond, const char* what, const std::string& ctx) {
  if (cond) return;
  long n = ++g_fail;
  if (n <= 40) fprintf(stderr, "FAIL %s: %s\n", what, ctx.c_str());
}

std::string fmt(const char* f, ...) __attribute__((format(printf, 1, 2)));
std::string fmt(const char* f, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof(buf), f, ap);
  va_end(ap);
  return buf;
}

// A call's status against the expected one; a failure must leave a message.
void expect(i8a_status got, i8a_status want, const std::string& ctx) {
  ++g_calls;
  if (want <= 0 && want >= -4) ++g_by_status[-want];
  if (got != want) {
    check(false, "status", fmt("%s: got %d (%s) want %d; last error: %.200s", ctx.c_str(), got,
                               i8a_status_string(got), want, i8a_last_error()));
    return;
  }
  if (got != I8A_OK) {
    const char* e = i8a_last_error();
    size_t n = strnlen(e, 512);
    check(n > 0 && n < 512, "last_error", ctx);
  }
}

// A pointer argument: valid most of the time, else null or off its alignment.
struct Ptr {
  void* p;
  bool ok;
};
Ptr pick_ptr(Rng& r, int align, int bad_pct) {
  if (!r.coin(bad_pct)) return {FAKE, true};
  if (r.coin(50) || align == 1) return {nullptr, false};
  return {addr((1 << 20) + (uint64_t)(align / 2)), false};
}

// Lower bound of the forward workspace: int8 K, fp16 V and a K scale for every kv
// token, int8 Q codes and fp32 scales for every query token.
unsigned __int128 fwd_ws_floor(int64_t T, int32_t Hq, int32_t Hkv, int32_t D) {
  return (unsigned __int128)T * Hkv * (3 * (unsigned)D + 4) +
         (unsigned __int128)T * Hq * ((unsigned)D + 4);
}

void check_ws(size_t need, bool valid, unsigned __int128 floor, const std::string& ctx) {
  check((need > 0) == valid, "bytes nonzero iff sizes valid", ctx);
  if (need > 0) {
    check(need % 256 == 0, "bytes multiple of 256", ctx);
    check((unsigned __int128)need >= floor, "bytes below the tensors' own size", ctx);
  }
}

// ---- dense forward entry points ---------------------------------------------------
void dense_case(Rng& r) {
  const int32_t B = r.coin(10) ? edge(r) : pick_pos(r, r.coin(50) ? 64 : kMaxYZ);
  const int32_t S = r.coin(10) ? edge(r) : pick_pos(r, r.coin(50) ? 8192 : 1 << 30);
  int32_t Hq, Hkv;
  pick_heads(r, &Hq, &Hkv);
  const int32_t D = pick_dim(r);
  const bool valid = dense_ok(B, S) && heads_ok(Hq, Hkv) && dim_ok(D);
  const std::string ctx = fmt("dense B=%d Hq=%d Hkv=%d S=%d D=%d", B, Hq, Hkv, S, D);
  const size_t need = attn_int8_workspace_bytes(B, Hq, Hkv, S, D);
  check_ws(need, valid, valid ? fwd_ws_floor((int64_t)B * S, Hq, Hkv, D) : 0, ctx);

  // One optional bad argument besides the sizes.
  bool scale_ok;
  const float scale = pick_scale(r, &scale_ok);
  const int32_t causal = r.coin(10) ? edge(r) : r.below(2);
  const bool causal_ok = causal == 0 || causal == 1;
  const Ptr q = pick_ptr(r, 16, 5), k = pick_ptr(r, 16, 5), v = pick_ptr(r, 16, 5),
            o = pick_ptr(r, 16, 5), ws = pick_ptr(r, 256, 5);
  const size_t wsb = need > 0 ? need - 1 : (r.coin(50) ? SIZE_MAX : 0);

  // attn_int8_fwd: pointers, head dim, heads, scale, causal, workspace pointer, B and S,
  // then the workspace size.
  auto fwd_want = [&](bool qok, bool kok, bool vok, bool ook, bool sc_ok, bool ca_ok,
                      bool ws_ok = true) {
    if (!qok || !kok || !vok || !ook) return I8A_ERR_INVALID_ARG;
    if (!dim_ok(D)) return I8A_ERR_UNSUPPORTED_HEAD_DIM;
    if (!heads_ok(Hq, Hkv) || !sc_ok || !ca_ok || !ws_ok || !dense_ok(B, S))
      return I8A_ERR_INVALID_ARG;
    return I8A_ERR_WORKSPACE_TOO_SMALL;
  };
  const i8a_status want = fwd_want(q.ok, k.ok, v.ok, o.ok, scale_ok, causal_ok, ws.ok);
  expect(attn_int8_fwd(q.p, k.p, v.p, o.p, B, Hq, Hkv, S, D, scale, causal, ws.p, wsb, nullptr),
         want, "fwd " + ctx);

  // attn_int8_fwd_ex: the flags are checked after B and S.
  const int32_t flags = r.coin(15) ? (int32_t)(r.next() & 0xff) : r.below(16);
  i8a_status want_ex = want;
  if (want == I8A_ERR_WORKSPACE_TOO_SMALL) {
    if (flags & ~15) want_ex = I8A_ERR_INVALID_ARG;
    else if ((flags & I8A_FWD_Q_OUTLIERS) && (flags & I8A_FWD_HADAMARD))
      want_ex = I8A_ERR_INVALID_ARG;
    else if ((flags & I8A_FWD_Q_OUTLIERS) && D > 128)
      want_ex = I8A_ERR_UNSUPPORTED_HEAD_DIM;
  }
  expect(attn_int8_fwd_ex(q.p, k.p, v.p, o.p, B, Hq, Hkv, S, D, scale, causal, flags, ws.p, wsb,
                          nullptr),
         want_ex, fmt("fwd_ex flags=%d ", flags) + ctx);
  expect(attn_int8_fwd_hadamard(q.p, k.p, v.p, o.p, B, Hq, Hkv, S, D, scale, causal, ws.p, wsb,
                                nullptr),
         want, "fwd_hadamard " + ctx);

  // The split phases check only the tensors they touch (the others stand in).
  expect(attn_int8_prepare_kv(k.p, v.p, B, Hq, Hkv, S, D, ws.p, wsb, nullptr),
         fwd_want(k.ok, k.ok, v.ok, k.ok, true, true, ws.ok), "prepare_kv " + ctx);
  expect(attn_int8_prepare_q(q.p, B, Hq, Hkv, S, D, ws.p, wsb, nullptr),
         fwd_want(q.ok, q.ok, q.ok, q.ok, true, true, ws.ok), "prepare_q " + ctx);
  expect(attn_int8_attend(o.p, B, Hq, Hkv, S, D, scale, causal, ws.p, wsb, nullptr),
         fwd_want(o.ok, o.ok, o.ok, o.ok, scale_ok, causal_ok, ws.ok), "attend " + ctx);
  expect(attn_int8_fwd_prepared(q.p, o.p, B, Hq, Hkv, S, D, scale, causal, ws.p, wsb, nullptr),
         fwd_want(q.ok, q.ok, q.ok, o.ok, scale_ok, causal_ok, ws.ok), "fwd_prepared " + ctx);

  // attn_int8_fwd_noalloc (no workspace argument): only where it cannot reach the
  // device, i.e. rejected arguments or a workspace larger than its scratch array.
  const i8a_status w = fwd_want(q.ok, k.ok, v.ok, o.ok, scale_ok, causal_ok);
  if (w != I8A_ERR_WORKSPACE_TOO_SMALL || need > kScratch) {
    expect(attn_int8_fwd_noalloc(q.p, k.p, v.p, o.p, B, Hq, Hkv, S, D, scale, causal, nullptr),
           w, "fwd_noalloc " + ctx);
  }
}

// ---- varlen forward and the debug dump -------------------------------------------
void varlen_case(Rng& r) {
  const int32_t nseq = r.coin(15) ? edge(r) : pick_pos(r, r.coin(50) ? 64 : kMaxYZ);
  int64_t T = r.coin(15) ? edge64(r) : (r.coin(10) ? 0 : 1 + (int64_t)(r.next() % kMaxTok));
  int32_t maxlen;
  if (r.coin(15)) maxlen = edge(r);
  else if (T <= 0) maxlen = 0;
  else maxlen = r.coin(10) ? 0 : 1 + (int32_t)(r.next() % (uint64_t)(T < INT32_MAX ? T : INT32_MAX));
  int32_t Hq, Hkv;
  pick_heads(r, &Hq, &Hkv);
  const int32_t D = pick_dim(r);
  const int32_t flags = r.coin(10) ? (int32_t)(r.next() & 0xff) : r.below(16);
  const bool sizes_ok = nseq >= 1 && nseq <= kMaxYZ && T >= 0 && T <= kMaxTok && maxlen >= 0 &&
                        maxlen <= T && heads_ok(Hq, Hkv) && dim_ok(D);
  const std::string ctx = fmt("varlen nseq=%d T=%lld max=%d Hq=%d Hkv=%d D=%d flags=%d", nseq,
                              (long long)T, maxlen, Hq, Hkv, D, flags);
  const size_t need = attn_int8_varlen_workspace_bytes(nseq, T, maxlen, Hq, Hkv, D);
  check_ws(need, sizes_ok, sizes_ok ? fwd_ws_floor(T, Hq, Hkv, D) : 0, ctx);

  bool scale_ok;
  const float scale = pick_scale(r, &scale_ok);
  const int32_t causal = r.coin(10) ? edge(r) : r.below(2);
  const bool causal_ok = causal == 0 || causal == 1;
  const Ptr q = pick_ptr(r, 16, 5), k = pick_ptr(r, 16, 5), v = pick_ptr(r, 16, 5),
            o = pick_ptr(r, 16, 5), ws = pick_ptr(r, 256, 5), cu = pick_ptr(r, 4, 5);
  const size_t wsb = need > 0 ? need - 1 : SIZE_MAX;

  // Flags first (as a probe), then cu_seqlens and the sizes; an empty batch returns
  // after the head checks; else the forward's own checks and the workspace size.
  auto flags_status = [&](int32_t f) {
    if (f & ~15) return I8A_ERR_INVALID_ARG;
    if ((f & I8A_FWD_Q_OUTLIERS) && (f & I8A_FWD_HADAMARD)) return I8A_ERR_INVALID_ARG;
    if ((f & I8A_FWD_Q_OUTLIERS) && D > 128) return I8A_ERR_UNSUPPORTED_HEAD_DIM;
    return I8A_OK;
  };
  i8a_status want = flags_status(flags);
  if (want == I8A_OK) {
    if (!cu.ok || nseq < 1 || nseq > kMaxYZ || T < 0 || T > kMaxTok || maxlen < 0 || maxlen > T)
      want = I8A_ERR_INVALID_ARG;
    else if (T == 0 || maxlen == 0)
      want = !dim_ok(D) ? I8A_ERR_UNSUPPORTED_HEAD_DIM
                        : (heads_ok(Hq, Hkv) ? I8A_OK : I8A_ERR_INVALID_ARG);
    else if (!q.ok || !k.ok || !v.ok || !o.ok)
      want = I8A_ERR_INVALID_ARG;
    else if (!dim_ok(D))
      want = I8A_ERR_UNSUPPORTED_HEAD_DIM;
    else if (!heads_ok(Hq, Hkv) || !scale_ok || !causal_ok || !ws.ok)
      want = I8A_ERR_INVALID_ARG;
    else
      want = I8A_ERR_WORKSPACE_TOO_SMALL;
  }
  expect(attn_int8_varlen_fwd_ex(q.p, k.p, v.p, o.p, (const int32_t*)cu.p, nseq, maxlen, T, Hq,
                                 Hkv, D, scale, causal, flags, ws.p, wsb, nullptr),
         want, "varlen_fwd_ex " + ctx);
  if (flags == 0)
    expect(attn_int8_varlen_fwd(q.p, k.p, v.p, o.p, (const int32_t*)cu.p, nseq, maxlen, T, Hq,
                                Hkv, D, scale, causal, ws.p, wsb, nullptr),
           want, "varlen_fwd " + ctx);

  // attn_int8_debug_qk_ex over the same geometry, dense (no cu_seqlens) or varlen.
  const bool dense = r.coin(40);
  const int32_t seq = r.coin(10) ? edge(r) : (nseq > 0 ? r.below(nseq) : 0);
  const int32_t h = r.coin(10) ? edge(r) : (Hq > 0 ? r.below(Hq) : 0);
  int32_t row0, rows, col0, cols;
  if (r.coin(20)) {
    row0 = edge(r), rows = edge(r), col0 = edge(r), cols = edge(r);
  } else {
    row0 = maxlen > 0 ? r.below(maxlen) : 0;
    rows = 1 + (maxlen > row0 ? r.below(maxlen - row0) : 0);
    col0 = maxlen > 0 ? r.below(maxlen) : 0;
    cols = 1 + (maxlen > col0 ? r.below(maxlen - col0) : 0);
  }
  const Ptr s32 = pick_ptr(r, 4, 5), vhat = pick_ptr(r, 2, 5);
  const bool vch = (flags & I8A_FWD_V_PER_CHANNEL) != 0, qout = (flags & I8A_FWD_Q_OUTLIERS) != 0;
  void* vscale = r.coin(50) ? FAKE : nullptr;
  void* vchan = r.coin(50) ? FAKE : nullptr;
  const Ptr ochan = r.coin(50) ? pick_ptr(r, 4, 10) : Ptr{nullptr, true};
  const int64_t Td = dense ? (r.coin(80) ? (int64_t)nseq * maxlen : T) : T;
  const size_t dneed = dense ? ((int64_t)nseq * maxlen == Td && maxlen >= 1
                                    ? attn_int8_workspace_bytes(nseq, Hq, Hkv, maxlen, D)
                                    : 0)
                             : need;
  i8a_status dw;
  if (!q.ok || !k.ok || !v.ok) dw = I8A_ERR_INVALID_ARG;
  else if (!dim_ok(D)) dw = I8A_ERR_UNSUPPORTED_HEAD_DIM;
  else if (!heads_ok(Hq, Hkv) || !ws.ok) dw = I8A_ERR_INVALID_ARG;
  else if ((dw = flags_status(flags)) != I8A_OK) {
  } else if (nseq < 1 || nseq > kMaxYZ || maxlen < 1 || Td < 1 || Td > kMaxTok || maxlen > Td)
    dw = I8A_ERR_INVALID_ARG;
  else if (!dense && !cu.ok && cu.p != nullptr) dw = I8A_ERR_INVALID_ARG;
  else if (dense && Td != (int64_t)nseq * maxlen) dw = I8A_ERR_INVALID_ARG;
  else if (seq < 0 || seq >= nseq || h < 0 || h >= Hq) dw = I8A_ERR_INVALID_ARG;
  else if (rows < 1 || cols < 1 || row0 < 0 || col0 < 0 || (int64_t)row0 + rows > maxlen ||
           (int64_t)col0 + cols > maxlen)
    dw = I8A_ERR_INVALID_ARG;
  else if (!s32.ok || (vhat.p && !vhat.ok) || (vch && vscale) || (!vch && vchan) ||
           (ochan.p && !qout) || (ochan.p && !ochan.ok))
    dw = I8A_ERR_INVALID_ARG;
  else dw = I8A_ERR_WORKSPACE_TOO_SMALL;
  // A null cu_seqlens selects the dense geometry; the varlen form needs a real one.
  const int32_t* cup = dense ? nullptr : (const int32_t*)(cu.p ? cu.p : FAKE);
  if (dw == I8A_ERR_WORKSPACE_TOO_SMALL && dneed == 0) return;  // cannot make it fail
  const size_t dwsb = dneed > 0 ? dneed - 1 : SIZE_MAX;
  expect(attn_int8_debug_qk_ex(q.p, k.p, v.p, cup, nseq, maxlen, Td, Hq, Hkv, D, flags, seq, h,
                               row0, rows, col0, cols, (int32_t*)s32.p, nullptr, nullptr,
                               (float*)vscale, nullptr, vhat.p, (float*)vchan,
                               (int32_t*)ochan.p, ws.p, dwsb, nullptr),
         dw, fmt("debug_qk_ex dense=%d seq=%d h=%d tile=%d+%d,%d+%d ", dense, seq, h, row0, rows,
                 col0, cols) + ctx);
}

// ---- decode over the int8 KV cache ------------------------------------------------
void decode_case(Rng& r) {
  const int32_t B = r.coin(10) ? edge(r) : pick_pos(r, r.coin(50) ? 64 : kMaxYZ);
  const int32_t S = r.coin(10) ? edge(r) : pick_pos(r, r.coin(50) ? 32768 : 1 << 30);
  int32_t Hq, Hkv;
  pick_heads(r, &Hq, &Hkv);
  const int32_t D = pick_dim(r);
  const int32_t vf = r.coin(10) ? edge(r) : 1 + r.below(2);
  const bool vf_ok = vf == I8A_VCACHE_INT8 || vf == I8A_VCACHE_FP16;
  const bool kv_ok = B >= 1 && B <= kMaxYZ && Hkv >= 1 && Hkv <= kMaxYZ && S >= 1 &&
                     (int64_t)B * S <= kMaxTok && dim_ok(D) && vf_ok &&
                     (int64_t)B * Hkv <= ((int64_t)1 << 24);
  const std::string ctx =
      fmt("decode B=%d Hq=%d Hkv=%d S=%d D=%d vf=%d", B, Hq, Hkv, S, D, vf);
  const size_t cneed = attn_int8_kvcache_bytes(B, Hkv, S, D, vf);
  // The cache holds at least the int8 K codes and a V code or value per element.
  check_ws(cneed, kv_ok,
           kv_ok ? (unsigned __int128)B * Hkv * (uint64_t)S * D * (vf == I8A_VCACHE_FP16 ? 3 : 2)
                 : 0,
           "kvcache_bytes " + ctx);
  const Ptr k = pick_ptr(r, 16, 5), v = pick_ptr(r, 16, 5), cache = pick_ptr(r, 256, 5);
  auto kvc_want = [&]() {
    if (!dim_ok(D)) return I8A_ERR_UNSUPPORTED_HEAD_DIM;
    if (!vf_ok || !kv_ok || !cache.ok) return I8A_ERR_INVALID_ARG;
    return I8A_ERR_WORKSPACE_TOO_SMALL;
  };
  const size_t short_cache = cneed > 0 ? cneed - 1 : SIZE_MAX;
  expect(attn_int8_kvcache_fill(k.p, v.p, B, Hkv, S, D, vf, cache.p, short_cache, nullptr),
         (!k.ok || !v.ok) ? I8A_ERR_INVALID_ARG : kvc_want(), "kvcache_fill " + ctx);

  const bool hq_ok = Hkv >= 1 && Hq >= Hkv && Hq <= kMaxYZ && Hq % Hkv == 0;
  const size_t wneed = attn_int8_decode_workspace_bytes(B, Hq, Hkv, S, D, vf);
  check(wneed == 0 || (kv_ok && hq_ok), "decode ws nonzero only for valid sizes", ctx);
  bool scale_ok;
  const float scale = pick_scale(r, &scale_ok);
  const Ptr q = pick_ptr(r, 16, 5), o = pick_ptr(r, 16, 5), ws = pick_ptr(r, 256, 5);
  // (a) the cache one byte short.
  expect(attn_int8_decode(q.p, o.p, B, Hq, Hkv, S, D, scale, vf, cache.p, short_cache, ws.p,
                          SIZE_MAX, nullptr),
         (!q.ok || !o.ok) ? I8A_ERR_INVALID_ARG : kvc_want(), "decode short cache " + ctx);
  // The growing cache.  (c) A prefix fill, an append and a decode of per-sequence lengths
  // with the cache one byte short: the cache checks decide, after the pointers that are
  // checked first.
  const int32_t S_fill =
      r.coin(20) ? edge(r) : 1 + (int32_t)(r.next() % (uint64_t)(S > 0 ? S : 1));
  const int32_t n_new =
      r.coin(20) ? edge(r) : (int32_t)(r.next() % (uint64_t)(S > 0 ? (int64_t)S + 1 : 1));
  const Ptr pos = pick_ptr(r, 4, 10), lens = pick_ptr(r, 4, 10);
  expect(attn_int8_kvcache_fill_prefix(k.p, v.p, B, Hkv, S_fill, S, D, vf, cache.p, short_cache,
                                       nullptr),
         (!k.ok || !v.ok) ? I8A_ERR_INVALID_ARG : kvc_want(),
         fmt("kvcache_fill_prefix S_fill=%d ", S_fill) + ctx);
  expect(attn_int8_kvcache_append(k.p, v.p, B, Hkv, n_new, (const int32_t*)pos.p, S, D, vf,
                                  cache.p, short_cache, nullptr),
         kvc_want(), fmt("kvcache_append n_new=%d ", n_new) + ctx);
  expect(attn_int8_decode_lens(q.p, o.p, B, Hq, Hkv, S, D, scale, vf, (const int32_t*)lens.p,
                               cache.p, short_cache, ws.p, SIZE_MAX, nullptr),
         (!lens.ok || !q.ok || !o.ok) ? I8A_ERR_INVALID_ARG : kvc_want(),
         "decode_lens short cache " + ctx);
  // (d) The cache whole: a prefix length or an append count out of range, or an append
  // with a bad pointer, fails; an empty append succeeds without touching the device.
  if (cneed > 0 && cache.ok) {
    const bool fill_ok = S_fill >= 1 && S_fill <= S;
    if (!fill_ok || !k.ok || !v.ok)
      expect(attn_int8_kvcache_fill_prefix(k.p, v.p, B, Hkv, S_fill, S, D, vf, cache.p, cneed,
                                           nullptr),
             I8A_ERR_INVALID_ARG, fmt("kvcache_fill_prefix whole S_fill=%d ", S_fill) + ctx);
    const bool n_ok = n_new >= 0 && n_new <= S;
    if (!n_ok || n_new == 0 || !k.ok || !v.ok || !pos.ok)
      expect(attn_int8_kvcache_append(k.p, v.p, B, Hkv, n_new, (const int32_t*)pos.p, S, D, vf,
                                      cache.p, cneed, nullptr),
             !n_ok ? I8A_ERR_INVALID_ARG : n_new == 0 ? I8A_OK : I8A_ERR_INVALID_ARG,
             fmt("kvcache_append whole n_new=%d ", n_new) + ctx);
  }
  // (b) the cache whole and the workspace one byte short; skipped where nothing fails.
  if (cneed == 0 || !cache.ok) return;
  i8a_status want;
  if (!q.ok || !o.ok || !hq_ok || !scale_ok) want = I8A_ERR_INVALID_ARG;
  else if (wneed > 0) want = I8A_ERR_WORKSPACE_TOO_SMALL;
  else return;
  expect(attn_int8_decode(q.p, o.p, B, Hq, Hkv, S, D, scale, vf, cache.p, cneed, ws.p,
                          wneed > 0 ? wneed - 1 : 0, nullptr),
         want, "decode short workspace " + ctx);
}

// ---- backward ---------------------------------------------------------------------
void bwd_case(Rng& r) {
  const int32_t B = r.coin(10) ? edge(r) : pick_pos(r, r.coin(50) ? 64 : kMaxYZ);
  const int32_t S = r.coin(10) ? edge(r) : pick_pos(r, r.coin(50) ? 8192 : 1 << 30);
  int32_t Hq, Hkv;
  pick_heads(r, &Hq, &Hkv);
  const int32_t D = pick_dim(r);
  const bool sizes_ok = dense_ok(B, S) && heads_ok(Hq, Hkv);
  const std::string ctx = fmt("bwd B=%d Hq=%d Hkv=%d S=%d D=%d", B, Hq, Hkv, S, D);
  const size_t need = attn_bwd_workspace_bytes(B, Hq, Hkv, S, D);
  // The workspace holds the fp16 inputs again (q, k, v, dout) at least.
  check_ws(need, sizes_ok && dim_ok(D),
           sizes_ok && dim_ok(D)
               ? (unsigned __int128)B * (uint64_t)S * D * 2 * (2 * (uint64_t)Hq + 2 * Hkv)
               : 0,
           ctx);
  bool scale_ok;
  const float scale = pick_scale(r, &scale_ok);
  const int32_t causal = r.coin(10) ? edge(r) : r.below(2);
  Ptr p[7];
  bool ptrs_ok = true;
  for (auto& x : p) {
    x = pick_ptr(r, 16, 3);
    ptrs_ok = ptrs_ok && x.ok;
  }
  const Ptr ws = pick_ptr(r, 256, 5);
  i8a_status want;
  if (!ptrs_ok) want = I8A_ERR_INVALID_ARG;
  else if (!dim_ok(D)) want = I8A_ERR_UNSUPPORTED_HEAD_DIM;
  else if (!sizes_ok || !scale_ok || (causal != 0 && causal != 1) || !ws.ok)
    want = I8A_ERR_INVALID_ARG;
  else want = I8A_ERR_WORKSPACE_TOO_SMALL;
  expect(attn_bwd(p[0].p, p[1].p, p[2].p, p[3].p, (float*)p[4].p, (float*)p[5].p,
                  (float*)p[6].p, B, Hq, Hkv, S, D, scale, causal, ws.p,
                  need > 0 ? need - 1 : SIZE_MAX, nullptr),
         want, ctx);
}

// ---- per-row quantization ---------------------------------------------------------
void quant_case(Rng& r) {
  const int64_t rows = r.coin(20) ? edge64(r) : (r.coin(20) ? 0 : 1 + r.below(100000));
  const int32_t d = r.coin(20) ? edge(r) : 8 * (1 + r.below(64));
  const int32_t bits = r.coin(10) ? edge(r) : (r.coin(50) ? I8A_SCALE_FP32 : I8A_SCALE_V4);
  const bool with_mean = r.coin(50);
  const int64_t rpg = r.coin(20) ? edge64(r) : 1 + r.below(4096);
  // At least one pointer is bad whenever the call would otherwise launch.
  Ptr x = pick_ptr(r, 16, 30), c = pick_ptr(r, 8, 30), s = pick_ptr(r, 4, 30);
  Ptr m = with_mean ? pick_ptr(r, 4, 20) : Ptr{nullptr, true};
  if (with_mean && !m.p) m = {FAKE, true};
  if (x.ok && c.ok && s.ok && m.ok) x = {nullptr, false};
  i8a_status want;
  if (rows < 0 || d < 8 || d > 512 || d % 8 || (bits != I8A_SCALE_FP32 && bits != I8A_SCALE_V4) ||
      (with_mean && rpg < 1))
    want = I8A_ERR_INVALID_ARG;
  else if (rows == 0) want = I8A_OK;
  else want = I8A_ERR_INVALID_ARG;
  expect(quant_rowwise_i8(x.p, rows, d, (const float*)m.p, rpg, bits, (int8_t*)c.p,
                          (float*)s.p, nullptr),
         want, fmt("quant rows=%lld d=%d bits=%d rpg=%lld", (long long)rows, d, bits,
                   (long long)rpg));
}

// Each thread's last error is its own: a head-dim failure's message names the head dim
// even while other threads fail in other ways.
void thread_local_errors(Rng& r) {
  static const int32_t bad[] = {40, 48, 96, 512};  // none of 32, 64, 128, 256
  const int32_t bad_d = bad[r.below(4)];
  i8a_status st = attn_int8_fwd(FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, bad_d, 0.125f, 0, FAKE,
                                SIZE_MAX, nullptr);
  std::this_thread::yield();
  check(st == I8A_ERR_UNSUPPORTED_HEAD_DIM && strstr(i8a_last_error(), "head dim") &&
            strstr(i8a_last_error(), std::to_string(bad_d).c_str()),
        "per-thread last error", fmt("D=%d: %s", bad_d, i8a_last_error()));
}

void worker(uint64_t seed, long iters) {
  Rng r{seed};
  for (long i = 0; i < iters; ++i) {
    switch (i % 6) {
      case 0: dense_case(r); break;
      case 1: varlen_case(r); break;
      case 2: decode_case(r); break;
      case 3: bwd_case(r); break;
      case 4: quant_case(r); break;
      default: thread_local_errors(r); break;
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  // No call here should reach the device; hide every device all the same, so that a
  // call that slipped through validation fails in the HIP runtime instead of launching.
  setenv("HIP_VISIBLE_DEVICES", "-1", 1);
  setenv("ROCR_VISIBLE_DEVICES", "-1", 1);
  const long iters = argc > 1 ? atol(argv[1]) : 20000;
  const int nthreads = argc > 2 ? atoi(argv[2]) : 4;
  for (int s = -8; s <= 8; ++s) {
    const char* n = i8a_status_string(s);
    if (!n || !*n) check(false, "status string", fmt("%d", s));
  }
  std::vector<std::thread> ts;
  for (int t = 0; t < nthreads; ++t) ts.emplace_back(worker, 0x5eed0000ull + t, iters);
  for (auto& t : ts) t.join();
  printf("calls=%ld ok=%ld invalid_arg=%ld head_dim=%ld workspace_too_small=%ld failures=%ld\n",
         g_calls.load(), g_by_status[0].load(), g_by_status[1].load(), g_by_status[2].load(),
         g_by_status[3].load(), g_fail.load());
  return g_fail.load() == 0 ? 0 : 1;
}
