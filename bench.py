"""Benchmark of the INT8 W8A8 attention forward on one MI355X.

One step = one ``attn_int8_fwd`` call on the causal GQA workload B=1, Hq=32,
Hkv=8, S=4096, D=128 (fp16 q/k/v ~ N(0,1), seeded): K-smoothing mean, K/V
quantization and the attention kernel, which quantizes Q itself, every kernel the call
launches.  Inputs, output and workspace are resident in HBM before timing starts.
The phases are also timed alone (K/V preparation, attention kernel) through the split
entry points, which enqueue the same kernels.

Prints one JSON line.  ``value`` is effective TOPS = algorithmic ops / time per
step, with ops = 4*D*Hq*S^2/2 (two products of 2*D ops per (query, key) pair,
S^2/2 causal pairs per head, the usual FlashAttention count).  ``roofline``
describes the attention kernel alone (timed with HIP events on the stream it runs
on) against the 5.0 POPS dense int8 MFMA peak.  ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload.  Also reported: the share of the
mixed int8/fp16 MFMA ceiling, per-call median and min (as is, and after writing a
512 MiB buffer that evicts the caches), the preparation kernels' GB/s, and on sampled
rows the fp16 rounding floor of the oracle's output and the SQNR of the output
against unquantized fp64 attention.

The ``decode`` object measures the split-KV decode over an int8 KV cache on the batched
serving shape B=16 sequences x S=8192 cached tokens, Hq=32, Hkv=8, D=128: one step is one
``attn_int8_decode`` call (the decode kernel and the merge of its chunks) for one new
token per sequence, with the cache filled beforehand, for both V formats.  Its
roofline is HBM: algorithmic bytes per call (the cache's K codes, V codes or values
and scales, the query rows read, the output written) over the call time, against
8 TB/s.  Its ``cpu_baseline`` times the oracle's decode over a cache quantized
beforehand, on a sample of sequences.

The ``variants`` object times the forward's variants (``attn_int8_fwd_ex`` with Q and K
Hadamard-rotated, with V per channel, with both, with Q per 32-row block and with Q
outlier detection) on the same workload and reports each one's quality (SQNR against
unquantized attention) on the outlier-channel workload next to the plain forward's.

The ``configs`` object measures the other workloads of the benchmark set the same way
(one forward call per step, inputs resident): the non-causal MHA head-dim sweep B4 H16
S2048 D32/64/128/256 with outlier channels, the varlen causal prefill of 16 sequences
(lengths drawn U[1,4096]) at Hq64 Hkv8 D128, and the long-context causal GQA B1 Hq40
Hkv8 S32768 D128.  Each has its whole-call TOPS, the attention kernel alone against the
int8 peak (dense ones), a parity guard on sampled rows and the CPU oracle's rate on a
bounded sample (heads and rows stated; the long-context one from one kv group).

The ``backward`` object times ``attn_bwd`` (the gradients of the attention, the
quantization taken as the identity) on the same workload against the fp16 MFMA peak.

Only one GPU is used: ``--gpus`` above 1 exits with a message.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POPS
FP16_PEAK_TOPS = 2500.0  # MI355X dense fp16 MFMA, 2.5 PFLOP/s
# Half of the ops run on each engine (int8 Q.K^T, fp16 P.V): the mixed ceiling.
MIXED_PEAK_TOPS = 1.0 / (0.5 / INT8_PEAK_TOPS + 0.5 / FP16_PEAK_TOPS)
WORKLOAD = dict(B=1, Hq=32, Hkv=8, S=4096, D=128, causal=True)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_cfg2_traffic.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_b16_s8192_traffic.json")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_cfg2_traffic.json")
DECODE_FP16_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_b16_s8192_fp16v_traffic.json")
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch of the dominant kernel from the stored FETCH_SIZE /
    WRITE_SIZE counter runs (scaled by a plain copy's readings), or None when the kernel
    sources have changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        n = rec["bytes_per_launch"] if "bytes_per_launch" in rec else rec["bytes_per_call"]
        return n if h.hexdigest() == rec["sources_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float):
    """Time the CPU oracle on whole heads of the same workload until the budget is
    spent; ops per second scaled to TOPS."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    B, Hq, S, D = w.q.shape
    t0 = time.perf_counter()
    z = oracle.quantize_qkv(w.q, w.k, w.v)  # quantization of the whole input
    G = Hq // w.k.shape[1]
    heads = 0
    for h in range(Hq):
        g = h // G
        oracle.attn_core(z["q8"][0, h], z["sq"][0, h], z["k8"][0, g], z["sk"][0, g],
                         z["v8"][0, g], z["sv"][0, g], oracle.default_softmax_scale(D), True)
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    ops = 4.0 * D * heads * S * S / 2.0
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{heads} of {Hq} query heads (all {S} rows each) plus the quantization "
                      f"of the whole input, {dt:.1f} s; numpy fp64 BLAS with {blas_threads} "
                      f"threads, the rest single-threaded; host has {os.cpu_count()} CPUs "
                      f"({cpu_model()})"}


def decode_bytes(B, Hq, Hkv, S, D, v_format):
    """Algorithmic bytes of one decode call: per cached token and kv head the int8 K
    codes and fp32 K scale, then the int8 V codes and their scale (stored as fp16) or
    the fp16 V values; the fp16 query rows read and output rows written."""
    per_tok = D + 4 + (D + 2 if v_format == "int8" else 2 * D)
    return B * Hkv * S * per_tok + 2 * B * Hq * D * 2


def decode_cpu_baseline(w, budget_s: float):
    """The oracle's decode on whole sequences of the same workload (each cache quantized
    beforehand, not timed) until the budget is spent; bytes of the cache attended per
    second."""
    import numpy as np

    import oracle
    B, Hq, D = w.q.shape
    Hkv, S = w.k.shape[1], w.k.shape[2]
    G = Hq // Hkv
    sm = oracle.default_softmax_scale(D)
    done, dt = 0, 0.0
    for b in range(B):
        q8, sq = oracle.quant_rows(w.q[b].astype(np.float32))
        m = oracle.kmean(w.k[b:b + 1])[0]
        k8, sk = oracle.quant_rows(w.k[b].astype(np.float32) - m[:, None, :])
        v8, sv = oracle.quant_rows(w.v[b].astype(np.float32), oracle.V_SCALE_BITS)
        t0 = time.perf_counter()
        for h in range(Hq):
            oracle.attn_core(q8[h][None], sq[h][None], k8[h // G], sk[h // G], v8[h // G],
                             sv[h // G], sm, False)
        dt += time.perf_counter() - t0
        done += 1
        if dt > budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    nbytes = decode_bytes(done, Hq, Hkv, S, D, "int8")
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{done} of {B} sequences (all {Hq} query heads over {S} cached tokens), "
                      f"int8 V, caches quantized beforehand (not timed); {dt:.1f} s of numpy "
                      f"fp64, BLAS with {blas_threads} threads ({cpu_model()})"}


def bench_decode(args, i8, torch, dev):
    """The decode measurement (both V formats) on the batched serving shape."""
    import numpy as np

    import oracle
    from int8_w8a8_flashattention_amd import workloads
    w = workloads.decode_bench()
    B, Hq, D = w.q.shape
    Hkv, S = w.k.shape[1], w.k.shape[2]
    q, k, v = (torch.from_numpy(a).to(dev) for a in (w.q, w.k, w.v))
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"workload": f"{w.name}: decode of one token per sequence, B{B} Hq{Hq} Hkv{Hkv} "
                       f"S{S} D{D}, fp16 N(0,1) with K channel offsets U(-3,3), seed 6",
           "step": "one attn_int8_decode call (decode kernel + chunk merge), cache filled "
                   "beforehand"}
    for vf in ("int8", "fp16"):
        cache = i8.attn_int8_kvcache_fill(k, v, vf)
        ws = torch.zeros(max(i8.attn_int8_decode_workspace_bytes(B, Hq, Hkv, S, D, vf), 1),
                         dtype=torch.uint8, device=dev)

        def call():
            i8.attn_int8_decode(q, cache, out=out, workspace=ws)

        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / args.steps * 1e3
        nbytes = decode_bytes(B, Hq, Hkv, S, D, vf)
        got = out.float().cpu().numpy()
        err = 0.0
        for b in (0, B - 1):
            ref = oracle.attn_int8_decode(w.q[b:b + 1], w.k[b:b + 1], w.v[b:b + 1], v_format=vf)
            err = max(err, float(np.abs(got[b:b + 1] - ref).max()))
        if not err <= 2e-3:
            raise RuntimeError(f"decode output differs from the oracle: max_abs={err}")
        # cache fill (K sums, K and V quantization): fp16 K read twice, V once, cache written
        for _ in range(5):
            i8.attn_int8_kvcache_fill(k, v, vf, cache=cache.buf)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(10):
            i8.attn_int8_kvcache_fill(k, v, vf, cache=cache.buf)
        e1.record(stream)
        torch.cuda.synchronize()
        fill_us = e0.elapsed_time(e1) / 10 * 1e3
        # a generation step on a growing cache: one new token per sequence appended into
        # the last slot, then the decode over every sequence's S tokens (lengths on the
        # device); and the append alone
        kn, vn = k[:, :, S - 1:S].contiguous(), v[:, :, S - 1:S].contiguous()
        pos = torch.full((B,), S - 1, dtype=torch.int32, device=dev)
        lens = torch.full((B,), S, dtype=torch.int32, device=dev)

        def gen_step():
            i8.attn_int8_kvcache_append(cache, kn, vn, pos)
            i8.attn_int8_decode_lens(q, cache, lens, out=out, workspace=ws)

        def timed_us(fn, n):
            for _ in range(max(n // 5, 5)):
                fn()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n * 1e3

        gen_us = timed_us(gen_step, args.steps)
        append_us = timed_us(lambda: i8.attn_int8_kvcache_append(cache, kn, vn, pos), args.steps)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[f"{vf}_v"] = {
            "call_us": round(us, 2), "bytes_per_call": nbytes, "gbs": round(gbs, 1),
            "parity_sample_max_abs": err, "fill_us": round(fill_us, 2),
            "append_decode_step_us": round(gen_us, 2), "append_us": round(append_us, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(DECODE_TRAFFIC_FILE if vf == "int8"
                                                     else DECODE_FP16_TRAFFIC_FILE)}}
        log(f"bench: decode {vf} V {us:.1f} us/call, {gbs:.0f} GB/s, fill {fill_us:.1f} us, "
            f"append + decode {gen_us:.1f} us, append {append_us:.1f} us")
        del cache, ws
    if not args.no_cpu_baseline:
        log(f"bench: timing the CPU oracle's decode (~{args.cpu_budget / 2:.0f} s)")
        res["cpu_baseline"] = decode_cpu_baseline(w, args.cpu_budget / 2)
    return res


def bench_variants(args, i8, torch, dev, q, k, v, out, ws, ms_step):
    """The forward's variants (NEXT-3 Hadamard-rotated Q/K, NEXT-2 V per channel, and
    both): their step times on the same workload, and their quality on the
    outlier-channel workload (B4 H16 S2048 D128 non-causal, 1 % of channels x20) as SQNR
    against unquantized attention on sampled heads and rows."""
    import numpy as np

    import oracle
    from int8_w8a8_flashattention_amd import workloads
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flags = {"hadamard": i8.FWD_HADAMARD, "v_per_channel": i8.FWD_V_PER_CHANNEL,
             "hadamard+v_per_channel": i8.FWD_HADAMARD | i8.FWD_V_PER_CHANNEL,
             "q_per_block": i8.FWD_Q_PER_BLOCK, "q_outliers": i8.FWD_Q_OUTLIERS,
             "q_per_block+q_outliers": i8.FWD_Q_PER_BLOCK | i8.FWD_Q_OUTLIERS}
    kw = {"hadamard": dict(hadamard=True), "v_per_channel": dict(v_per_channel=True),
          "hadamard+v_per_channel": dict(hadamard=True, v_per_channel=True),
          "q_per_block": dict(q_per_block=True), "q_outliers": dict(q_outliers=True),
          "q_per_block+q_outliers": dict(q_per_block=True, q_outliers=True)}
    res = {"outlier_workload": "cfg3_mha_s2048_d128_outliers: B4 H16 S2048 D128 non-causal, "
                               "1 % of channels x20 in Q and K, 4 heads x 293 rows"}
    w = workloads.cfg3(128)
    qq, kk, vv = (torch.from_numpy(a).to(dev) for a in (w.q, w.k, w.v))
    heads = [(0, 0), (1, 7), (2, 11), (3, 15)]
    rows = np.arange(0, 2048, 7)
    exact = oracle.attn_exact(w.q, w.k, w.v, False, heads=heads, rows=rows)

    def pick(o):
        return np.stack([o[b, h][rows] for b, h in heads]).astype(np.float64)

    def sqnr(o):
        return round(float(10 * np.log10(np.sum(exact ** 2) / np.sum((pick(o) - exact) ** 2))),
                     2)
    res["sqnr_db_plain"] = sqnr(i8.attn_int8_fwd(qq, kk, vv, False).float().cpu().numpy())
    for name, fl in flags.items():
        def step():
            i8.attn_int8_fwd_ex(q, k, v, True, fl, out=out, workspace=ws)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        o = i8.attn_int8_fwd_ex(qq, kk, vv, False, fl).float().cpu().numpy()
        ref = oracle.attn_int8_fwd(w.q, w.k, w.v, False, heads=heads, rows=rows, **kw[name])
        err = float(np.abs(pick(o) - ref).max())
        if not err <= 2e-3:
            raise RuntimeError(f"{name} output differs from the oracle: max_abs={err}")
        res[name] = {"step_us": round(ms * 1e3, 2),
                     "extra_us_over_plain": round((ms - ms_step) * 1e3, 2),
                     "sqnr_db": sqnr(o), "parity_sample_max_abs": err}
        log(f"bench: {name} forward {res[name]['step_us']} us/step; SQNR "
            f"{res['sqnr_db_plain']} -> {res[name]['sqnr_db']} dB on the outlier workload")
    return res


def oracle_rate(q16, k16, v16, heads, rows, causal, budget_s: float):
    """The CPU oracle on a bounded sample: the quantization of the given fp16 q/k/v
    (dense ``[1, H, S, D]``, only the heads the sample needs), then the listed query heads
    over the listed rows until the budget is spent.  Returns (algorithmic ops done,
    seconds, heads done); a row's ops are 4 D per (query, key) pair it attends."""
    import numpy as np

    import oracle
    S, D = q16.shape[2], q16.shape[3]
    G = q16.shape[1] // k16.shape[1]
    t0 = time.perf_counter()
    z = oracle.quantize_qkv(q16, k16, v16)
    sm = oracle.default_softmax_scale(D)
    rows = np.asarray(rows)
    pairs = float(np.sum(rows + 1)) if causal else float(rows.size * S)
    ops, done = 0.0, 0
    for h in heads:
        g = h // G
        oracle.attn_core(z["q8"][0, h], z["sq"][0, h], z["k8"][0, g], z["sk"][0, g],
                         z["v8"][0, g], z["sv"][0, g], sm, causal, rows)
        ops += 4.0 * D * pairs
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    return ops, time.perf_counter() - t0, done


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return 1


def bench_configs(args, i8, torch, dev):
    """The benchmark set's other workloads (see the module docstring)."""
    import numpy as np

    import oracle
    from int8_w8a8_flashattention_amd import workloads
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm, n = max(args.warmup // 10, 5), max(args.steps // 2, 10)

    def timed(fn, warmup=warm, steps=n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3  # us

    def tops(ops, us):
        return ops / (us * 1e-6) / 1e12

    def roofline(ops, us):
        a = tops(ops, us)
        return {"bound": "mfma", "achieved": round(a, 2), "peak": INT8_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(a / INT8_PEAK_TOPS, 4), "traffic": None}

    def guard(got, ref, what):
        err = float(np.abs(got.astype(np.float64) - ref).max())
        if not err <= 2e-3:
            raise RuntimeError(f"{what} output differs from the oracle: max_abs={err}")
        return err

    def cpu(ops, dt, what):
        th = blas_threads()
        return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": int(th),
                "kind": "oracle", "sample": f"{what}; {dt:.1f} s of numpy fp64 with BLAS on "
                                            f"{th} threads ({cpu_model()})"}

    budget = args.cpu_budget / 3
    res = {}
    dense_cases = [(f"mha_s2048_d{D}", workloads.cfg3(D), False) for D in (32, 64, 128, 256)]
    for name, w, causal in dense_cases + [("causal_gqa_s32768", None, True)]:
        if w is None:
            log("bench: generating the S=32768 inputs")
            w = workloads.cfg5()
        B, Hq, S, D = w.q.shape
        Hkv = w.k.shape[1]
        q, k, v = (torch.from_numpy(a).to(dev) for a in (w.q, w.k, w.v))
        out = torch.empty_like(q)
        ws = torch.empty(i8.attn_int8_workspace_bytes(B, Hq, Hkv, S, D), dtype=torch.uint8,
                         device=dev)
        ops = workloads.attn_ops(Hq, D, [S] * B, causal)
        long = S > 8192
        us = timed(lambda: i8.attn_int8_fwd(q, k, v, causal, out=out, workspace=ws),
                   *((3, 5) if long else (warm, n)))
        # The attention kernel alone: over prepared K/V, the kernel that quantizes its own
        # Q rows (D <= 128), or over prepared Q as well (D = 256).
        i8.attn_int8_prepare_kv(k, v, Hq, workspace=ws)
        if D <= 128:
            ua = timed(lambda: i8.attn_int8_fwd_prepared(q, Hkv, ws, causal, out=out),
                       *((3, 5) if long else (warm, n)))
        else:
            i8.attn_int8_prepare_q(q, Hkv, ws)
            ua = timed(lambda: i8.attn_int8_attend(ws, B, Hq, Hkv, S, D, causal, out=out))
        i8.attn_int8_fwd(q, k, v, causal, out=out, workspace=ws)
        heads = [(0, 0), (B - 1, Hq - 1)]
        rows = np.unique(np.linspace(0, S - 1, 24).astype(np.int64))
        ridx = torch.from_numpy(rows).to(dev)
        got = np.stack([out[b, h][ridx].float().cpu().numpy() for b, h in heads])
        ref = oracle.attn_int8_fwd(w.q, w.k, w.v, causal, heads=heads, rows=rows)
        err = guard(got, ref, name)
        e = {"workload": w.name, "B": B, "Hq": Hq, "Hkv": Hkv, "S": S, "D": D, "causal": causal,
             "algorithmic_ops": ops, "step_us": round(us, 2), "value": round(tops(ops, us), 2),
             "unit": "TOPS", "frac_int8_peak": round(tops(ops, us) / INT8_PEAK_TOPS, 4),
             "attn_kernel_us": round(ua, 2), "roofline": roofline(ops, ua),
             "parity_sample_max_abs": err}
        if not args.no_cpu_baseline:
            if long:  # one kv group, every 64th row of its heads
                G = Hq // Hkv
                rr = np.arange(0, S, 64)
                o_, dt, hd = oracle_rate(w.q[:1, :G], w.k[:1, :1], w.v[:1, :1], range(G), rr,
                                         causal, budget)
                what = (f"{hd} of the {G} query heads of kv group 0 (one of {Hkv}), every 64th "
                        f"of their {S} rows, plus that group's quantization; extrapolated: "
                        f"the rate on the sample stands for the whole call")
            else:
                o_, dt, hd = oracle_rate(w.q[:1], w.k[:1], w.v[:1], range(Hq), np.arange(S),
                                         causal, budget)
                what = (f"{hd} of the {Hq} heads of batch 0 (all {S} rows each), plus batch "
                        f"0's quantization")
            e["cpu_baseline"] = cpu(o_, dt, what)
        res[name] = e
        log(f"bench: {name}: {us:.1f} us/call ({e['value']} TOPS), attention kernel "
            f"{ua:.1f} us ({e['roofline']['achieved']} TOPS)")
        del q, k, v, out, ws, w
    # Varlen prefill: 16 sequences, lengths drawn U[1, 4096].
    w = workloads.cfg4()
    T, Hq, D = w.q.shape
    Hkv = w.k.shape[1]
    cu = w.cu_seqlens
    lens = np.diff(cu).tolist()
    q, k, v = (torch.from_numpy(a).to(dev) for a in (w.q, w.k, w.v))
    cud = torch.from_numpy(cu.astype(np.int32)).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(i8.attn_int8_varlen_workspace_bytes(len(lens), T, w.max_seqlen, Hq, Hkv, D),
                     dtype=torch.uint8, device=dev)
    ops = workloads.attn_ops(Hq, D, lens, True)
    us = timed(lambda: i8.attn_int8_varlen_fwd(q, k, v, cud, w.max_seqlen, True, out=out,
                                               workspace=ws))
    s0 = int(np.argmax(lens))
    a0, b0 = int(cu[s0]), int(cu[s0 + 1])
    rows = np.unique(np.linspace(0, b0 - a0 - 1, 16).astype(np.int64))
    got = out[a0:b0][torch.from_numpy(rows).to(dev)][:, [0, Hq - 1]].float().cpu().numpy()
    qs_, ks_, vs_ = (np.ascontiguousarray(x[a0:b0].transpose(1, 0, 2))[None]
                     for x in (w.q, w.k, w.v))
    ref = oracle.attn_int8_fwd(qs_, ks_, vs_, True, heads=[(0, 0), (0, Hq - 1)], rows=rows)
    err = guard(got.transpose(1, 0, 2), ref, "varlen")
    e = {"workload": w.name, "nseq": len(lens), "lengths": lens, "total_tokens": T,
         "Hq": Hq, "Hkv": Hkv, "D": D, "causal": True, "algorithmic_ops": ops,
         "step_us": round(us, 2), "value": round(tops(ops, us), 2), "unit": "TOPS",
         "frac_int8_peak": round(tops(ops, us) / INT8_PEAK_TOPS, 4),
         "roofline": roofline(ops, us), "roofline_note": "the whole call (no split entry for "
                                                         "varlen attention alone)",
         "parity_sample_max_abs": err}
    if not args.no_cpu_baseline:
        o_, dt, hd = oracle_rate(qs_, ks_, vs_, range(Hq), np.arange(b0 - a0), True, budget)
        e["cpu_baseline"] = cpu(o_, dt, f"{hd} of the {Hq} heads of the longest sequence "
                                       f"({b0 - a0} tokens, all rows), plus its quantization")
    res["varlen_16x_u4096"] = e
    log(f"bench: varlen: {us:.1f} us/call ({e['value']} TOPS)")
    return res


def bench_backward(args, i8, torch, dev, q, k, v):
    """The backward (NEXT-4) on the same workload: one attn_bwd call per step (operand
    preparation, dQ kernel, dK/dV kernel).  Its roofline is the fp16 MFMA: algorithmic
    flops = 10 * D per (query, key) pair (five products of 2 * D: the recomputed scores,
    dP, dV, dK and dQ; the FlashAttention-2 count), S^2/2 pairs per causal head."""
    import numpy as np

    B, Hq, S, D = q.shape
    do = torch.from_numpy(np.random.Generator(np.random.PCG64(214)).standard_normal(
        tuple(q.shape)).astype(np.float16)).to(dev)
    ws = torch.empty(i8.attn_bwd_workspace_bytes(B, Hq, k.shape[1], S, D), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def step():
        i8.attn_bwd(q, k, v, do, True, workspace=ws)

    for _ in range(max(args.warmup // 4, 5)):
        step()
    torch.cuda.synchronize()
    n = max(args.steps // 2, 5)
    e0.record(stream)
    for _ in range(n):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    flops = 10.0 * D * Hq * B * S * S / 2.0
    tf = flops / (us * 1e-6) / 1e12
    log(f"bench: backward {us:.1f} us/call, {tf:.1f} TFLOP/s")
    return {"call_us": round(us, 2), "algorithmic_flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP16_PEAK_TOPS,
                         "unit": "TFLOP/s", "frac": round(tf / FP16_PEAK_TOPS, 4),
                         "traffic": measured_traffic(BWD_TRAFFIC_FILE),
                         "traffic_note": "HBM bytes of one whole call (its four kernels)"},
            "note": "fp32 dq, dk, dv; the quantization taken as the identity; the "
                    "implementation computes the scores and dP three times per pair "
                    "(18 D flops per pair), the roofline counts the algorithmic 10 D"}


def profile_backward(n, i8, torch, dev):
    """Profiling mode: n backward calls on the causal GQA workload."""
    import numpy as np
    from int8_w8a8_flashattention_amd import workloads
    w = workloads.cfg2()
    q, k, v = (torch.from_numpy(a).to(dev) for a in (w.q, w.k, w.v))
    do = torch.from_numpy(np.random.Generator(np.random.PCG64(214)).standard_normal(
        w.q.shape).astype(np.float16)).to(dev)
    for _ in range(n):
        i8.attn_bwd(q, k, v, do, True)
    torch.cuda.synchronize()
    log(f"bench: {n} backward calls")


def profile_decode(n, i8, torch, dev):
    """Profiling mode: per V format (int8, then fp16), fill the cache once, then n
    decode calls."""
    from int8_w8a8_flashattention_amd import workloads
    w = workloads.decode_bench()
    B, Hq, D = w.q.shape
    q, k, v = (torch.from_numpy(a).to(dev) for a in (w.q, w.k, w.v))
    out = torch.empty_like(q)
    for vf in ("int8", "fp16"):
        cache = i8.attn_int8_kvcache_fill(k, v, vf)
        for _ in range(n):
            i8.attn_int8_decode(q, cache, out=out)
        torch.cuda.synchronize()
        del cache
    log(f"bench: {n} decode calls per V format")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # Back-to-back forwards settle at the sustained clock only after tens of ms; 300
    # untimed steps (~50 ms) get there, 10 do not (the first timed steps then run ~15 %
    # slower).
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of CPU oracle work for the cpu_baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calls", type=int, default=100,
                    help="individually timed calls for the median/min, with and without a "
                         "512 MiB cache flush before each")
    ap.add_argument("--profile-attn", type=int, default=0, metavar="N",
                    help="profiling mode: prepare Q, K and V once, launch only the attention "
                         "kernel N times, print nothing else")
    ap.add_argument("--profile-decode", type=int, default=0, metavar="N",
                    help="profiling mode: per V format, fill the decode cache once, then N "
                         "decode calls")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (head-dim sweep, varlen, S=32768)")
    ap.add_argument("--profile-bwd", type=int, default=0, metavar="N",
                    help="profiling mode: N backward calls on the causal GQA workload")
    ap.add_argument("--profile-copy", type=int, default=0, metavar="MIB",
                    help="profiling mode: 10 plain device copies of MIB MiB (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards by kv-head groups with no communication)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int8_w8a8_flashattention_amd as i8
    from int8_w8a8_flashattention_amd import workloads

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    i8.load_library()
    dev = torch.device("cuda:0")
    if args.profile_decode:
        profile_decode(args.profile_decode, i8, torch, dev)
        return
    if args.profile_bwd:
        profile_backward(args.profile_bwd, i8, torch, dev)
        return
    w = workloads.cfg2()
    B, Hq, Hkv, S, D = (WORKLOAD[k] for k in ("B", "Hq", "Hkv", "S", "D"))
    assert w.q.shape == (B, Hq, S, D) and w.k.shape == (B, Hkv, S, D)
    if args.profile_copy:
        src = torch.ones(args.profile_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copied {args.profile_copy} MiB 10 times")
        return
    q, k, v = (torch.from_numpy(a).to(dev) for a in (w.q, w.k, w.v))
    out = torch.empty_like(q)
    ws = torch.empty(i8.attn_int8_workspace_bytes(B, Hq, Hkv, S, D), dtype=torch.uint8, device=dev)
    if args.profile_attn:
        i8.attn_int8_prepare_kv(k, v, Hq, workspace=ws)
        for _ in range(args.profile_attn):
            i8.attn_int8_fwd_prepared(q, Hkv, ws, True, out=out)
        torch.cuda.synchronize()
        log(f"bench: {args.profile_attn} attention launches")
        return
    ops = workloads.attn_ops(Hq, D, [S] * B, True)
    stream = torch.cuda.current_stream(dev)

    def step():
        i8.attn_int8_fwd(q, k, v, True, out=out, workspace=ws)

    log(f"bench: warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"bench: {args.steps} steps, {ms_step * 1e3:.1f} us/step (host wall {t_wall * 1e6 / args.steps:.1f} us/step)")

    # The phases alone: the attention kernel (dominant; over prepared K/V it quantizes
    # its own Q rows, as in the step), then the K/V preparation.
    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    i8.attn_int8_prepare_kv(k, v, Hq, workspace=ws)
    ms_attn = timed(lambda: i8.attn_int8_fwd_prepared(q, Hkv, ws, True, out=out))
    ms_prep_kv = timed(lambda: i8.attn_int8_prepare_kv(k, v, Hq, workspace=ws))
    log(f"bench: attention kernel {ms_attn * 1e3:.1f} us, K/V preparation {ms_prep_kv * 1e3:.1f} us")

    # Per-call times (each call between its own pair of events): median and min, as they
    # stand and with a 512 MiB buffer written before each call, which evicts the inputs
    # and the workspace from the L2s and the 256 MB last-level cache.
    def per_call(flush):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.calls)]
        for a, b in evs:
            if flush is not None:
                flush.fill_(1)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        return {"median": round(t[len(t) // 2], 2), "min": round(t[0], 2), "n": len(t)}

    call_us = per_call(None)
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flushed_call_us = per_call(flush_buf)
    del flush_buf
    log(f"bench: per call {call_us}, after a cache flush {flushed_call_us}")

    # Parity guard on the benchmarked output (sampled rows of two heads), the fp16
    # rounding floor of the oracle's output there, and the quantization's SQNR against
    # unquantized fp64 attention on the same rows (quality, not a gate).
    import oracle
    i8.attn_int8_fwd(q, k, v, True, out=out, workspace=ws)
    rows = np.array([0, 1, 127, 128, 2047, 4095])
    heads = [(0, 0), (0, 31)]
    ref = oracle.attn_int8_fwd(w.q, w.k, w.v, True, heads=heads, rows=rows)
    got = out[0, [h for _, h in heads]][:, rows].float().cpu().numpy()
    max_abs = float(np.abs(got - ref).max())
    if not max_abs <= 2e-3:
        raise RuntimeError(f"benchmarked output differs from the oracle: max_abs={max_abs}")
    floor = float(np.abs(ref.astype(np.float16).astype(np.float64) - ref).max())
    exact = oracle.attn_exact(w.q, w.k, w.v, True, heads=heads, rows=rows)
    sqnr_db = float(10.0 * np.log10(np.sum(exact ** 2) / np.sum((got - exact) ** 2)))

    # Algorithmic bytes of the K/V preparation: fp16 K and V read once, the K/V tile
    # blocks (int8 K, exact fp16 V, fp32 K scales) written.
    prep_kv_bytes = 2 * B * Hkv * S * D * 2 + B * Hkv * S * (D + 2 * D + 4)
    value = ops / (ms_step * 1e-3) / 1e12
    achieved = ops / (ms_attn * 1e-3) / 1e12
    traffic = measured_traffic()
    res = {
        "metric": "INT8 attn fwd effective TOPS & % int8 MFMA peak, Hq32/Hkv8 S4096 D128 causal",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp16",
        "data": "synthetic",
        "config": {"workload": "causal GQA attention B1 Hq32 Hkv8 S4096 D128, fp16 N(0,1), seed 2",
                   "B": B, "Hq": Hq, "Hkv": Hkv, "S": S, "D": D, "causal": True,
                   "algorithmic_ops": ops},
        "pct_int8_peak": round(100.0 * value / INT8_PEAK_TOPS, 2),
        "pct_mixed_ceiling": round(100.0 * value / MIXED_PEAK_TOPS, 2),
        "call_us": call_us,
        "flushed_call_us": flushed_call_us,
        "attn_kernel_us": round(ms_attn * 1e3, 2),
        "prep_kv_us": round(ms_prep_kv * 1e3, 2),
        "prep_kv_gbs": round(prep_kv_bytes / (ms_prep_kv * 1e-3) / 1e9, 1),
        "parity_sample_max_abs": max_abs,
        "parity_sample_fp16_floor": floor,
        "sqnr_db_vs_exact": round(sqnr_db, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        log(f"bench: timing the CPU oracle (~{args.cpu_budget:.0f} s)")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    res["variants"] = bench_variants(args, i8, torch, dev, q, k, v, out, ws, ms_step)
    res["backward"] = bench_backward(args, i8, torch, dev, q, k, v)
    del q, k, v, out, ws
    if not args.no_configs:
        res["configs"] = bench_configs(args, i8, torch, dev)
    if not args.no_decode:
        res["decode"] = bench_decode(args, i8, torch, dev)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
