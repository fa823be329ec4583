"""Pins for the CPU oracle: checks against things other than the oracle itself.

Every check here compares the oracle with exact rational arithmetic, brute
force, a library routine (torch's CPU fp64 scaled-dot-product attention), an
invariance the method must have, a closed form, or a value derived by hand
(``tests/golden``).  None of them re-types the oracle's own formulas.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import scipy.linalg as sla
import pytest
import torch

import oracle
from int8_w8a8_flashattention_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def rn32(f: Fraction) -> Fraction:
    """Exact value of the fp32 nearest to f (ties to even), from first principles."""
    if f == 0:
        return Fraction(0)
    sign = -1 if f < 0 else 1
    a = abs(f)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = round(a / ulp)  # Python rounds a Fraction half to even
    return sign * n * ulp


def smallest_at_least(t: Fraction, bits: int) -> Fraction:
    """Smallest number >= t whose binary significand fits in ``bits`` bits."""
    if t == 0:
        return Fraction(0)
    e = t.numerator.bit_length() - t.denominator.bit_length()
    if Fraction(2) ** e > t:
        e -= 1
    while Fraction(2) ** (e + 1) <= t:
        e += 1
    step = Fraction(2) ** (e - bits + 1)
    return math.ceil(t / step) * step


def exact_quant_row(row, bits=24):
    """Quantize one fp32 row with rational arithmetic; returns (scale, codes)."""
    xs = [Fraction(float(x)) for x in row]
    a = max(abs(x) for x in xs)
    if a == 0:
        return Fraction(0), [0] * len(xs)
    t = rn32(a / 127)
    s = smallest_at_least(t, bits)
    codes = []
    for x in xs:
        r = rn32(x / s)
        c = round(r)  # half to even
        codes.append(max(-127, min(127, c)))
    return s, codes


def dequant(codes, scales):
    return scales.astype(np.float64)[..., None] * codes.astype(np.float64)


def sdpa64(q, k, v, causal, scale):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))  # noqa: E731
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=float(scale)).numpy()


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- K mean

@pytest.mark.parametrize("L", [1, 3, 17, 128, 1000])
def test_kmean_equals_exact_rational_mean(L):
    g = rng(100 + L)
    D = 8
    k = (g.standard_normal((2, L, D)) * np.exp(g.uniform(-12, 10, (2, L, D)))).astype(np.float16)
    k[0, 0, 0] = np.float16(6e-8)  # a subnormal
    m = oracle.kmean(k)
    for h in range(2):
        for d in range(D):
            exact = sum(Fraction(float(x)) for x in k[h, :, d]) / L
            want = np.float32(float(exact))  # float(Fraction) is correctly rounded
            assert m[h, d] == want, (h, d)


# ---------------------------------------------------------------- quantization

def _rows_for_quant():
    g = rng(7)
    rows = [g.standard_normal(64).astype(np.float16).astype(np.float32) for _ in range(30)]
    rows += [(g.standard_normal(16) * 1e-3).astype(np.float16).astype(np.float32) for _ in range(10)]
    # K-smoothing-like rows: fp16 values minus an arbitrary fp32 mean
    for _ in range(20):
        m = np.float32(g.uniform(-3, 3))
        rows.append(g.standard_normal(32).astype(np.float16).astype(np.float32) - m)
    # rows built to hit exact .5 ties of x/scale (scale of absmax 127/64 is 1/64)
    tie = np.array([127 / 64, 0.5 / 64, 2.5 / 64, -3.5 / 64, 6.5 / 64], np.float32)
    assert np.float32(tie[0] / np.float32(127)) == np.float32(1 / 64)
    rows.append(tie)
    rows.append(np.zeros(8, np.float32))
    rows.append(np.array([65504.0, -65504.0, 1.0], np.float32))
    return rows


@pytest.mark.parametrize("bits", [oracle.QK_SCALE_BITS, oracle.V_SCALE_BITS])
def test_quant_rows_match_exact_rational_rule(bits):
    for row in _rows_for_quant():
        codes, scale = oracle.quant_rows(row[None, :], bits)
        s, c = exact_quant_row(row, bits)
        assert Fraction(float(scale[0])) == s
        assert codes[0].tolist() == c


def test_quant_rows_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "quant_rows_worked.json")))
    for key, bits in (("qk_cases", oracle.QK_SCALE_BITS), ("v_cases", oracle.V_SCALE_BITS)):
        for case in g[key]:
            codes, scale = oracle.quant_rows(np.array([case["x"]], np.float32), bits)
            assert Fraction(float(scale[0])) == Fraction(case["scale_num"], case["scale_den"])
            assert codes[0].tolist() == case["codes"]
    kc = g["kmean_case"]
    k = np.array(kc["k"], np.float16)[None]  # [1, L, D]
    m = oracle.kmean(k)[0]
    assert m.tolist() == kc["mean"]
    codes, scale = oracle.quant_rows(k.astype(np.float32)[0] - m[None, :])
    for r in kc["rows"]:
        assert Fraction(float(scale[r["row"]])) == Fraction(r["scale_num"], r["scale_den"])
        assert codes[r["row"]].tolist() == r["codes"]


def test_quant_rows_properties():
    g = rng(11)
    x = g.standard_normal((200, 128)).astype(np.float16).astype(np.float32)
    x[5] = 0
    codes, scale = oracle.quant_rows(x)
    nz = scale > 0
    assert not nz[5] and np.all(codes[5] == 0)
    # the row maximum maps to +-127
    assert np.all(np.abs(codes[nz]).max(axis=1) == 127)
    # |x/scale - code| <= 1/2 (up to the fp32 rounding of the quotient)
    r = x[nz].astype(np.float64) / scale[nz, None].astype(np.float64)
    assert np.all(np.abs(r - codes[nz]) <= 0.5 + 1e-5)
    # the scale is absmax/127 to fp32 precision
    a = np.abs(x[nz]).max(axis=1).astype(np.float64)
    np.testing.assert_allclose(scale[nz].astype(np.float64), a / 127, rtol=2**-24, atol=0)
    # power-of-two scaling is exact: same codes, scale times 2^k
    for kexp in (-7, 3):
        c2, s2 = oracle.quant_rows((x * np.float32(2.0**kexp)).astype(np.float32))
        assert np.array_equal(c2, codes)
        assert np.array_equal(s2, (scale * np.float32(2.0**kexp)).astype(np.float32))


def test_v_quant_dequantizes_to_exact_fp16():
    """V rows: 4-bit scale significand, row max maps to at least 113, and every
    code * scale is exactly an fp16 number (including fp16 subnormals for
    rows whose scale is at least 2^-21)."""
    g = rng(12)
    x = (g.standard_normal((300, 64)) * np.exp(g.uniform(-9, 9, (300, 1)))).astype(np.float16)
    x = x.astype(np.float32)
    codes, scale = oracle.quant_rows(x, oracle.V_SCALE_BITS)
    assert np.all(scale.view(np.uint32) & 0xFFFFF == 0)
    a = np.abs(x).max(axis=1).astype(np.float64)
    assert np.all(scale >= a / 127 * (1 - 2**-23))
    assert np.all(scale <= a / 127 * 1.125 * (1 + 2**-23))
    assert np.all(np.abs(codes).max(axis=1) >= 113)
    ok = scale >= 2.0**-21
    vhat = scale[ok, None].astype(np.float64) * codes[ok].astype(np.float64)
    assert np.array_equal(vhat.astype(np.float16).astype(np.float64), vhat)


# ---------------------------------------------------------------- integer scores

def test_qk_int32_brute_force():
    g = rng(3)
    q8 = g.integers(-127, 128, (5, 7)).astype(np.int8)
    k8 = g.integers(-127, 128, (6, 7)).astype(np.int8)
    s = oracle.qk_int32(q8, k8)
    for i in range(5):
        for j in range(6):
            assert s[i, j] == sum(int(q8[i, d]) * int(k8[j, d]) for d in range(7))


def test_qk_int32_extremes_d256():
    q8 = np.full((2, 256), 127, np.int8)
    k8 = np.full((3, 256), -127, np.int8)
    s = oracle.qk_int32(q8, k8)
    assert np.all(s == -127 * 127 * 256)
    g = rng(4)
    a = g.integers(-127, 128, (64, 256)).astype(np.int8)
    b = g.integers(-127, 128, (80, 256)).astype(np.int8)
    assert np.array_equal(oracle.qk_int32(a, b), np.einsum("id,jd->ij", a.astype(np.int64), b.astype(np.int64)))


# ---------------------------------------------------------------- attention on quantized operands

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv,S,D", [(4, 2, 37, 32), (2, 1, 64, 64), (3, 3, 20, 128)])
def test_forward_equals_library_attention_on_dequantized(causal, Hq, Hkv, S, D):
    w = workloads.dense(21, 2, Hq, Hkv, S, D, causal, k_offset=2.0)
    out = oracle.attn_int8_fwd(w.q, w.k, w.v, causal)
    z = oracle.quantize_qkv(w.q, w.k, w.v)
    G = Hq // Hkv
    qh = dequant(z["q8"], z["sq"])
    kh = np.repeat(dequant(z["k8"], z["sk"]), G, axis=1)
    vh = np.repeat(dequant(z["v8"], z["sv"]), G, axis=1)
    ref = sdpa64(qh, kh, vh, causal, oracle.default_softmax_scale(D))
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_exact_attention_equals_library():
    w = workloads.dense(22, 1, 4, 2, 33, 64, True)
    ref = sdpa64(w.q, np.repeat(w.k, 2, 1), np.repeat(w.v, 2, 1), True, oracle.default_softmax_scale(64))
    np.testing.assert_allclose(oracle.attn_exact(w.q, w.k, w.v, True), ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_exact_attention_sampled_rows_equal_library(causal):
    w = workloads.dense(24, 2, 4, 2, 40, 32, causal)
    ref = sdpa64(w.q, np.repeat(w.k, 2, 1), np.repeat(w.v, 2, 1), causal,
                 oracle.default_softmax_scale(32))
    heads, rows = [(1, 3), (0, 0)], np.array([0, 7, 39])
    got = oracle.attn_exact(w.q, w.k, w.v, causal, heads=heads, rows=rows)
    want = np.stack([ref[b, h][rows] for b, h in heads])
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_k_smoothing_exact_invariance_unquantized():
    w = workloads.dense(23, 1, 2, 1, 50, 32, True, k_offset=3.0)
    k = w.k.astype(np.float64)
    ks = k - k.mean(axis=2, keepdims=True)
    a = oracle.attn_exact(w.q, k, w.v, True)
    b = oracle.attn_exact(w.q, ks, w.v, True)
    assert np.max(np.abs(a - b)) < 1e-12


def test_k_smoothing_removes_channel_offsets():
    """With K-smoothing a per-channel K offset changes nothing: codes, scales
    and outputs are bit-identical.  Inputs are chosen so every step is exact
    (K on a 2^-4 grid, integer offsets, 16 tokens)."""
    g = rng(24)
    B, H, S, D = 1, 2, 16, 32
    q = g.standard_normal((B, H, S, D)).astype(np.float16)
    v = g.standard_normal((B, H, S, D)).astype(np.float16)
    k = (np.round(g.uniform(-4, 4, (B, H, S, D)) * 16) / 16).astype(np.float16)
    off = g.integers(-3, 4, (1, H, 1, D)).astype(np.float16)
    k2 = (k.astype(np.float32) + off).astype(np.float16)
    assert np.array_equal(k2.astype(np.float32) - off, k.astype(np.float32))
    za, zb = oracle.quantize_qkv(q, k, v), oracle.quantize_qkv(q, k2, v)
    assert np.array_equal(za["k8"], zb["k8"]) and np.array_equal(za["sk"], zb["sk"])
    assert np.array_equal(oracle.attn_int8_fwd(q, k, v, True), oracle.attn_int8_fwd(q, k2, v, True))
    # without the subtraction the codes would differ
    c_raw, _ = oracle.quant_rows(k2.astype(np.float32))
    assert not np.array_equal(c_raw, za["k8"])


def test_causal_rows_equal_prefix_attention():
    g = rng(25)
    S, D = 40, 64
    q8 = g.integers(-127, 128, (S, D)).astype(np.int8)
    k8 = g.integers(-127, 128, (S, D)).astype(np.int8)
    v8 = g.integers(-127, 128, (S, D)).astype(np.int8)
    sq, sk, sv = (g.uniform(0.001, 0.03, S).astype(np.float32) for _ in range(3))
    sm = oracle.default_softmax_scale(D)
    full = oracle.attn_core(q8, sq, k8, sk, v8, sv, sm, True)
    for i in (0, 1, 7, S - 1):
        pre = oracle.attn_core(q8[i:i + 1], sq[i:i + 1], k8[:i + 1], sk[:i + 1], v8[:i + 1], sv[:i + 1], sm, False)
        np.testing.assert_allclose(full[i], pre[0], rtol=1e-13, atol=1e-15)
    # row 0 sees one key: exactly that key's dequantized value
    assert np.array_equal(full[0], sv[0].astype(np.float64) * v8[0].astype(np.float64))


def test_gqa_equals_repeated_heads():
    w = workloads.dense(26, 2, 6, 2, 45, 32, True, k_offset=1.0)
    a = oracle.attn_int8_fwd(w.q, w.k, w.v, True)
    b = oracle.attn_int8_fwd(w.q, np.repeat(w.k, 3, 1), np.repeat(w.v, 3, 1), True)
    assert np.array_equal(a, b)


def test_varlen_equal_lengths_equals_dense():
    w = workloads.dense(27, 3, 4, 2, 30, 32, True)
    B, Hq, S, D = w.q.shape
    tq = w.q.transpose(0, 2, 1, 3).reshape(B * S, Hq, D)
    tk = w.k.transpose(0, 2, 1, 3).reshape(B * S, 2, D)
    tv = w.v.transpose(0, 2, 1, 3).reshape(B * S, 2, D)
    cu = np.arange(0, B * S + 1, S, dtype=np.int32)
    a = oracle.attn_int8_varlen_fwd(tq, tk, tv, cu, True)
    b = oracle.attn_int8_fwd(w.q, w.k, w.v, True).transpose(0, 2, 1, 3).reshape(B * S, Hq, D)
    assert np.array_equal(a, b)


def test_varlen_sequences_are_independent():
    w = workloads.varlen(28, 4, 30, 4, 2, 32, True, lengths=[5, 0, 30, 1])
    a = oracle.attn_int8_varlen_fwd(w.q, w.k, w.v, w.cu_seqlens, True)
    # changing one sequence leaves every other sequence's rows unchanged
    k2 = w.k.copy()
    k2[5:35] = (k2[5:35].astype(np.float32) * 3).astype(np.float16)
    b = oracle.attn_int8_varlen_fwd(w.q, k2, w.v, w.cu_seqlens, True)
    assert np.array_equal(a[:5], b[:5]) and np.array_equal(a[35:], b[35:])
    assert not np.array_equal(a[5:35], b[5:35])


def test_zero_queries_give_prefix_means():
    g = rng(29)
    B, H, S, D = 1, 1, 25, 32
    q = np.zeros((B, H, S, D), np.float16)
    k = g.standard_normal((B, H, S, D)).astype(np.float16)
    v = g.standard_normal((B, H, S, D)).astype(np.float16)
    out = oracle.attn_int8_fwd(q, k, v, True)[0, 0]
    v8, sv = oracle.quant_rows(v.astype(np.float32)[0, 0], oracle.V_SCALE_BITS)
    vh = dequant(v8, sv)
    want = np.cumsum(vh, axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)
    out_nc = oracle.attn_int8_fwd(q, k, v, False)[0, 0]
    np.testing.assert_allclose(out_nc, np.broadcast_to(vh.mean(axis=0), out_nc.shape), rtol=1e-12, atol=1e-14)


def test_dominant_key_gives_its_value():
    g = rng(30)
    S, D = 20, 64
    q = g.standard_normal((1, 1, S, D)).astype(np.float16)
    k = (g.standard_normal((1, 1, S, D)) * 0.01).astype(np.float16)
    j = 13
    k[0, 0, j] = (q[0, 0, S - 1].astype(np.float32) * 40).astype(np.float16)
    v = g.standard_normal((1, 1, S, D)).astype(np.float16)
    out = oracle.attn_int8_fwd(q, k, v, False)[0, 0, S - 1]
    v8, sv = oracle.quant_rows(v.astype(np.float32)[0, 0], oracle.V_SCALE_BITS)
    np.testing.assert_allclose(out, dequant(v8, sv)[j], rtol=0, atol=1e-9)


def test_noncausal_key_permutation_invariance():
    w = workloads.dense(31, 1, 2, 2, 24, 32, False, k_offset=1.0)
    perm = rng(31).permutation(24)
    a = oracle.attn_int8_fwd(w.q, w.k, w.v, False)
    b = oracle.attn_int8_fwd(w.q, w.k[:, :, perm], w.v[:, :, perm], False)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- whole method vs exact attention

@pytest.mark.parametrize("causal", [True, False])
def test_quantized_forward_within_a_posteriori_bound(causal):
    """|O_int8 - O_exact| <= max_j|dv_jd| + (exp(2 eps_i) - 1) max_j|v_jd| with
    eps_i = sm * max_j sum_d(|q||dk| + |dq||k| + |dq||dk|), the dequantization
    errors measured on the actual inputs (a score perturbation of at most eps
    moves every softmax weight by a factor within exp(+-2 eps))."""
    w = workloads.cfg1() if causal else workloads.dense(32, 1, 2, 1, 96, 32, False, outlier_frac=0.05)
    q = w.q.astype(np.float64)
    z = oracle.quantize_qkv(w.q, w.k, w.v)
    ks = (w.k.astype(np.float32) - z["kmean"][..., None, :]).astype(np.float64)
    v = w.v.astype(np.float64)
    dq = dequant(z["q8"], z["sq"]) - q
    dk = dequant(z["k8"], z["sk"]) - ks
    dv = dequant(z["v8"], z["sv"]) - v
    o = oracle.attn_int8_fwd(w.q, w.k, w.v, causal)
    ex = oracle.attn_exact(q, ks, v, causal)
    D = q.shape[-1]
    sm = float(oracle.default_softmax_scale(D))
    B, Hq, S, _ = q.shape
    G = Hq // w.k.shape[1]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            e = (np.abs(q[b, h]) @ np.abs(dk[b, g]).T + np.abs(dq[b, h]) @ np.abs(ks[b, g]).T
                 + np.abs(dq[b, h]) @ np.abs(dk[b, g]).T) * sm
            for i in range(S):
                jmax = i + 1 if causal else S
                eps = e[i, :jmax].max()
                bound = (np.abs(dv[b, g, :jmax]).max(axis=0)
                         + np.expm1(2 * eps) * np.abs(v[b, g, :jmax]).max(axis=0))
                assert np.all(np.abs(o[b, h, i] - ex[b, h, i]) <= bound + 1e-12), (b, h, i)


# ---------------------------------------------------------------- decode (R12)

@pytest.mark.parametrize("Hq,Hkv,S,D", [(4, 2, 37, 32), (2, 1, 64, 64), (8, 8, 20, 128), (32, 1, 9, 256)])
def test_decode_equals_library_attention_on_dequantized(Hq, Hkv, S, D):
    w = workloads.dense(40 + D, 2, Hq, Hkv, S, D, False, k_offset=2.0)
    q1 = w.q[:, :, 0]  # one new query token per sequence
    out = oracle.attn_int8_decode(q1, w.k, w.v)
    q8, sq = oracle.quant_rows(q1.astype(np.float32))
    z = oracle.quantize_qkv(w.q, w.k, w.v)
    G = Hq // Hkv
    qh = dequant(q8, sq)[:, :, None]
    kh = np.repeat(dequant(z["k8"], z["sk"]), G, axis=1)
    vh = np.repeat(dequant(z["v8"], z["sv"]), G, axis=1)
    ref = sdpa64(qh, kh, vh, False, oracle.default_softmax_scale(D))[:, :, 0]
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_decode_equals_noncausal_forward_row():
    # The query row placed at any position of a full query block gives the same row
    # of the non-causal forward: rows are quantized and attended independently (equal
    # up to the fp64 summation order of a one-row against a block matrix product).
    w = workloads.dense(41, 2, 4, 2, 50, 64, False)
    r = 17
    out = oracle.attn_int8_decode(w.q[:, :, r], w.k, w.v)
    fwd = oracle.attn_int8_fwd(w.q, w.k, w.v, False)[:, :, r]
    np.testing.assert_allclose(out, fwd, rtol=1e-12, atol=1e-14)


def test_decode_zero_query_gives_mean_value():
    g = rng(42)
    B, Hkv, S, D = 1, 2, 33, 32
    q = np.zeros((B, 4, D), np.float16)
    k = g.standard_normal((B, Hkv, S, D)).astype(np.float16)
    v = g.standard_normal((B, Hkv, S, D)).astype(np.float16)
    out = oracle.attn_int8_decode(q, k, v)
    v8, sv = oracle.quant_rows(v.astype(np.float32), oracle.V_SCALE_BITS)
    want = dequant(v8, sv).mean(axis=2)  # [B, Hkv, D]
    np.testing.assert_allclose(out, np.repeat(want, 2, axis=1), rtol=1e-12, atol=1e-14)


def test_decode_gqa_equals_repeated_heads():
    w = workloads.dense(43, 1, 8, 2, 40, 64, False, k_offset=1.0)
    q1 = w.q[:, :, 3]
    a = oracle.attn_int8_decode(q1, w.k, w.v)
    b = oracle.attn_int8_decode(q1, np.repeat(w.k, 4, axis=1), np.repeat(w.v, 4, axis=1))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("D", [32, 128])
def test_decode_fp16_v_equals_library_attention(D):
    # fp16-V cache: the values are used as given, K as in the int8-V cache.
    w = workloads.dense(44 + D, 2, 6, 3, 29, D, False, k_offset=-1.5)
    q1 = w.q[:, :, 5]
    out = oracle.attn_int8_decode(q1, w.k, w.v, v_format="fp16")
    q8, sq = oracle.quant_rows(q1.astype(np.float32))
    z = oracle.quantize_qkv(w.q, w.k, w.v)
    kh = np.repeat(dequant(z["k8"], z["sk"]), 2, axis=1)
    vh = np.repeat(w.v.astype(np.float64), 2, axis=1)
    ref = sdpa64(dequant(q8, sq)[:, :, None], kh, vh, False, oracle.default_softmax_scale(D))
    np.testing.assert_allclose(out, ref[:, :, 0], rtol=1e-11, atol=1e-12)


def test_decode_fp16_v_zero_query_gives_exact_mean():
    g = rng(45)
    k = g.standard_normal((2, 1, 21, 64)).astype(np.float16)
    v = g.standard_normal((2, 1, 21, 64)).astype(np.float16)
    out = oracle.attn_int8_decode(np.zeros((2, 3, 64), np.float16), k, v, v_format="fp16")
    want = v.astype(np.float64).mean(axis=2)
    np.testing.assert_allclose(out, np.repeat(want, 3, axis=1), rtol=1e-13, atol=1e-15)


# ------------------------------------------------- decode over a grown cache (R20)

def test_cache_appended_rows_quantize_against_the_filled_mean():
    # Rows past n_fill are appended: K against the mean of the filled tokens only (exact
    # rational rule), V per token; a copy of a filled token gets that token's codes.
    g = rng(60)
    B, Hkv, S, D, n_fill = 2, 2, 40, 32, 25
    k = (g.standard_normal((B, Hkv, S, D)) + g.uniform(-3, 3, (1, 1, 1, D))).astype(np.float16)
    v = g.standard_normal((B, Hkv, S, D)).astype(np.float16)
    k[:, :, 30] = k[:, :, 7]
    v[:, :, 30] = v[:, :, 7]
    k8, sk, v8, sv, m = oracle.kvcache_quantize(k, v, n_fill)
    np.testing.assert_array_equal(m, oracle.kmean(k[:, :, :n_fill]))
    assert not np.array_equal(m, oracle.kmean(k))
    for b, h, t in [(0, 0, 26), (1, 1, 39), (0, 1, 30), (1, 0, 3)]:
        s_k, c_k = exact_quant_row(k[b, h, t].astype(np.float32) - m[b, h])
        assert Fraction(float(sk[b, h, t])) == s_k and list(k8[b, h, t]) == c_k
        s_v, c_v = exact_quant_row(v[b, h, t].astype(np.float32), bits=oracle.V_SCALE_BITS)
        assert Fraction(float(sv[b, h, t])) == s_v and list(v8[b, h, t]) == c_v
    assert np.array_equal(k8[:, :, 30], k8[:, :, 7]) and np.array_equal(sk[:, :, 30], sk[:, :, 7])
    assert np.array_equal(v8[:, :, 30], v8[:, :, 7]) and np.array_equal(sv[:, :, 30], sv[:, :, 7])


@pytest.mark.parametrize("v_format", ["int8", "fp16"])
def test_cache_decode_equals_library_attention_on_each_prefix(v_format):
    w = workloads.dense(61, 3, 8, 2, 70, 64, False, k_offset=1.5)
    q1 = w.q[:, :, 9]
    n_fill, lens = 33, np.array([70, 1, 48])
    out = oracle.attn_int8_decode_cache(q1, w.k, w.v, n_fill, lens, v_format=v_format)
    q8, sq = oracle.quant_rows(q1.astype(np.float32))
    k8, sk, v8, sv, _ = oracle.kvcache_quantize(w.k, w.v, n_fill, v_format)
    qh = dequant(q8, sq)[:, :, None]
    kh = np.repeat(dequant(k8, sk), 4, axis=1)
    vh = np.repeat(dequant(v8, sv) if v_format == "int8" else w.v.astype(np.float64), 4, axis=1)
    for b, n in enumerate(lens):
        ref = sdpa64(qh[b:b + 1], kh[b:b + 1, :, :n], vh[b:b + 1, :, :n], False,
                     oracle.default_softmax_scale(64))[0, :, 0]
        np.testing.assert_allclose(out[b], ref, rtol=1e-11, atol=1e-12)
    # one cached token: softmax weight 1, the output is that token's value row
    np.testing.assert_array_equal(out[1], np.repeat(vh[1, ::4, 0], 4, axis=0))


def test_cache_decode_full_fill_equals_decode_and_empty_rows_are_zero():
    w = workloads.dense(62, 2, 6, 3, 45, 32, False, k_offset=-2.0)
    q1 = w.q[:, :, 0]
    a = oracle.attn_int8_decode_cache(q1, w.k, w.v, 45, [45, 45])
    np.testing.assert_allclose(a, oracle.attn_int8_decode(q1, w.k, w.v), rtol=1e-13, atol=1e-15)
    z = oracle.attn_int8_decode_cache(q1, w.k, w.v, 45, [0, 45])
    assert not z[0].any() and np.array_equal(z[1], a[1])


def test_cache_decode_mean_choice_stays_within_quantization_error():
    # Exact attention does not depend on which per-channel vector is subtracted from K;
    # the stored mean (here of a third of the tokens, or of all of them) only moves the
    # int8 rounding, so both stay within the quantization error of exact attention.
    w = workloads.dense(63, 2, 4, 2, 96, 128, False, k_offset=3.0)
    q1 = w.q[:, :, 4]
    lens = np.array([96, 80])
    exact = np.stack([oracle.attn_exact(q1[b:b + 1, :, None], w.k[b:b + 1, :, :n],
                                        w.v[b:b + 1, :, :n], False)[0, :, 0]
                      for b, n in enumerate(lens)])
    for n_fill in (32, 96):
        out = oracle.attn_int8_decode_cache(q1, w.k, w.v, n_fill, lens)
        rel = np.linalg.norm(out - exact) / np.linalg.norm(exact)
        assert rel < 2e-2, (n_fill, rel)



# ---------------------------------------------------------------- Hadamard rotation (R13)

def test_fwht_butterfly_order_worked_example():
    case = json.load(open(os.path.join(GOLDEN, "fwht_order_worked.json")))
    x = np.array(case["x"], dtype=np.float32)
    got = oracle.fwht_f32(x)
    assert got.dtype == np.float32
    assert got.tolist() == case["fp32_result"]
    assert (x.astype(np.float64) @ sla.hadamard(4)).tolist() == case["exact_result"]


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_fwht_equals_library_hadamard_on_integers(D):
    # Integer rows: every fp32 partial sum is exact, so the transform equals the
    # product with the library's Sylvester-Hadamard matrix exactly, and applying it
    # twice gives D times the row (H H = D I).
    x = rng(60 + D).integers(-2000, 2000, (5, 3, D)).astype(np.float32)
    y = oracle.fwht_f32(x)
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) @ sla.hadamard(D))
    assert np.array_equal(oracle.fwht_f32(y).astype(np.float64), D * x.astype(np.float64))


@pytest.mark.parametrize("causal", [True, False])
def test_hadamard_forward_equals_library_attention_on_rotated_operands(causal):
    # The rotated forward is plain attention on the dequantized rotated Q and K rows
    # (each scaled by 1/sqrt(D), which makes H orthonormal) and the dequantized V.
    w = workloads.dense(61, 1, 4, 2, 70, 64, causal, k_offset=2.0)
    D = 64
    out = oracle.attn_int8_fwd(w.q, w.k, w.v, causal, hadamard=True)
    z = oracle.quantize_qkv(w.q, w.k, w.v, hadamard=True)
    qh = dequant(z["q8"], z["sq"]) / np.sqrt(D)
    kh = np.repeat(dequant(z["k8"], z["sk"]), 2, axis=1) / np.sqrt(D)
    vh = np.repeat(dequant(z["v8"], z["sv"]), 2, axis=1)
    ref = sdpa64(qh, kh, vh, causal, oracle.default_softmax_scale(D))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_hadamard_rows_are_rotations_of_the_smoothed_rows():
    # The quantized rotated K rows approximate (k - mean) H to within half a code step
    # per element, and the rotation preserves row norms up to the factor sqrt(D).
    w = workloads.dense(62, 1, 2, 1, 40, 128, False, k_offset=3.0)
    z = oracle.quantize_qkv(w.q, w.k, w.v, hadamard=True)
    ksm = w.k.astype(np.float64) - z["kmean"][..., None, :].astype(np.float64)
    rot = ksm @ sla.hadamard(128)
    deq = dequant(z["k8"], z["sk"])
    assert np.all(np.abs(deq - rot) <= 0.5 * z["sk"][..., None] * (1 + 1e-5) + 1e-3)
    np.testing.assert_allclose(np.linalg.norm(rot, axis=-1),
                               np.sqrt(128) * np.linalg.norm(ksm, axis=-1), rtol=1e-12)


def test_hadamard_improves_quantization_on_outlier_channels():
    # The point of the rotation: with a few channels x20 in Q and K, rotated rows
    # quantize with far less error; measured against unquantized attention.
    w = workloads.dense(63, 1, 4, 4, 256, 64, False, outlier_frac=0.03)
    exact = oracle.attn_exact(w.q, w.k, w.v, False)

    def sqnr(o):
        return 10 * np.log10(np.sum(exact ** 2) / np.sum((o - exact) ** 2))
    plain = sqnr(oracle.attn_int8_fwd(w.q, w.k, w.v, False))
    rot = sqnr(oracle.attn_int8_fwd(w.q, w.k, w.v, False, hadamard=True))
    assert rot > plain + 3.0, (plain, rot)


# ---------------------------------------------------------------- V per channel (R14)

def test_v_per_channel_worked_example():
    case = json.load(open(os.path.join(GOLDEN, "v_per_channel_worked.json")))
    codes, scales = oracle.quant_cols(np.array(case["v"], dtype=np.float32))
    assert codes.tolist() == case["codes"]
    assert (scales * np.float32(1024)).tolist() == case["scales_times_1024"]


@pytest.mark.parametrize("causal", [True, False])
def test_v_per_channel_forward_equals_library_attention(causal):
    w = workloads.dense(64, 2, 4, 2, 90, 64, causal, k_offset=1.0)
    out = oracle.attn_int8_fwd(w.q, w.k, w.v, causal, v_per_channel=True)
    z = oracle.quantize_qkv(w.q, w.k, w.v, v_per_channel=True)
    assert z["sv"].shape == (2, 2, 64)
    qh = dequant(z["q8"], z["sq"])
    kh = np.repeat(dequant(z["k8"], z["sk"]), 2, axis=1)
    vh = np.repeat(z["v8"].astype(np.float64) * z["sv"][..., None, :].astype(np.float64), 2,
                   axis=1)
    ref = sdpa64(qh, kh, vh, causal, oracle.default_softmax_scale(64))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_v_per_channel_scaling_a_channel_by_two_scales_its_output_exactly():
    # Per-channel scales absorb a power-of-two gain of one V channel exactly (same
    # codes, doubled scale), so that output channel doubles and the others are
    # untouched; per-token scales do not have this property.
    w = workloads.dense(65, 1, 2, 1, 50, 32, True)
    v2 = w.v.copy()
    v2[..., 5] *= np.float16(2.0)
    a = oracle.attn_int8_fwd(w.q, w.k, w.v, True, v_per_channel=True)
    b = oracle.attn_int8_fwd(w.q, w.k, v2, True, v_per_channel=True)
    assert np.array_equal(b[..., 5], 2.0 * a[..., 5])
    keep = [d for d in range(32) if d != 5]
    assert np.array_equal(b[..., keep], a[..., keep])
    a_t = oracle.attn_int8_fwd(w.q, w.k, w.v, True)
    b_t = oracle.attn_int8_fwd(w.q, w.k, v2, True)
    assert not np.array_equal(b_t[..., keep], a_t[..., keep])


def test_v_per_channel_varlen_scales_per_sequence():
    # Each sequence of a packed batch gets its own channel scales: the packed result
    # equals the dense result of every sequence alone.
    w = workloads.varlen(66, 3, 40, 4, 2, 32, True, lengths=[17, 1, 40])
    out = oracle.attn_int8_varlen_fwd(w.q, w.k, w.v, w.cu_seqlens, True, v_per_channel=True)
    for i in range(3):
        a, b = int(w.cu_seqlens[i]), int(w.cu_seqlens[i + 1])
        tr = lambda x: np.ascontiguousarray(x[a:b].transpose(1, 0, 2))[None]
        ref = oracle.attn_int8_fwd(tr(w.q), tr(w.k), tr(w.v), True, v_per_channel=True)[0]
        assert np.array_equal(out[a:b], ref.transpose(1, 0, 2))


# ---------------------------------------------------------------- backward (R17)

def _autograd_grads(w, do, causal, scale=None):
    # torch's CPU fp64 autograd through its own attention (library routine)
    q = torch.tensor(w.q, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(w.k, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(w.v, dtype=torch.float64, requires_grad=True)
    G = q.shape[1] // k.shape[1]
    s = float(oracle.default_softmax_scale(q.shape[-1])) if scale is None else float(np.float32(scale))
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1), is_causal=causal, scale=s)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv,S,D", [(2, 2, 17, 32), (4, 2, 40, 64), (3, 1, 9, 16)])
def test_bwd_equals_torch_autograd(Hq, Hkv, S, D, causal):
    w = workloads.dense(67 + S, 2, Hq, Hkv, S, D, causal, k_offset=1.0)
    do = rng(68).standard_normal(w.q.shape).astype(np.float16)
    got = oracle.attn_bwd_exact(w.q, w.k, w.v, do, causal)
    want = _autograd_grads(w, do, causal)
    for g, r in zip(got, want):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)


def test_bwd_finite_differences():
    # Gradient check: the directional derivative of <dO, O(q, k, v)> along a random
    # direction equals <grad, direction>, by central differences in fp64.
    w = workloads.dense(69, 1, 2, 1, 12, 16, True)
    do = rng(70).standard_normal(w.q.shape)
    q, k, v = (x.astype(np.float64) for x in (w.q, w.k, w.v))
    dq, dk, dv = oracle.attn_bwd_exact(w.q, w.k, w.v, do, True)
    s = float(oracle.default_softmax_scale(16))

    def loss(qq, kk, vv):
        out = 0.0
        for h in range(2):
            lg = s * qq[0, h] @ kk[0, 0].T
            lg = np.where(np.tril(np.ones((12, 12), bool)), lg, -np.inf)
            p = np.exp(lg - lg.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            out += np.sum(do[0, h] * (p @ vv[0, 0]))
        return out
    g = rng(71)
    eq, ek, ev = (g.standard_normal(x.shape) for x in (q, k, v))
    eps = 1e-6
    fd = (loss(q + eps * eq, k + eps * ek, v + eps * ev)
          - loss(q - eps * eq, k - eps * ek, v - eps * ev)) / (2 * eps)
    an = np.sum(dq * eq) + np.sum(dk * ek) + np.sum(dv * ev)
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_bwd_uniform_attention_closed_form():
    # q = 0: every row attends uniformly (non-causal, P_ij = 1/S), so dV_j is the mean
    # of the dO rows, dK_j = s * sum_i dS_ij q_i = 0, and
    # dQ_i = s * sum_j (dP_ij - mean_j dP_ij) k_j / S with dP = dO V^T.
    w = workloads.dense(72, 1, 1, 1, 10, 8, False)
    q = np.zeros_like(w.q)
    do = rng(73).standard_normal(w.q.shape).astype(np.float16)
    dq, dk, dv = oracle.attn_bwd_exact(q, w.k, w.v, do, False)
    np.testing.assert_allclose(dv[0, 0], np.repeat(do[0, 0].astype(np.float64).sum(0, keepdims=True) / 10, 10, 0),
                               rtol=1e-13, atol=1e-14)
    assert np.all(np.abs(dk) < 1e-15)
    vv, kk, dd = w.v[0, 0].astype(np.float64), w.k[0, 0].astype(np.float64), do[0, 0].astype(np.float64)
    dp = dd @ vv.T
    dsc = (dp - dp.mean(1, keepdims=True)) / 10
    np.testing.assert_allclose(dq[0, 0], float(oracle.default_softmax_scale(8)) * dsc @ kk,
                               rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- R18 Q per block

def test_q_per_block_scale_is_the_blocks_largest_row_scale():
    # One scale per 32 rows: exactly the largest of the per-row scales of the block (a
    # max of |x| / 127 is the max of the rows' values), ragged last block included.
    x = np.random.default_rng(31).standard_normal((2, 3, 70, 16)).astype(np.float32)
    x[0, 1, 40] *= 50.0  # one outlier row in the second block
    c, s = oracle.quant_row_blocks(x)
    _, sr = oracle.quant_rows(x)
    for b0 in range(0, 70, 32):
        blk = sr[..., b0:b0 + 32]
        assert np.array_equal(s[..., b0:b0 + 32],
                              np.broadcast_to(blk.max(axis=-1, keepdims=True), blk.shape))
    assert s[0, 1, 40] == sr[0, 1, 40] and s[0, 1, 63] == sr[0, 1, 40]


def test_q_per_block_row_with_the_block_max_keeps_its_row_codes():
    # The row that holds a block's maximum is quantized against its own row scale, so
    # its codes equal the per-row codes; other rows of the block have coarser codes
    # (never larger in magnitude than their per-row codes).
    x = np.random.default_rng(32).standard_normal((4, 64, 32)).astype(np.float32)
    c, s = oracle.quant_row_blocks(x)
    cr, sr = oracle.quant_rows(x)
    for h in range(4):
        for b0 in (0, 32):
            r = b0 + int(np.argmax(sr[h, b0:b0 + 32]))
            assert np.array_equal(c[h, r], cr[h, r])
            assert np.all(np.abs(c[h, b0:b0 + 32].astype(int)) <= np.abs(cr[h, b0:b0 + 32].astype(int)))


def test_q_per_block_forward_equals_sdpa_on_its_dequantized_operands():
    # The forward with per-block Q is attention on the dequantized operands of that
    # quantization (torch's fp64 SDPA), causal GQA with a ragged tail.
    import torch
    w = workloads.dense(33, 1, 4, 2, 70, 32, True, k_offset=1.0)
    got = oracle.attn_int8_fwd(w.q, w.k, w.v, True, q_per_block=True)
    z = oracle.quantize_qkv(w.q, w.k, w.v, q_per_block=True)
    qd = torch.from_numpy(z["q8"].astype(np.float64) * z["sq"][..., None])
    kd = torch.from_numpy(z["k8"].astype(np.float64) * z["sk"][..., None])
    vd = torch.from_numpy(z["v8"].astype(np.float64) * z["sv"][..., None])
    kd = kd.repeat_interleave(2, dim=1)
    vd = vd.repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qd, kd, vd, is_causal=True, scale=float(np.float32(1 / np.sqrt(32)))).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-12)


def exact_block_codes(rows, scale):
    """Codes of fp32 rows against a given scale with rational arithmetic (R3)."""
    return [[max(-127, min(127, round(rn32(Fraction(float(x)) / scale)))) for x in r]
            for r in rows]


def test_q_per_block_hand_derived_case():
    # tests/golden/q_per_block_worked.json: blocks of 2 rows, a ragged last block; the
    # non-maximal row of block 0 is quantized against the block's scale.
    g = json.load(open(os.path.join(GOLDEN, "q_per_block_worked.json")))
    x = np.array(g["rows"], dtype=np.float32)
    c, s = oracle.quant_row_blocks(x, block=g["block"])
    for b in g["blocks"]:
        want_s = Fraction(b["scale_num"], b["scale_den"])
        for r, want_c in zip(b["rows"], b["codes"]):
            assert Fraction(float(s[r])) == want_s
            assert c[r].tolist() == want_c


def test_q_per_block_every_row_follows_the_rational_rule_at_the_block_scale():
    # Every code of every row: rint(fp32(x / s_b)) clamped, with s_b = fp32(absmax of
    # the block / 127) in exact arithmetic -- the rows that do not hold the block's
    # maximum included, ragged last block (70 = 32 + 32 + 6 rows) included.
    g = np.random.default_rng(34)
    x = (g.standard_normal((2, 70, 16)) * np.exp(g.standard_normal((2, 70, 1)))).astype(np.float16)
    x = x.astype(np.float32)
    x[1, 45] *= 40.0  # one dominant row in the second block
    c, s = oracle.quant_row_blocks(x)
    for h in range(2):
        for b0 in range(0, 70, 32):
            rows = x[h, b0:b0 + 32]
            a = max(abs(Fraction(float(v))) for v in rows.ravel())
            sb = rn32(a / 127)
            assert all(Fraction(float(v)) == sb for v in s[h, b0:b0 + 32])
            assert c[h, b0:b0 + 32].tolist() == exact_block_codes(rows, sb)


def test_q_per_block_varlen_blocks_start_at_each_sequence():
    # In a packed batch the 32-row blocks are counted from each sequence's first token
    # (sequences at rows 0 and 40 here): the varlen forward equals torch's fp64 SDPA on
    # operands dequantized with exact block scales per sequence.
    w = workloads.varlen(35, 2, 80, 2, 1, 16, True, lengths=[40, 50])
    cu = w.cu_seqlens
    got = oracle.attn_int8_varlen_fwd(w.q, w.k, w.v, cu, True, q_per_block=True)
    sm = float(oracle.default_softmax_scale(16))
    for i in range(2):
        a, b = int(cu[i]), int(cu[i + 1])
        z = oracle.quantize_qkv(np.ascontiguousarray(w.q[a:b].transpose(1, 0, 2))[None],
                                np.ascontiguousarray(w.k[a:b].transpose(1, 0, 2))[None],
                                np.ascontiguousarray(w.v[a:b].transpose(1, 0, 2))[None])
        qd = np.empty((2, b - a, 16))
        for h in range(2):
            q32 = w.q[a:b, h].astype(np.float32)
            for b0 in range(0, b - a, 32):
                rows = q32[b0:b0 + 32]
                sb = rn32(max(abs(Fraction(float(v))) for v in rows.ravel()) / 127)
                qd[h, b0:b0 + 32] = np.array(exact_block_codes(rows, sb), dtype=np.float64) * float(sb)
        kd = dequant(z["k8"][0], z["sk"][0]).repeat(2, axis=0)
        vd = dequant(z["v8"][0], z["sv"][0]).repeat(2, axis=0)
        ref = sdpa64(qd, kd, vd, True, sm)
        np.testing.assert_allclose(got[a:b].transpose(1, 0, 2), ref, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- Q outlier detection (R19)

def test_q_outlier_detection_hand_derived_cases():
    # tests/golden/q_outliers_worked.json: the threshold is strict (a peak of exactly 6
    # is not an outlier), the peak is taken over every head of the group and every
    # token, and past 16 candidates the largest peaks win with ties to the lower channel.
    g = json.load(open(os.path.join(GOLDEN, "q_outliers_worked.json")))
    for case in g["detect_cases"]:
        q = np.array(case["q"], dtype=np.float16)
        assert oracle.q_outlier_channels(q).tolist() == case["channels"], case["what"]
    rc = g["row_case"]
    q = np.zeros((1, 1, 1, 4), dtype=np.float16)
    q[0, 0, 0] = rc["row"]
    kv = np.ones((1, 1, 1, 4), dtype=np.float16)
    z = oracle.quantize_qkv(q, kv, kv, q_outliers=True)
    assert z["ochan"][0, 0][z["ochan"][0, 0] >= 0].tolist() == rc["outliers"]
    assert Fraction(float(z["sq"][0, 0, 0])) == Fraction(rc["scale_num"], rc["scale_den"])
    assert z["q8"][0, 0, 0].tolist() == rc["codes"]
    assert z["qo"][0, 0, 0, :1].tolist() == [-10.0]


def _outlier_inputs(seed, B=1, Hq=4, Hkv=2, S=96, D=32, chans=(3, 17), gain=20.0):
    g = rng(seed)
    q = g.standard_normal((B, Hq, S, D)).astype(np.float32)
    k = g.standard_normal((B, Hkv, S, D)).astype(np.float32) + g.uniform(-2, 2, (1, Hkv, 1, D)).astype(np.float32)
    v = g.standard_normal((B, Hkv, S, D)).astype(np.float32)
    q[..., list(chans)] *= gain
    k[..., list(chans)] *= gain
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


def test_q_outliers_without_outliers_reduce_to_the_plain_rows():
    # No |q| above the threshold: nothing is detected and every code, scale and output
    # is the plain per-row (and per-block) quantization's.
    g = rng(81)
    q = np.clip(g.standard_normal((1, 4, 70, 32)), -5.9, 5.9).astype(np.float16)
    k = g.standard_normal((1, 2, 70, 32)).astype(np.float16)
    v = g.standard_normal((1, 2, 70, 32)).astype(np.float16)
    for blk in (False, True):
        a = oracle.quantize_qkv(q, k, v, q_per_block=blk)
        b = oracle.quantize_qkv(q, k, v, q_per_block=blk, q_outliers=True)
        assert (b["ochan"] == -1).all()
        for key in ("q8", "sq", "k8", "sk", "v8", "sv"):
            assert np.array_equal(a[key], b[key]), key
        o1 = oracle.attn_int8_fwd(q, k, v, True, q_per_block=blk)
        o2 = oracle.attn_int8_fwd(q, k, v, True, q_per_block=blk, q_outliers=True)
        assert np.array_equal(o1, o2)


@pytest.mark.parametrize("blk", [False, True])
def test_q_outliers_int8_part_follows_the_rational_rule(blk):
    # Every Q and K row of the int8 part: the outlier channels hold code 0 and the row
    # (or 32-row block) scale and codes are the exact rational rule applied to the row
    # with those channels set to zero.
    q, k, v = _outlier_inputs(82, S=70)
    z = oracle.quantize_qkv(q, k, v, q_per_block=blk, q_outliers=True)
    ksm = k.astype(np.float32) - z["kmean"][..., None, :]
    for g in range(2):
        ch = z["ochan"][0, g][z["ochan"][0, g] >= 0]
        assert ch.tolist() == [3, 17]
        for t in range(70):
            row = ksm[0, g, t].copy()
            row[ch] = 0
            s, c = exact_quant_row(row)
            assert Fraction(float(z["sk"][0, g, t])) == s
            assert z["k8"][0, g, t].tolist() == c
        for h in (2 * g, 2 * g + 1):
            x = q[0, h].astype(np.float32)
            x[:, ch] = 0
            for b0 in range(0, 70, 32 if blk else 1):
                rows = x[b0:b0 + (32 if blk else 1)]
                sb = rn32(max(abs(Fraction(float(e))) for e in rows.ravel()) / 127)
                n = rows.shape[0]
                assert all(Fraction(float(e)) == sb for e in z["sq"][0, h, b0:b0 + n])
                assert z["q8"][0, h, b0:b0 + n].tolist() == exact_block_codes(rows, sb)
                assert (z["q8"][0, h, b0:b0 + n][:, ch] == 0).all()


@pytest.mark.parametrize("causal", [True, False])
def test_q_outliers_forward_equals_sdpa_on_the_decomposed_operands(causal):
    # The logits are the int8 part dequantized plus the exact products of the outlier
    # channels: torch's fp64 attention on Q^ = sq*q8 (zeros on the outlier channels)
    # plus q on them, and K^ = sk*k8 plus k on them, must give the oracle's output.
    q, k, v = _outlier_inputs(83, S=80)
    z = oracle.quantize_qkv(q, k, v, q_outliers=True)
    qd = dequant(z["q8"], z["sq"])
    kd = dequant(z["k8"], z["sk"])
    for g in range(2):
        ch = z["ochan"][0, g][z["ochan"][0, g] >= 0]
        qd[0, 2 * g:2 * g + 2][..., ch] = q[0, 2 * g:2 * g + 2][..., ch].astype(np.float64)
        kd[0, g][..., ch] = k[0, g][..., ch].astype(np.float64)
    vd = dequant(z["v8"], z["sv"])
    ref = sdpa64(qd, kd.repeat(2, axis=1), vd.repeat(2, axis=1), causal,
                 oracle.default_softmax_scale(32))
    got = oracle.attn_int8_fwd(q, k, v, causal, q_outliers=True)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-12)


def test_q_outliers_are_detected_per_kv_group():
    # A large value in one query head marks that channel for the whole group (the
    # other head's int8 part loses it too), and not for the other group.
    g = rng(84)
    q = g.standard_normal((1, 4, 40, 16)).astype(np.float16)
    k = g.standard_normal((1, 2, 40, 16)).astype(np.float16)
    q = np.clip(q, -5, 5)
    q[0, 1, 7, 9] = 30.0  # head 1 is in group 0
    z = oracle.quantize_qkv(q, k, k, q_outliers=True)
    assert z["ochan"][0, 0].tolist() == [9] + [-1] * 15
    assert (z["ochan"][0, 1] == -1).all()
    assert (z["q8"][0, 0][:, 9] == 0).all() and (z["q8"][0, 1][:, 9] == 0).all()
    assert (z["k8"][0, 0][:, 9] == 0).all() and (z["k8"][0, 1][:, 9] != 0).any()


def test_q_outliers_varlen_sets_are_per_sequence():
    # A sequence without outliers is attended exactly as the plain forward attends it,
    # whatever the other sequences of the batch hold.
    w = workloads.varlen(85, 2, 60, 2, 1, 16, True, lengths=[50, 60])
    q = np.clip(w.q, -5, 5)
    q[10, 0, 4] = 25.0  # sequence 0 only
    cu = w.cu_seqlens
    got = oracle.attn_int8_varlen_fwd(q, w.k, w.v, cu, True, q_outliers=True)
    plain = oracle.attn_int8_varlen_fwd(q, w.k, w.v, cu, True)
    assert np.array_equal(got[50:], plain[50:])
    assert not np.array_equal(got[:50], plain[:50])


def test_q_outliers_recover_quantization_quality_on_outlier_channels():
    # The point of the detection: with 1 % of the channels x20 in Q and K, against
    # unquantized attention, per-row and per-block Q both gain more than 8 dB.
    w = workloads.dense(86, 1, 4, 4, 256, 128, False, outlier_frac=0.01)
    exact = oracle.attn_exact(w.q, w.k, w.v, False)

    def sqnr(o):
        return 10 * np.log10(np.sum(exact ** 2) / np.sum((o - exact) ** 2))
    for blk in (False, True):
        plain = sqnr(oracle.attn_int8_fwd(w.q, w.k, w.v, False, q_per_block=blk))
        det = sqnr(oracle.attn_int8_fwd(w.q, w.k, w.v, False, q_per_block=blk, q_outliers=True))
        assert det > plain + 8.0, (blk, plain, det)
