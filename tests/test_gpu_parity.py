"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer and byte results (K mean, codes, scales, int32 scores) must be bit-exact.
The fp16 output must satisfy max|o - O| <= 2e-3 and ||o - O||_2 / ||O||_2 <= 1e-3
over each compared set, with O the unrounded fp64 oracle.  Every input is seeded
and synthetic (int8_w8a8_flashattention_amd.workloads).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import int8_w8a8_flashattention_amd as i8
from int8_w8a8_flashattention_amd import workloads

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
REL_L2 = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_close(o16, ref, what):
    o = o16.astype(np.float64)
    err = np.abs(o - ref)
    mx = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(o - ref) / max(np.linalg.norm(ref), 1e-30))
    floor = float(np.abs(ref.astype(np.float16).astype(np.float64) - ref).max()) if ref.size else 0.0
    say(f"  {what}: max_abs={mx:.3e} rel_l2={rel:.3e} (fp16 floor {floor:.3e})")
    assert np.all(np.isfinite(o)), what
    assert mx <= MAX_ABS, (what, mx)
    assert rel <= REL_L2, (what, rel)


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ------------------------------------------------------------------ quantizer

@pytest.mark.parametrize("bits", [i8.SCALE_FP32, i8.SCALE_V4])
@pytest.mark.parametrize("d", [8, 32, 96, 128, 256, 512])
def test_quant_rowwise_bit_exact(bits, d):
    say(f"quant_rowwise d={d} bits={bits}")
    g = rng(1000 + d + bits)
    x = (g.standard_normal((333, d)) * np.exp(g.uniform(-8, 8, (333, 1)))).astype(np.float16)
    x[3] = 0
    x[4, :] = np.float16(1e-7)
    x[5, 0] = np.float16(60000.0)
    codes, scales = i8.quant_rowwise_i8(dev(x), scale_bits=bits)
    c_ref, s_ref = oracle.quant_rows(x.astype(np.float32), bits)
    assert np.array_equal(host(scales), s_ref)
    assert np.array_equal(host(codes), c_ref)


def test_quant_rowwise_with_mean_bit_exact():
    say("quant_rowwise with group means")
    g = rng(77)
    rows, d, rpg = 200, 128, 7
    x = g.standard_normal((rows, d)).astype(np.float16)
    mean = g.uniform(-3, 3, ((rows + rpg - 1) // rpg, d)).astype(np.float32)
    codes, scales = i8.quant_rowwise_i8(dev(x), dev(mean), rpg)
    xs = x.astype(np.float32) - np.repeat(mean, rpg, axis=0)[:rows]
    c_ref, s_ref = oracle.quant_rows(xs)
    assert np.array_equal(host(scales), s_ref)
    assert np.array_equal(host(codes), c_ref)


# ------------------------------------------------------------------ debug score dump

def _debug_case(w, b, h, row0, rows, col0, cols, z):
    r = i8.attn_int8_debug_qk(dev(w.q), dev(w.k), dev(w.v), b, h, row0, rows, col0, cols)
    G = w.q.shape[1] // w.k.shape[1]
    gk = h // G
    s_ref = oracle.qk_int32(z["q8"][b, h], z["k8"][b, gk])[row0:row0 + rows, col0:col0 + cols]
    assert np.array_equal(host(r["s32"]).astype(np.int64), s_ref), (b, h, row0, col0)
    assert np.array_equal(host(r["qscale"]), z["sq"][b, h, row0:row0 + rows])
    assert np.array_equal(host(r["kscale"]), z["sk"][b, gk, col0:col0 + cols])
    assert np.array_equal(host(r["vscale"]), z["sv"][b, gk, col0:col0 + cols])
    assert np.array_equal(host(r["kmean"]), z["kmean"][b, gk])


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_debug_scores_bit_exact(D):
    say(f"debug scores D={D}")
    w = workloads.dense(40 + D, 2, 4, 2, 300, D, True, k_offset=3.0, outlier_frac=0.02)
    z = oracle.quantize_qkv(w.q, w.k, w.v)
    S = 300
    for (b, h, r0, nr, c0, nc) in [(0, 0, 0, 64, 0, 64),        # first tiles
                                   (1, 3, 100, 37, 90, 50),     # around the diagonal
                                   (1, 2, 236, 64, 236, 64),    # last tiles, ragged tail
                                   (0, 1, 0, S, 0, S)]:         # everything
        _debug_case(w, b, h, r0, nr, c0, nc, z)


def test_debug_scores_cfg1_and_extremes():
    say("debug scores cfg1 + extreme codes")
    w = workloads.cfg1()
    z = oracle.quantize_qkv(w.q, w.k, w.v)
    _debug_case(w, 0, 1, 0, 128, 0, 128, z)
    # rows whose codes saturate at +-127 everywhere (largest |S32| = 127^2 * 256)
    q = np.ones((1, 1, 64, 256), np.float16)
    k = np.ones((1, 1, 64, 256), np.float16)
    k[0, 0, ::2] = -1  # mean 0 per channel, rows alternate +-1
    wx = workloads.Dense(q, k, q.copy(), False)
    _debug_case(wx, 0, 0, 0, 64, 0, 64, oracle.quantize_qkv(q, k, q.copy()))


# ------------------------------------------------------------------ forward, small shapes

SMALL = [
    # B, Hq, Hkv, S, D
    (2, 4, 2, 300, 32),
    (2, 4, 2, 300, 64),
    (2, 4, 2, 300, 128),
    (1, 2, 1, 300, 256),
    (1, 3, 1, 517, 128),   # MQA, ragged
    (1, 2, 2, 64, 64),     # exactly one tile
    (1, 2, 1, 1, 128),     # a single token
    (1, 2, 1, 65, 32),     # one tile plus one
    (3, 8, 8, 129, 128),   # MHA, one block plus one
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_forward_small_shapes(shape, causal):
    B, Hq, Hkv, S, D = shape
    say(f"forward {shape} causal={causal}")
    w = workloads.dense(sum(shape) + causal, B, Hq, Hkv, S, D, causal, k_offset=2.0)
    o = host(i8.attn_int8_fwd(dev(w.q), dev(w.k), dev(w.v), causal))
    ref = oracle.attn_int8_fwd(w.q, w.k, w.v, causal)
    check_close(o, ref, f"{shape} causal={causal}")


def test_forward_softmax_scale_argument():
    say("forward with a non-default softmax scale")
    w = workloads.dense(55, 1, 4, 2, 200, 64, True)
    o = host(i8.attn_int8_fwd(dev(w.q), dev(w.k), dev(w.v), True, softmax_scale=0.3))
    ref = oracle.attn_int8_fwd(w.q, w.k, w.v, True, softmax_scale=0.3)
    check_close(o, ref, "scale 0.3")


def _special_rows(vgain):
    g = rng(56)
    B, H, S, D = 1, 2, 150, 128
    q = g.standard_normal((B, H, S, D)).astype(np.float16)
    q[0, 0, :40] = 0  # zero rows: uniform attention over the prefix
    k = g.standard_normal((B, H, S, D)).astype(np.float16)
    q[0, 1] = (q[0, 1].astype(np.float32) * 30).astype(np.float16)  # near one-hot rows
    v = (g.standard_normal((B, H, S, D)) * vgain).astype(np.float16)
    return q, k, v


def test_forward_zero_rows_and_one_hot():
    say("forward with zero queries and one-hot rows")
    q, k, v = _special_rows(1.0)
    for causal in (True, False):
        o = host(i8.attn_int8_fwd(dev(q), dev(k), dev(v), causal))
        check_close(o, oracle.attn_int8_fwd(q, k, v, causal), f"special rows causal={causal}")


def test_forward_large_outputs_within_fp16_floor():
    """Outputs of magnitude >= 4 sit on an fp16 grid coarser than 2 * 2e-3, so no
    fp16 result can meet max-abs 2e-3 there; the bound is the oracle's own fp16
    rounding error of that element plus 2e-3."""
    say("forward with |O| up to ~12")
    q, k, v = _special_rows(3.0)
    for causal in (True, False):
        o = host(i8.attn_int8_fwd(dev(q), dev(k), dev(v), causal)).astype(np.float64)
        ref = oracle.attn_int8_fwd(q, k, v, causal)
        floor = np.abs(ref.astype(np.float16).astype(np.float64) - ref)
        excess = np.abs(o - ref) - floor
        say(f"  large |O| causal={causal}: max |O|={np.abs(ref).max():.2f} "
            f"max excess over fp16 floor={excess.max():.3e}")
        assert np.all(np.isfinite(o))
        assert excess.max() <= MAX_ABS
        assert np.linalg.norm(o - ref) / np.linalg.norm(ref) <= REL_L2


def test_cfg1_tiny_causal_gqa():
    say("cfg1")
    w = workloads.cfg1()
    o = host(i8.attn_int8_fwd(dev(w.q), dev(w.k), dev(w.v), True))
    check_close(o, oracle.attn_int8_fwd(w.q, w.k, w.v, True), "cfg1")


# ------------------------------------------------------------------ identities on the GPU

def test_deterministic_and_gqa_equals_repeated_heads():
    say("determinism + GQA identity")
    w = workloads.dense(60, 1, 8, 2, 700, 128, True, k_offset=1.0)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    a = host(i8.attn_int8_fwd(q, k, v, True))
    b = host(i8.attn_int8_fwd(q, k, v, True))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    kr = dev(np.repeat(w.k, 4, axis=1))
    vr = dev(np.repeat(w.v, 4, axis=1))
    c = host(i8.attn_int8_fwd(q, kr, vr, True))
    assert np.array_equal(a.view(np.uint16), c.view(np.uint16))


def test_prepare_then_prepared_equals_fwd():
    say("prepare_kv + fwd_prepared == fwd")
    w = workloads.dense(63, 2, 6, 3, 333, 128, True, k_offset=1.0)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    a = host(i8.attn_int8_fwd(q, k, v, True))
    ws = i8.attn_int8_prepare_kv(k, v, 6)
    b = host(i8.attn_int8_fwd_prepared(q, 3, ws, True))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_split_phases_equal_fwd_and_reuse_kv():
    say("prepare_kv + prepare_q + attend == fwd; one K/V preparation serves two query batches")
    w = workloads.dense(64, 1, 8, 2, 517, 64, True, k_offset=0.5)
    w2 = workloads.dense(65, 1, 8, 2, 517, 64, True)
    q, k, v, q2 = dev(w.q), dev(w.k), dev(w.v), dev(w2.q)
    a = host(i8.attn_int8_fwd(q, k, v, True))
    a2 = host(i8.attn_int8_fwd(q2, k, v, True))
    ws = i8.attn_int8_prepare_kv(k, v, 8)
    i8.attn_int8_prepare_q(q, 2, ws)
    b = host(i8.attn_int8_attend(ws, 1, 8, 2, 517, 64, True))
    i8.attn_int8_prepare_q(q2, 2, ws)
    b2 = host(i8.attn_int8_attend(ws, 1, 8, 2, 517, 64, True))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(a2.view(np.uint16), b2.view(np.uint16))
    check_close(b2, oracle.attn_int8_fwd(w2.q, w.k, w.v, True), "second query batch")


def test_varlen_equal_lengths_equals_dense():
    say("varlen == dense for equal lengths")
    w = workloads.dense(61, 3, 4, 2, 192, 64, True)
    B, Hq, S, D = w.q.shape
    a = host(i8.attn_int8_fwd(dev(w.q), dev(w.k), dev(w.v), True))
    tq = w.q.transpose(0, 2, 1, 3).reshape(B * S, Hq, D)
    tk = w.k.transpose(0, 2, 1, 3).reshape(B * S, 2, D)
    tv = w.v.transpose(0, 2, 1, 3).reshape(B * S, 2, D)
    cu = np.arange(0, B * S + 1, S, dtype=np.int32)
    b = host(i8.attn_int8_varlen_fwd(dev(tq), dev(tk), dev(tv), dev(cu), S, True))
    a_t = a.transpose(0, 2, 1, 3).reshape(B * S, Hq, D)
    assert np.array_equal(a_t.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_ragged_with_empty_sequences(causal):
    say(f"varlen ragged causal={causal}")
    w = workloads.varlen(62, 6, 300, 4, 2, 128, causal, lengths=[1, 0, 300, 65, 0, 130])
    o = host(i8.attn_int8_varlen_fwd(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens),
                                     w.max_seqlen, causal))
    ref = oracle.attn_int8_varlen_fwd(w.q, w.k, w.v, w.cu_seqlens, causal)
    check_close(o, ref, "ragged varlen")


# ------------------------------------------------------------------ the five workloads

def test_cfg2_causal_gqa_s4096_sampled_heads():
    say("cfg2 (B1 Hq32 Hkv8 S4096 D128 causal), 6 heads, all rows")
    w = workloads.cfg2()
    o = host(i8.attn_int8_fwd(dev(w.q), dev(w.k), dev(w.v), True))
    heads = [(0, 0), (0, 5), (0, 13), (0, 22), (0, 27), (0, 31)]
    ref = oracle.attn_int8_fwd(w.q, w.k, w.v, True, heads=heads)
    got = np.stack([o[b, h] for b, h in heads])
    check_close(got, ref, "cfg2")


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_cfg3_mha_outliers_sampled_heads(D):
    say(f"cfg3 D={D} (B4 H16 S2048 non-causal, outlier channels)")
    w = workloads.cfg3(D)
    o = host(i8.attn_int8_fwd(dev(w.q), dev(w.k), dev(w.v), False))
    heads = [(0, 0), (1, 7), (2, 11), (3, 15)]
    ref = oracle.attn_int8_fwd(w.q, w.k, w.v, False, heads=heads)
    got = np.stack([o[b, h] for b, h in heads])
    check_close(got, ref, f"cfg3 D={D}")


def test_cfg4_varlen_sampled_rows():
    say("cfg4 varlen (16 seqs, L~U[1,4096], Hq64 Hkv8 D128 causal)")
    w = workloads.cfg4()
    o = host(i8.attn_int8_varlen_fwd(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens),
                                     w.max_seqlen, True))
    g = rng(404)
    got, ref = [], []
    for s in range(len(w.cu_seqlens) - 1):
        a, b = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
        L = b - a
        rows = np.unique(np.concatenate([[0, L - 1, min(L - 1, 127), min(L - 1, 128)],
                                         g.integers(0, L, 24)]))
        heads = [(0, int(h)) for h in (0, 63, g.integers(1, 63))]
        qs = np.ascontiguousarray(w.q[a:b].transpose(1, 0, 2))[None]
        ks = np.ascontiguousarray(w.k[a:b].transpose(1, 0, 2))[None]
        vs = np.ascontiguousarray(w.v[a:b].transpose(1, 0, 2))[None]
        ref.append(oracle.attn_int8_fwd(qs, ks, vs, True, heads=heads, rows=rows))
        got.append(np.stack([o[a + rows, h] for _, h in heads]))
    check_close(np.concatenate([x.reshape(-1) for x in got]),
                np.concatenate([x.reshape(-1) for x in ref]), "cfg4")


def test_cfg5_long_context_sampled_rows():
    say("cfg5 (B1 Hq40 Hkv8 S32768 D128 causal, K offset), sampled rows")
    w = workloads.cfg5()
    o = host(i8.attn_int8_fwd(dev(w.q), dev(w.k), dev(w.v), True))
    g = rng(505)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 4095, 16384, 32767],
                                     g.integers(0, 32768, 40)]))
    heads = [(0, 0), (0, 4), (0, 5), (0, 39)]
    ref = oracle.attn_int8_fwd(w.q, w.k, w.v, True, heads=heads, rows=rows)
    got = np.stack([o[0, h][rows] for _, h in heads])
    check_close(got, ref, "cfg5")


# ------------------------------------------------------------------ workspace contents

def nan_workspace(nbytes):
    return torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("flags", [0, i8.FWD_HADAMARD | i8.FWD_V_PER_CHANNEL])
def test_forward_needs_no_workspace_initialization(flags):
    # The workspace is filled with NaN bytes first: every value the kernels read from it
    # (padding slots of the K/V tiles and Q rows included) is written by the same call.
    say(f"forward on a NaN-filled workspace, flags={flags}")
    B, Hq, Hkv, S, D = 2, 4, 2, 300, 64
    w = workloads.dense(63, B, Hq, Hkv, S, D, True, k_offset=1.0)
    ws = nan_workspace(i8.attn_int8_workspace_bytes(B, Hq, Hkv, S, D))
    o = host(i8.attn_int8_fwd_ex(dev(w.q), dev(w.k), dev(w.v), True, flags, workspace=ws))
    ref = oracle.attn_int8_fwd(w.q, w.k, w.v, True, hadamard=bool(flags & i8.FWD_HADAMARD),
                               v_per_channel=bool(flags & i8.FWD_V_PER_CHANNEL))
    check_close(o, ref, f"dense flags={flags}")
    v = workloads.varlen(64, 5, 200, 4, 2, 128, True, lengths=[1, 0, 200, 65, 33])
    T = int(v.cu_seqlens[-1])
    ws = nan_workspace(i8.attn_int8_varlen_workspace_bytes(5, T, 200, 4, 2, 128))
    o = host(i8.attn_int8_varlen_fwd_ex(dev(v.q), dev(v.k), dev(v.v), dev(v.cu_seqlens), 200,
                                        True, flags, workspace=ws))
    ref = oracle.attn_int8_varlen_fwd(v.q, v.k, v.v, v.cu_seqlens, True,
                                      hadamard=bool(flags & i8.FWD_HADAMARD),
                                      v_per_channel=bool(flags & i8.FWD_V_PER_CHANNEL))
    check_close(o, ref, f"varlen flags={flags}")
