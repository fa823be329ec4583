"""GPU parity of the forward's variants against the CPU oracle's: the Hadamard-rotated
Q/K (attn_int8_fwd_hadamard, flag FWD_HADAMARD) and V quantized per channel (flag
FWD_V_PER_CHANNEL), dense and varlen, alone and combined.  The rotated Q and K codes,
their scales and the int32 scores are bit-exact (through the debug dump); the fp16
output is within max-abs 2e-3 and rel-L2 1e-3 of the unrounded fp64 oracle; and on the
outlier-channel workload the rotation improves the SQNR against unquantized attention."""

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
    """max-abs 2e-3 wherever |O| < 4; where |O| >= 4 (an fp16 grid coarser than
    2 * 2e-3, which no fp16 result can meet) 2e-3 over the oracle's own fp16 rounding
    error of that element; rel-L2 1e-3 over all."""
    o = o16.astype(np.float64)
    err = np.abs(o - ref)
    small = np.abs(ref) < 4.0
    mx = float(err[small].max()) if small.any() else 0.0
    floor = np.abs(ref.astype(np.float16).astype(np.float64) - ref)
    ex = float((err - floor)[~small].max()) if (~small).any() else 0.0
    rel = float(np.linalg.norm(o - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"  {what}: max_abs={mx:.3e} (|O| < 4), max excess over the fp16 floor={ex:.3e} "
        f"(|O| >= 4), rel_l2={rel:.3e} (max |O| {np.abs(ref).max():.2f})")
    assert np.all(np.isfinite(o)), what
    assert mx <= MAX_ABS, (what, mx)
    assert ex <= MAX_ABS, (what, ex)
    assert rel <= REL_L2, (what, rel)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_rotated_codes_scales_and_scores_bit_exact(D):
    say(f"rotated debug dump D={D}")
    w = workloads.dense(70 + D, 2, 4, 2, 300, D, True, k_offset=3.0, outlier_frac=0.02)
    z = oracle.quantize_qkv(w.q, w.k, w.v, hadamard=True)
    for (b, h, r0, nr, c0, nc) in [(0, 0, 0, 64, 0, 64), (1, 3, 100, 37, 90, 50),
                                   (1, 2, 0, 300, 0, 300)]:
        r = i8.attn_int8_debug_qk(dev(w.q), dev(w.k), dev(w.v), b, h, r0, nr, c0, nc,
                                  hadamard=True)
        gk = h // 2
        s_ref = oracle.qk_int32(z["q8"][b, h], z["k8"][b, gk])[r0:r0 + nr, c0:c0 + nc]
        assert np.array_equal(host(r["s32"]).astype(np.int64), s_ref), (b, h, r0, c0)
        assert np.array_equal(host(r["qscale"]), z["sq"][b, h, r0:r0 + nr])
        assert np.array_equal(host(r["kscale"]), z["sk"][b, gk, c0:c0 + nc])
        assert np.array_equal(host(r["kmean"]), z["kmean"][b, gk])


SMALL = [(2, 4, 2, 300, 32), (2, 4, 2, 300, 64), (1, 3, 1, 517, 128), (1, 2, 1, 300, 256),
         (1, 2, 1, 1, 128), (3, 8, 8, 129, 64)]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_rotated_forward_small_shapes(shape, causal):
    B, Hq, Hkv, S, D = shape
    say(f"rotated forward {shape} causal={causal}")
    w = workloads.dense(90 + S + D, B, Hq, Hkv, S, D, causal, k_offset=2.0, outlier_frac=0.03)
    out = host(i8.attn_int8_fwd_hadamard(dev(w.q), dev(w.k), dev(w.v), causal))
    check_close(out, oracle.attn_int8_fwd(w.q, w.k, w.v, causal, hadamard=True), f"{shape}")


@pytest.mark.parametrize("D", [64, 128])
def test_rotated_forward_outlier_workload_gains_sqnr(D):
    # cfg3 (B4 H16 S2048 non-causal, 1 % of channels x20): parity on sampled heads, and
    # the rotated output is closer to unquantized attention than the plain one.
    w = workloads.cfg3(D)
    say(f"cfg3 D={D} rotated")
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    rot = host(i8.attn_int8_fwd_hadamard(q, k, v, False))
    plain = host(i8.attn_int8_fwd(q, k, v, False))
    heads = [(0, 0), (2, 11)]
    ref = oracle.attn_int8_fwd(w.q, w.k, w.v, False, heads=heads, hadamard=True)
    check_close(np.stack([rot[b, h] for b, h in heads]), ref, f"cfg3 D={D} rotated")
    exact = oracle.attn_exact(w.q, w.k, w.v, False, heads=heads)

    def sqnr(o):
        got = np.stack([o[b, h] for b, h in heads]).astype(np.float64)
        return 10 * np.log10(np.sum(exact ** 2) / np.sum((got - exact) ** 2))
    s_plain, s_rot = sqnr(plain), sqnr(rot)
    say(f"  SQNR vs exact: plain {s_plain:.2f} dB, rotated {s_rot:.2f} dB")
    assert s_rot > s_plain + 1.0


VARIANTS = [(i8.FWD_V_PER_CHANNEL, dict(v_per_channel=True)),
            (i8.FWD_HADAMARD | i8.FWD_V_PER_CHANNEL, dict(hadamard=True, v_per_channel=True)),
            (i8.FWD_Q_PER_BLOCK, dict(q_per_block=True)),
            (i8.FWD_HADAMARD | i8.FWD_V_PER_CHANNEL | i8.FWD_Q_PER_BLOCK,
             dict(hadamard=True, v_per_channel=True, q_per_block=True))]
VARIANT_IDS = ["vch", "rot+vch", "qblk", "rot+vch+qblk"]


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_flagged_forward_small_shapes(shape, causal, variant):
    flags, kw = variant
    B, Hq, Hkv, S, D = shape
    say(f"forward flags={flags} {shape} causal={causal}")
    w = workloads.dense(110 + S + D, B, Hq, Hkv, S, D, causal, k_offset=2.0, outlier_frac=0.03)
    # A V channel with a gain of 8 and one that is all zero.  The output of the amplified
    # channel is compared divided by 8 (exact on both sides): its absolute error scales
    # with its magnitude through the fp16 rounding of P.
    w.v[..., 1] *= np.float16(8.0)
    w.v[..., 2] = 0
    out = host(i8.attn_int8_fwd_ex(dev(w.q), dev(w.k), dev(w.v), causal, flags))
    ref = oracle.attn_int8_fwd(w.q, w.k, w.v, causal, **kw)
    out = out.astype(np.float64)
    out[..., 1] /= 8.0
    ref[..., 1] /= 8.0
    assert np.all(out[..., 2] == 0)
    check_close(out, ref, f"{shape} flags={flags}")


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_flagged_varlen_ragged_with_empty_sequences(variant):
    flags, kw = variant
    say(f"varlen flags={flags}")
    w = workloads.varlen(120, 6, 700, 8, 2, 128, True, lengths=[300, 0, 1, 700, 65, 129])
    out = host(i8.attn_int8_varlen_fwd_ex(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens),
                                          w.max_seqlen, True, flags))
    ref = oracle.attn_int8_varlen_fwd(w.q, w.k, w.v, w.cu_seqlens, True, **kw)
    check_close(out, ref, f"varlen flags={flags}")


def test_v_per_channel_cfg2_sampled_heads():
    w = workloads.cfg2()
    say("cfg2 with V per channel, 3 heads")
    o = host(i8.attn_int8_fwd_ex(dev(w.q), dev(w.k), dev(w.v), True, i8.FWD_V_PER_CHANNEL))
    heads = [(0, 0), (0, 17), (0, 31)]
    ref = oracle.attn_int8_fwd(w.q, w.k, w.v, True, heads=heads, v_per_channel=True)
    check_close(np.stack([o[b, h] for b, h in heads]), ref, "cfg2 vch")
