"""GPU parity of the forward with Q outlier detection (I8A_FWD_Q_OUTLIERS) against the
CPU oracle: the output within the forward's tolerance, dense and varlen, with the other
flags; and, bit for bit through the debug dump, the channel sets in the cases the rule
singles out (more than 16 candidates, a channel large in one head of a group only)."""

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
OUT = i8.FWD_Q_OUTLIERS


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
    say(f"  {what}: max_abs={mx:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(o)), what
    assert mx <= MAX_ABS, (what, mx)
    assert rel <= REL_L2, (what, rel)


def kw(flags):
    return dict(v_per_channel=bool(flags & i8.FWD_V_PER_CHANNEL),
                q_per_block=bool(flags & i8.FWD_Q_PER_BLOCK), q_outliers=True)


@pytest.mark.parametrize("flags", [OUT, OUT | i8.FWD_Q_PER_BLOCK,
                                   OUT | i8.FWD_V_PER_CHANNEL | i8.FWD_Q_PER_BLOCK])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_dense_outliers_against_oracle(D, causal, flags):
    say(f"dense outliers D={D} causal={causal} flags={flags}")
    # 3 % of the channels x20 in Q and K, GQA 2:1, a ragged last query tile.
    w = workloads.dense(500 + D, 2, 4, 2, 333, D, causal, k_offset=1.0, outlier_frac=0.03)
    out = host(i8.attn_int8_fwd_ex(dev(w.q), dev(w.k), dev(w.v), causal, flags))
    check_close(out, oracle.attn_int8_fwd(w.q, w.k, w.v, causal, **kw(flags)), (D, causal, flags))


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_outliers_against_oracle(causal):
    say(f"varlen outliers causal={causal}")
    w = workloads.varlen(510, 5, 300, 8, 2, 128, causal, lengths=[37, 0, 300, 64, 129])
    q = w.q.copy()
    q[40:100, 3, 77] = np.float16(25.0)  # an outlier channel in sequence 2 only
    out = host(i8.attn_int8_varlen_fwd_ex(dev(q), dev(w.k), dev(w.v), dev(w.cu_seqlens),
                                          w.max_seqlen, causal, OUT))
    ref = oracle.attn_int8_varlen_fwd(q, w.k, w.v, w.cu_seqlens, causal, q_outliers=True)
    check_close(out, ref, ("varlen", causal))


def test_more_than_sixteen_candidates_and_group_scope():
    # D = 64 with 20 channels x20 in every head: the 16 largest maxima are kept; a
    # channel large in one head of the second group only joins that group's set.
    g = np.random.default_rng(520)
    q = g.standard_normal((1, 4, 200, 64)).astype(np.float32)
    k = g.standard_normal((1, 2, 200, 64)).astype(np.float32)
    v = g.standard_normal((1, 2, 200, 64)).astype(np.float32)
    big = np.arange(0, 60, 3)  # 20 channels
    q[..., big] *= 20 * (1 + np.arange(20) / 40)
    k[..., big] *= 20
    q = np.clip(q, -60000, 60000)
    q[0, 3, 5, 1] = 900.0  # head 3 is in group 1
    q16, k16, v16 = (a.astype(np.float16) for a in (q, k, v))
    z = oracle.quantize_qkv(q16, k16, v16, q_outliers=True)
    assert (z["ochan"] >= 0).sum(axis=-1).tolist() == [[16, 16]]
    assert 1 in z["ochan"][0, 1] and 1 not in z["ochan"][0, 0]
    for h in (0, 3):
        r = i8.attn_int8_debug_qk(dev(q16), dev(k16), dev(v16), 0, h, 0, 200, 0, 200, flags=OUT)
        assert np.array_equal(host(r["ochan"]).astype(np.int64), z["ochan"][0, h // 2])
        s_ref = oracle.qk_int32(z["q8"][0, h], z["k8"][0, h // 2])
        assert np.array_equal(host(r["s32"]).astype(np.int64), s_ref)
        assert np.array_equal(host(r["qscale"]), z["sq"][0, h])
        assert np.array_equal(host(r["kscale"]), z["sk"][0, h // 2])
    out = host(i8.attn_int8_fwd_ex(dev(q16), dev(k16), dev(v16), True, OUT))
    check_close(out, oracle.attn_int8_fwd(q16, k16, v16, True, q_outliers=True), "cap")


def test_rows_whose_int8_part_is_zero():
    # Query rows that live only on the outlier channels: the int8 part has scale 0 and
    # the logits are the exact outlier products alone.
    g = np.random.default_rng(530)
    q = g.standard_normal((1, 2, 130, 64)).astype(np.float32)
    k = g.standard_normal((1, 1, 130, 64)).astype(np.float32)
    v = g.standard_normal((1, 1, 130, 64)).astype(np.float32)
    q[..., 10] *= 30
    k[..., 10] *= 3
    q[0, 0, 7] = 0.0
    q[0, 0, 7, 10] = 12.0
    q[0, 1, 100:] = 0.0
    q[0, 1, 100:, 10] = -9.5
    q16, k16, v16 = (a.astype(np.float16) for a in (q, k, v))
    for causal in (True, False):
        out = host(i8.attn_int8_fwd_ex(dev(q16), dev(k16), dev(v16), causal, OUT))
        check_close(out, oracle.attn_int8_fwd(q16, k16, v16, causal, q_outliers=True),
                    ("zero int8 part", causal))


def test_outliers_improve_sqnr_on_outlier_channels():
    # The quality gain the detection exists for, on the GPU: cfg3's shape at D = 128
    # (1 % of the channels x20), two heads, against unquantized attention.
    w = workloads.cfg3(128)
    q, k, v = w.q[:1, :2], w.k[:1, :2], w.v[:1, :2]
    exact = oracle.attn_exact(q, k, v, False)

    def sqnr(o):
        return 10 * np.log10(np.sum(exact ** 2) / np.sum((o.astype(np.float64) - exact) ** 2))
    plain = sqnr(host(i8.attn_int8_fwd(dev(q), dev(k), dev(v), False)))
    det = sqnr(host(i8.attn_int8_fwd_ex(dev(q), dev(k), dev(v), False, OUT)))
    say(f"  SQNR plain {plain:.2f} dB, with outlier detection {det:.2f} dB")
    assert det > plain + 8.0
