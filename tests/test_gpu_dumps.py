"""GPU parity of every code and scale the forward prepares, bit for bit, through the
debug dump (attn_int8_debug_qk_ex) against the CPU oracle's quantization: the int32
scores, the Q row (or per-block) scales, the K scales and K-smoothing mean, the
prepared V rows (the exact fp16 values scale * code the P.V product consumes, compared
by value: with the scale bit-exact, equal values are equal codes) and the V scales per
token or per channel, and the Q outlier channels -- for every head dim, with and without
each variant flag, dense and varlen (blocks, means and outlier channels per sequence)."""

import sys

import numpy as np
import pytest
import torch

import oracle
import int8_w8a8_flashattention_amd as i8
from int8_w8a8_flashattention_amd import workloads

pytestmark = pytest.mark.gpu

FLAGS = [0, i8.FWD_V_PER_CHANNEL, i8.FWD_Q_PER_BLOCK,
         i8.FWD_HADAMARD | i8.FWD_V_PER_CHANNEL | i8.FWD_Q_PER_BLOCK]
# Q outlier detection (head dims up to 128).
FLAGS_OUT = [i8.FWD_Q_OUTLIERS, i8.FWD_Q_OUTLIERS | i8.FWD_Q_PER_BLOCK | i8.FWD_V_PER_CHANNEL]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def zflags(q, k, v, flags):
    return oracle.quantize_qkv(q, k, v, hadamard=bool(flags & i8.FWD_HADAMARD),
                               v_per_channel=bool(flags & i8.FWD_V_PER_CHANNEL),
                               q_per_block=bool(flags & i8.FWD_Q_PER_BLOCK),
                               q_outliers=bool(flags & i8.FWD_Q_OUTLIERS))


def vhat_ref(z, b, g, c0, nc, per_channel):
    """The oracle's dequantized V rows, which its 4-bit V scale makes exact in fp16."""
    v8 = z["v8"][b, g, c0:c0 + nc].astype(np.float64)
    sv = z["sv"][b, g].astype(np.float64)
    vh = v8 * (sv[None, :] if per_channel else sv[c0:c0 + nc, None])
    assert np.array_equal(vh.astype(np.float16).astype(np.float64), vh)
    return vh.astype(np.float16)


def check_dump(r, z, b, h, G, r0, nr, c0, nc, flags, what):
    g = h // G
    pc = bool(flags & i8.FWD_V_PER_CHANNEL)
    s_ref = oracle.qk_int32(z["q8"][b, h], z["k8"][b, g])[r0:r0 + nr, c0:c0 + nc]
    assert np.array_equal(host(r["s32"]).astype(np.int64), s_ref), what
    assert np.array_equal(host(r["qscale"]), z["sq"][b, h, r0:r0 + nr]), what
    assert np.array_equal(host(r["kscale"]), z["sk"][b, g, c0:c0 + nc]), what
    assert np.array_equal(host(r["kmean"]), z["kmean"][b, g]), what
    # Exact values (a negative entry whose code is 0 may come back as -0.0).
    assert np.array_equal(host(r["vhat"]).astype(np.float64),
                          vhat_ref(z, b, g, c0, nc, pc).astype(np.float64)), what
    if pc:
        assert np.array_equal(host(r["vchan"]), z["sv"][b, g]), what
    else:
        assert np.array_equal(host(r["vscale"]), z["sv"][b, g, c0:c0 + nc]), what
    if flags & i8.FWD_Q_OUTLIERS:
        assert np.array_equal(host(r["ochan"]).astype(np.int64), z["ochan"][b, g]), what


@pytest.mark.parametrize("flags", FLAGS + FLAGS_OUT)
@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_dense_dump_bit_exact(D, flags):
    if D == 256 and flags & i8.FWD_Q_OUTLIERS:
        pytest.skip("Q outlier detection is built for D <= 128")
    say(f"dense dump D={D} flags={flags}")
    w = workloads.dense(300 + D + flags, 2, 4, 2, 150, D, True, k_offset=2.5, outlier_frac=0.02)
    z = zflags(w.q, w.k, w.v, flags)
    for (b, h, r0, nr, c0, nc) in [(0, 0, 0, 150, 0, 150), (1, 3, 33, 70, 64, 86)]:
        r = i8.attn_int8_debug_qk(dev(w.q), dev(w.k), dev(w.v), b, h, r0, nr, c0, nc,
                                  flags=flags)
        check_dump(r, z, b, h, 2, r0, nr, c0, nc, flags, (D, flags, b, h))


@pytest.mark.parametrize("flags", FLAGS + FLAGS_OUT)
@pytest.mark.parametrize("D", [64, 128])
def test_varlen_dump_bit_exact(D, flags):
    # Sequences of 37, 0, 150 and 64 tokens: each dumped sequence against the oracle's
    # quantization of that sequence alone (its own mean, V channel scales and Q blocks).
    say(f"varlen dump D={D} flags={flags}")
    w = workloads.varlen(400 + D + flags, 4, 150, 4, 2, D, True, lengths=[37, 0, 150, 64])
    cu = w.cu_seqlens
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    cud = dev(cu.astype(np.int32))
    for s in (0, 2, 3):
        a, b_ = int(cu[s]), int(cu[s + 1])
        L = b_ - a
        z = zflags(np.ascontiguousarray(w.q[a:b_].transpose(1, 0, 2))[None],
                   np.ascontiguousarray(w.k[a:b_].transpose(1, 0, 2))[None],
                   np.ascontiguousarray(w.v[a:b_].transpose(1, 0, 2))[None], flags)
        for h in (0, 3):
            r = i8.attn_int8_varlen_debug_qk(q, k, v, cud, w.max_seqlen, s, h, 0, L, 0, L,
                                             flags=flags)
            check_dump(r, z, 0, h, 2, 0, L, 0, L, flags, (D, flags, s, h))


def test_dump_leaves_entries_past_the_sequence_unwritten():
    # Varlen rows and keys past a sequence's own length (inside max_seqlen) stay as the
    # caller left them.
    w = workloads.varlen(450, 2, 100, 2, 1, 64, True, lengths=[40, 100])
    cu = dev(w.cu_seqlens.astype(np.int32))
    r = i8.attn_int8_varlen_debug_qk(dev(w.q), dev(w.k), dev(w.v), cu, w.max_seqlen, 0, 1, 0,
                                     100, 0, 100)
    s32 = host(r["s32"])
    assert np.all(s32[40:] == 0) and np.all(s32[:, 40:] == 0)
    assert np.any(s32[:40, :40] != 0)
    assert np.all(host(r["vhat"])[40:] == 0)
