"""GPU parity of the backward (attn_bwd, through the C ABI) against the CPU oracle's
gradient of exact attention, and of the autograd wrapper.

Bar: the gradients come from fp16 MFMA products with fp32 accumulation, with P and dS
rounded to fp16 as operands (a relative error of at most 2^-12 = 2.4e-4 per operand,
which is also what the measured gradients show: rel-L2 about 2e-4).  For each of dq,
dk, dv over the compared set, ||g - G||_2 / ||G||_2 <= 1e-3 and
max |g - G| <= 1e-3 * max |G|, with G the fp64 oracle: about four times the rounding
level.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import int8_w8a8_flashattention_amd as i8
from int8_w8a8_flashattention_amd import workloads

pytestmark = pytest.mark.gpu

REL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_grad(g, ref, what):
    g = g.astype(np.float64)
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30))
    mx = float(np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30))
    say(f"  {what}: rel_l2={rel:.3e} max_abs/max|G|={mx:.3e}")
    assert np.all(np.isfinite(g)), what
    assert rel <= REL, (what, rel)
    assert mx <= REL, (what, mx)


def run(w, do, causal, scale=None):
    return [host(t) for t in i8.attn_bwd(dev(w.q), dev(w.k), dev(w.v), dev(do), causal, scale)]


SHAPES = [(1, 2, 2, 64, 64), (2, 4, 2, 100, 32), (1, 4, 1, 300, 128), (1, 2, 1, 1, 64),
          (2, 8, 2, 129, 128), (1, 3, 3, 33, 32),
          # one query block in the last 128-key group with G = 1: the causal split's second
          # part has no items there and must still write its (zero) partial rows
          (1, 2, 2, 160, 64), (1, 1, 1, 129, 32),
          # a large query group (MQA, G = 16)
          (1, 16, 1, 200, 64),
          # D = 256 (the plain dK/dV loop, the dQ kernel with its results in accumulation
          # registers), GQA and MHA, ragged tails
          (1, 4, 2, 150, 256), (2, 2, 2, 70, 256)]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_matches_oracle(shape, causal):
    B, Hq, Hkv, S, D = shape
    say(f"bwd {shape} causal={causal}")
    w = workloads.dense(200 + S + D, B, Hq, Hkv, S, D, causal, k_offset=1.0)
    do = np.random.Generator(np.random.PCG64(201 + S)).standard_normal(w.q.shape).astype(np.float16)
    got = run(w, do, causal)
    ref = oracle.attn_bwd_exact(w.q, w.k, w.v, do, causal)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        check_grad(g, r, f"{shape} {name}")


def test_bwd_softmax_scale_argument():
    w = workloads.dense(210, 1, 4, 2, 150, 64, True)
    do = np.random.Generator(np.random.PCG64(211)).standard_normal(w.q.shape).astype(np.float16)
    got = run(w, do, True, 0.3)
    ref = oracle.attn_bwd_exact(w.q, w.k, w.v, do, True, 0.3)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        check_grad(g, r, f"scale 0.3 {name}")


def test_autograd_wrapper_uses_the_backward():
    w = workloads.dense(212, 1, 4, 2, 96, 64, True)
    do = np.random.Generator(np.random.PCG64(213)).standard_normal(w.q.shape).astype(np.float16)
    q, k, v = (dev(x).requires_grad_(True) for x in (w.q, w.k, w.v))
    out = i8.int8_attention(q, k, v, True)
    ref_out = i8.attn_int8_fwd(dev(w.q), dev(w.k), dev(w.v), True)
    assert torch.equal(out.detach(), ref_out)
    out.backward(dev(do))
    dq, dk, dv = run(w, do, True)
    for name, a, b in (("dq", q.grad, dq), ("dk", k.grad, dk), ("dv", v.grad, dv)):
        assert a.dtype == torch.float16
        assert np.array_equal(host(a), b.astype(np.float16)), name


def test_bwd_cfg2_one_kv_group():
    # The quick-start shape (B1 Hq32 Hkv8 S4096 D128 causal) runs in full on the GPU;
    # the oracle checks kv head 3 and its 4 query heads (groups are independent).
    w = workloads.cfg2()
    say("bwd cfg2, kv group 3")
    do = np.random.Generator(np.random.PCG64(214)).standard_normal(w.q.shape).astype(np.float16)
    dq, dk, dv = run(w, do, True)
    sl = slice(12, 16)
    ref = oracle.attn_bwd_exact(w.q[:, sl], w.k[:, 3:4], w.v[:, 3:4], do[:, sl], True)
    check_grad(dq[:, sl], ref[0], "cfg2 dq")
    check_grad(dk[:, 3:4], ref[1], "cfg2 dk")
    check_grad(dv[:, 3:4], ref[2], "cfg2 dv")


def test_bwd_needs_no_workspace_initialization():
    # The workspace is filled with NaN bytes first: every value the kernels read from it
    # must have been written by the same call (the combine kernel adds every partial row,
    # including those of a part with no items).
    B, Hq, Hkv, S, D = 1, 2, 2, 160, 64
    w = workloads.dense(215, B, Hq, Hkv, S, D, True, k_offset=1.0)
    do = np.random.Generator(np.random.PCG64(216)).standard_normal(w.q.shape).astype(np.float16)
    ws = torch.full((i8.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    got = [host(t) for t in i8.attn_bwd(dev(w.q), dev(w.k), dev(w.v), dev(do), True,
                                        workspace=ws)]
    ref = oracle.attn_bwd_exact(w.q, w.k, w.v, do, True)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        check_grad(g, r, f"NaN-filled workspace {name}")


def test_bwd_is_deterministic():
    # No atomics: two calls give bit-identical gradients (here with the causal split and
    # its combine, GQA, a ragged tail).
    w = workloads.dense(217, 2, 8, 2, 300, 128, True)
    do = np.random.Generator(np.random.PCG64(218)).standard_normal(w.q.shape).astype(np.float16)
    a = run(w, do, True)
    b = run(w, do, True)
    for name, x, y in zip(("dq", "dk", "dv"), a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), name


def test_bwd_noncausal_large_one_kv_group():
    # Non-causal (no split, no combine) at S = 2048, D = 128, GQA: the whole call runs on
    # the GPU, the oracle checks kv head 1 and its 4 query heads.
    w = workloads.dense(219, 1, 8, 2, 2048, 128, False, k_offset=1.0)
    say("bwd non-causal S2048 D128, kv group 1")
    do = np.random.Generator(np.random.PCG64(220)).standard_normal(w.q.shape).astype(np.float16)
    dq, dk, dv = run(w, do, False)
    sl = slice(4, 8)
    ref = oracle.attn_bwd_exact(w.q[:, sl], w.k[:, 1:2], w.v[:, 1:2], do[:, sl], False)
    check_grad(dq[:, sl], ref[0], "non-causal dq")
    check_grad(dk[:, 1:2], ref[1], "non-causal dk")
    check_grad(dv[:, 1:2], ref[2], "non-causal dv")
