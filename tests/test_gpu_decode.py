"""GPU parity of the split-KV int8 decode (cache fill + decode through the C ABI)
against the CPU oracle's decode.

The fp16 output must satisfy max|o - O| <= 2e-3 and ||o - O||_2 / ||O||_2 <= 1e-3 over
each compared set, with O the unrounded fp64 oracle.  The shapes cover every head dim,
both V formats, ragged cache lengths (not a multiple of the 32-token tile), a single
cached token, caches split over several chunks, GQA groups wider than 32 heads and the
batched serving shape (checked on sampled sequences).
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
    mx = float(err.max())
    rel = float(np.linalg.norm(o - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"  {what}: max_abs={mx:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(o)), what
    assert mx <= MAX_ABS, (what, mx)
    assert rel <= REL_L2, (what, rel)


def run_decode(w, v_format, softmax_scale=None):
    cache = i8.attn_int8_kvcache_fill(dev(w.k), dev(w.v), v_format)
    return host(i8.attn_int8_decode(dev(w.q), cache, softmax_scale))


# (B, Hq, Hkv, S, D): tiny, ragged, one token, several chunks, wide GQA groups
SHAPES = [
    (1, 2, 1, 1, 64),
    (2, 4, 2, 37, 32),
    (1, 8, 2, 100, 128),
    (2, 8, 8, 95, 64),
    (1, 4, 2, 3000, 128),
    (1, 8, 1, 2049, 256),
    (1, 40, 1, 300, 128),
    (3, 70, 2, 650, 64),
]


@pytest.mark.parametrize("v_format", ["int8", "fp16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_matches_oracle(shape, v_format):
    B, Hq, Hkv, S, D = shape
    say(f"decode {shape} v={v_format}")
    w = workloads.decode(500 + S + D + Hq, B, Hq, Hkv, S, D, k_offset=2.0)
    out = run_decode(w, v_format)
    ref = oracle.attn_int8_decode(w.q, w.k, w.v, v_format=v_format)
    check_close(out, ref, f"decode {shape} {v_format}")


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_decode_every_head_dim_multi_chunk(D):
    say(f"decode D={D} multi-chunk")
    w = workloads.decode(600 + D, 1, 4, 1, 4000, D, k_offset=3.0)
    for vf in ("int8", "fp16"):
        check_close(run_decode(w, vf), oracle.attn_int8_decode(w.q, w.k, w.v, v_format=vf),
                    f"D={D} {vf}")


def test_decode_softmax_scale_and_zero_query():
    say("decode softmax_scale argument and zero query rows")
    w = workloads.decode(700, 2, 8, 2, 777, 128)
    w.q[1, 3] = 0  # an all-zero query row attends uniformly: the mean of the values
    for vf in ("int8", "fp16"):
        out = run_decode(w, vf, softmax_scale=0.3)
        ref = oracle.attn_int8_decode(w.q, w.k, w.v, softmax_scale=0.3, v_format=vf)
        check_close(out, ref, f"scale 0.3 {vf}")


def test_decode_gqa_equals_repeated_heads_and_deterministic():
    say("decode GQA vs repeated kv heads")
    w = workloads.decode(701, 1, 16, 4, 1500, 64, k_offset=1.0)
    a = run_decode(w, "int8")
    rep = workloads.Decode(w.q, np.repeat(w.k, 4, axis=1), np.repeat(w.v, 4, axis=1))
    b = run_decode(rep, "int8")
    assert np.array_equal(a, b)
    assert np.array_equal(a, run_decode(w, "int8"))


def test_decode_cache_reused_across_steps():
    say("one cache, several query batches")
    w = workloads.decode(702, 2, 8, 2, 513, 128, k_offset=2.0)
    cache = i8.attn_int8_kvcache_fill(dev(w.k), dev(w.v), "int8")
    g = np.random.Generator(np.random.PCG64(703))
    for step in range(3):
        q = g.standard_normal(w.q.shape).astype(np.float16)
        out = host(i8.attn_int8_decode(dev(q), cache))
        check_close(out, oracle.attn_int8_decode(q, w.k, w.v), f"step {step}")


def test_decode_serving_shape_sampled_sequences():
    # The full batched shape runs on the GPU; the oracle checks three sequences
    # (sequences are independent: each has its own cache and K mean).
    w = workloads.decode_bench()
    say(f"decode {w.name} (sampled sequences)")
    for vf in ("int8", "fp16"):
        out = run_decode(w, vf)
        for b in (0, 7, 15):
            ref = oracle.attn_int8_decode(w.q[b:b + 1], w.k[b:b + 1], w.v[b:b + 1], v_format=vf)
            check_close(out[b:b + 1], ref, f"{vf} sequence {b}")


def test_decode_rejects_bad_arguments():
    lib = i8.load_library()
    w = workloads.decode(704, 1, 4, 2, 64, 64)
    cache = i8.attn_int8_kvcache_fill(dev(w.k), dev(w.v), "int8")
    q, out = dev(w.q), torch.empty((1, 4, 64), dtype=torch.float16, device="cuda")
    args = lambda **kw: dict(dict(q=q.data_ptr(), out=out.data_ptr(), B=1, Hq=4, Hkv=2, S=64,
                                  D=64, scale=0.125, vf=1, cache=cache.buf.data_ptr(),
                                  cb=cache.nbytes), **kw)

    def call(a):
        return lib.attn_int8_decode(a["q"], a["out"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"],
                                    a["scale"], a["vf"], a["cache"], a["cb"], None, 0, None)
    assert call(args()) == 0
    assert call(args(Hq=5)) == -1
    assert call(args(D=48)) == -2
    assert call(args(vf=3)) == -1
    assert call(args(cb=cache.nbytes - 1)) == -3
    assert call(args(scale=0.0)) == -1
    assert call(args(cache=cache.buf.data_ptr() + 16)) == -1
    torch.cuda.synchronize()


def test_decode_workspace_reused_across_calls_and_shapes():
    # One workspace, filled with NaN bytes first, serves several multi-chunk calls and
    # shapes: every chunk partial the merge reads is written by the same call.
    say("one NaN-filled workspace, several multi-chunk calls and shapes")
    shapes = [(1, 4, 2, 3000, 128), (2, 8, 2, 1500, 64), (1, 40, 1, 2500, 128)]
    need = max(i8.attn_int8_decode_workspace_bytes(B, Hq, Hkv, S, D, "int8")
               for B, Hq, Hkv, S, D in shapes)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for n, (B, Hq, Hkv, S, D) in enumerate(shapes):
            w = workloads.decode(800 + n, B, Hq, Hkv, S, D, k_offset=1.5)
            cache = i8.attn_int8_kvcache_fill(dev(w.k), dev(w.v), "int8")
            out = host(i8.attn_int8_decode(dev(w.q), cache, workspace=ws))
            check_close(out, oracle.attn_int8_decode(w.q, w.k, w.v), f"rep {rep} shape {n}")
