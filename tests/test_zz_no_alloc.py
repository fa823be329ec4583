"""attn_int8_fwd_noalloc (the forward with the library's own per-GPU scratch as its
workspace, for callers that cannot allocate) against attn_int8_fwd with a workspace:
bit-identical outputs on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents), both within the oracle's tolerance; and a
size beyond the scratch rejected before any work.  Called through the C ABI."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import int8_w8a8_flashattention_amd as i8
from int8_w8a8_flashattention_amd import workloads

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_noalloc_forward_equals_the_workspace_forward_twice():
    lib = i8.load_library()
    dev = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    for (seed, B, Hq, Hkv, S, D, causal) in [(501, 2, 8, 2, 700, 128, True),
                                             (502, 1, 4, 1, 300, 64, False)]:
        say(f"noalloc B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} causal={causal}")
        w = workloads.dense(seed, B, Hq, Hkv, S, D, causal, k_offset=2.0)
        q, k, v = (torch.from_numpy(a).to(dev) for a in (w.q, w.k, w.v))
        scale = float(np.float32(1.0 / np.sqrt(D)))
        out_ref = torch.full_like(q, float("nan"))
        nb = lib.attn_int8_workspace_bytes(B, Hq, Hkv, S, D)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        assert lib.attn_int8_fwd(P(q), P(k), P(v), P(out_ref), B, Hq, Hkv, S, D, scale,
                                 int(causal), P(ws), nb, stream) == 0
        out = torch.full_like(q, float("nan"))
        st = lib.attn_int8_fwd_noalloc(P(q), P(k), P(v), P(out), B, Hq, Hkv, S, D, scale,
                                       int(causal), stream)
        assert st == 0, lib.i8a_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref)
        ref = oracle.attn_int8_fwd(w.q, w.k, w.v, causal)
        o = out.cpu().numpy().astype(np.float64)
        assert np.abs(o - ref).max() <= 2e-3
        assert np.linalg.norm(o - ref) / np.linalg.norm(ref) <= 1e-3


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lib = i8.load_library()
    x = torch.zeros(16, dtype=torch.float16, device="cuda:0")
    p = ctypes.c_void_p(x.data_ptr())
    st = lib.attn_int8_fwd_noalloc(p, p, p, p, 1, 32, 8, 16384, 128, 0.088, 1, None)
    assert st == -3
    assert b"scratch" in lib.i8a_last_error()
