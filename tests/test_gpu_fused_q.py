"""GPU: the forward's attention kernel quantizes (and, with the rotation, rotates) Q itself.

Its codes and scales follow the same row rule as the Q preparation pass, so the output
must equal, bit for bit, that of the staged path: K/V and Q prepared into a workspace
(the debug dump's preparation, which honours the variant flags) and then
``attn_int8_attend``, whose kernel reads the prepared Q fragments.  Rows that are all
zero, rows of large values, rows of fp16 subnormals, the largest finite fp16 values with
both signs, negative zeros and query tiles that end inside a 32-row block are included.
"""

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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def staged(q, k, v, causal, flags):
    """Prepare K/V and Q (with the flags) into a workspace, then attend over it."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    ws = torch.empty(i8.attn_int8_workspace_bytes(B, Hq, Hkv, S, D), dtype=torch.uint8,
                     device=q.device)
    i8.attn_int8_debug_qk(q, k, v, 0, 0, 0, 1, 0, 1, workspace=ws, flags=flags)
    # The attention phase takes no flags: rotated rows carry H H^T = D I, the forward's
    # extra factor 1/D (a power of two, so fp32(1/sqrt(D)) / D is exact), given here
    # through the softmax scale.
    scale = float(np.float32(1.0 / np.sqrt(D))) / D if flags & i8.FWD_HADAMARD else None
    return i8.attn_int8_attend(ws, B, Hq, Hkv, S, D, causal, softmax_scale=scale)


@pytest.mark.parametrize("flags", [0, i8.FWD_Q_PER_BLOCK, i8.FWD_V_PER_CHANNEL,
                                   i8.FWD_V_PER_CHANNEL | i8.FWD_Q_PER_BLOCK, i8.FWD_HADAMARD,
                                   i8.FWD_HADAMARD | i8.FWD_Q_PER_BLOCK | i8.FWD_V_PER_CHANNEL])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_fused_q_equals_prepared_q(D, causal, flags):
    say(f"fused Q == prepared Q: D={D} causal={causal} flags={flags}")
    w = workloads.dense(70 + D, 2, 4, 2, 700, D, causal, k_offset=1.0)
    qn = w.q.copy()
    qn[0, 1, 5] = 0                    # an all-zero row: scale 0, zero codes
    qn[1, 2, 33] *= np.float16(3000)   # a row of large values (still finite in fp16)
    qn[1, 3, 690:] = 0                 # zero rows inside the last, ragged 32-row block
    # fp16 subnormals only (the absolute maximum from bit patterns), the largest finite
    # fp16 values with both signs, and negative zeros
    qn[0, 0, 7] = (w.q[0, 0, 7].astype(np.float32) * 2.0 ** -20).astype(np.float16)
    qn[0, 2, 11, :4] = [65504, -65504, -0.0, 0.0]
    qn[1, 0, 40] = -np.abs(qn[1, 0, 40])
    qn[1, 0, 40, ::3] = -0.0
    assert np.isfinite(qn).all()
    assert (np.abs(qn[0, 0, 7]) < np.float16(2.0 ** -14)).all() and np.abs(qn[0, 0, 7]).max() > 0
    q, k, v = dev(qn), dev(w.k), dev(w.v)
    a = host(i8.attn_int8_fwd_ex(q, k, v, causal, flags))
    b = host(staged(q, k, v, causal, flags))
    diff = np.argwhere(a.view(np.uint16) != b.view(np.uint16))
    if diff.size:
        d = np.abs(a.astype(np.float64) - b.astype(np.float64))
        say(f"  {len(diff)} elements differ, max |a - b| = {d.max():.3e}, "
            f"first at (b, h, row, d) = {tuple(diff[0])}, rows {np.unique(diff[:, 2])[:16]}")
    assert diff.size == 0
    if flags == 0:
        c = host(i8.attn_int8_fwd(q, k, v, causal))
        assert np.array_equal(a.view(np.uint16), c.view(np.uint16))


def test_fused_q_varlen_tolerance_and_tail_rows():
    say("fused Q, varlen with ragged and empty sequences, against the oracle")
    w = workloads.varlen(71, 5, 300, 8, 2, 128, True, lengths=[37, 0, 150, 64, 300])
    lens = np.diff(w.cu_seqlens)
    out = host(i8.attn_int8_varlen_fwd(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens),
                                       w.max_seqlen, True))
    ref = oracle.attn_int8_varlen_fwd(w.q, w.k, w.v, w.cu_seqlens, True)
    err = np.abs(out.astype(np.float64) - ref)
    say(f"  lengths {lens.tolist()} max_abs={err.max():.3e}")
    assert err.max() <= 2e-3
    rel = np.linalg.norm(out.astype(np.float64) - ref) / np.linalg.norm(ref)
    assert rel <= 1e-3
