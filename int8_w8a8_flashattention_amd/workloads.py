"""Seeded synthetic inputs for the INT8 attention forward.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic.  Both the GPU path's tests and the oracle's tests
consume the same bytes from here.

Recipe (all workloads): ``numpy.random.Generator(PCG64(seed))``; draw q, k,
v as fp32 ``standard_normal`` in that order, then the structure draws; apply
the structure in fp32; cast to fp16 with round-to-nearest-even.  The shapes
follow the page's quick-start call (q ``[1,32,4096,128]``, k/v
``[1,8,4096,128]``) and the head-dim, GQA and ragged-prefill claims of its
*Attention kernels* table.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass
class Dense:
    q: np.ndarray  # fp16 [B, Hq, S, D]
    k: np.ndarray  # fp16 [B, Hkv, S, D]
    v: np.ndarray  # fp16 [B, Hkv, S, D]
    causal: bool
    name: str = ""
    meta: dict = field(default_factory=dict)


@dataclass
class Varlen:
    q: np.ndarray  # fp16 [T, Hq, D]
    k: np.ndarray  # fp16 [T, Hkv, D]
    v: np.ndarray  # fp16 [T, Hkv, D]
    cu_seqlens: np.ndarray  # int32 [nseq + 1]
    max_seqlen: int
    causal: bool
    name: str = ""
    meta: dict = field(default_factory=dict)


@dataclass
class Decode:
    q: np.ndarray  # fp16 [B, Hq, D]: the new token's query rows
    k: np.ndarray  # fp16 [B, Hkv, S, D]: the cached tokens
    v: np.ndarray  # fp16 [B, Hkv, S, D]
    name: str = ""
    meta: dict = field(default_factory=dict)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def dense(seed, B, Hq, Hkv, S, D, causal, k_offset=0.0, outlier_frac=0.0,
          outlier_gain=20.0, name=""):
    """Dense BHSD inputs.

    ``k_offset``: if > 0, a per-(kv head, channel) offset ~ U(-k_offset,
    k_offset) is added to K (broadcast over batch and tokens).
    ``outlier_frac``: if > 0, ``ceil(frac * D)`` channel indices drawn once are
    multiplied by ``outlier_gain`` in both Q and K (all heads).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (B, Hq, S, D))
    k = _normal(rng, (B, Hkv, S, D))
    v = _normal(rng, (B, Hkv, S, D))
    meta = {}
    if k_offset > 0:
        off = rng.uniform(-k_offset, k_offset, size=(Hkv, D)).astype(np.float32)
        k += off[None, :, None, :]
        meta["k_offset"] = off
    if outlier_frac > 0:
        n = int(math.ceil(outlier_frac * D))
        ch = rng.choice(D, size=n, replace=False)
        q[..., ch] *= np.float32(outlier_gain)
        k[..., ch] *= np.float32(outlier_gain)
        meta["outlier_channels"] = np.sort(ch)
    return Dense(q.astype(np.float16), k.astype(np.float16), v.astype(np.float16),
                 causal, name, meta)


def varlen(seed, nseq, max_len, Hq, Hkv, D, causal, lengths=None, name=""):
    """Packed ``[T, H, D]`` inputs with lengths ~ U[1, max_len] (or given)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if lengths is None:
        lengths = rng.integers(1, max_len + 1, size=nseq)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.size + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q = _normal(rng, (T, Hq, D)).astype(np.float16)
    k = _normal(rng, (T, Hkv, D)).astype(np.float16)
    v = _normal(rng, (T, Hkv, D)).astype(np.float16)
    return Varlen(q, k, v, cu, int(lengths.max()) if lengths.size else 0, causal, name,
                  {"lengths": lengths})


def decode(seed, B, Hq, Hkv, S, D, k_offset=0.0, name=""):
    """One decode step: the new token's query rows ``q [B, Hq, D]`` and the ``S``
    cached tokens ``k, v [B, Hkv, S, D]`` (fp16, standard normal; ``k_offset`` as in
    :func:`dense`)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (B, Hq, D))
    k = _normal(rng, (B, Hkv, S, D))
    v = _normal(rng, (B, Hkv, S, D))
    meta = {}
    if k_offset > 0:
        off = rng.uniform(-k_offset, k_offset, size=(Hkv, D)).astype(np.float32)
        k += off[None, :, None, :]
        meta["k_offset"] = off
    return Decode(q.astype(np.float16), k.astype(np.float16), v.astype(np.float16), name, meta)


# The five workloads the method is measured and checked on.

def cfg1():
    """Tiny causal GQA: B1 Hq2 Hkv1 S128 D64, K offset U(-3,3)."""
    return dense(1, 1, 2, 1, 128, 64, True, k_offset=3.0, name="cfg1_tiny_causal_gqa")


def cfg2():
    """Causal GQA at the quick-start shape: B1 Hq32 Hkv8 S4096 D128."""
    return dense(2, 1, 32, 8, 4096, 128, True, name="cfg2_causal_gqa_s4096_d128")


def cfg3(D):
    """Non-causal MHA head-dim sweep: B4 H16 S2048, 1% outlier channels x20."""
    assert D in (32, 64, 128, 256)
    return dense(3, 4, 16, 16, 2048, D, False, outlier_frac=0.01,
                 name=f"cfg3_mha_s2048_d{D}_outliers")


def cfg4():
    """Varlen ragged causal prefill: 16 seqs, L ~ U[1,4096], Hq64 Hkv8 D128."""
    return varlen(4, 16, 4096, 64, 8, 128, True, name="cfg4_varlen_16x_u4096")


def cfg5():
    """Long-context causal GQA: B1 Hq40 Hkv8 S32768 D128, K offset U(-3,3)."""
    return dense(5, 1, 40, 8, 32768, 128, True, k_offset=3.0, name="cfg5_causal_gqa_s32768")


def decode_bench():
    """Batched decode at a GQA serving shape: 16 sequences with 8192 cached tokens each,
    Hq32 Hkv8 D128, K offset U(-3,3)."""
    return decode(6, 16, 32, 8, 8192, 128, k_offset=3.0, name="decode_b16_s8192_gqa_d128")


def attn_ops(Hq, D, lengths, causal):
    """Algorithmic operation count: 4*D*Hq per (query, key) pair, S^2/2 pairs
    per causal head (the usual FlashAttention convention)."""
    tot = 0.0
    for L in lengths:
        L = float(L)
        pairs = L * L / 2.0 if causal else L * L
        tot += 4.0 * D * Hq * pairs
    return tot
