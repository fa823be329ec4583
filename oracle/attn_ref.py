"""Plain, slow CPU definition of the INT8 W8A8 attention forward (fp64).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Imported only by
tests, the smoke check and the CPU-baseline leg of the benchmark.

What is computed follows the "SuperL8" README: the *Attention kernels* table
(``attn_int8_fwd``: W8A8 FlashAttention-2, causal, GQA/MQA, head dims
32/64/128/256; ``attn_varlen_fwd``: ragged prefill), the *Supporting kernels*
table (``quant_rowwise``: symmetric per-row int8), the *Quantization* table
("Per-row int8: symmetric, K-smoothing"; "V per-channel / per-token") and the
*Quick start* call, which takes fp16 q/k/v and quantizes internally.

The page prints no formulas, so each step below is the plainest reading of
those rows.  Readings taken where the page is silent:

R1  Codes are symmetric: integers in [-127, 127]; -128 is never produced.
R2  Row scale of Q and K: ``fp32(absmax / 127)`` (IEEE round-to-nearest-even),
    stored as fp32.  Row scale of V (the per-token choice of the
    *Quantization* table's "V per-channel / per-token" row): the same value
    rounded *up* to the next number whose significand has 4 bits.  Then every
    dequantized value ``code * scale`` (7-bit code times 4-bit significand)
    is exactly an fp16 number, so the fp16 P.V product can consume V without
    rounding it; rounding up keeps every ``|x| / scale`` at most 127.
R3  ``code = clamp(rint(fp32(x / scale)), -127, 127)`` with a correctly
    rounded fp32 division and round-half-to-even.
R4  An all-zero row gets scale 0 and codes 0.
R5  K-smoothing subtracts, per (batch, kv head, channel), the mean of K over
    all tokens of that sequence (future tokens included under the causal
    mask).  The mean is the exact sum (fp16 values are integer multiples of
    2^-24), divided in fp64, rounded to fp32; K rows are quantized from the
    fp32 difference ``fp32(k) - mean``.
R6  Q and V are quantized per row (per token and head) like K, without the
    mean subtraction; V uses its 4-bit scale (R2).
R7  Scores are the exact integer dot products of the codes; logits are
    ``S32 * sq_i * sk_j * softmax_scale``; the softmax scale defaults to
    ``fp32(1 / sqrt(D))`` and is not folded into Q before quantization.
R8  Causal means equal query and key lengths and query i sees keys j <= i.
R9  GQA/MQA: query head h reads kv head ``h // (Hq / Hkv)``.
R10 Output ``O = softmax(logits) @ (sv * v8)``, exact softmax over the whole
    row, in fp64 and left unrounded (a GPU result is compared against it).
R11 Varlen input is packed ``[T, H, D]`` with ``cu_seqlens[nseq + 1]``; every
    sequence is an independent causal (or full) attention with its own K mean.
R12 Decode (the *Attention kernels* table's ``attn_decode`` row: split-KV decode
    with an int8 KV cache, in its int8-V and fp16-V variants): one new query token
    per sequence attends every token of that sequence's cache.  K is cached as in
    the forward (K-smoothing mean over the cached tokens, R5, then per-row int8).
    V is cached per token as in the forward (R2) in the int8-V variant, and as the
    fp16 values themselves in the fp16-V variant.  The query row is quantized like
    Q (R6).  The split over the keys is an implementation choice and does not
    change what is computed.

R13 Hadamard rotation (the *Quantization* table's "Hadamard rotation" row: an
    incoherence rotation for outlier-heavy activations).  The page gives no
    formula; the plainest reading rotates Q and the mean-smoothed K by the
    Sylvester-Hadamard matrix before their rows are quantized, so that an outlier
    channel's energy spreads over all D channels.  Concretely, each fp32 row x
    (``fp32(q)``, or ``fp32(k) - mean`` as in R5) becomes the unnormalized fast
    Walsh-Hadamard transform ``x H`` computed in fp32 with the butterflies taken in
    the fixed order of stages s = 0, 1, ..., log2(D)-1, each stage replacing the
    pair (x[i], x[i + 2^s]) (bit s of i clear) by (x[i] + x[i + 2^s],
    x[i] - x[i + 2^s]).  Since ``H H^T = D I``, the dequantized scores of the
    rotated rows are D times the unrotated ones: the logits take an extra exact
    factor 1/D.  V is not rotated.

R14 V per channel (the *Quantization* table's "V per-channel / per-token" row:
    configurable KV cache quantization).  Per token is R2's default.  Per channel,
    V is quantized with one scale per (sequence, kv head, channel) over the
    sequence's tokens: the scale is fp32(absmax/127) rounded up to a 4-bit
    significand (the V rule of R2, so that every dequantized value is exactly an
    fp16 number) and the codes follow R3 with that channel's scale.

R19 Q outlier detection (the *Quantization* table's "Per-row int8" row: symmetric,
    K-smoothing, Q outlier detection; the *Attention kernels* table's
    ``attn_w8a8_fwd`` row: outlier-aware).  The page gives no rule; the plainest
    reading is the mixed-precision decomposition of int8 products with outlier
    feature dimensions (LLM.int8(), Dettmers et al. 2022), with the outliers
    detected on Q.  Per (sequence, kv head), channel d is an outlier channel when
    ``max |q[t, h, d]|`` over the sequence's tokens t and the query heads h of the
    kv head's group exceeds 6 (the published magnitude threshold); at most 16 are
    kept, the largest maxima first, ties to the lower channel.  Q rows and the
    mean-smoothed K rows are quantized (R2/R3, per row or per block) with those
    channels set to zero; the channels themselves stay as the fp16 inputs, K
    without the mean (a per-row constant of the logits), and the logits become
    ``(S32 * sq_i * sk_j + sum_{d in set} q_id * k_jd) * softmax_scale``.

R20 A growing decode cache (the *Attention kernels* table's ``attn_decode`` row serves
    generation, where every step adds a token to each sequence; the page gives no
    rule for the K-smoothing mean of a cache that grows).  The plainest reading:
    the mean is taken once, over the tokens the cache is filled with (R5), and
    every later K row is quantized against that stored mean (``fp32(k) - mean``,
    then R2/R3), V rows as in R12.  Subtracting any fixed per-channel vector from
    K adds a per-query constant to the logits, so exact attention does not depend
    on which mean is stored; re-taking the mean would requantize the whole cache
    at every step.  A sequence attends its first ``lens[b]`` cached tokens; with
    none, its output row is zero (the empty sum).

Quantization steps are emulated op for op in numpy float32, which is IEEE
single precision with round-to-nearest-even; everything after the integer
codes is exact or fp64.
"""

from __future__ import annotations

import numpy as np

#: Significand width (implicit bit included) of the row scales, reading R2.
QK_SCALE_BITS = 24  # a plain fp32 scale
V_SCALE_BITS = 4

_ROW_BLOCK = 512  # query rows per block: keeps the [rows, keys] logits small

#: Outlier channels of Q (R19): the magnitude threshold and the most channels kept.
Q_OUTLIER_THRESHOLD = 6.0
Q_OUTLIER_MAX = 16


def default_softmax_scale(d: int) -> np.float32:
    """fp32(1/sqrt(D)), reading R7."""
    return np.float32(1.0 / np.sqrt(np.float64(d)))


def kmean(k16: np.ndarray) -> np.ndarray:
    """Per-channel mean of K over the token axis (K-smoothing statistic, R5).

    ``k16`` is fp16 ``[..., L, D]`` with L >= 1; returns fp32 ``[..., D]``.
    Every fp16 value times 2^24 is an integer of magnitude below 2^40, so the
    int64 sum is exact for any L below 2^23.
    """
    if k16.dtype != np.float16:
        raise TypeError("kmean expects fp16 input")
    L = k16.shape[-2]
    if L < 1:
        raise ValueError("kmean needs at least one token")
    fixed = (k16.astype(np.float64) * 2.0**24).astype(np.int64)
    isum = fixed.sum(axis=-2)
    return (isum.astype(np.float64) / (np.float64(L) * 2.0**24)).astype(np.float32)


def _round_up_significand(t: np.ndarray, bits: int) -> np.ndarray:
    """Smallest fp32 with a ``bits``-bit significand that is >= t (t >= 0,
    finite, normal or zero)."""
    drop = 24 - bits  # fp32 has a 24-bit significand
    u = np.ascontiguousarray(t, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + ((1 << drop) - 1)) & (0xFFFFFFFF ^ ((1 << drop) - 1))).astype(np.uint32)
    return r.view(np.float32)


def quant_rows(x32: np.ndarray, scale_bits: int = QK_SCALE_BITS):
    """Symmetric per-row int8 quantization of fp32 rows (R1-R4).

    ``x32`` is fp32 ``[..., D]``; ``scale_bits`` is 24 for Q and K rows and 4
    for V rows.  Returns ``(codes int8 [..., D], scales fp32 [...])``.
    """
    x32 = np.asarray(x32)
    if x32.dtype != np.float32:
        raise TypeError("quant_rows expects fp32 rows")
    a = np.max(np.abs(x32), axis=-1)
    t = a / np.float32(127.0)
    assert t.dtype == np.float32
    scale = _round_up_significand(t, scale_bits) if scale_bits < 24 else t
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = x32 / safe[..., None]
    assert ratio.dtype == np.float32
    codes = np.clip(np.rint(ratio), -127, 127)
    codes = np.where(scale[..., None] > 0, codes, 0).astype(np.int8)
    return codes, scale.astype(np.float32)


def quant_row_blocks(x32: np.ndarray, block: int = 32):
    """Q quantized per warp (R18): rows ``[..., S, D]`` in blocks of ``block`` rows from
    row 0; each block's scale is ``fp32(max over its rows of max |x| / 127)`` (the Q/K
    rule, no significand rounding), and each row's codes follow R3 against its block's
    scale.  Returns ``(codes int8 [..., S, D], scales fp32 [..., S])`` (a row carries its
    block's scale).
    """
    x32 = np.asarray(x32)
    if x32.dtype != np.float32:
        raise TypeError("quant_row_blocks expects fp32 rows")
    S = x32.shape[-2]
    a = np.max(np.abs(x32), axis=-1)  # [..., S]
    nb = (S + block - 1) // block
    pad = np.zeros(a.shape[:-1] + (nb * block,), dtype=np.float32)
    pad[..., :S] = a
    bmax = pad.reshape(a.shape[:-1] + (nb, block)).max(axis=-1)  # [..., nb]
    t = np.repeat(bmax, block, axis=-1)[..., :S] / np.float32(127.0)
    assert t.dtype == np.float32
    safe = np.where(t > 0, t, np.float32(1.0)).astype(np.float32)
    ratio = x32 / safe[..., None]
    assert ratio.dtype == np.float32
    codes = np.clip(np.rint(ratio), -127, 127)
    codes = np.where(t[..., None] > 0, codes, 0).astype(np.int8)
    return codes, t.astype(np.float32)


def fwht_f32(x32: np.ndarray) -> np.ndarray:
    """Unnormalized fast Walsh-Hadamard transform of the last axis (R13), in fp32,
    stages in the order s = 0, 1, ...: the pair (x[i], x[i + 2^s]) with bit s of i
    clear becomes (x[i] + x[i + 2^s], x[i] - x[i + 2^s]).  Equals ``x @ H`` for the
    Sylvester-Hadamard matrix H (symmetric, entries +-1) up to fp32 rounding."""
    x = np.array(x32, dtype=np.float32, copy=True)
    D = x.shape[-1]
    if D & (D - 1):
        raise ValueError("the row length must be a power of two")
    h = 1
    while h < D:
        y = x.reshape(x.shape[:-1] + (D // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        x = y.reshape(x.shape)
        h *= 2
    return x


def quant_cols(x32: np.ndarray, scale_bits: int = 4):
    """Symmetric int8 quantization of fp32 ``[..., T, D]`` with one scale per column
    (channel) over the T rows (R14): the row rule of :func:`quant_rows` applied along
    the token axis.  Returns ``(codes int8 [..., T, D], scales fp32 [..., D])``."""
    codes, scale = quant_rows(np.ascontiguousarray(np.swapaxes(x32, -1, -2)), scale_bits)
    return np.ascontiguousarray(np.swapaxes(codes, -1, -2)), scale


def q_outlier_channels(qg16):
    """Outlier channels of Q (R19) for one (sequence, kv head): ``qg16`` is fp16
    ``[G, L, D]``, the group's query heads over the sequence's tokens.  A channel is an
    outlier when its largest magnitude exceeds the threshold; at most
    ``Q_OUTLIER_MAX`` of them, the largest magnitudes first, ties to the lower channel.
    Returns the channel indices in increasing order (int64)."""
    qg = np.asarray(qg16)
    if qg.dtype != np.float16:
        raise TypeError("q_outlier_channels expects fp16 input")
    D = qg.shape[-1]
    if qg.size == 0:
        return np.zeros(0, dtype=np.int64)
    a = np.abs(qg.astype(np.float64)).reshape(-1, D).max(axis=0)
    cand = [d for d in range(D) if a[d] > Q_OUTLIER_THRESHOLD]
    cand.sort(key=lambda d: (-a[d], d))
    return np.array(sorted(cand[:Q_OUTLIER_MAX]), dtype=np.int64)


def quantize_qkv(q16, k16, v16, hadamard=False, v_per_channel=False, q_per_block=False,
                 q_outliers=False):
    """Quantize dense BHSD q/k/v as the forward does internally (with ``hadamard``,
    Q and the mean-smoothed K rows rotated first, R13; with ``v_per_channel``, V
    quantized per channel over the tokens, R14; with ``q_per_block``, Q quantized with
    one scale per 32-row block, R18; with ``q_outliers``, Q's outlier channels taken
    out of the int8 part, R19).

    Returns a dict with ``q8, sq, k8, sk, v8, sv, kmean``; ``sv`` is ``[B, Hkv, S]``
    per token or ``[B, Hkv, D]`` per channel.  With ``q_outliers`` it also holds
    ``ochan`` (int64 ``[B, Hkv, 16]``, the outlier channels in increasing order,
    padded with -1) and the outlier part ``qo`` (fp64 ``[B, Hq, S, 16]``) and ``ko``
    (fp64 ``[B, Hkv, S, 16]``): the fp16 inputs at those channels, 0 in the padding.
    """
    if hadamard and q_outliers:
        raise ValueError("the rotation and Q outlier detection do not combine")
    B, Hq, S, D = q16.shape
    Hkv = k16.shape[1]
    G = Hq // Hkv
    q32 = q16.astype(np.float32)
    m = kmean(k16)  # [B, Hkv, D]
    ksm = k16.astype(np.float32) - m[..., None, :]
    assert ksm.dtype == np.float32
    extra = {}
    if q_outliers:
        ochan = np.full((B, Hkv, Q_OUTLIER_MAX), -1, dtype=np.int64)
        qo = np.zeros((B, Hq, S, Q_OUTLIER_MAX))
        ko = np.zeros((B, Hkv, S, Q_OUTLIER_MAX))
        q32 = q32.copy()
        ksm = ksm.copy()
        for b in range(B):
            for g in range(Hkv):
                ch = q_outlier_channels(q16[b, g * G:(g + 1) * G])
                ochan[b, g, :ch.size] = ch
                qo[b, g * G:(g + 1) * G, :, :ch.size] = q16[b, g * G:(g + 1) * G][..., ch]
                ko[b, g, :, :ch.size] = k16[b, g][..., ch]
                q32[b, g * G:(g + 1) * G][..., ch] = 0.0
                ksm[b, g][..., ch] = 0.0
        extra = dict(ochan=ochan, qo=qo, ko=ko)
    qx = fwht_f32(q32) if hadamard else q32
    q8, sq = quant_row_blocks(qx) if q_per_block else quant_rows(qx)
    k8, sk = quant_rows(fwht_f32(ksm) if hadamard else ksm)
    if v_per_channel:
        v8, sv = quant_cols(v16.astype(np.float32), V_SCALE_BITS)
    else:
        v8, sv = quant_rows(v16.astype(np.float32), V_SCALE_BITS)
    return dict(q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv, kmean=m, **extra)


def qk_int32(q8: np.ndarray, k8: np.ndarray) -> np.ndarray:
    """Exact integer scores ``q8 @ k8.T`` for one head (R7).

    Computed with an fp64 matrix product, which is exact here: every partial
    sum is an integer of magnitude at most 127*127*256 < 2^53.
    """
    s = q8.astype(np.float64) @ k8.astype(np.float64).T
    return s.astype(np.int64)


def attn_core(q8, sq, k8, sk, v8, sv, softmax_scale, causal, rows=None, logit_factor=1.0,
              v_per_channel=False, qo=None, ko=None):
    """Attention of one head on quantized operands (R7, R8, R10).

    ``q8 [Sq, D]``, ``k8/v8 [Sk, D]`` int8; ``sq [Sq]``, ``sk [Sk]`` fp32; ``sv [Sk]``
    per key, or ``[D]`` per channel with ``v_per_channel`` (R14).
    ``rows`` optionally selects query rows (each row is independent).
    ``logit_factor`` multiplies every logit (1/D for rotated rows, R13).
    ``qo [Sq, n]``, ``ko [Sk, n]``: the outlier channels' values (R19), whose exact
    products are added to the dequantized scores.
    Returns fp64 ``[len(rows), D]``.
    """
    Sq, Sk = q8.shape[0], k8.shape[0]
    if causal and Sq != Sk:
        raise ValueError("causal attention needs equal query and key lengths")
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    sm = np.float64(np.float32(softmax_scale)) * np.float64(logit_factor)
    if v_per_channel:
        vhat = v8.astype(np.float64) * sv.astype(np.float64)[None, :]
    else:
        vhat = sv.astype(np.float64)[:, None] * v8.astype(np.float64)
    kk = k8.astype(np.float64)
    skd = sk.astype(np.float64)
    out = np.empty((rows.size, q8.shape[1]), dtype=np.float64)
    for r0 in range(0, rows.size, _ROW_BLOCK):
        rr = rows[r0:r0 + _ROW_BLOCK]
        s32 = q8[rr].astype(np.float64) @ kk.T  # exact integers
        if qo is None:
            logits = s32 * sq.astype(np.float64)[rr][:, None] * skd[None, :] * sm
        else:  # fp16 products are exact in fp64, and so is a sum of 16 of them
            deq = s32 * sq.astype(np.float64)[rr][:, None] * skd[None, :]
            logits = (deq + qo[rr] @ ko.T) * sm
        if causal:
            logits = np.where(np.arange(Sk)[None, :] <= rr[:, None], logits, -np.inf)
        mx = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - mx)
        p /= p.sum(axis=1, keepdims=True)
        out[r0:r0 + rr.size] = p @ vhat
    return out


def attn_int8_fwd(q16, k16, v16, causal=True, softmax_scale=None, heads=None, rows=None,
                  hadamard=False, v_per_channel=False, q_per_block=False, q_outliers=False):
    """The dense forward: fp16 ``q[B,Hq,S,D]``, ``k/v[B,Hkv,S,D]`` -> fp64 O.

    ``heads`` (list of (b, h)) and ``rows`` restrict the output to a sample;
    the result then has shape ``[len(heads), len(rows), D]``, otherwise
    ``[B, Hq, S, D]``.  ``hadamard`` selects the rotated variant (R13): Q and K
    rows rotated before quantization and the logits scaled by an extra 1/D.
    ``v_per_channel`` quantizes V per channel (R14), ``q_per_block`` Q per 32-row block
    (R18), ``q_outliers`` detects Q's outlier channels (R19).
    """
    B, Hq, S, D = q16.shape
    Hkv = k16.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    sm = default_softmax_scale(D) if softmax_scale is None else np.float32(softmax_scale)
    qz = quantize_qkv(q16, k16, v16, hadamard, v_per_channel, q_per_block, q_outliers)
    # The 1/D of the rotation multiplies the logits exactly (D is a power of two).
    extra = 1.0 / D if hadamard else 1.0
    sel = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    outs = []
    for b, h in sel:
        g = h // G
        outs.append(attn_core(qz["q8"][b, h], qz["sq"][b, h], qz["k8"][b, g], qz["sk"][b, g],
                              qz["v8"][b, g], qz["sv"][b, g], sm, causal, rows, extra,
                              v_per_channel,
                              qz["qo"][b, h] if q_outliers else None,
                              qz["ko"][b, g] if q_outliers else None))
    o = np.stack(outs)
    if heads is None and rows is None:
        o = o.reshape(B, Hq, S, D)
    return o


def attn_int8_varlen_fwd(q16, k16, v16, cu_seqlens, causal=True, softmax_scale=None,
                         hadamard=False, v_per_channel=False, q_per_block=False,
                         q_outliers=False):
    """The varlen forward (R11): packed ``q[T,Hq,D]``, ``k/v[T,Hkv,D]``.

    Each sequence ``cu[i]:cu[i+1]`` is quantized (its own K mean, its own V channel
    scales with ``v_per_channel``, its own outlier channels with ``q_outliers``) and
    attended independently.  Returns fp64
    ``[T, Hq, D]``.
    """
    T, Hq, D = q16.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for i in range(cu.size - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if b == a:
            continue
        qs = np.ascontiguousarray(q16[a:b].transpose(1, 0, 2))[None]
        ks = np.ascontiguousarray(k16[a:b].transpose(1, 0, 2))[None]
        vs = np.ascontiguousarray(v16[a:b].transpose(1, 0, 2))[None]
        o = attn_int8_fwd(qs, ks, vs, causal, softmax_scale, hadamard=hadamard,
                          v_per_channel=v_per_channel, q_per_block=q_per_block,
                          q_outliers=q_outliers)[0]
        out[a:b] = o.transpose(1, 0, 2)
    return out


def attn_int8_decode(q16, k16, v16, softmax_scale=None, v_format="int8"):
    """Decode (R12): fp16 ``q[B,Hq,D]`` (one token per sequence) against the cache
    built from fp16 ``k/v[B,Hkv,S,D]`` -> fp64 ``[B, Hq, D]``.

    ``v_format`` is ``"int8"`` (V quantized per token) or ``"fp16"`` (V as given).
    """
    B, Hq, D = q16.shape
    Hkv, S = k16.shape[1], k16.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if v_format not in ("int8", "fp16"):
        raise ValueError("v_format must be 'int8' or 'fp16'")
    G = Hq // Hkv
    sm = default_softmax_scale(D) if softmax_scale is None else np.float32(softmax_scale)
    q8, sq = quant_rows(q16.astype(np.float32))  # [B, Hq, D], [B, Hq]
    m = kmean(k16)
    k8, sk = quant_rows(k16.astype(np.float32) - m[..., None, :])
    if v_format == "int8":
        v8, sv = quant_rows(v16.astype(np.float32), V_SCALE_BITS)
    else:  # the fp16 values are the dequantized V: unit scales, fp64 "codes"
        v8, sv = v16.astype(np.float64), np.ones((B, Hkv, S), dtype=np.float32)
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            out[b, h] = attn_core(q8[b, h][None], sq[b, h][None], k8[b, g], sk[b, g],
                                  v8[b, g], sv[b, g], sm, False)[0]
    return out


def kvcache_quantize(k16, v16, n_fill, v_format="int8"):
    """The contents of a decode cache (R12, R20): fp16 ``k/v[B,Hkv,S,D]`` hold every
    token the cache holds, tokens ``[0, n_fill)`` filled and the later ones appended.

    Returns ``(k8, sk, v8, sv, mean)``: K rows quantized against the mean of the
    filled tokens' K (R5), V rows per token (R2; ``v_format="fp16"``: the fp16
    values as fp64 "codes" with unit scales), and that fp32 mean ``[B, Hkv, D]``.
    """
    if v_format not in ("int8", "fp16"):
        raise ValueError("v_format must be 'int8' or 'fp16'")
    S = k16.shape[2]
    if not 1 <= n_fill <= S:
        raise ValueError("need 1 <= n_fill <= S")
    m = kmean(k16[:, :, :n_fill])
    k8, sk = quant_rows(k16.astype(np.float32) - m[..., None, :])
    if v_format == "int8":
        v8, sv = quant_rows(v16.astype(np.float32), V_SCALE_BITS)
    else:
        v8, sv = v16.astype(np.float64), np.ones(v16.shape[:3], dtype=np.float32)
    return k8, sk, v8, sv, m


def attn_int8_decode_cache(q16, k16, v16, n_fill, lens, softmax_scale=None, v_format="int8"):
    """Decode against a grown cache (R12, R20): fp16 ``q[B,Hq,D]``, the cache of
    :func:`kvcache_quantize` over ``k/v[B,Hkv,S,D]`` with ``n_fill`` filled tokens, and
    ``lens[B]`` (0 <= lens[b] <= S): sequence b's query rows attend its cached tokens
    ``[0, lens[b])``.  Returns fp64 ``[B, Hq, D]``; rows of a sequence with no token
    are zero.
    """
    B, Hq, D = q16.shape
    Hkv, S = k16.shape[1], k16.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    lens = np.asarray(lens, dtype=np.int64)
    if lens.shape != (B,) or (lens < 0).any() or (lens > S).any():
        raise ValueError("need lens[B] with 0 <= lens[b] <= S")
    G = Hq // Hkv
    sm = default_softmax_scale(D) if softmax_scale is None else np.float32(softmax_scale)
    q8, sq = quant_rows(q16.astype(np.float32))
    k8, sk, v8, sv, _ = kvcache_quantize(k16, v16, n_fill, v_format)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(Hq):
            g = h // G
            out[b, h] = attn_core(q8[b, h][None], sq[b, h][None], k8[b, g, :n], sk[b, g, :n],
                                  v8[b, g, :n], sv[b, g, :n], sm, False)[0]
    return out


def attn_exact(q, k, v, causal=True, softmax_scale=None, heads=None, rows=None):
    """Unquantized attention in fp64 (reference for the quantization bound).

    ``q[B,Hq,S,D]``, ``k/v[B,Hkv,S,D]`` of any float dtype.  ``heads`` (list of (b, h))
    and ``rows`` restrict the output to a sample of shape ``[len(heads), len(rows), D]``,
    as in :func:`attn_int8_fwd`; otherwise it is ``[B, Hq, S, D]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    sm = np.float64(default_softmax_scale(D) if softmax_scale is None else np.float32(softmax_scale))
    sel = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    rr = np.arange(S) if rows is None else np.asarray(rows)
    out = np.empty((len(sel), rr.size, D))
    for n, (b, h) in enumerate(sel):
        lg = (q[b, h][rr] @ k[b, h // G].T) * sm
        if causal:
            lg = np.where(np.arange(k.shape[2])[None, :] <= rr[:, None], lg, -np.inf)
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[n] = p @ v[b, h // G]
    if heads is None and rows is None:
        out = out.reshape(B, Hq, S, D)
    return out
