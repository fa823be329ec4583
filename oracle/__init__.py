"""CPU oracle for the INT8 W8A8 attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything under ``oracle/``; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library: no kernels, headers, helpers, tables or pre/post-processing.

The method it defines comes from the "SuperL8" README (the page titled
"SuperL8 - DP4A FlashAttention-2 and GEMM for Volta GPUs"):

* *Attention kernels* table, row ``attn_int8_fwd``: W8A8 FlashAttention-2
  forward, causal, GQA/MQA, head dims 32/64/128/256.
* *Attention kernels* table, row ``attn_varlen_fwd``: variable-length
  (ragged, non-tile-multiple) prefill.
* *Attention kernels* table, row ``attn_decode``: split-KV decode with an int8
  KV cache, in its int8-V and fp16-V variants (one query token per sequence), over
  a cache that grows by appended tokens (``attn_int8_decode_cache``).
* *Attention kernels* table, row ``attn_bwd``, and the *Infrastructure* table's
  autograd row: the backward of the differentiable int8 attention (gradient of exact
  attention, the quantization taken as the identity).
* *Supporting kernels* table, row ``quant_rowwise``: symmetric per-row int8
  quantization.
* *Quantization* table, rows "Per-row int8" (symmetric, K-smoothing) and
  "V per-channel / per-token" (V is quantized per token here).
* *Quantization* table, row "Hadamard rotation": Q and K rows rotated before
  quantization (the ``hadamard`` option of the forward).
* *Quantization* table, row "V per-channel / per-token": V quantized per token
  (default) or per channel over the tokens (the ``v_per_channel`` option).
* *Quantization* table, row "Per-row int8" (Q outlier detection) and the
  *Attention kernels* table's ``attn_w8a8_fwd`` row (per-warp, outlier-aware): Q
  quantized per 32-row block, and Q's outlier channels multiplied in fp16 beside the
  int8 product (the ``q_per_block`` and ``q_outliers`` options).
* *Quick start*: ``attn_int8_fwd(q, k, v, causal=True)`` takes fp16
  ``q[B,Hq,S,D]``, ``k/v[B,Hkv,S,D]`` and quantizes internally.

Where the page is silent the oracle takes the readings listed in the
module docstring of :mod:`oracle.attn_ref`.

Pinning status: every public function is pinned by ``tests/test_oracle_pins.py``
against exact rational arithmetic, brute force, library routines or closed
forms, except the fp32 rounding of the fp16 output, which only the stated
tolerance constrains.
"""

from .attn_ref import (  # noqa: F401
    QK_SCALE_BITS,
    V_SCALE_BITS,
    default_softmax_scale,
    kmean,
    quant_rows,
    quant_cols,
    quant_row_blocks,
    q_outlier_channels,
    Q_OUTLIER_THRESHOLD,
    Q_OUTLIER_MAX,
    quantize_qkv,
    fwht_f32,
    qk_int32,
    attn_core,
    attn_int8_fwd,
    attn_int8_decode,
    attn_int8_decode_cache,
    kvcache_quantize,
    attn_int8_varlen_fwd,
    attn_exact,
)
from .attn_bwd import attn_bwd_exact  # noqa: F401
