"""INT8 W8A8 FlashAttention forward for AMD MI355X (gfx950).

Thin ctypes binding of ``libi8attn.so`` (the C ABI in ``include/i8attn.h``).  It
only checks and marshals arguments: every step of the forward runs in the HIP
kernels of the library.  PyTorch provides device memory and the stream.  There is
no CPU fallback: if the library is missing or no GPU is present, the calls raise.

Entry points (same names as the C ABI):

* :func:`quant_rowwise_i8` - symmetric per-row int8 quantization.
* :func:`attn_int8_fwd` - dense forward, q ``[B,Hq,S,D]``, k/v ``[B,Hkv,S,D]``.
* :func:`attn_int8_fwd_hadamard` - the same with Q and K Hadamard-rotated first.
* :func:`attn_int8_fwd_ex` / :func:`attn_int8_varlen_fwd_ex` - the forwards with variant
  flags (``FWD_HADAMARD``, ``FWD_V_PER_CHANNEL``, ``FWD_Q_PER_BLOCK``).
* :func:`attn_int8_varlen_fwd` - packed ragged batch, q ``[T,Hq,D]`` + ``cu_seqlens``.
* :func:`attn_int8_debug_qk` - the forward's exact int32 scores and scales.
* :func:`attn_int8_kvcache_fill` / :func:`attn_int8_decode` - an int8 KV cache and
  split-KV decode of one query token per sequence against it.
* :func:`attn_bwd` - the backward (gradients of the attention, the quantization taken
  as the identity); :class:`Int8Attention` / :func:`int8_attention` - the forward as a
  ``torch.autograd.Function`` with that backward.
"""

from __future__ import annotations

import ctypes
import math
import os
import re

import torch

__all__ = [
    "quant_rowwise_i8", "attn_int8_fwd", "attn_int8_varlen_fwd", "attn_int8_debug_qk",
    "attn_int8_varlen_debug_qk", "attn_int8_fwd_noalloc",
    "attn_int8_fwd_hadamard", "attn_int8_fwd_ex", "attn_int8_varlen_fwd_ex", "FWD_HADAMARD",
    "FWD_V_PER_CHANNEL", "FWD_Q_PER_BLOCK", "FWD_Q_OUTLIERS", "attn_int8_prepare_kv", "attn_int8_prepare_q",
    "attn_int8_attend", "attn_int8_fwd_prepared",
    "attn_int8_workspace_bytes", "attn_int8_varlen_workspace_bytes", "library_path",
    "load_library", "SCALE_FP32", "SCALE_V4", "HEAD_DIMS", "attn_int8_kvcache_bytes",
    "attn_int8_kvcache_fill", "attn_int8_decode_workspace_bytes", "attn_int8_decode",
    "attn_int8_kvcache_fill_prefix", "attn_int8_kvcache_append", "attn_int8_decode_lens", "KVCache",
    "VCACHE_INT8", "VCACHE_FP16", "attn_bwd", "attn_bwd_workspace_bytes", "Int8Attention",
    "int8_attention",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libi8attn.so")
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "i8attn.h")

SCALE_FP32 = 24
SCALE_V4 = 4
HEAD_DIMS = (32, 64, 128, 256)
FWD_HADAMARD = 1
FWD_V_PER_CHANNEL = 2
FWD_Q_PER_BLOCK = 4
FWD_Q_OUTLIERS = 8
VCACHE_INT8 = 1
VCACHE_FP16 = 2
_VFORMATS = {"int8": VCACHE_INT8, "fp16": VCACHE_FP16}

_c_i32, _c_i64, _c_sz, _c_f32, _c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                        ctypes.c_float, ctypes.c_void_p)
_SIGS = {
    "quant_rowwise_i8": (_c_i32, [_c_vp, _c_i64, _c_i32, _c_vp, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp]),
    "attn_int8_workspace_bytes": (_c_sz, [_c_i32] * 5),
    "attn_int8_fwd": (_c_i32, [_c_vp] * 4 + [_c_i32] * 5 + [_c_f32, _c_i32, _c_vp, _c_sz, _c_vp]),
    "attn_int8_varlen_workspace_bytes": (_c_sz, [_c_i32, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32]),
    "attn_int8_varlen_fwd": (_c_i32, [_c_vp] * 5 + [_c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_i32,
                                                     _c_f32, _c_i32, _c_vp, _c_sz, _c_vp]),
    "attn_int8_debug_qk_ex": (_c_i32, [_c_vp] * 4 + [_c_i32, _c_i32, _c_i64] + [_c_i32] * 10
                              + [_c_vp] * 8 + [_c_vp, _c_sz, _c_vp]),
    "attn_int8_debug_qk": (_c_i32, [_c_vp] * 3 + [_c_i32] * 11 + [_c_vp] * 5 + [_c_i32, _c_vp,
                                                                                 _c_sz, _c_vp]),
    "attn_int8_fwd_hadamard": (_c_i32, [_c_vp] * 4 + [_c_i32] * 5 + [_c_f32, _c_i32, _c_vp, _c_sz,
                                                                    _c_vp]),
    "attn_int8_fwd_noalloc": (_c_i32, [_c_vp] * 4 + [_c_i32] * 5 + [_c_f32, _c_i32, _c_vp]),
    "attn_int8_fwd_ex": (_c_i32, [_c_vp] * 4 + [_c_i32] * 5 + [_c_f32, _c_i32, _c_i32, _c_vp, _c_sz,
                                                              _c_vp]),
    "attn_int8_varlen_fwd_ex": (_c_i32, [_c_vp] * 5 + [_c_i32, _c_i32, _c_i64, _c_i32, _c_i32,
                                                        _c_i32, _c_f32, _c_i32, _c_i32, _c_vp, _c_sz,
                                                        _c_vp]),
    "attn_int8_prepare_kv": (_c_i32, [_c_vp] * 2 + [_c_i32] * 5 + [_c_vp, _c_sz, _c_vp]),
    "attn_int8_prepare_q": (_c_i32, [_c_vp] + [_c_i32] * 5 + [_c_vp, _c_sz, _c_vp]),
    "attn_int8_attend": (_c_i32, [_c_vp] + [_c_i32] * 5 + [_c_f32, _c_i32, _c_vp, _c_sz, _c_vp]),
    "attn_int8_fwd_prepared": (_c_i32, [_c_vp] * 2 + [_c_i32] * 5 + [_c_f32, _c_i32, _c_vp, _c_sz,
                                                                     _c_vp]),
    "attn_int8_kvcache_bytes": (_c_sz, [_c_i32] * 5),
    "attn_int8_kvcache_fill": (_c_i32, [_c_vp] * 2 + [_c_i32] * 5 + [_c_vp, _c_sz, _c_vp]),
    "attn_int8_kvcache_fill_prefix": (_c_i32, [_c_vp] * 2 + [_c_i32] * 6 + [_c_vp, _c_sz, _c_vp]),
    "attn_int8_kvcache_append": (_c_i32, [_c_vp] * 2 + [_c_i32] * 3 + [_c_vp] + [_c_i32] * 3
                                 + [_c_vp, _c_sz, _c_vp]),
    "attn_int8_decode_lens": (_c_i32, [_c_vp] * 2 + [_c_i32] * 5 + [_c_f32, _c_i32, _c_vp, _c_vp,
                                                                    _c_sz, _c_vp, _c_sz, _c_vp]),
    "attn_int8_decode_workspace_bytes": (_c_sz, [_c_i32] * 6),
    "attn_int8_decode": (_c_i32, [_c_vp] * 2 + [_c_i32] * 5 + [_c_f32, _c_i32, _c_vp, _c_sz,
                                                               _c_vp, _c_sz, _c_vp]),
    "attn_bwd_workspace_bytes": (_c_sz, [_c_i32] * 5),
    "attn_bwd": (_c_i32, [_c_vp] * 7 + [_c_i32] * 5 + [_c_f32, _c_i32, _c_vp, _c_sz, _c_vp]),
    "i8a_status_string": (ctypes.c_char_p, [_c_i32]),
    "i8a_last_error": (ctypes.c_char_p, []),
}

_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libi8attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m int8_w8a8_flashattention_amd.build_lib` (there is no CPU fallback)")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions():
    """Names of the functions declared in include/i8attn.h."""
    text = open(_HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|size_t|i8a_status)\s+(\w+)\s*\(",
                                 text, re.M)))


def _check(status: int, what: str):
    if status != 0:
        lib = load_library()
        raise RuntimeError(f"{what} failed: {lib.i8a_status_string(status).decode()}: "
                           f"{lib.i8a_last_error().decode()}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_gpu_fp16(name, t, ndim):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float16:
        raise ValueError(f"{name} must be float16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _scale(softmax_scale, D):
    s = (1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale)
    return ctypes.c_float(s)  # rounded to fp32 here, the value the kernels use


def _workspace(workspace, nbytes, dev):
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must be a buffer of >= {nbytes} bytes on {dev}")
    return workspace


def quant_rowwise_i8(x, mean=None, rows_per_group=None, scale_bits=SCALE_FP32):
    """Per-row symmetric int8 codes and fp32 scales of fp16 ``x[..., d]``.

    ``mean`` (fp32 ``[groups, d]``) is subtracted from row r in group
    ``r // rows_per_group`` before quantizing (the K-smoothing subtraction).
    """
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float16 or not x.is_cuda:
        raise ValueError("x must be a float16 GPU tensor")
    if not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x must be contiguous with at least one dim")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    codes = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if mean is not None:
        if mean.dtype != torch.float32 or mean.device != x.device or not mean.is_contiguous():
            raise ValueError("mean must be a contiguous float32 tensor on x's device")
        if mean.shape[-1] != d:
            raise ValueError("mean's last dim must match x's")
        if rows_per_group is None or rows_per_group < 1:
            raise ValueError("rows_per_group must be >= 1 with mean")
        if mean.numel() // d < -(-rows // rows_per_group):
            raise ValueError("mean has fewer groups than the rows need")
    lib = load_library()
    with torch.cuda.device(x.device):
        st = lib.quant_rowwise_i8(_ptr(x), rows, d, _ptr(mean), rows_per_group or 1, scale_bits,
                                  _ptr(codes), _ptr(scales), _stream(x.device))
    _check(st, "quant_rowwise_i8")
    return codes, scales


def attn_int8_workspace_bytes(B, Hq, Hkv, S, D) -> int:
    return int(load_library().attn_int8_workspace_bytes(B, Hq, Hkv, S, D))


def attn_int8_varlen_workspace_bytes(nseq, total_tokens, max_seqlen, Hq, Hkv, D) -> int:
    return int(load_library().attn_int8_varlen_workspace_bytes(nseq, total_tokens, max_seqlen,
                                                               Hq, Hkv, D))


def _dense_shapes(q, k, v):
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_gpu_fp16(n, t, 4)
    B, Hq, S, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError(f"k/v must be [B, Hkv, S, D] matching q {tuple(q.shape)}; "
                         f"got {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    Hkv = k.shape[1]
    if D not in HEAD_DIMS:
        raise ValueError(f"head dim {D} not in {HEAD_DIMS}")
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} must be a multiple of Hkv={Hkv}")
    return B, Hq, Hkv, S, D


def attn_int8_fwd(q, k, v, causal=True, softmax_scale=None, out=None, workspace=None):
    """INT8 W8A8 attention forward; returns fp16 ``out[B,Hq,S,D]``."""
    B, Hq, Hkv, S, D = _dense_shapes(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_gpu_fp16("out", out, 4)
        if out.shape != q.shape or out.device != q.device:
            raise ValueError("out must match q")
    lib = load_library()
    nbytes = lib.attn_int8_workspace_bytes(B, Hq, Hkv, S, D)
    ws = _workspace(workspace, nbytes, q.device)
    with torch.cuda.device(q.device):
        st = lib.attn_int8_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                               _scale(softmax_scale, D), int(bool(causal)), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(q.device))
    _check(st, "attn_int8_fwd")
    return out


def attn_int8_fwd_noalloc(q, k, v, out, causal=True, softmax_scale=None):
    """:func:`attn_int8_fwd` into the caller's fp16 ``out[B,Hq,S,D]`` with the library's
    own per-GPU scratch as the workspace: the call allocates nothing (for callers that
    cannot).  Calls that overlap on one GPU race (they share the scratch)."""
    B, Hq, Hkv, S, D = _dense_shapes(q, k, v)
    _need_gpu_fp16("out", out, 4)
    if out.shape != q.shape or out.device != q.device:
        raise ValueError("out must match q")
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_int8_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                                       _scale(softmax_scale, D), int(bool(causal)),
                                       _stream(q.device))
    _check(st, "attn_int8_fwd_noalloc")
    return out


def attn_int8_fwd_ex(q, k, v, causal=True, flags=0, softmax_scale=None, out=None,
                     workspace=None):
    """:func:`attn_int8_fwd` with variant ``flags`` (``FWD_HADAMARD``: Q and K rows
    Hadamard-rotated before quantization; ``FWD_V_PER_CHANNEL``: V quantized per channel
    over the tokens); returns fp16 ``out[B,Hq,S,D]``."""
    B, Hq, Hkv, S, D = _dense_shapes(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_gpu_fp16("out", out, 4)
        if out.shape != q.shape or out.device != q.device:
            raise ValueError("out must match q")
    lib = load_library()
    nbytes = lib.attn_int8_workspace_bytes(B, Hq, Hkv, S, D)
    ws = _workspace(workspace, nbytes, q.device)
    with torch.cuda.device(q.device):
        st = lib.attn_int8_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                                  _scale(softmax_scale, D), int(bool(causal)), int(flags),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(q.device))
    _check(st, "attn_int8_fwd_ex")
    return out


def attn_int8_fwd_hadamard(q, k, v, causal=True, softmax_scale=None, out=None, workspace=None):
    """:func:`attn_int8_fwd` with Q and K rows Hadamard-rotated before quantization (an
    incoherence rotation for outlier channels); returns fp16 ``out[B,Hq,S,D]``."""
    B, Hq, Hkv, S, D = _dense_shapes(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_gpu_fp16("out", out, 4)
        if out.shape != q.shape or out.device != q.device:
            raise ValueError("out must match q")
    lib = load_library()
    nbytes = lib.attn_int8_workspace_bytes(B, Hq, Hkv, S, D)
    ws = _workspace(workspace, nbytes, q.device)
    with torch.cuda.device(q.device):
        st = lib.attn_int8_fwd_hadamard(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                                        _scale(softmax_scale, D), int(bool(causal)), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(q.device))
    _check(st, "attn_int8_fwd_hadamard")
    return out


def attn_int8_prepare_kv(k, v, Hq, workspace=None):
    """K/V phase of :func:`attn_int8_fwd`: K-smoothing mean and K/V quantization of
    dense k/v ``[B,Hkv,S,D]`` into a workspace, returned for
    :func:`attn_int8_fwd_prepared` (or :func:`attn_int8_prepare_q` and
    :func:`attn_int8_attend`)."""
    for n, t in (("k", k), ("v", v)):
        _need_gpu_fp16(n, t, 4)
    if k.shape != v.shape or k.device != v.device:
        raise ValueError("k and v must match")
    B, Hkv, S, D = k.shape
    if D not in HEAD_DIMS or Hq % Hkv:
        raise ValueError("bad head dim or Hq")
    lib = load_library()
    ws = _workspace(workspace, lib.attn_int8_workspace_bytes(B, Hq, Hkv, S, D), k.device)
    with torch.cuda.device(k.device):
        st = lib.attn_int8_prepare_kv(_ptr(k), _ptr(v), B, Hq, Hkv, S, D, _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(k.device))
    _check(st, "attn_int8_prepare_kv")
    return ws


def attn_int8_prepare_q(q, Hkv, workspace):
    """Q phase of :func:`attn_int8_fwd`: quantization of dense q ``[B,Hq,S,D]`` into a
    workspace sized for the same problem (e.g. one from :func:`attn_int8_prepare_kv`)."""
    _need_gpu_fp16("q", q, 4)
    B, Hq, S, D = q.shape
    if D not in HEAD_DIMS or Hkv < 1 or Hq % Hkv:
        raise ValueError("bad head dim or Hkv")
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_int8_prepare_q(_ptr(q), B, Hq, Hkv, S, D, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(q.device))
    _check(st, "attn_int8_prepare_q")
    return workspace


def attn_int8_attend(workspace, B, Hq, Hkv, S, D, causal=True, softmax_scale=None, out=None):
    """Attention phase of :func:`attn_int8_fwd` over a workspace holding prepared Q, K
    and V for these sizes; returns (or fills) fp16 ``out [B,Hq,S,D]``."""
    if D not in HEAD_DIMS or Hkv < 1 or Hq % Hkv:
        raise ValueError("bad head dim or Hkv")
    if out is None:
        out = torch.empty((B, Hq, S, D), dtype=torch.float16, device=workspace.device)
    _need_gpu_fp16("out", out, 4)
    if tuple(out.shape) != (B, Hq, S, D):
        raise ValueError("out must be [B, Hq, S, D]")
    lib = load_library()
    with torch.cuda.device(out.device):
        st = lib.attn_int8_attend(_ptr(out), B, Hq, Hkv, S, D, _scale(softmax_scale, D),
                                  int(bool(causal)), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _stream(out.device))
    _check(st, "attn_int8_attend")
    return out


def attn_int8_fwd_prepared(q, Hkv, workspace, causal=True, softmax_scale=None, out=None):
    """Q and attention phases of :func:`attn_int8_fwd`: dense q ``[B,Hq,S,D]`` against a
    workspace filled by :func:`attn_int8_prepare_kv` for the same sizes."""
    _need_gpu_fp16("q", q, 4)
    B, Hq, S, D = q.shape
    if D not in HEAD_DIMS or Hkv < 1 or Hq % Hkv:
        raise ValueError("bad head dim or Hkv")
    if out is None:
        out = torch.empty_like(q)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_int8_fwd_prepared(_ptr(q), _ptr(out), B, Hq, Hkv, S, D,
                                        _scale(softmax_scale, D), int(bool(causal)),
                                        _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(q.device))
    _check(st, "attn_int8_fwd_prepared")
    return out


def attn_int8_varlen_fwd(q, k, v, cu_seqlens, max_seqlen, causal=True, softmax_scale=None,
                         out=None, workspace=None):
    """See :func:`attn_int8_varlen_fwd_ex` (no variant flags)."""
    return attn_int8_varlen_fwd_ex(q, k, v, cu_seqlens, max_seqlen, causal, 0, softmax_scale,
                                   out, workspace)


def attn_int8_varlen_fwd_ex(q, k, v, cu_seqlens, max_seqlen, causal=True, flags=0,
                            softmax_scale=None, out=None, workspace=None):
    """Forward over packed sequences: q ``[T,Hq,D]``, k/v ``[T,Hkv,D]``, int32
    ``cu_seqlens[nseq+1]`` on the same GPU; ``max_seqlen`` (host int) bounds
    every sequence length.  Returns fp16 ``out[T,Hq,D]``."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_gpu_fp16(n, t, 3)
    T, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != T or k.shape[2] != D:
        raise ValueError("k/v must be [T, Hkv, D] matching q")
    Hkv = k.shape[1]
    if D not in HEAD_DIMS:
        raise ValueError(f"head dim {D} not in {HEAD_DIMS}")
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} must be a multiple of Hkv={Hkv}")
    if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32
            or cu_seqlens.device != q.device or cu_seqlens.dim() != 1
            or cu_seqlens.numel() < 2 or not cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 [nseq+1] tensor on q's device")
    nseq = cu_seqlens.numel() - 1
    max_seqlen = int(max_seqlen)
    if out is None:
        out = torch.empty_like(q)
    lib = load_library()
    nbytes = lib.attn_int8_varlen_workspace_bytes(nseq, T, max_seqlen, Hq, Hkv, D)
    if nbytes == 0 and T > 0:
        raise ValueError("invalid varlen sizes")
    ws = _workspace(workspace, nbytes, q.device)
    with torch.cuda.device(q.device):
        st = lib.attn_int8_varlen_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(cu_seqlens),
                                         nseq, max_seqlen, T, Hq, Hkv, D,
                                         _scale(softmax_scale, D), int(bool(causal)), int(flags),
                                         _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(q.device))
    _check(st, "attn_int8_varlen_fwd_ex")
    return out


def _debug_call(q, k, v, cu, nseq, max_len, T, Hq, Hkv, D, flags, seq, h, row0, rows, col0,
                cols, nbytes, workspace):
    dev = q.device
    vch = bool(flags & FWD_V_PER_CHANNEL)
    r = dict(s32=torch.zeros((rows, cols), dtype=torch.int32, device=dev),
             qscale=torch.zeros(rows, dtype=torch.float32, device=dev),
             kscale=torch.zeros(cols, dtype=torch.float32, device=dev),
             kmean=torch.zeros(D, dtype=torch.float32, device=dev),
             vhat=torch.zeros((cols, D), dtype=torch.float16, device=dev))
    if vch:
        r["vchan"] = torch.zeros(D, dtype=torch.float32, device=dev)
    else:
        r["vscale"] = torch.zeros(cols, dtype=torch.float32, device=dev)
    if flags & FWD_Q_OUTLIERS:
        r["ochan"] = torch.zeros(16, dtype=torch.int32, device=dev)
    lib = load_library()
    ws = _workspace(workspace, nbytes, dev)
    with torch.cuda.device(dev):
        st = lib.attn_int8_debug_qk_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(cu), nseq, max_len, T, Hq, Hkv, D, int(flags), seq, h,
            row0, rows, col0, cols, _ptr(r["s32"]), _ptr(r["qscale"]), _ptr(r["kscale"]),
            _ptr(r.get("vscale")), _ptr(r["kmean"]), _ptr(r["vhat"]), _ptr(r.get("vchan")),
            _ptr(r.get("ochan")),
            _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check(st, "attn_int8_debug_qk_ex")
    return r


def attn_int8_debug_qk(q, k, v, b, h, row0, rows, col0, cols, workspace=None, hadamard=False,
                       flags=None):
    """The dense forward's exact int32 scores ``S32[row0:row0+rows, col0:col0+cols]``
    of (batch b, query head h), with the row scales, the K mean and the prepared V rows
    it used (``flags``: the variant flags of :func:`attn_int8_fwd_ex`; ``hadamard`` is
    the same as ``flags=FWD_HADAMARD``).  Returns a dict of tensors: ``s32``,
    ``qscale``, ``kscale``, ``kmean``, ``vhat`` (fp16 ``[cols, D]``) and ``vscale``
    (per token) or ``vchan`` (per channel, with ``FWD_V_PER_CHANNEL``), and with
    ``FWD_Q_OUTLIERS`` ``ochan`` (int32 ``[16]``: the kv group's Q outlier channels,
    -1 padded; the scores and scales are then the int8 part's)."""
    B, Hq, Hkv, S, D = _dense_shapes(q, k, v)
    if flags is None:
        flags = FWD_HADAMARD if hadamard else 0
    nbytes = load_library().attn_int8_workspace_bytes(B, Hq, Hkv, S, D)
    return _debug_call(q, k, v, None, B, S, B * S, Hq, Hkv, D, flags, b, h, row0, rows, col0,
                       cols, nbytes, workspace)


def attn_int8_varlen_debug_qk(q, k, v, cu_seqlens, max_seqlen, seq, h, row0, rows, col0, cols,
                              flags=0, workspace=None):
    """:func:`attn_int8_debug_qk` for the varlen forward: sequence ``seq`` of the packed
    batch, rows and keys counted from its first token (entries past its length stay 0)."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_gpu_fp16(n, t, 3)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if D not in HEAD_DIMS or Hkv < 1 or Hq % Hkv:
        raise ValueError("bad head dim or Hq/Hkv")
    if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32
            or cu_seqlens.device != q.device or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2):
        raise ValueError("cu_seqlens must be an int32 [nseq+1] tensor on q's device")
    nseq = cu_seqlens.numel() - 1
    nbytes = load_library().attn_int8_varlen_workspace_bytes(nseq, T, int(max_seqlen), Hq, Hkv, D)
    return _debug_call(q, k, v, cu_seqlens, nseq, int(max_seqlen), T, Hq, Hkv, D, flags, seq, h,
                       row0, rows, col0, cols, nbytes, workspace)


def _vformat(v_format):
    if v_format not in _VFORMATS:
        raise ValueError(f"v_format must be one of {sorted(_VFORMATS)}")
    return _VFORMATS[v_format]


def attn_int8_kvcache_bytes(B, Hkv, S, D, v_format="int8") -> int:
    return int(load_library().attn_int8_kvcache_bytes(B, Hkv, S, D, _vformat(v_format)))


def attn_int8_decode_workspace_bytes(B, Hq, Hkv, S, D, v_format="int8") -> int:
    return int(load_library().attn_int8_decode_workspace_bytes(B, Hq, Hkv, S, D,
                                                               _vformat(v_format)))


class KVCache:
    """A filled decode cache: the device buffer and the sizes it was built for."""

    def __init__(self, buf, B, Hkv, S, D, v_format):
        self.buf, self.B, self.Hkv, self.S, self.D, self.v_format = buf, B, Hkv, S, D, v_format

    @property
    def nbytes(self) -> int:
        return self.buf.numel() * self.buf.element_size()


def attn_int8_kvcache_fill(k, v, v_format="int8", cache=None):
    """Quantize fp16 ``k, v [B,Hkv,S,D]`` into a decode cache (K with its K-smoothing
    mean, per-row int8; V per-token int8 or kept in fp16).  Returns a :class:`KVCache`
    (``cache``, a uint8 buffer of at least :func:`attn_int8_kvcache_bytes` bytes, is
    reused when given)."""
    for n, t in (("k", k), ("v", v)):
        _need_gpu_fp16(n, t, 4)
    if k.shape != v.shape or k.device != v.device:
        raise ValueError("k and v must match")
    B, Hkv, S, D = k.shape
    vf = _vformat(v_format)
    lib = load_library()
    nbytes = lib.attn_int8_kvcache_bytes(B, Hkv, S, D, vf)
    if nbytes == 0:
        raise ValueError(f"invalid cache sizes B={B} Hkv={Hkv} S={S} D={D}")
    buf = _workspace(cache, nbytes, k.device)
    with torch.cuda.device(k.device):
        st = lib.attn_int8_kvcache_fill(_ptr(k), _ptr(v), B, Hkv, S, D, vf, _ptr(buf),
                                        buf.numel() * buf.element_size(), _stream(k.device))
    _check(st, "attn_int8_kvcache_fill")
    return KVCache(buf, B, Hkv, S, D, v_format)


def attn_int8_kvcache_fill_prefix(k, v, S, v_format="int8", cache=None):
    """A decode cache of capacity ``S`` tokens whose first ``k.shape[2]`` slots are filled
    from fp16 ``k, v [B,Hkv,S_fill,D]`` (the K-smoothing mean over those tokens); later
    slots hold zeros until :func:`attn_int8_kvcache_append` writes them.  Returns a
    :class:`KVCache`."""
    for n, t in (("k", k), ("v", v)):
        _need_gpu_fp16(n, t, 4)
    if k.shape != v.shape or k.device != v.device:
        raise ValueError("k and v must match")
    B, Hkv, S_fill, D = k.shape
    vf = _vformat(v_format)
    lib = load_library()
    nbytes = lib.attn_int8_kvcache_bytes(B, Hkv, S, D, vf)
    if nbytes == 0:
        raise ValueError(f"invalid cache sizes B={B} Hkv={Hkv} S={S} D={D}")
    buf = _workspace(cache, nbytes, k.device)
    with torch.cuda.device(k.device):
        st = lib.attn_int8_kvcache_fill_prefix(_ptr(k), _ptr(v), B, Hkv, S_fill, S, D, vf,
                                               _ptr(buf), buf.numel() * buf.element_size(),
                                               _stream(k.device))
    _check(st, "attn_int8_kvcache_fill_prefix")
    return KVCache(buf, B, Hkv, S, D, v_format)


def _need_gpu_i32(name, t, B):
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.int32
            and t.is_contiguous() and tuple(t.shape) == (B,)):
        raise ValueError(f"{name} must be a contiguous int32 CUDA tensor of shape ({B},)")


def attn_int8_kvcache_append(cache, k, v, pos):
    """Append fp16 ``k, v [B,Hkv,n,D]`` to a :class:`KVCache`: token i of sequence b goes to
    slot ``pos[b] + i`` (``pos`` an int32 CUDA tensor ``[B]``); slots outside the capacity
    are not written."""
    if not isinstance(cache, KVCache):
        raise ValueError("cache must come from attn_int8_kvcache_fill or _fill_prefix")
    for n, t in (("k", k), ("v", v)):
        _need_gpu_fp16(n, t, 4)
    if k.shape != v.shape or k.device != v.device or cache.buf.device != k.device:
        raise ValueError("k and v must match each other and the cache's device")
    B, Hkv, n, D = k.shape
    if (B, Hkv, D) != (cache.B, cache.Hkv, cache.D):
        raise ValueError("k/v do not match the cache")
    _need_gpu_i32("pos", pos, B)
    lib = load_library()
    with torch.cuda.device(k.device):
        st = lib.attn_int8_kvcache_append(_ptr(k), _ptr(v), B, Hkv, n, _ptr(pos), cache.S, D,
                                          _vformat(cache.v_format), _ptr(cache.buf),
                                          cache.nbytes, _stream(k.device))
    _check(st, "attn_int8_kvcache_append")


def attn_int8_decode_lens(q, cache, lens, softmax_scale=None, out=None, workspace=None):
    """:func:`attn_int8_decode` where sequence b attends its first ``lens[b]`` cached
    tokens (``lens`` an int32 CUDA tensor ``[B]``; a sequence with none gets zeros)."""
    return attn_int8_decode(q, cache, softmax_scale, out, workspace, lens=lens)


def attn_int8_decode(q, cache, softmax_scale=None, out=None, workspace=None, lens=None):
    """One decode step: fp16 ``q [B,Hq,D]`` (the new token's query rows) against a
    :class:`KVCache`; returns fp16 ``out [B,Hq,D]``.  With ``lens`` (int32 CUDA tensor
    ``[B]``) sequence b attends only its first ``lens[b]`` cached tokens."""
    _need_gpu_fp16("q", q, 3)
    B, Hq, D = q.shape
    if not isinstance(cache, KVCache):
        raise ValueError("cache must come from attn_int8_kvcache_fill")
    if B != cache.B or D != cache.D or cache.buf.device != q.device:
        raise ValueError("q does not match the cache")
    Hkv, S = cache.Hkv, cache.S
    if Hq % Hkv:
        raise ValueError(f"Hq={Hq} must be a multiple of Hkv={Hkv}")
    vf = _vformat(cache.v_format)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_gpu_fp16("out", out, 3)
        if out.shape != q.shape or out.device != q.device:
            raise ValueError("out must match q")
    lib = load_library()
    nbytes = lib.attn_int8_decode_workspace_bytes(B, Hq, Hkv, S, D, vf)
    ws = _workspace(workspace, nbytes, q.device) if nbytes else workspace
    wsz = ws.numel() * ws.element_size() if ws is not None else 0
    with torch.cuda.device(q.device):
        if lens is None:
            st = lib.attn_int8_decode(_ptr(q), _ptr(out), B, Hq, Hkv, S, D,
                                      _scale(softmax_scale, D), vf, _ptr(cache.buf),
                                      cache.nbytes, _ptr(ws), wsz, _stream(q.device))
        else:
            _need_gpu_i32("lens", lens, B)
            st = lib.attn_int8_decode_lens(_ptr(q), _ptr(out), B, Hq, Hkv, S, D,
                                           _scale(softmax_scale, D), vf, _ptr(lens),
                                           _ptr(cache.buf), cache.nbytes, _ptr(ws), wsz,
                                           _stream(q.device))
    _check(st, "attn_int8_decode" if lens is None else "attn_int8_decode_lens")
    return out


def attn_bwd_workspace_bytes(B, Hq, Hkv, S, D) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, Hq, Hkv, S, D))


def attn_bwd(q, k, v, dout, causal=True, softmax_scale=None, workspace=None):
    """Gradients ``(dq, dk, dv)`` (fp32, shapes of q, k, v) of the attention for the
    output gradient ``dout [B,Hq,S,D]`` (fp16); the quantization of the forward is taken
    as the identity."""
    B, Hq, Hkv, S, D = _dense_shapes(q, k, v)
    _need_gpu_fp16("dout", dout, 4)
    if dout.shape != q.shape or dout.device != q.device:
        raise ValueError("dout must match q")
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    lib = load_library()
    nbytes = lib.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D)
    if nbytes == 0:
        raise ValueError(f"backward sizes not supported: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} "
                         f"(needs B, S >= 1, Hq a multiple of Hkv, D in {HEAD_DIMS})")
    ws = _workspace(workspace, nbytes, q.device)
    with torch.cuda.device(q.device):
        st = lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                          B, Hq, Hkv, S, D, _scale(softmax_scale, D), int(bool(causal)),
                          _ptr(ws), ws.numel() * ws.element_size(), _stream(q.device))
    _check(st, "attn_bwd")
    return dq, dk, dv


class Int8Attention(torch.autograd.Function):
    """The int8 attention forward (:func:`attn_int8_fwd`) with the backward of
    :func:`attn_bwd` (gradients in the inputs' fp16)."""

    @staticmethod
    def forward(ctx, q, k, v, causal=True, softmax_scale=None):
        ctx.save_for_backward(q, k, v)
        ctx.causal, ctx.softmax_scale = causal, softmax_scale
        return attn_int8_fwd(q, k, v, causal, softmax_scale)

    @staticmethod
    def backward(ctx, dout):
        q, k, v = ctx.saved_tensors
        dq, dk, dv = attn_bwd(q, k, v, dout.contiguous().to(torch.float16), ctx.causal,
                              ctx.softmax_scale)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None


def int8_attention(q, k, v, causal=True, softmax_scale=None):
    """Differentiable int8 attention: :class:`Int8Attention` applied to fp16 q, k, v."""
    return Int8Attention.apply(q, k, v, causal, softmax_scale)
