"""Host-side checks of the C ABI: the library loads without a GPU, exports every
function include/i8attn.h declares, and rejects bad arguments on the host before
any launch (these calls never reach the device, so they run without a GPU)."""

import ctypes
import os
import subprocess

import pytest

import int8_w8a8_flashattention_amd as i8

LIB = i8.library_path()
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libi8attn.so not built")

OK, INVALID, HEADDIM, WSSMALL = 0, -1, -2, -3
FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    return i8.load_library()


def test_header_declares_the_entry_points():
    names = i8.header_functions()
    for n in ("quant_rowwise_i8", "attn_int8_fwd", "attn_int8_varlen_fwd", "attn_int8_debug_qk",
              "attn_int8_workspace_bytes", "attn_int8_varlen_workspace_bytes",
              "attn_int8_prepare_kv", "attn_int8_prepare_q", "attn_int8_attend",
              "attn_int8_fwd_prepared",
              "i8a_status_string", "i8a_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for n in i8.header_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    assert lib.i8a_status_string(OK) == b"I8A_OK"
    assert lib.i8a_status_string(INVALID) == b"I8A_ERR_INVALID_ARG"
    assert lib.i8a_status_string(HEADDIM) == b"I8A_ERR_UNSUPPORTED_HEAD_DIM"
    assert lib.i8a_status_string(WSSMALL) == b"I8A_ERR_WORKSPACE_TOO_SMALL"
    assert lib.i8a_status_string(-4) == b"I8A_ERR_HIP"
    assert lib.i8a_status_string(7) == b"I8A_UNKNOWN_STATUS"


def test_workspace_sizes(lib):
    assert lib.attn_int8_workspace_bytes(1, 32, 8, 4096, 128) > 0
    assert lib.attn_int8_workspace_bytes(1, 32, 8, 4096, 96) == 0
    assert lib.attn_int8_workspace_bytes(1, 30, 8, 4096, 128) == 0
    assert lib.attn_int8_workspace_bytes(0, 32, 8, 4096, 128) == 0
    a = lib.attn_int8_workspace_bytes(1, 32, 8, 1000, 128)
    b = lib.attn_int8_workspace_bytes(1, 32, 8, 2000, 128)
    assert 0 < a < b and a % 256 == 0
    # the workspace holds at least int8 K and fp16 V for every kv token
    assert a >= 8 * 1000 * 128 * 3
    assert lib.attn_int8_varlen_workspace_bytes(3, 100, 60, 4, 2, 64) > 0
    assert lib.attn_int8_varlen_workspace_bytes(3, 100, 101, 4, 2, 64) == 0
    assert lib.attn_int8_varlen_workspace_bytes(0, 100, 60, 4, 2, 64) == 0
    assert lib.attn_int8_varlen_workspace_bytes(70000, 100000, 60, 4, 2, 64) == 0
    assert lib.attn_int8_workspace_bytes(70000, 32, 8, 16, 128) == 0
    # the workspace also holds the int8 Q codes and their scales
    assert a >= 8 * 1000 * 128 * 3 + 32 * 1000 * (128 + 4)


def _fwd(lib, D=128, Hq=32, Hkv=8, S=64, B=1, scale=0.1, causal=1, ws=FAKE, wsb=1 << 40,
         q=FAKE, out=FAKE):
    return lib.attn_int8_fwd(q, FAKE, FAKE, out, B, Hq, Hkv, S, D, scale, causal, ws, wsb, None)


def test_forward_rejects_bad_arguments(lib):
    assert _fwd(lib, D=96) == HEADDIM
    assert b"head dim" in lib.i8a_last_error()
    assert _fwd(lib, D=512) == HEADDIM
    assert _fwd(lib, Hq=30) == INVALID
    assert _fwd(lib, Hkv=0) == INVALID
    assert _fwd(lib, S=0) == INVALID
    assert _fwd(lib, B=0) == INVALID
    assert _fwd(lib, B=70000) == INVALID
    assert _fwd(lib, Hq=70000, Hkv=1) == INVALID
    assert _fwd(lib, scale=0.0) == INVALID
    assert _fwd(lib, scale=float("inf")) == INVALID
    assert _fwd(lib, scale=float("nan")) == INVALID
    assert _fwd(lib, causal=2) == INVALID
    assert _fwd(lib, q=None) == INVALID
    assert _fwd(lib, out=ctypes.c_void_p((1 << 20) + 8)) == INVALID  # misaligned
    assert _fwd(lib, ws=None) == INVALID
    assert _fwd(lib, ws=ctypes.c_void_p((1 << 20) + 128)) == INVALID
    need = lib.attn_int8_workspace_bytes(1, 32, 8, 64, 128)
    assert _fwd(lib, wsb=need - 1) == WSSMALL
    assert b"workspace needs" in lib.i8a_last_error()


def test_split_phases_reject_bad_arguments(lib):
    need = lib.attn_int8_workspace_bytes(1, 8, 2, 256, 64)
    assert lib.attn_int8_prepare_q(None, 1, 8, 2, 256, 64, FAKE, need, None) == INVALID
    assert lib.attn_int8_prepare_q(FAKE, 1, 8, 3, 256, 64, FAKE, need, None) == INVALID
    assert lib.attn_int8_prepare_q(FAKE, 1, 8, 2, 256, 48, FAKE, need, None) == HEADDIM
    assert lib.attn_int8_prepare_q(FAKE, 1, 8, 2, 256, 64, FAKE, need - 1, None) == WSSMALL
    assert lib.attn_int8_attend(None, 1, 8, 2, 256, 64, 0.1, 1, FAKE, need, None) == INVALID
    assert lib.attn_int8_attend(FAKE, 1, 8, 2, 256, 64, 0.0, 1, FAKE, need, None) == INVALID
    assert lib.attn_int8_attend(FAKE, 1, 8, 2, 256, 64, 0.1, 3, FAKE, need, None) == INVALID
    assert lib.attn_int8_attend(FAKE, 1, 8, 2, 256, 64, 0.1, 1, None, need, None) == INVALID
    assert lib.attn_int8_attend(FAKE, 1, 8, 2, 256, 64, 0.1, 1, FAKE, need - 1, None) == WSSMALL


def test_varlen_rejects_bad_arguments(lib):
    def call(nseq=2, maxlen=10, T=20, D=64, cu=FAKE, wsb=1 << 40):
        return lib.attn_int8_varlen_fwd(FAKE, FAKE, FAKE, FAKE, cu, nseq, maxlen, T, 4, 2, D, 0.1,
                                        1, FAKE, wsb, None)
    assert call(cu=None) == INVALID
    assert call(nseq=0) == INVALID
    assert call(nseq=70000, maxlen=10, T=100000) == INVALID
    assert call(maxlen=21) == INVALID
    assert call(T=-1) == INVALID
    assert call(D=48) == HEADDIM
    assert call(T=0, maxlen=0) == OK  # nothing to do, nothing launched
    assert call(wsb=10) == WSSMALL


def test_quant_rejects_bad_arguments(lib):
    def call(rows=4, d=64, mean=None, rpg=1, bits=24, x=FAKE):
        return lib.quant_rowwise_i8(x, rows, d, mean, rpg, bits, FAKE, FAKE, None)
    assert call(rows=0) == OK  # empty input: no launch
    assert call(rows=-1) == INVALID
    assert call(d=12) == INVALID
    assert call(d=520) == INVALID
    assert call(bits=8) == INVALID
    assert call(mean=FAKE, rpg=0) == INVALID
    assert call(x=None) == INVALID
    assert call(x=ctypes.c_void_p((1 << 20) + 4)) == INVALID


def test_debug_rejects_bad_tiles(lib):
    def call(b=0, h=0, r0=0, r=8, c0=0, c=8, s32=FAKE):
        return lib.attn_int8_debug_qk(FAKE, FAKE, FAKE, 1, 4, 2, 64, 64, b, h, r0, r, c0, c, s32,
                                      None, None, None, None, 0, FAKE, 1 << 40, None)
    assert call(b=1) == INVALID
    assert call(h=4) == INVALID
    assert call(r0=60, r=8) == INVALID
    assert call(c=0) == INVALID
    assert call(s32=None) == INVALID
    assert lib.attn_int8_debug_qk(FAKE, FAKE, FAKE, 1, 4, 2, 64, 64, 0, 0, 0, 8, 0, 8, FAKE,
                                  None, None, None, None, 2, FAKE, 1 << 40, None) == INVALID


def test_python_binding_validates_before_the_library():
    import torch
    x = torch.zeros(4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        i8.quant_rowwise_i8(x)  # CPU tensor
    with pytest.raises(ValueError):
        i8.attn_int8_fwd(x.view(1, 1, 4, 64), x.view(1, 1, 4, 64), x.view(1, 1, 4, 64))


def test_forward_ex_rejects_unknown_flags(lib):
    st = lib.attn_int8_fwd_ex(FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 64, 64, 0.125, 1, 16, FAKE,
                              1 << 40, None)
    assert st == INVALID
    assert b"flags" in lib.i8a_last_error()


def test_q_outlier_flag_limits(lib):
    # Q outlier detection does not combine with the rotation and is built for D <= 128:
    # both rejected on the host, for the dense and the varlen entries.
    def dense(flags, d):
        return lib.attn_int8_fwd_ex(FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 64, d, 0.125, 1, flags,
                                    FAKE, 1 << 40, None)

    def varlen(flags, d):
        return lib.attn_int8_varlen_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 2, 1, d,
                                           0.125, 1, flags, FAKE, 1 << 40, None)
    for call in (dense, varlen):
        assert call(i8.FWD_Q_OUTLIERS | i8.FWD_HADAMARD, 64) == INVALID
        assert b"HADAMARD" in lib.i8a_last_error()
        assert call(i8.FWD_Q_OUTLIERS, 256) == HEADDIM


def test_backward_head_dims_and_arguments(lib):
    # Head dims 32, 64, 128 and 256 are supported (workspace size > 0); others are
    # rejected on the host before any launch, as are bad sizes and a short workspace.
    for d in (32, 64, 128, 256):
        assert lib.attn_bwd_workspace_bytes(1, 4, 2, 300, d) > 0
    assert lib.attn_bwd_workspace_bytes(1, 4, 2, 300, 48) == 0
    assert lib.attn_bwd_workspace_bytes(1, 4, 3, 300, 64) == 0  # Hq % Hkv != 0
    need = lib.attn_bwd_workspace_bytes(1, 4, 2, 300, 256)
    args = [FAKE] * 7 + [1, 4, 2, 300]
    assert lib.attn_bwd(*args, 48, 0.1, 1, FAKE, need, None) == HEADDIM
    assert lib.attn_bwd(*args, 256, 0.0, 1, FAKE, need, None) == INVALID
    assert lib.attn_bwd(*args, 256, 0.1, 1, FAKE, need - 1, None) == WSSMALL


def test_debug_ex_rejects_bad_arguments(lib):
    # Dense geometry (no cu_seqlens) must have total = nseq * max_seqlen; unknown flags,
    # a per-token V scale output with V per channel (and the reverse), and misaligned
    # pointers are rejected on the host.
    def call(cu=None, nseq=1, L=64, T=64, flags=0, seq=0, h=0, r0=0, r=8, c0=0, c=8,
             vscale=None, vhat=None, vchan=None, ochan=None):
        return lib.attn_int8_debug_qk_ex(FAKE, FAKE, FAKE, cu, nseq, L, T, 4, 2, 64, flags, seq,
                                         h, r0, r, c0, c, FAKE, None, None, vscale, None, vhat,
                                         vchan, ochan, FAKE, 1 << 40, None)
    assert call(T=65) == INVALID
    assert call(flags=16) == INVALID
    assert call(flags=0, ochan=FAKE) == INVALID
    assert call(flags=i8.FWD_Q_OUTLIERS, ochan=ctypes.c_void_p((1 << 20) + 2)) == INVALID
    assert call(flags=i8.FWD_V_PER_CHANNEL, vscale=FAKE) == INVALID
    assert call(flags=0, vchan=FAKE) == INVALID
    assert call(vhat=ctypes.c_void_p((1 << 20) + 1)) == INVALID
    assert call(cu=ctypes.c_void_p((1 << 20) + 2), nseq=2, L=40, T=64) == INVALID
    assert call(seq=1) == INVALID
    assert call(r0=60, r=8) == INVALID
    assert b"tile" in lib.i8a_last_error()
