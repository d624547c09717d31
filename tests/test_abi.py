"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments before touching the HIP runtime."""
import ctypes
import os
import re
import subprocess

import pytest

import joint_attention_non_amd as dit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_attn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x7f0000000000          # 256-byte aligned, never dereferenced on these paths


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*]+\s+)+\**(dit_attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_expected_calls():
    names = _declared()
    for n in ("dit_attn_fwd", "dit_attn_fwd_ws", "dit_attn_fwd_workspace_bytes",
              "dit_attn_fwd_fp8", "dit_attn_fwd_fp8_workspace_bytes",
              "dit_attn_fp8_quantize", "dit_attn_fwd_blocksparse", "dit_attn_status_string",
              "dit_attn_last_error", "dit_attn_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = dit.load()
    out = subprocess.run(["nm", "-D", "--defined-only", dit.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dit_attn_\w+)", out))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)
    assert lib.dit_attn_version() >= 10000


def _shape(B=1, H=2, N=320, D=128, scale=0.088, flags=0):
    s = dit._Shape()
    s.batch, s.heads, s.seqlen, s.head_dim = B, H, N, D
    for st in (s.q_stride, s.k_stride, s.v_stride, s.o_stride):
        st[0], st[1], st[2] = H * N * D, N * D, D
    s.softmax_scale, s.flags = scale, flags
    return s


def _fwd(s, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None):
    lib = dit.load()
    return lib.dit_attn_fwd(ctypes.byref(s) if s is not None else None, q, k, v, o, lse, None)


@pytest.mark.parametrize("mutate,status", [
    (lambda s: setattr(s, "head_dim", 64), UNSUPPORTED),
    (lambda s: setattr(s, "seqlen", 0), INVALID),
    (lambda s: setattr(s, "batch", -1), INVALID),
    (lambda s: setattr(s, "heads", 0), INVALID),
    (lambda s: setattr(s, "softmax_scale", 0.0), INVALID),
    (lambda s: setattr(s, "softmax_scale", float("nan")), INVALID),
    (lambda s: setattr(s, "softmax_scale", -0.1), INVALID),
    (lambda s: setattr(s, "flags", 0x80), INVALID),
    (lambda s: s.q_stride.__setitem__(2, 100), INVALID),     # not a multiple of 8
    (lambda s: s.k_stride.__setitem__(2, 64), INVALID),      # rows overlap
    (lambda s: s.v_stride.__setitem__(1, -8), INVALID),
    (lambda s: s.o_stride.__setitem__(0, 12), INVALID),
    (lambda s: (setattr(s, "seqlen", 1 << 22), s.q_stride.__setitem__(2, 1024)), UNSUPPORTED),
])
def test_fwd_rejects_bad_shapes(mutate, status):
    s = _shape()
    mutate(s)
    assert _fwd(s) == status
    assert dit.load().dit_attn_last_error().decode() != ""


def test_fwd_rejects_null_and_misaligned_pointers():
    s = _shape()
    assert _fwd(None) == INVALID
    assert _fwd(s, q=None) == INVALID
    assert _fwd(s, o=None) == INVALID
    assert _fwd(s, k=FAKE + 8) == INVALID
    assert _fwd(s, lse=FAKE + 2) == INVALID
    msg = dit.load().dit_attn_last_error().decode()
    assert "lse" in msg


def test_blocksparse_rejects_bad_mask_arguments():
    lib = dit.load()
    s = _shape()
    f = lib.dit_attn_fwd_blocksparse
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, None, 0, 128, None) == INVALID
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 64, None) == UNSUPPORTED
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, -1, 128, None) == INVALID


def test_fp8_workspace_size_and_checks():
    lib = dit.load()
    s = _shape(B=1, H=2, N=320)
    need = lib.dit_attn_fwd_fp8_workspace_bytes(ctypes.byref(s))
    # 3 code tensors of 2*384*128 bytes + 3 scale arrays of 2*3 floats, 256-aligned regions
    assert need == 3 * 98304 + 3 * 256
    assert lib.dit_attn_fwd_fp8_workspace_bytes(None) == 0
    f = lib.dit_attn_fwd_fp8
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, None, need, None) == WORKSPACE
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 1, None) == WORKSPACE
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE + 16, need, None) == WORKSPACE
    s.head_dim = 96
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, need, None) == UNSUPPORTED
    g = lib.dit_attn_fp8_quantize
    s.head_dim = 128
    assert g(ctypes.byref(s), FAKE, FAKE, None, FAKE, need, None) == INVALID


def test_status_strings():
    lib = dit.load()
    for st in range(0, 6):
        assert lib.dit_attn_status_string(st)
    assert lib.dit_attn_status_string(0).decode() == "ok"


@pytest.mark.parametrize("mutate,status", [
    (lambda s: setattr(s, "head_dim", 64), UNSUPPORTED),
    (lambda s: setattr(s, "seqlen", 0), INVALID),
    (lambda s: setattr(s, "softmax_scale", float("inf")), INVALID),
    (lambda s: s.o_stride.__setitem__(2, 120), INVALID),
])
def test_fwd_ws_rejects_bad_shapes_before_any_device_call(mutate, status):
    lib = dit.load()
    s = _shape()
    mutate(s)
    assert lib.dit_attn_fwd_ws(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == status
    assert lib.dit_attn_fwd_ws(None, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == INVALID
    assert lib.dit_attn_fwd_ws(ctypes.byref(_shape()), None, FAKE, FAKE, FAKE, None, FAKE, 1 << 20,
                               None) == INVALID
    assert lib.dit_attn_fwd_workspace_bytes(None) == 0
    bad = _shape()
    bad.seqlen = 0
    assert lib.dit_attn_fwd_workspace_bytes(ctypes.byref(bad)) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback path: without the built library every call raises."""
    import torch
    monkeypatch.setattr(dit, "_lib", None)
    monkeypatch.setattr(dit, "_LIB_PATH", str(tmp_path / "libdit_attn.so"))
    with pytest.raises(RuntimeError, match="is missing"):
        dit.load()

    # and host tensors are refused rather than computed on the CPU
    q = torch.zeros((1, 1, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        dit.attn_fwd(q, q, q)
