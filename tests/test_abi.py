"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments before touching the HIP runtime."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

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
              "dit_attn_fp8_quantize", "dit_attn_fwd_blocksparse",
              "dit_attn_fwd_blocksparse_workspace_bytes", "dit_attn_fwd_noalloc",
              "dit_attn_fwd_noalloc_scratch_bytes", "dit_attn_select_blocks",
              "dit_attn_select_blocks_workspace_bytes", "dit_attn_status_string",
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
    # a row stride above 2^22 elements (the staged key tiles' 32-bit offsets
    # past the last row could wrap), even where the slice itself is small
    (lambda s: (setattr(s, "seqlen", 2), s.k_stride.__setitem__(2, (1 << 22) + 8)), UNSUPPORTED),
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
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, None, 0, 128, None, 0, None) == INVALID
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 64, None, 0, None) == UNSUPPORTED
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, -1, 128, None, 0, None) == INVALID
    # the workspace this build needs is none; a misaligned one is still refused
    assert lib.dit_attn_fwd_blocksparse_workspace_bytes(ctypes.byref(s)) == 0
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 128, FAKE + 16, 64, None) == WORKSPACE


class _DeviceLike(torch.Tensor):
    """A host tensor that reports itself as a device tensor, so the binding's
    argument checks (which all run before any library call) can be exercised
    without a GPU."""

    @property
    def is_cuda(self):
        return True


def _dev(t):
    return t.as_subclass(_DeviceLike)


def _qkv(B=1, H=2, N=300):
    q = _dev(torch.zeros((B, H, N, 128), dtype=torch.bfloat16))
    return q, q, q


@pytest.mark.parametrize("make_out,msg", [
    (lambda: torch.zeros((1, 2, 300, 128), dtype=torch.bfloat16), "device tensor"),       # host tensor
    (lambda: _dev(torch.zeros((1, 2, 300, 128), dtype=torch.float32)), "bfloat16"),       # wrong dtype
    (lambda: _dev(torch.zeros((1, 2, 299, 128), dtype=torch.bfloat16)), "shape"),         # too short
    (lambda: _dev(torch.zeros((1, 2, 128, 300), dtype=torch.bfloat16)).transpose(2, 3), "contiguous"),
])
def test_binding_rejects_bad_out(make_out, msg):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match=msg):
        dit.attn_fwd(q, k, v, out=make_out())


def test_binding_rejects_fp32_flag_with_bf16_out_and_bad_lse_out():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="float32"):
        dit.attn_fwd(q, k, v, out_fp32=True, out=_dev(torch.zeros((1, 2, 300, 128), dtype=torch.bfloat16)))
    with pytest.raises(ValueError, match="lse_out"):
        dit.attn_fwd(q, k, v, lse_out=_dev(torch.zeros((1, 2, 299), dtype=torch.float32)))
    with pytest.raises(ValueError, match="lse_out"):
        dit.attn_fwd_fp8(q, k, v, lse_out=_dev(torch.zeros((1, 2, 300), dtype=torch.float64)))


def test_binding_rejects_bad_workspace():
    q, k, v = _qkv()
    for ws in (torch.zeros(4096, dtype=torch.uint8),                 # host memory
               _dev(torch.zeros(1024, dtype=torch.float32)),         # not bytes
               _dev(torch.zeros((2, 4096), dtype=torch.uint8))[:, ::2]):   # not contiguous
        with pytest.raises(ValueError, match="workspace"):
            dit.attn_fwd(q, k, v, workspace=ws)
        with pytest.raises(ValueError, match="workspace"):
            dit.attn_fwd_fp8(q, k, v, workspace=ws)


@pytest.mark.parametrize("shape", [(2, 3), (3, 2), (3, 3, 3), (1, 3, 3), (2, 1, 3, 3), (4, 4)])
def test_binding_rejects_masks_that_do_not_cover_every_slice(shape):
    """N = 300 gives nb = 3; B*H = 2.  A short mask, one built for another N,
    or a [1, nb, nb] mask used with two heads would be read past its end."""
    q, k, v = _qkv()
    mask = _dev(torch.ones(shape, dtype=torch.uint8))
    with pytest.raises(ValueError, match="block_mask"):
        dit.attn_fwd_blocksparse(q, k, v, mask)


def test_binding_mask_strides():
    q, _, _ = _qkv(B=1, H=2, N=300)
    for shape, stride in (((3, 3), 0), ((2, 3, 3), 9), ((1, 2, 3, 3), 9)):
        assert dit._mask_stride(_dev(torch.ones(shape, dtype=torch.uint8)), q, 128) == stride


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


def test_noalloc_checks_arguments_before_any_device_call():
    lib = dit.load()
    assert lib.dit_attn_fwd_noalloc_scratch_bytes() == 64 << 20
    bad = _shape()
    bad.head_dim = 64
    assert lib.dit_attn_fwd_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None, None) == UNSUPPORTED
    assert lib.dit_attn_fwd_noalloc(None, FAKE, FAKE, FAKE, FAKE, None, None) == INVALID
    assert lib.dit_attn_fwd_noalloc(ctypes.byref(_shape()), FAKE, None, FAKE, FAKE, None, None) == INVALID


def test_select_blocks_checks_arguments_before_any_device_call():
    lib = dit.load()
    s = _shape(B=1, H=2, N=320)
    need = lib.dit_attn_select_blocks_workspace_bytes(ctypes.byref(s))
    assert need == 2 * 2 * 3 * 128 * 4          # fp32 block means of Q and K
    assert lib.dit_attn_select_blocks_workspace_bytes(None) == 0
    f = lib.dit_attn_select_blocks
    assert f(ctypes.byref(s), FAKE, FAKE, 1.0, 0, FAKE, FAKE, need - 1, None) == WORKSPACE
    assert f(ctypes.byref(s), FAKE, FAKE, 1.0, 0, FAKE, None, need, None) == WORKSPACE
    assert f(ctypes.byref(s), FAKE, FAKE, 1.0, 0, FAKE, FAKE + 16, need, None) == WORKSPACE
    assert f(ctypes.byref(s), FAKE, FAKE, 1.0, 0, None, FAKE, need, None) == INVALID       # no mask
    assert f(ctypes.byref(s), FAKE, None, 1.0, 0, FAKE, FAKE, need, None) == INVALID       # no k
    assert f(ctypes.byref(s), FAKE, FAKE, -0.5, 0, FAKE, FAKE, need, None) == INVALID      # tau < 0
    assert f(ctypes.byref(s), FAKE, FAKE, float("nan"), 0, FAKE, FAKE, need, None) == INVALID
    assert f(ctypes.byref(s), FAKE, FAKE, float("inf"), 0, FAKE, FAKE, need, None) == INVALID
    assert f(ctypes.byref(s), FAKE, FAKE, 1.0, -1, FAKE, FAKE, need, None) == INVALID      # text < 0
    assert f(ctypes.byref(s), FAKE, FAKE, 1.0, 321, FAKE, FAKE, need, None) == INVALID     # text > N
    assert f(None, FAKE, FAKE, 1.0, 0, FAKE, FAKE, need, None) == INVALID
    big = _shape(B=1, H=1, N=4097 * 128)       # 4097 blocks: beyond the selection kernel
    nbig = lib.dit_attn_select_blocks_workspace_bytes(ctypes.byref(big))
    assert f(ctypes.byref(big), FAKE, FAKE, 1.0, 0, FAKE, FAKE, nbig, None) == UNSUPPORTED
    assert "4096" in lib.dit_attn_last_error().decode()


def test_binding_select_blocks_rejects_bad_out():
    q, k, _ = _qkv()
    with pytest.raises(ValueError, match="out"):
        dit.select_blocks(q, k, 1.0, 0, out=_dev(torch.zeros((1, 2, 3, 2), dtype=torch.uint8)))
    with pytest.raises(ValueError, match="out"):
        dit.select_blocks(q, k, 1.0, 0, out=_dev(torch.zeros((1, 2, 3, 3), dtype=torch.int32)))


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
