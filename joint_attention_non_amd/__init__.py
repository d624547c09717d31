"""Python binding of the dit_attn C ABI (joint attention forward on MI355X).

Argument marshalling only: every step of the attention runs in the HIP
kernels of ``libdit_attn.so``.  PyTorch supplies device memory and the
current stream.  There is no fallback: if the library is not built, or a
call fails, an exception is raised.

    attn_fwd(q, k, v, scale=None, return_lse=False, out_fp32=False, out=None, workspace=None, lse_out=None)
    attn_fwd_fp8(q, k, v, scale=None, return_lse=False, workspace=None, out_fp32=False, out=None, lse_out=None)
    attn_fwd_blocksparse(q, k, v, block_mask, scale=None, return_lse=False, out_fp32=False, out=None,
                         workspace=None, lse_out=None)
    fp8_quantize(q, k, v, workspace=None) -> Fp8Workspace views
    select_blocks(q, k, tau, text_tokens, scale=None, out=None, workspace=None) -> uint8 [B, H, nb, nb]

q, k, v: CUDA (HIP) bfloat16 tensors [B, H, N, 128] whose last dimension is
contiguous (any other strides that are multiples of 8 elements).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import torch

__all__ = ["attn_fwd", "attn_fwd_fp8", "attn_fwd_blocksparse", "fp8_quantize",
           "fp8_workspace_bytes", "fwd_workspace_bytes", "fwd_workspace",
           "blocksparse_workspace_bytes", "attn_fwd_noalloc", "select_blocks",
           "select_blocks_workspace_bytes", "DitAttnError",
           "library_path", "load"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdit_attn.so")
_lib = None

FLAG_OUT_F32 = 1


class DitAttnError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str, text: str):
        super().__init__(f"{fn} failed with status {status} ({text}): {detail}")
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("seqlen", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
                ("softmax_scale", ctypes.c_float), ("flags", ctypes.c_uint32)]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libdit_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, sp = ctypes.c_void_p, ctypes.POINTER(_Shape)
        lib.dit_attn_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        lib.dit_attn_fwd.restype = ctypes.c_int
        lib.dit_attn_fwd_workspace_bytes.argtypes = [sp]
        lib.dit_attn_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.dit_attn_fwd_ws.argtypes = [sp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.dit_attn_fwd_ws.restype = ctypes.c_int
        lib.dit_attn_fwd_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        lib.dit_attn_fwd_noalloc.restype = ctypes.c_int
        lib.dit_attn_fwd_noalloc_scratch_bytes.argtypes = []
        lib.dit_attn_fwd_noalloc_scratch_bytes.restype = ctypes.c_size_t
        lib.dit_attn_fwd_fp8_workspace_bytes.argtypes = [sp]
        lib.dit_attn_fwd_fp8_workspace_bytes.restype = ctypes.c_size_t
        lib.dit_attn_fwd_fp8.argtypes = [sp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.dit_attn_fwd_fp8.restype = ctypes.c_int
        lib.dit_attn_fp8_quantize.argtypes = [sp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.dit_attn_fp8_quantize.restype = ctypes.c_int
        lib.dit_attn_fwd_blocksparse_workspace_bytes.argtypes = [sp]
        lib.dit_attn_fwd_blocksparse_workspace_bytes.restype = ctypes.c_size_t
        lib.dit_attn_fwd_blocksparse.argtypes = [sp, vp, vp, vp, vp, vp, vp, ctypes.c_int64,
                                                 ctypes.c_int32, vp, ctypes.c_size_t, vp]
        lib.dit_attn_fwd_blocksparse.restype = ctypes.c_int
        lib.dit_attn_select_blocks_workspace_bytes.argtypes = [sp]
        lib.dit_attn_select_blocks_workspace_bytes.restype = ctypes.c_size_t
        lib.dit_attn_select_blocks.argtypes = [sp, vp, vp, ctypes.c_float, ctypes.c_int32, vp, vp,
                                               ctypes.c_size_t, vp]
        lib.dit_attn_select_blocks.restype = ctypes.c_int
        lib.dit_attn_status_string.argtypes = [ctypes.c_int]
        lib.dit_attn_status_string.restype = ctypes.c_char_p
        lib.dit_attn_last_error.argtypes = []
        lib.dit_attn_last_error.restype = ctypes.c_char_p
        lib.dit_attn_version.argtypes = []
        lib.dit_attn_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc: int, fn: str):
    if rc != 0:
        lib = load()
        raise DitAttnError(rc, fn, lib.dit_attn_last_error().decode(),
                           lib.dit_attn_status_string(rc).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_inputs(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, D], got {tuple(t.shape)}")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")


def _shape(q, k, v, o, scale, flags) -> _Shape:
    _check_inputs(q, k, v)
    B, H, N, D = q.shape
    s = _Shape()
    s.batch, s.heads, s.seqlen, s.head_dim = B, H, N, D
    for dst, t in ((s.q_stride, q), (s.k_stride, k), (s.v_stride, v), (s.o_stride, o)):
        dst[0], dst[1], dst[2] = t.stride(0), t.stride(1), t.stride(2)
    s.softmax_scale = float(1.0 / math.sqrt(D) if scale is None else scale)
    s.flags = flags
    return s


def _outputs(q, return_lse, out_fp32, out=None, lse_out=None):
    """Output tensors: caller-supplied ones are checked against what the
    kernels will write (the C ABI cannot see an allocation's size), missing
    ones are allocated."""
    _check_inputs(q, q, q)
    B, H, N, D = q.shape
    dtype = torch.float32 if out_fp32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, H, N, D), device=q.device, dtype=dtype)
    else:
        if not isinstance(out, torch.Tensor) or not out.is_cuda or out.device != q.device:
            raise ValueError("out must be a device tensor on q's device")
        if tuple(out.shape) != (B, H, N, D):
            raise ValueError(f"out must have shape {(B, H, N, D)}, got {tuple(out.shape)}")
        if out.dtype != dtype:
            raise ValueError(f"out must be {dtype} (out_fp32={out_fp32}), got {out.dtype}")
        if out.stride(3) != 1:
            raise ValueError("out must have a contiguous last dimension")
    lse = None
    if return_lse or lse_out is not None:
        if lse_out is None:
            lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
        else:
            if (not isinstance(lse_out, torch.Tensor) or not lse_out.is_cuda or lse_out.device != q.device
                    or lse_out.dtype != torch.float32 or tuple(lse_out.shape) != (B, H, N)
                    or not lse_out.is_contiguous()):
                raise ValueError(f"lse_out must be a contiguous float32 device tensor of shape {(B, H, N)}")
            lse = lse_out
    return out, lse


def _check_workspace(ws, q, name="workspace"):
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != q.device:
        raise ValueError(f"{name} must be a device tensor on q's device")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError(f"{name} must be a contiguous uint8 tensor")
    return ws


def fwd_workspace_bytes(q) -> int:
    """Bytes of the tail-split workspace dit_attn_fwd_ws needs for q's shape
    on the current device (0: no split applies)."""
    B, H, N, D = q.shape
    s = _Shape()
    s.batch, s.heads, s.seqlen, s.head_dim = B, H, N, D
    return int(load().dit_attn_fwd_workspace_bytes(ctypes.byref(s)))


def _ret(o, lse, return_lse):
    return (o, lse) if return_lse else o


def attn_fwd(q, k, v, scale=None, return_lse=False, out_fp32=False, out=None, workspace=None,
             lse_out=None):
    """Dense bf16 joint attention; returns O (and lse if asked).  With a
    workspace (uint8 device tensor of at least fwd_workspace_bytes(q) bytes)
    the last partial round of query blocks is split over key ranges
    (dit_attn_fwd_ws).  `out` / `lse_out` receive the results when given."""
    o, lse = _outputs(q, return_lse, out_fp32, out, lse_out)
    s = _shape(q, k, v, o, scale, FLAG_OUT_F32 if out_fp32 else 0)
    if workspace is None:
        _check(load().dit_attn_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   _stream()), "dit_attn_fwd")
    else:
        _check_workspace(workspace, q)
        _check(load().dit_attn_fwd_ws(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      _ptr(workspace), workspace.numel(), _stream()), "dit_attn_fwd_ws")
    return _ret(o, lse, return_lse)


def attn_fwd_noalloc(q, k, v, scale=None, return_lse=False, out_fp32=False, out=None, lse_out=None):
    """dit_attn_fwd_noalloc: dit_attn_fwd_ws with the library's own static
    scratch instead of a workspace (allocates nothing when `out` -- and
    `lse_out` if lse is wanted -- are given)."""
    o, lse = _outputs(q, return_lse, out_fp32, out, lse_out)
    s = _shape(q, k, v, o, scale, FLAG_OUT_F32 if out_fp32 else 0)
    _check(load().dit_attn_fwd_noalloc(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       _stream()), "dit_attn_fwd_noalloc")
    return _ret(o, lse, return_lse)


def fwd_workspace(q):
    """A workspace tensor for attn_fwd(..., workspace=...) (at least 256 bytes)."""
    return torch.empty(max(fwd_workspace_bytes(q), 256), dtype=torch.uint8, device=q.device)


def blocksparse_workspace_bytes(q) -> int:
    """Bytes of workspace dit_attn_fwd_blocksparse needs for q's shape."""
    B, H, N, D = q.shape
    s = _Shape()
    s.batch, s.heads, s.seqlen, s.head_dim = B, H, N, D
    return int(load().dit_attn_fwd_blocksparse_workspace_bytes(ctypes.byref(s)))


def _mask_stride(block_mask, q, block_size):
    """Element offset between consecutive (b, h) masks; refuses a mask that
    does not cover every (b, h) slice with [nb, nb] entries."""
    if (not isinstance(block_mask, torch.Tensor) or block_mask.dtype != torch.uint8
            or not block_mask.is_cuda or block_mask.device != q.device or not block_mask.is_contiguous()):
        raise ValueError("block_mask must be a contiguous uint8 tensor on q's device")
    B, H, N, _ = q.shape
    nb = (N + block_size - 1) // block_size if block_size > 0 else 0
    if block_mask.dim() < 2 or tuple(block_mask.shape[-2:]) != (nb, nb):
        raise ValueError(f"block_mask must end in [{nb}, {nb}] (ceil(N / {block_size})), "
                         f"got {tuple(block_mask.shape)}")
    lead = tuple(block_mask.shape[:-2])
    if lead == ():
        return 0
    if lead in ((B * H,), (B, H)):
        return nb * nb
    raise ValueError(f"block_mask must be [nb, nb], [B*H, nb, nb] or [B, H, nb, nb] with B*H = {B * H}, "
                     f"got {tuple(block_mask.shape)}")


def attn_fwd_blocksparse(q, k, v, block_mask, scale=None, return_lse=False, out_fp32=False,
                         block_size=128, out=None, workspace=None, lse_out=None):
    """Block-sparse attention.  block_mask: uint8 device tensor [nb, nb]
    (shared by all heads) or [B, H, nb, nb] / [B*H, nb, nb]."""
    o, lse = _outputs(q, return_lse, out_fp32, out, lse_out)
    s = _shape(q, k, v, o, scale, FLAG_OUT_F32 if out_fp32 else 0)
    stride_bh = _mask_stride(block_mask, q, block_size)
    need = blocksparse_workspace_bytes(q)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_workspace(workspace, q)
    _check(load().dit_attn_fwd_blocksparse(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                           _ptr(lse), _ptr(block_mask), stride_bh, block_size,
                                           _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                           _stream()), "dit_attn_fwd_blocksparse")
    return _ret(o, lse, return_lse)


def select_blocks_workspace_bytes(q) -> int:
    """Bytes of workspace dit_attn_select_blocks needs for q's shape."""
    B, H, N, D = q.shape
    s = _Shape()
    s.batch, s.heads, s.seqlen, s.head_dim = B, H, N, D
    return int(load().dit_attn_select_blocks_workspace_bytes(ctypes.byref(s)))


def select_blocks(q, k, tau, text_tokens, scale=None, out=None, workspace=None):
    """Block-mask selection (dit_attn_select_blocks): returns a uint8 device
    tensor [B, H, nb, nb] (1 = keep) that attn_fwd_blocksparse takes as is.
    `out`, when given, must be a contiguous uint8 tensor of that shape."""
    _check_inputs(q, k, k)
    B, H, N, D = q.shape
    nb = (N + 127) // 128
    if out is None:
        out = torch.empty((B, H, nb, nb), dtype=torch.uint8, device=q.device)
    elif (not isinstance(out, torch.Tensor) or not out.is_cuda or out.device != q.device
          or out.dtype != torch.uint8 or not out.is_contiguous() or out.numel() != B * H * nb * nb):
        raise ValueError(f"out must be a contiguous uint8 device tensor of {B * H * nb * nb} elements")
    need = select_blocks_workspace_bytes(q)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q)
    s = _shape(q, k, k, q, scale, 0)
    _check(load().dit_attn_select_blocks(ctypes.byref(s), _ptr(q), _ptr(k), float(tau), int(text_tokens),
                                         _ptr(out), _ptr(workspace), workspace.numel(), _stream()),
           "dit_attn_select_blocks")
    return out


def fp8_workspace_bytes(q) -> int:
    B, H, N, D = q.shape
    s = _Shape()
    s.batch, s.heads, s.seqlen, s.head_dim = B, H, N, D
    return int(load().dit_attn_fwd_fp8_workspace_bytes(ctypes.byref(s)))


def _workspace(q, workspace):
    need = fp8_workspace_bytes(q)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    return _check_workspace(workspace, q)


def attn_fwd_fp8(q, k, v, scale=None, return_lse=False, workspace=None, out_fp32=False, out=None,
                 lse_out=None):
    """fp8 (e4m3) joint attention with on-device dynamic per-block scaling."""
    o, lse = _outputs(q, return_lse, out_fp32, out, lse_out)
    s = _shape(q, k, v, o, scale, FLAG_OUT_F32 if out_fp32 else 0)
    ws = _workspace(q, workspace)
    _check(load().dit_attn_fwd_fp8(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   _ptr(ws), ws.numel(), _stream()), "dit_attn_fwd_fp8")
    return _ret(o, lse, return_lse)


@dataclasses.dataclass
class Fp8Workspace:
    buffer: torch.Tensor
    q8: torch.Tensor    # uint8 [B, H, Np, 128]
    k8: torch.Tensor    # uint8 [B, H, Np, 128]
    v8t: torch.Tensor   # uint8 [B, H, 128, Np], key order permuted per 64-key group
    sq: torch.Tensor    # float32 [B, H, nb]
    sk: torch.Tensor
    sv: torch.Tensor


def _r256(x):
    return (x + 255) // 256 * 256


def fp8_workspace_views(q, ws) -> Fp8Workspace:
    B, H, N, D = q.shape
    nb = (N + 127) // 128
    np_ = nb * 128
    codes = B * H * np_ * 128
    sc = B * H * nb * 4
    o_k8 = _r256(codes)
    o_v8 = _r256(o_k8 + codes)
    o_sq = _r256(o_v8 + codes)
    o_sk = _r256(o_sq + sc)
    o_sv = _r256(o_sk + sc)
    return Fp8Workspace(
        ws,
        ws[:codes].view(B, H, np_, 128),
        ws[o_k8:o_k8 + codes].view(B, H, np_, 128),
        ws[o_v8:o_v8 + codes].view(B, H, 128, np_),
        ws[o_sq:o_sq + sc].view(torch.float32).view(B, H, nb),
        ws[o_sk:o_sk + sc].view(torch.float32).view(B, H, nb),
        ws[o_sv:o_sv + sc].view(torch.float32).view(B, H, nb))


def fp8_quantize(q, k, v, workspace=None) -> Fp8Workspace:
    """Run only the e4m3 quantisation pass and return views of the workspace."""
    s = _shape(q, k, v, q, None, 0)
    ws = _workspace(q, workspace)
    _check(load().dit_attn_fp8_quantize(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(ws),
                                        ws.numel(), _stream()),
           "dit_attn_fp8_quantize")
    return fp8_workspace_views(q, ws)


def v8t_key_order(np_: int) -> torch.Tensor:
    """For each stored position of a V8t row, the key it holds (the documented
    per-64-key-group permutation of 4-key groups)."""
    pos = torch.arange(np_)
    grp64, p = pos // 64, pos % 64
    pg, byte = p // 4, p % 4
    kg = 8 * ((pg >> 2) & 1) + 2 * (pg & 3) + (pg >> 3)
    return grp64 * 64 + 4 * kg + byte
