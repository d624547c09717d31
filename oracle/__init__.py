"""fp64 CPU oracle for the joint-attention forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP path
(``joint_attention_non_amd``); the only thing both sides consume is the seeded
input generator in ``workloads``, which holds no attention arithmetic.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, OpenMP over rows);
this module only builds and loads that library and marshals numpy arrays.

Functions and what pins them (tests/test_oracle.py):

* ``attn``              -- two-pass softmax attention in fp64; pinned against
  an mpmath 60-digit brute force, torch's float64 CPU
  ``scaled_dot_product_attention`` (also with a boolean block mask) and the
  closed forms / invariants (rows of P sum to one, constant V, key/value
  permutation, one-hot key, N = 1, Q = 0).
* ``e4m3_decode`` / ``e4m3_encode`` -- OCP E4M3 codec; pinned exhaustively
  against torch's ``float8_e4m3fn`` and hand-checked code points.
* ``fp8_quantize``      -- per-block absmax quantiser; pinned by its defining
  properties (block absmax lands on +-448, dequantised values within half an
  e4m3 step, zero block) and against torch's float8 cast.
* ``attn_fp8_recipe``   -- the fp8 attention recipe; with P quantisation off it
  must equal ``attn`` on the dequantised inputs, with it on a one-hot key must
  return the dequantised value row exactly, its running max across key blocks
  must match a restatement with torch's e4m3 cast (and differ from the
  final-max variant), and its error against ``attn`` on the unquantised inputs
  must sit in the band the e4m3 step implies.
* ``attn_fp8_recipe(..., nsplit=S)`` -- the recipe with each row's key
  blocks cut into S ranges, each from a fresh running max, merged exactly;
  pinned by S = 1 being the recipe bit for bit, by S = 3 without P
  quantisation equalling ``attn`` on the dequantised inputs, by one range
  per key block matching a numpy / torch-codec restatement, and by S = 3
  with P quantisation differing from the unsplit recipe (negative control).
* ``select_blocks``     -- the block-mask selection rule; pinned against
  torch's block pooling and scipy's softmax, the softmax's shift invariance,
  key-block permutation, identical key blocks (every share exactly 1/nb),
  tau = 0, and a planted dominant block.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile attn_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, dp, fp, u8p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        lib.oracle_attn_f64.argtypes = [i64, i64, i64, dp, dp, dp, u8p, i64, i64,
                                        ctypes.c_double, dp, i64, dp, dp]
        lib.oracle_attn_f64.restype = ctypes.c_int
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_fp8_quantize.argtypes = [i64, i64, i64, i64, fp, u8p, fp]
        lib.oracle_fp8_quantize.restype = None
        lib.oracle_attn_fp8_recipe.argtypes = [i64, i64, i64, i64, u8p, u8p, u8p, fp, fp, fp,
                                               ctypes.c_double, ctypes.c_int, dp, i64, dp, dp]
        lib.oracle_attn_fp8_recipe.restype = ctypes.c_int
        lib.oracle_attn_fp8_recipe_split.argtypes = [i64, i64, i64, i64, u8p, u8p, u8p, fp, fp, fp,
                                                     ctypes.c_double, ctypes.c_int, i64, dp, i64, dp, dp]
        lib.oracle_attn_fp8_recipe_split.restype = ctypes.c_int
        lib.oracle_select_blocks.argtypes = [i64, i64, i64, i64, dp, dp, ctypes.c_double,
                                             ctypes.c_double, i64, u8p, dp]
        lib.oracle_select_blocks.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_f64(x) -> np.ndarray:
    """bf16/float torch tensor or numpy array -> contiguous float64 numpy (exact upcast)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().cpu().to(torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def attn(q, k, v, scale: float, mask=None, mask_stride_bh: int = 0, block: int = 128,
         rows=None):
    """Exact-definition attention on [B, H, N, D] inputs.

    Returns (o, lse) as float64 numpy arrays: o is [B, H, N, D] (or
    [len(rows), D] when ``rows`` -- flat ids bh * N + i -- is given), lse is
    [B, H, N] (or [len(rows)]).  ``mask`` is uint8 [nb, nb] (shared by all
    (b, h) when mask_stride_bh == 0) or [B*H, nb, nb] with stride nb*nb."""
    qd, kd, vd = _as_f64(q), _as_f64(k), _as_f64(v)
    if qd.ndim != 4 or kd.shape != qd.shape or vd.shape != qd.shape:
        raise ValueError("q, k, v must all be [B, H, N, D] of one shape")
    B, H, N, D = qd.shape
    BH = B * H
    m = None
    if mask is not None:
        m = np.ascontiguousarray(np.asarray(mask.cpu() if hasattr(mask, "cpu") else mask,
                                            dtype=np.uint8))
        nb = (N + block - 1) // block
        if m.size < mask_stride_bh * (BH - 1) + nb * nb:
            raise ValueError("mask is smaller than the (b, h) slices it must cover")
    r = None
    if rows is not None:
        r = np.ascontiguousarray(np.asarray(rows.cpu() if hasattr(rows, "cpu") else rows,
                                            dtype=np.int64))
        nrows = r.size
    else:
        nrows = BH * N
    o = np.empty((nrows, D), dtype=np.float64)
    lse = np.empty((nrows,), dtype=np.float64)
    rc = _load().oracle_attn_f64(BH, N, D, _ptr(qd), _ptr(kd), _ptr(vd), _ptr(m),
                                 mask_stride_bh, block, float(scale), _ptr(r), nrows,
                                 _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attn_f64 rejected its arguments")
    if rows is None:
        return o.reshape(B, H, N, D), lse.reshape(B, H, N)
    return o, lse


def e4m3_decode(code: int) -> float:
    return float(_load().oracle_e4m3_decode(int(code) & 0xFF))


def e4m3_encode(x: float) -> int:
    return int(_load().oracle_e4m3_encode(float(x)))


def fp8_quantize(x, block: int = 128):
    """x: [B, H, N, D] bf16/float -> (codes uint8 [B,H,N,D], scales float32 [B,H,nb])."""
    xf = x
    try:
        import torch
        if isinstance(x, torch.Tensor):
            xf = x.detach().cpu().to(torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    xf = np.ascontiguousarray(np.asarray(xf, dtype=np.float32))
    B, H, N, D = xf.shape
    nb = (N + block - 1) // block
    codes = np.empty((B, H, N, D), dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    _load().oracle_fp8_quantize(B * H, N, D, block, _ptr(xf), _ptr(codes), _ptr(scales))
    return codes, scales


def e4m3_decode_array(codes: np.ndarray) -> np.ndarray:
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale: float, quantize_p: bool = True,
                    block: int = 128, rows=None, nsplit: int = 1):
    """The fp8 recipe on oracle-quantised codes; returns (o, lse) like ``attn``.
    nsplit > 1: each row's key blocks cut into nsplit consecutive ranges, each
    run from a fresh running max, merged exactly (see attn_oracle.c)."""
    q8, k8, v8 = (np.ascontiguousarray(a, dtype=np.uint8) for a in (q8, k8, v8))
    sq, sk, sv = (np.ascontiguousarray(a, dtype=np.float32) for a in (sq, sk, sv))
    if q8.ndim != 4 or k8.shape != q8.shape or v8.shape != q8.shape:
        raise ValueError("q8, k8, v8 must all be [B, H, N, D] of one shape")
    B, H, N, D = q8.shape
    nb = (N + block - 1) // block
    for s_ in (sq, sk, sv):
        if s_.shape != (B, H, nb):
            raise ValueError("scales must be [B, H, ceil(N / block)]")
    BH = B * H
    r = None
    if rows is not None:
        r = np.ascontiguousarray(np.asarray(rows.cpu() if hasattr(rows, "cpu") else rows,
                                            dtype=np.int64))
        nrows = r.size
    else:
        nrows = BH * N
    o = np.empty((nrows, D), dtype=np.float64)
    lse = np.empty((nrows,), dtype=np.float64)
    rc = _load().oracle_attn_fp8_recipe_split(BH, N, D, block, _ptr(q8), _ptr(k8), _ptr(v8),
                                              _ptr(sq), _ptr(sk), _ptr(sv), float(scale),
                                              1 if quantize_p else 0, int(nsplit), _ptr(r), nrows,
                                              _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attn_fp8_recipe_split rejected its arguments")
    if rows is None:
        return o.reshape(B, H, N, D), lse.reshape(B, H, N)
    return o, lse


def select_blocks(q, k, scale: float, tau: float, text_tokens: int, block: int = 128):
    """Sol-Attention-style block selection (see attn_oracle.c): returns
    (mask uint8 [B, H, nb, nb], share float64 [B, H, nb, nb])."""
    qd, kd = _as_f64(q), _as_f64(k)
    if qd.ndim != 4 or kd.shape != qd.shape:
        raise ValueError("q, k must be [B, H, N, D] of one shape")
    B, H, N, D = qd.shape
    nb = (N + block - 1) // block
    mask = np.empty((B, H, nb, nb), dtype=np.uint8)
    share = np.empty((B, H, nb, nb), dtype=np.float64)
    _load().oracle_select_blocks(B * H, N, D, block, _ptr(qd), _ptr(kd), float(scale), float(tau),
                                 int(text_tokens), _ptr(mask), _ptr(share))
    return mask, share
