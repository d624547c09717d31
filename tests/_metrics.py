"""Error metrics and tolerances shared by the parity tests.

Metrics are taken over the flattened output in float64, with b = oracle:
max |a - b|, mean |a - b|, cosine <a,b>/(|a||b|) and relative L2 |a-b|/|b|.

Tolerances (stated once here, used by every parity test):
* bf16 path: max-abs <= 1e-2 and mean-abs <= 1e-3 against the fp64 oracle on
  the kernel's fp32 output (DIT_ATTN_FLAG_OUT_F32).  The bf16 output is
  checked to be the round-to-nearest-even image of that fp32 output, bit for
  bit, and element-wise: an error above 1e-2 may exceed it by at most half a
  bf16 step of the oracle value plus 1e-3 (the fp32 output already meets the
  1e-2 gate; rounding it to bf16 adds up to half a step, which for |O| >= 2
  is 2^-7 or more).
* lse (bf16 paths): the kernel normalises by the sum of the bf16-rounded
  weights it multiplies V with; each weight carries a relative rounding
  error of at most 2^-8 (bf16 unit roundoff, 8 significant bits), so
  ln(sum) moves by at most ln(1 + 2^-8) < 2^-8.
* fp8 path: cosine >= 0.99 and relative L2 <= 5e-2 against the oracle on the
  unquantised inputs; against the oracle's fp8 recipe (same codes, same
  running-max blocks) relative L2 <= 5e-3.
"""
import numpy as np
import torch

BF16_MAX_ABS = 1e-2
BF16_MEAN_ABS = 1e-3
LSE_ABS = 2.0 ** -8 + 1e-5
FP8_COS = 0.99
FP8_REL_L2 = 5e-2
FP8_RECIPE_REL_L2 = 5e-3


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def errors(a, b) -> dict:
    a = to64(a).ravel()
    b = to64(b).ravel()
    d = a - b
    return {
        "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
        "mean_abs": float(np.mean(np.abs(d))) if d.size else 0.0,
        "cos": float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b))),
        "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(b)),
    }


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers around |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def bf16_elementwise_ok(o_bf16, ref) -> np.ndarray:
    a, b = to64(o_bf16), to64(ref)
    err = np.abs(a - b)
    return err - BF16_MAX_ABS <= half_ulp_bf16(b) + 1e-3


def rne_bf16(t: torch.Tensor) -> torch.Tensor:
    """fp32 tensor -> bf16 with round to nearest even (torch's cast)."""
    return t.to(torch.bfloat16)
