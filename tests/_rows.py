"""Output buffers pre-filled with NaN for parity checks at production shapes.

Full-size outputs are too large for the fp64 oracle to recompute whole, so
the tests check the rows ``workloads.block_rows`` picks (first, last and one
random row of every work-group's query block) -- and, to catch a work-group
that never stores its rows, they pass outputs filled with NaN and require
the whole result to be finite.
"""
import torch

from workloads import block_rows  # noqa: F401  (re-exported for the tests)


def nan_like_out(B: int, H: int, N: int, fp32: bool, device) -> torch.Tensor:
    dt = torch.float32 if fp32 else torch.bfloat16
    return torch.full((B, H, N, 128), float("nan"), dtype=dt, device=device)


def nan_lse(B: int, H: int, N: int, device) -> torch.Tensor:
    return torch.full((B, H, N), float("nan"), dtype=torch.float32, device=device)
