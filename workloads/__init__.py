"""Seeded synthetic inputs for the joint-attention forward.

This module only draws random numbers and lays them out. It holds none of the
attention arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path
(``joint_attention_non_amd``) can be fed from it without sharing any of the
method's code.

Workloads (all non-causal, head_dim 128, softmax scale 1/sqrt(128)):

* ``tiny``      B=1 H=2  N=64+256=320
* ``img1024``   B=1 H=24 N=512+4096=4608
* ``img2048``   B=2 H=24 N=512+16384=16896 (cond/uncond pair), 1% of key rows x8
* ``img2048_fp8``    B=1 H=24 N=16896, e4m3 recipe
* ``img2048_sparse`` B=1 H=24 N=16896, 128x128 block mask, density 0.25 with
  the diagonal and every text-token block forced on
* ``i2i2048``   B=2 H=24 N=512+16384+16384=33280: image-to-image at 2048^2,
  where the joint sequence also carries the reference image's latents (taken
  at the target resolution), 1% of key rows x8

The token order is text first, then image latents: joint attention in the
FLUX-family DiT concatenates the separately embedded text, target-image and
optional reference-image streams and runs one attention over all of them
(bpdata.com "FLUX 3 Image Klein optimalizálása", section "Modellezés és
pipeline jellemzők").  Seed 0 throughout: that section states that the
benchmarks were run with seed 0, and the page's run example passes --seed 0
(section "Telepítési és futtatási példák").

Random-number recipe (stated once, used by tests, smoke and the benchmark):

* ``q, k, v``: ``g = torch.Generator().manual_seed(seed)``, three
  ``torch.randn((B, H, N, D), generator=g)`` draws in that order, each rounded
  to bfloat16 (round to nearest even).
* peaked key rows: ``torch.randperm(N, generator=manual_seed(seed + 1))``,
  first ``floor(0.01 * N)`` indices; those key rows (all b, h, d) are
  multiplied by 8 in bfloat16 (a power of two, so exact).
* block mask: ``torch.rand((nb, nb), generator=manual_seed(seed + 2)) <
  density``, then rows and columns of the text blocks and the diagonal set to
  1.  ``nb = ceil(N / 128)``; text blocks are ``ceil(text_tokens / 128)``.
"""
from __future__ import annotations

import dataclasses
import math

import torch

HEAD_DIM = 128
BLOCK = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    text_tokens: int
    image_tokens: int
    head_dim: int = HEAD_DIM
    variant: str = "bf16"          # "bf16" | "fp8" | "sparse"
    peaked_key_frac: float = 0.0   # fraction of key rows scaled x8
    mask_density: float = 0.0      # Bernoulli density of the block mask

    @property
    def seqlen(self) -> int:
        return self.text_tokens + self.image_tokens

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def nblocks(self) -> int:
        return (self.seqlen + BLOCK - 1) // BLOCK

    @property
    def text_blocks(self) -> int:
        return (self.text_tokens + BLOCK - 1) // BLOCK

    def describe(self) -> dict:
        d = {"workload": self.name, "batch": self.batch, "heads": self.heads,
             "seqlen": self.seqlen, "text_tokens": self.text_tokens,
             "image_tokens": self.image_tokens, "head_dim": self.head_dim,
             "variant": self.variant}
        if self.peaked_key_frac:
            d["peaked_key_frac"] = self.peaked_key_frac
        if self.mask_density:
            d["mask_density"] = self.mask_density
        return d


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 256),
    "img1024": Workload("img1024", 1, 24, 512, 4096),
    "img2048": Workload("img2048", 2, 24, 512, 16384, peaked_key_frac=0.01),
    "img2048_fp8": Workload("img2048_fp8", 1, 24, 512, 16384, variant="fp8"),
    "img2048_sparse": Workload("img2048_sparse", 1, 24, 512, 16384, variant="sparse",
                               mask_density=0.25),
    # text + target latents + reference-image latents
    "i2i2048": Workload("i2i2048", 2, 24, 512, 16384 + 16384, peaked_key_frac=0.01),
}


def make_qkv(B: int, H: int, N: int, D: int = HEAD_DIM, seed: int = 0,
             peaked_key_frac: float = 0.0):
    """Return (q, k, v) as contiguous CPU bfloat16 tensors of shape [B, H, N, D]."""
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn((B, H, N, D), generator=g).to(torch.bfloat16) for _ in range(3))
    if peaked_key_frac:
        n_peak = int(math.floor(peaked_key_frac * N))
        idx = torch.randperm(N, generator=torch.Generator().manual_seed(seed + 1))[:n_peak]
        k[:, :, idx, :] *= 8
    return q.contiguous(), k.contiguous(), v.contiguous()


def make_local_qkv(B: int, H: int, N: int, text_tokens: int, D: int = HEAD_DIM, seed: int = 0,
                   amp: float = 16.0, length: float = 8.0):
    """(q, k, v) like ``make_qkv`` whose image tokens also carry a shared
    positional feature, so that tokens near each other on the latent grid
    have correlated queries and keys (the locality that block-sparse
    attention exploits).  Image token t sits at (t // side, t % side) of a
    grid of width side = ceil(sqrt(N - text_tokens)); per head h the feature
    is sqrt(2 / D) cos(<omega_h,d, pos> + phase_h,d) over d (random Fourier
    features: omega ~ N(0, I / length^2), phase ~ U[0, 2 pi), drawn from
    ``manual_seed(seed + 4)`` in that order), scaled by ``amp`` and added in
    float32 to the Gaussian q and k before the bfloat16 rounding.  Text
    tokens and v are unchanged."""
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn((B, H, N, D), generator=g) for _ in range(3))
    n_img = N - text_tokens
    if n_img > 0:
        side = math.ceil(math.sqrt(n_img))
        t = torch.arange(n_img)
        pos = torch.stack([(t // side).float(), (t % side).float()], dim=1)        # [n_img, 2]
        gf = torch.Generator().manual_seed(seed + 4)
        omega = torch.randn((H, D, 2), generator=gf) / length
        phase = torch.rand((H, D), generator=gf) * (2 * math.pi)
        feat = math.sqrt(2.0 / D) * torch.cos(torch.einsum("pc,hdc->hpd", pos, omega) + phase[:, None, :])
        q[:, :, text_tokens:, :] += amp * feat[None]
        k[:, :, text_tokens:, :] += amp * feat[None]
    return tuple(t.to(torch.bfloat16).contiguous() for t in (q, k, v))


def peaked_key_rows(N: int, seed: int = 0, frac: float = 0.01) -> torch.Tensor:
    n_peak = int(math.floor(frac * N))
    return torch.randperm(N, generator=torch.Generator().manual_seed(seed + 1))[:n_peak]


def make_block_mask(N: int, text_tokens: int, density: float = 0.25, seed: int = 0,
                    block: int = BLOCK) -> torch.Tensor:
    """uint8 [nb, nb] row-major mask over (query block, key block); nonzero = keep."""
    nb = (N + block - 1) // block
    tb = (text_tokens + block - 1) // block
    r = torch.rand((nb, nb), generator=torch.Generator().manual_seed(seed + 2)) < density
    r[:tb, :] = True
    r[:, :tb] = True
    r.fill_diagonal_(True)
    return r.to(torch.uint8).contiguous()


def make_workload_inputs(w: Workload, seed: int = 0):
    """(q, k, v, mask_or_None) on the CPU for a named workload."""
    q, k, v = make_qkv(w.batch, w.heads, w.seqlen, w.head_dim, seed, w.peaked_key_frac)
    mask = None
    if w.variant == "sparse":
        mask = make_block_mask(w.seqlen, w.text_tokens, w.mask_density, seed)
    return q, k, v, mask


def sample_rows(B: int, H: int, N: int, n: int, seed: int = 0) -> torch.Tensor:
    """n distinct flat row ids (bh * N + i), always including the first and last
    row of the first and last (b, h) slice and rows of the ragged last block."""
    total = B * H * N
    g = torch.Generator().manual_seed(seed + 3)
    picks = torch.randint(0, total, (n,), generator=g)
    fixed = torch.tensor([0, N - 1, total - N, total - 1, (N // BLOCK) * BLOCK,
                          total - 1 - (N % BLOCK)], dtype=torch.int64).clamp(0, total - 1)
    rows = torch.unique(torch.cat([fixed, picks]))
    return rows


def block_rows(B: int, H: int, N: int, rows: int, seed: int = 0) -> torch.Tensor:
    """Flat row ids (bh * N + i) that touch every block of `rows` query rows
    of every (batch, head) slice: the block's first and last row and one
    random row of it -- so a check on these rows sees every work-group of a
    launch that gives one such block to each work-group."""
    nqb = (N + rows - 1) // rows
    g = torch.Generator().manual_seed(seed + 77)
    lo = torch.arange(nqb) * rows
    hi = torch.clamp(lo + rows, max=N) - 1
    picks = []
    for bh in range(B * H):
        rnd = torch.minimum(lo + (torch.rand(nqb, generator=g) * rows).long(), hi)
        picks.append(bh * N + torch.stack([lo, hi, rnd], 1).reshape(-1))
    return torch.unique(torch.cat(picks))
