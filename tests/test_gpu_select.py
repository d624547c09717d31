"""GPU parity of the block-mask selection (dit_attn_select_blocks) against
the fp64 oracle, and of block-sparse attention run on the mask it selects.

The kernel decides p_ij >= tau / nb in fp32, the oracle in fp64: a share
within a relative 1e-4 of the threshold may be decided either way (fp32
block means and logits are good to about 1e-6 relative here; the margin is
a hundred times that).  Every other decision, and every forced entry, must
match exactly."""
import math

import numpy as np
import pytest
import torch

import joint_attention_non_amd as dit
import oracle
from tests._metrics import BF16_MAX_ABS, BF16_MEAN_ABS, LSE_ABS, errors, to64
from tests._rows import block_rows
from workloads import make_local_qkv, make_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"
MARGIN = 1e-4
SCALE = 1.0 / math.sqrt(128)


def _say(msg):
    print(msg, flush=True)


def _check_mask(got, q, k, tau, text_tokens, max_ambiguous_frac=1e-3):
    """Compare a device mask with the oracle's decisions; returns the oracle mask."""
    ref, share = oracle.select_blocks(q, k, SCALE, tau, text_tokens)
    g = got.cpu().numpy().reshape(ref.shape)
    assert set(np.unique(g)) <= {0, 1}
    nb = ref.shape[-1]
    thr = tau / nb
    ambiguous = np.abs(share - thr) <= MARGIN * thr
    tb = (text_tokens + 127) // 128
    forced = np.zeros((nb, nb), dtype=bool)
    forced[:tb, :] = True
    forced[:, :tb] = True
    forced[np.arange(nb), np.arange(nb)] = True
    assert (g[..., forced] == 1).all()
    bad = (g != ref) & ~ambiguous
    assert not bad.any(), (f"{int(bad.sum())} decisions differ outside the margin, first at "
                           f"{np.argwhere(bad)[0]}")
    free = np.broadcast_to(~forced, ambiguous.shape)
    if free.any():
        assert ambiguous[free].mean() <= max_ambiguous_frac
    return ref


@pytest.mark.parametrize("B,H,N,text,tau", [
    (1, 2, 1, 0, 1.0),            # one block
    (1, 2, 100, 0, 1.0),          # one ragged block
    (2, 3, 700, 77, 1.0),         # ragged last block, partial text block
    (2, 3, 1100, 300, 0.5),
    (1, 4, 4000, 512, 2.0),       # 32 blocks
    (1, 2, 40000, 512, 1.0),      # 313 blocks: two key blocks per thread
])
def test_select_matches_oracle_local_inputs(B, H, N, text, tau):
    _say(f"case: select B={B} H={H} N={N} text={text} tau={tau}")
    q, k, _ = make_local_qkv(B, H, N, text, seed=N)
    got = dit.select_blocks(q.to(DEV), k.to(DEV), tau, text)
    torch.cuda.synchronize()
    assert got.shape == (B, H, (N + 127) // 128, (N + 127) // 128)
    _check_mask(got, q, k, tau, text)


def test_select_matches_oracle_gaussian_inputs_and_strided_views():
    """Near-uniform shares (i.i.d. inputs) and q / k given as strided views
    of a packed [B, N, 3, H, D] tensor."""
    _say("case: select gaussian strided")
    B, H, N = 2, 3, 900
    g = torch.Generator().manual_seed(5)
    qkv = torch.randn((B, N, 3, H, 128), generator=g).to(torch.bfloat16)
    q, k = qkv[:, :, 0].permute(0, 2, 1, 3), qkv[:, :, 1].permute(0, 2, 1, 3)
    qkv_d = qkv.to(DEV)
    qd, kd = qkv_d[:, :, 0].permute(0, 2, 1, 3), qkv_d[:, :, 1].permute(0, 2, 1, 3)
    for tau in (0.9, 1.0, 1.1):
        got = dit.select_blocks(qd, kd, tau, 0)
        torch.cuda.synchronize()
        _check_mask(got, q.contiguous(), k.contiguous(), tau, 0, max_ambiguous_frac=2e-2)


def test_select_degenerate_cases():
    """tau = 0 keeps every block; text covering the sequence keeps every
    block; identical key blocks give every share exactly 1/nb, so tau = 1
    keeps all and tau slightly above 1 keeps only the forced entries."""
    _say("case: select degenerate")
    q, k, _ = make_local_qkv(1, 2, 1000, 64, seed=3)
    qd, kd = q.to(DEV), k.to(DEV)
    assert bool((dit.select_blocks(qd, kd, 0.0, 64) == 1).all())
    assert bool((dit.select_blocks(qd, kd, 5.0, 1000) == 1).all())
    kb = k[:, :, :128].repeat(1, 1, 8, 1)          # 8 identical key blocks, N = 1024
    qb, _, _ = make_qkv(1, 2, 1024, seed=4)
    m1 = dit.select_blocks(qb.to(DEV), kb.to(DEV), 1.0, 0).cpu()
    m2 = dit.select_blocks(qb.to(DEV), kb.to(DEV), 1.0 + 1e-3, 0).cpu()
    assert bool((m1 == 1).all())
    assert torch.equal(m2[0, 0], torch.eye(8, dtype=torch.uint8))


def test_select_is_deterministic_and_fills_out():
    _say("case: select determinism")
    q, k, _ = make_local_qkv(2, 3, 3000, 512, seed=8)
    qd, kd = q.to(DEV), k.to(DEV)
    a = dit.select_blocks(qd, kd, 1.0, 512)
    out = torch.full_like(a, 7)
    ws = torch.full((dit.select_blocks_workspace_bytes(q),), 0xFF, dtype=torch.uint8, device=DEV)
    b = dit.select_blocks(qd, kd, 1.0, 512, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert b is out and torch.equal(a, b)


def test_select_max_blocks():
    """4096 blocks (N = 524288), the largest the kernel takes."""
    _say("case: select nb=4096")
    N = 4096 * 128
    q, k, _ = make_local_qkv(1, 1, N, 0, seed=11, amp=16.0, length=48.0)
    got = dit.select_blocks(q.to(DEV), k.to(DEV), 1.0, 0)
    torch.cuda.synchronize()
    _check_mask(got, q, k, 1.0, 0)


def test_img2048_select_then_blocksparse():
    """The full img2048 step with selection: B1 H24 N16896 (512 text
    tokens), tau = 1.  The selected mask matches the oracle's decisions;
    block-sparse attention on it matches the oracle's masked attention on
    rows that touch every 128-row block of every head."""
    _say("case: img2048 select + blocksparse")
    B, H, N, text = 1, 24, 16896, 512
    q, k, v = make_local_qkv(B, H, N, text, seed=0)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    mask = dit.select_blocks(qd, kd, 1.0, text)
    o, lse = dit.attn_fwd_blocksparse(qd, kd, vd, mask, return_lse=True, out_fp32=True)
    torch.cuda.synchronize()
    _check_mask(mask, q, k, 1.0, text)
    density = float(mask.float().mean())
    _say(f"  realized density {density:.3f}")
    assert 0.05 < density < 0.6
    rows = block_rows(B, H, N, 128, seed=1)
    ref, ref_lse = oracle.attn(q, k, v, SCALE, mask=mask.cpu(), mask_stride_bh=mask.shape[-1] ** 2,
                               rows=rows)
    got = to64(o).reshape(-1, 128)[rows.numpy()]
    e = errors(got, ref)
    assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, e
    assert np.max(np.abs(to64(lse).reshape(-1)[rows.numpy()] - ref_lse)) <= LSE_ABS
