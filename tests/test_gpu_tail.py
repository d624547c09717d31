"""GPU parity of dit_attn_fwd_ws: the dense bf16 attention with the last,
partial round of 384-row query blocks split over key ranges and merged.

Every expected value comes from ``oracle/`` on the same seeded inputs; the
rows outside the split blocks must equal dit_attn_fwd's output bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import joint_attention_non_amd as dit
import oracle
from tests._metrics import (BF16_MAX_ABS, BF16_MEAN_ABS, LSE_ABS, bf16_elementwise_ok, errors,
                            rne_bf16, to64)
from workloads import WORKLOADS, make_qkv, make_workload_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


ROWS, TILE = 384, 32   # dense work-group rows and keys per tile


def _plan(B, H, N):
    """(first split block, blocks split, parts per block) as the library
    plans it: one 384-row block per compute unit at a time."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = B * H * ((N + ROWS - 1) // ROWS)
    r = units % cus
    split = min(cus // r, (N + TILE - 1) // TILE) if r > 0 else 1
    if split < 2:
        return units, 0, 1
    return units - r, r, split


def _tail_rows(B, H, N, first):
    """Flat row ids (bh * N + i) of the query blocks from `first` on."""
    nqb = (N + ROWS - 1) // ROWS
    rows = []
    for u in range(first, B * H * nqb):
        bh, qb = divmod(u, nqb)
        lo, hi = qb * ROWS, min(qb * ROWS + ROWS, N)
        rows.append(torch.arange(bh * N + lo, bh * N + hi))
    return torch.cat(rows) if rows else torch.zeros(0, dtype=torch.int64)


def _run_ws(q, k, v, ws, scale=None):
    o16, lse = dit.attn_fwd(q, k, v, scale=scale, return_lse=True, workspace=ws)
    o32 = dit.attn_fwd(q, k, v, scale=scale, out_fp32=True, workspace=ws)
    torch.cuda.synchronize()
    return o16, o32, lse


def _check_rows(o16, o32, lse, q, k, v, rows, scale):
    ref, ref_lse = oracle.attn(q, k, v, scale, rows=rows)
    r = rows.to(DEV)
    e32 = errors(o32.reshape(-1, 128)[r].cpu(), ref)
    e16 = errors(o16.reshape(-1, 128)[r].cpu(), ref)
    _say(f"rows={rows.numel()} fp32-out {e32}  bf16-out {e16}")
    assert e32["max_abs"] <= BF16_MAX_ABS and e32["mean_abs"] <= BF16_MEAN_ABS, e32
    assert bf16_elementwise_ok(o16.reshape(-1, 128)[r].cpu(), ref).all()
    assert e16["mean_abs"] <= BF16_MEAN_ABS, e16
    assert np.max(np.abs(to64(lse.reshape(-1)[r].cpu()) - ref_lse)) <= LSE_ABS


def test_img2048_split_tail_parity_and_untouched_rows():
    w = WORKLOADS["img2048"]
    B, H, N = w.batch, w.heads, w.seqlen
    first, ntail, split = _plan(B, H, N)
    _say(f"case: img2048 split plan first={first} tail={ntail} split={split}")
    assert ntail > 0, "the 2048^2 CFG shape leaves a partial round on this device"
    q, k, v, _ = make_workload_inputs(w, seed=0)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    need = dit.fwd_workspace_bytes(qd)
    assert need == ntail * split * ROWS * 132 * 4
    ws = dit.fwd_workspace(qd)
    o16, o32, lse = _run_ws(qd, kd, vd, ws)
    assert torch.equal(rne_bf16(o32).view(torch.int16), o16.view(torch.int16))
    base16, base_lse = dit.attn_fwd(qd, kd, vd, return_lse=True)
    torch.cuda.synchronize()
    tail = _tail_rows(B, H, N, first)
    keep = torch.ones(B * H * N, dtype=torch.bool)
    keep[tail] = False
    kd_ = keep.to(DEV)
    assert torch.equal(o16.reshape(-1, 128)[kd_].view(torch.int16),
                       base16.reshape(-1, 128)[kd_].view(torch.int16))
    assert torch.equal(lse.reshape(-1)[kd_], base_lse.reshape(-1)[kd_])
    g = torch.Generator().manual_seed(41)
    pick = tail[torch.randperm(tail.numel(), generator=g)[:192]]
    rows = torch.unique(torch.cat([pick, tail[:2], tail[-2:]]))
    _check_rows(o16, o32, lse, q, k, v, rows, w.scale)


def test_ragged_split_tail_parity_one_hot_and_determinism():
    B, H = 1, 1
    N = ROWS * 300 - 77
    first, ntail, split = _plan(B, H, N)
    _say(f"case: ragged N={N} split plan first={first} tail={ntail} split={split}")
    assert ntail > 0 and split >= 2
    q, k, v = make_qkv(B, H, N, 128, seed=51)
    # A dominant key for one query row inside a split block: P = 1 for it,
    # every other weight of the row underflows, so O is that V row exactly.
    i, j = first * ROWS + 100, 3000
    k[0, 0, j] = (40.0 * q[0, 0, i].float()).to(torch.bfloat16)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    ws = dit.fwd_workspace(qd)
    o16, o32, lse = _run_ws(qd, kd, vd, ws)
    assert torch.equal(o16[0, 0, i].cpu().view(torch.int16), v[0, 0, j].view(torch.int16))
    again = dit.attn_fwd(qd, kd, vd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), o16.view(torch.int16))
    assert torch.equal(rne_bf16(o32).view(torch.int16), o16.view(torch.int16))
    tail = _tail_rows(B, H, N, first)
    g = torch.Generator().manual_seed(52)
    pick = tail[torch.randperm(tail.numel(), generator=g)[:48]]
    rows = torch.unique(torch.cat([pick, torch.tensor([i, N - 1, N - 2, first * ROWS - 1, 0])]))
    rows = rows[rows != i]
    _check_rows(o16, o32, lse, q, k, v, rows, 1.0 / math.sqrt(128))


@pytest.mark.parametrize("B,H,N", [(1, 2, 4000), (1, 2, 320)])
def test_small_grid_split_full_parity(B, H, N):
    """A grid smaller than one round is split as a whole (every block over
    several key ranges); full parity against the oracle."""
    first, ntail, split = _plan(B, H, N)
    _say(f"case: small grid B{B} H{H} N{N} plan first={first} tail={ntail} split={split}")
    assert first == 0 and ntail > 0 and split >= 2
    q, k, v = make_qkv(B, H, N, 128, seed=55)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    ws = dit.fwd_workspace(qd)
    o16, o32, lse = _run_ws(qd, kd, vd, ws)
    assert torch.equal(rne_bf16(o32).view(torch.int16), o16.view(torch.int16))
    _check_rows(o16, o32, lse, q, k, v, torch.arange(B * H * N), 1.0 / math.sqrt(128))


def test_no_split_shapes_match_dit_attn_fwd_bitwise():
    # whole rounds on 256 CUs (16 x 16 blocks of 384 rows), and a grid that
    # keeps more than half the CUs busy (1 x 160 blocks)
    for (B, H, N) in ((1, 16, 6144), (1, 1, 384 * 160)):
        first, ntail, split = _plan(B, H, N)
        _say(f"case: B{B} H{H} N{N} plan tail={ntail} split={split}")
        q, k, v = (t.to(DEV) for t in make_qkv(B, H, N, 128, seed=53))
        need = dit.fwd_workspace_bytes(q)
        assert (need == 0) == (ntail == 0)
        ws = dit.fwd_workspace(q)
        a = dit.attn_fwd(q, k, v, workspace=ws)
        b = dit.attn_fwd(q, k, v)
        torch.cuda.synchronize()
        if ntail == 0:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workspace_too_small_is_rejected():
    w = WORKLOADS["img2048"]
    q, k, v = (t.to(DEV) for t in make_qkv(w.batch, w.heads, w.seqlen, 128, seed=54))
    need = dit.fwd_workspace_bytes(q)
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(dit.DitAttnError) as ei:
        dit.attn_fwd(q, k, v, workspace=small)
    assert ei.value.status == 3
