"""GPU parity of the block-sparse path against the fp64 oracle with the same
128x128 block mask, plus the properties that tie it to the dense path."""
import math

import numpy as np
import pytest
import torch

import joint_attention_non_amd as dit
import oracle
from tests._metrics import (BF16_MAX_ABS, BF16_MEAN_ABS, LSE_ABS, bf16_elementwise_ok, errors,
                            rne_bf16, to64)
from tests._rows import block_rows, nan_like_out, nan_lse
from workloads import WORKLOADS, make_block_mask, make_qkv, make_workload_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("N", [100, 128, 320, 700, 1100])
def test_random_mask_full_parity(N):
    _say(f"case: sparse N={N} B=1 H=2")
    q, k, v = make_qkv(1, 2, N, 128, seed=70 + N)
    mask = make_block_mask(N, 64, 0.3, seed=N)
    o32, lse = dit.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), mask.to(DEV),
                                        out_fp32=True, return_lse=True)
    o16 = dit.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), mask.to(DEV))
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attn(q, k, v, 1.0 / math.sqrt(128), mask=mask)
    e = errors(o32, ref)
    assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, e
    assert torch.equal(rne_bf16(o32).view(torch.int16), o16.view(torch.int16))
    assert bf16_elementwise_ok(o16, ref).all()
    assert np.max(np.abs(to64(lse) - ref_lse)) <= LSE_ABS


def test_all_ones_mask_equals_dense():
    """Every block kept: the sparse kernel (32-key tiles, 128-row blocks) and
    the dense one (32-key tiles, 384-row blocks) compute the same attention;
    both meet the oracle gates and agree with each other within them."""
    _say("case: all-ones mask vs dense")
    for N in (320, 1000):
        q, k, v = make_qkv(1, 3, N, 128, seed=80 + N)
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
        nb = (N + 127) // 128
        ones = torch.ones((nb, nb), dtype=torch.uint8, device=DEV)
        o_s, l_s = dit.attn_fwd_blocksparse(qd, kd, vd, ones, return_lse=True, out_fp32=True)
        o_d, l_d = dit.attn_fwd(qd, kd, vd, return_lse=True, out_fp32=True)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.attn(q, k, v, 1.0 / math.sqrt(128))
        for o, l in ((o_s, l_s), (o_d, l_d)):
            e = errors(o, ref)
            assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, e
            assert np.max(np.abs(to64(l) - ref_lse)) <= LSE_ABS
        e = errors(o_s, to64(o_d))
        assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, e


def test_diagonal_mask_is_segment_attention():
    """Only diagonal blocks kept: each 128-token segment attends to itself,
    which is the dense oracle run on that segment alone."""
    _say("case: diagonal mask")
    N = 400
    q, k, v = make_qkv(1, 2, N, 128, seed=90)
    nb = 4
    mask = torch.eye(nb, dtype=torch.uint8)
    o = dit.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), mask.to(DEV), out_fp32=True)
    torch.cuda.synchronize()
    for s in range(nb):
        a, b = s * 128, min(N, (s + 1) * 128)
        ref, _ = oracle.attn(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], 1.0 / math.sqrt(128))
        e = errors(o[:, :, a:b], ref)
        assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS


def test_masked_blocks_are_never_read():
    """Fill a key block that every query masks out with NaN: the output must
    be finite, equal the oracle on the clean inputs with the same mask, and
    match the kernel's own clean-input result bit for bit."""
    _say("case: NaN-poisoned masked block")
    N = 512
    q, k, v = make_qkv(1, 2, N, 128, seed=91)
    mask = torch.ones((4, 4), dtype=torch.uint8)
    mask[:, 2] = 0
    kp, vp = k.clone(), v.clone()
    kp[:, :, 256:384] = float("nan")
    vp[:, :, 256:384] = float("nan")
    md = mask.to(DEV)
    o = dit.attn_fwd_blocksparse(q.to(DEV), kp.to(DEV), vp.to(DEV), md, out_fp32=True)
    o_clean = dit.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), md, out_fp32=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    assert torch.equal(o, o_clean)
    ref, _ = oracle.attn(q, k, v, 1.0 / math.sqrt(128), mask=mask)
    e = errors(o, ref)
    assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, e


def test_fully_masked_row_gives_zero_and_neg_inf_lse():
    _say("case: empty mask row")
    N = 300
    q, k, v = make_qkv(1, 1, N, 128, seed=92)
    mask = torch.ones((3, 3), dtype=torch.uint8)
    mask[1] = 0
    o, lse = dit.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), mask.to(DEV),
                                      out_fp32=True, return_lse=True)
    torch.cuda.synchronize()
    assert float(o[0, 0, 128:256].abs().max()) == 0.0
    assert bool(torch.isneginf(lse[0, 0, 128:256]).all())
    ref, _ = oracle.attn(q, k, v, 1.0 / math.sqrt(128), mask=mask)
    e = errors(o, ref)
    assert e["max_abs"] <= BF16_MAX_ABS


def test_per_head_masks():
    _say("case: per-(b,h) masks")
    N = 384
    q, k, v = make_qkv(1, 3, N, 128, seed=93)
    masks = torch.stack([make_block_mask(N, 0, 0.4, seed=s) for s in range(3)])
    o = dit.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), masks.to(DEV), out_fp32=True)
    torch.cuda.synchronize()
    ref, _ = oracle.attn(q, k, v, 1.0 / math.sqrt(128), mask=masks, mask_stride_bh=9)
    e = errors(o, ref)
    assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, e


def test_img2048_sparse_blockwise_parity():
    """Every 128-row work-group: first, last and one random row of each mask
    block of every head against the oracle, outputs pre-filled with NaN."""
    w = WORKLOADS["img2048_sparse"]
    B, H, N = w.batch, w.heads, w.seqlen
    _say(f"case: {w.describe()} blockwise")
    q, k, v, mask = make_workload_inputs(w, seed=0)
    _say(f"active blocks: {int(mask.sum())} of {mask.numel()}")
    qd, kd, vd, md = (t.to(DEV) for t in (q, k, v, mask))
    o32 = dit.attn_fwd_blocksparse(qd, kd, vd, md, out_fp32=True, out=nan_like_out(B, H, N, True, DEV))
    o16, lse = dit.attn_fwd_blocksparse(qd, kd, vd, md, return_lse=True, out=nan_like_out(B, H, N, False, DEV),
                                        lse_out=nan_lse(B, H, N, DEV))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o32).all()) and bool(torch.isfinite(lse).all())
    assert torch.equal(rne_bf16(o32).view(torch.int16), o16.view(torch.int16))
    rows = block_rows(B, H, N, 128, seed=0)
    ref, ref_lse = oracle.attn(q, k, v, w.scale, mask=mask, rows=rows)
    got = o32.reshape(-1, 128)[rows.to(DEV)].cpu()
    e = errors(got, ref)
    _say(f"rows={rows.numel()} sparse fp32-out {e}")
    assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, e
    assert bf16_elementwise_ok(o16.reshape(-1, 128)[rows.to(DEV)].cpu(), ref).all()
    assert np.max(np.abs(to64(lse.reshape(-1)[rows.to(DEV)].cpu()) - ref_lse)) <= LSE_ABS


def test_long_sequence_sparse_sampled_parity():
    """One head of 2^19 + 77 tokens (4097 mask blocks, ragged last block),
    density 0.02 plus the forced diagonal and first block."""
    N = (1 << 19) + 77
    _say(f"case: long sequence block-sparse B1 H1 N{N}")
    q, k, v = make_qkv(1, 1, N, 128, seed=91)
    mask = make_block_mask(N, 64, 0.02, seed=92)
    o32 = dit.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), mask.to(DEV), out_fp32=True)
    torch.cuda.synchronize()
    rows = torch.unique(torch.cat([torch.tensor([0, 127, 128, N // 2, N - 78, N - 77, N - 1]),
                                   torch.randint(0, N, (25,), generator=torch.Generator().manual_seed(93))]))
    ref, _ = oracle.attn(q, k, v, 1.0 / math.sqrt(128), mask=mask, rows=rows)
    e = errors(o32.reshape(-1, 128)[rows.to(DEV)].cpu(), ref)
    _say(f"fp32-out {e}")
    assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, e


def test_blocksparse_bitwise_determinism():
    """Repeated calls give the same bits (O and lse): per-head masks of mixed
    density on a ragged shape, three launches, and the img2048_sparse
    workload, two launches."""
    _say("case: block-sparse determinism B1 H4 N3000 and img2048_sparse")
    N = 3000
    nb = (N + 127) // 128
    q, k, v = (t.to(DEV) for t in make_qkv(1, 4, N, 128, seed=97))
    masks = torch.stack([make_block_mask(N, 64, d, seed=60 + i)
                         for i, d in enumerate([0.1, 0.3, 0.6, 1.0])]).reshape(1, 4, nb, nb).to(DEV)
    runs = [dit.attn_fwd_blocksparse(q, k, v, masks, return_lse=True) for _ in range(3)]
    torch.cuda.synchronize()
    for o, lse in runs[1:]:
        assert torch.equal(o.view(torch.int16), runs[0][0].view(torch.int16))
        assert torch.equal(lse.view(torch.int32), runs[0][1].view(torch.int32))
    w = WORKLOADS["img2048_sparse"]
    qw, kw, vw, mw = (t.to(DEV) for t in make_workload_inputs(w, seed=0))
    a = dit.attn_fwd_blocksparse(qw, kw, vw, mw)
    b = dit.attn_fwd_blocksparse(qw, kw, vw, mw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_blocksparse_strided_inputs_and_output_match_contiguous_bitwise():
    """Q and V stored [B, N, H, D], K contiguous, O written into a
    [B, N, H, D] view, per-head masks: bit-identical to the all-contiguous
    call."""
    B, H, N = 1, 4, 333
    nb = (N + 127) // 128
    _say(f"case: block-sparse strided B{B} H{H} N{N}")
    q, k, v = make_qkv(B, H, N, 128, seed=25)
    qs, vs = (t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for t in (q, v))
    kd = k.to(DEV)
    masks = torch.stack([make_block_mask(N, 64, 0.4, seed=70 + i) for i in range(H)]).reshape(B, H, nb, nb).to(DEV)
    out = torch.empty((B, N, H, 128), dtype=torch.float32, device=DEV).transpose(1, 2)
    o_s = dit.attn_fwd_blocksparse(qs, kd, vs, masks, out_fp32=True, out=out)
    o_c = dit.attn_fwd_blocksparse(q.to(DEV), kd, v.to(DEV), masks, out_fp32=True)
    torch.cuda.synchronize()
    assert o_s.data_ptr() == out.data_ptr()
    assert torch.equal(o_s, o_c)
