"""GPU parity of the bf16 path (dit_attn_fwd) against the fp64 oracle.

Every call goes through the C ABI (ctypes binding); every expected value comes
from ``oracle/`` on the same seeded inputs (``workloads``).
"""
import math

import numpy as np
import pytest
import torch

import joint_attention_non_amd as dit
import oracle
from tests._metrics import (BF16_MAX_ABS, BF16_MEAN_ABS, LSE_ABS, bf16_elementwise_ok, errors,
                            rne_bf16, to64)
from workloads import WORKLOADS, make_qkv, make_workload_inputs, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _run_both(q, k, v, scale=None):
    """bf16 output, fp32 output and lse from one set of inputs."""
    o16, lse = dit.attn_fwd(q, k, v, scale=scale, return_lse=True)
    o32 = dit.attn_fwd(q, k, v, scale=scale, out_fp32=True)
    torch.cuda.synchronize()
    return o16, o32, lse


def _check_full(q, k, v, scale=None, lse_tol=LSE_ABS):
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    o16, o32, lse = _run_both(q.to(DEV), k.to(DEV), v.to(DEV), scale)
    ref, ref_lse = oracle.attn(q, k, v, scale)
    e32 = errors(o32, ref)
    assert e32["max_abs"] <= BF16_MAX_ABS and e32["mean_abs"] <= BF16_MEAN_ABS, e32
    assert torch.equal(rne_bf16(o32).view(torch.int16), o16.view(torch.int16)), \
        "bf16 output is not the RNE image of the fp32 output"
    assert bf16_elementwise_ok(o16, ref).all()
    e16 = errors(o16, ref)
    assert e16["mean_abs"] <= BF16_MEAN_ABS, e16
    assert np.max(np.abs(to64(lse) - ref_lse)) <= lse_tol
    return e32, e16


def test_tiny_workload_full_parity():
    w = WORKLOADS["tiny"]
    _say(f"case: {w.describe()}")
    q, k, v, _ = make_workload_inputs(w, seed=0)
    e32, e16 = _check_full(q, k, v)
    _say(f"fp32-out {e32}  bf16-out {e16}")


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 320, 511, 700])
def test_ragged_lengths(N):
    _say(f"case: ragged N={N} B=1 H=2")
    q, k, v = make_qkv(1, 2, N, 128, seed=N)
    _check_full(q, k, v)


def test_batch_heads_and_scale():
    _say("case: B=2 H=3 N=200 scale=0.05")
    q, k, v = make_qkv(2, 3, 200, 128, seed=21)
    _check_full(q, k, v, scale=0.05)


def test_strided_bnhd_layout_matches_contiguous_bitwise():
    """[B, N, H, D] storage viewed as [B, H, N, D] (strides (N*H*D, D, H*D))."""
    _say("case: BNHD strides B=1 H=4 N=333")
    q, k, v = make_qkv(1, 4, 333, 128, seed=22)
    qs, ks, vs = (t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for t in (q, k, v))
    assert qs.stride(2) == 4 * 128
    o_strided = dit.attn_fwd(qs, ks, vs)
    o_contig = dit.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV))
    # the workspace entry point splits this small grid over key ranges; the
    # strides must not matter there either
    o_ws_strided = dit.attn_fwd(qs, ks, vs, workspace=dit.fwd_workspace(qs))
    o_ws_contig = dit.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), workspace=dit.fwd_workspace(qs))
    torch.cuda.synchronize()
    assert torch.equal(o_strided.view(torch.int16), o_contig.view(torch.int16))
    assert torch.equal(o_ws_strided.view(torch.int16), o_ws_contig.view(torch.int16))


def test_bitwise_determinism():
    _say("case: determinism B=1 H=4 N=1000")
    q, k, v = (t.to(DEV) for t in make_qkv(1, 4, 1000, 128, seed=23))
    outs = [dit.attn_fwd(q, k, v) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


# (query row, dominant key) pairs for N = 300 (the dense kernel's 32-key
# tiles, the last one ragged): the key sits in each of the four 4-key lane
# groups (key % 16 // 4) and in both 16-key halves of its tile, in the
# first, a middle and the ragged last tile, and the rows cover several
# waves and 16-row blocks.
ONE_HOT_CASES = [(17, 250), (3, 68), (40, 36), (63, 299), (100, 270), (299, 7), (150, 131), (255, 190)]


@pytest.mark.parametrize("i,j", ONE_HOT_CASES)
def test_one_hot_key_returns_value_row_bitwise(i, j):
    """A dominant key: P = 2^0 = 1 for it, every other weight underflows to
    0, l = 1, so O is that V row exactly -- which also needs the running max
    to be the max over every key of the row, whichever lanes hold it."""
    _say(f"case: one-hot key i={i} j={j}")
    N = 300
    q, k, v = make_qkv(1, 1, N, 128, seed=24)
    k[0, 0, j] = (40.0 * q[0, 0, i].float()).to(torch.bfloat16)
    o = dit.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o[0, 0, i].cpu().view(torch.int16), v[0, 0, j].view(torch.int16))


def test_constant_v():
    _say("case: constant V")
    q, k, _ = make_qkv(1, 2, 400, 128, seed=25)
    v = torch.full_like(q, 0.75)
    o = dit.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out_fp32=True)
    torch.cuda.synchronize()
    assert float((o - 0.75).abs().max()) <= 1e-3


def _sampled_parity(name, n_rows):
    w = WORKLOADS[name]
    _say(f"case: {w.describe()} sampled rows={n_rows}")
    q, k, v, _ = make_workload_inputs(w, seed=0)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o16, o32, lse = _run_both(qd, kd, vd)
    assert torch.equal(rne_bf16(o32).view(torch.int16), o16.view(torch.int16))
    assert bool(torch.isfinite(o32).all())
    rows = sample_rows(w.batch, w.heads, w.seqlen, n_rows, seed=0)
    ref, ref_lse = oracle.attn(q, k, v, w.scale, rows=rows)
    o32r = o32.reshape(-1, 128)[rows.to(DEV)].cpu()
    o16r = o16.reshape(-1, 128)[rows.to(DEV)].cpu()
    e32, e16 = errors(o32r, ref), errors(o16r, ref)
    _say(f"fp32-out {e32}  bf16-out {e16}")
    assert e32["max_abs"] <= BF16_MAX_ABS and e32["mean_abs"] <= BF16_MEAN_ABS, e32
    assert bf16_elementwise_ok(o16r, ref).all()
    assert e16["mean_abs"] <= BF16_MEAN_ABS
    lse_r = lse.reshape(-1)[rows.to(DEV)].cpu().double().numpy()
    assert np.max(np.abs(lse_r - ref_lse)) <= LSE_ABS


def test_img1024_sampled_parity():
    _sampled_parity("img1024", 512)


def test_img2048_cfg_pair_sampled_parity():
    _sampled_parity("img2048", 384)


def test_i2i2048_sampled_parity():
    """Image-to-image joint sequence: text + target + reference latents."""
    _sampled_parity("i2i2048", 256)


def test_long_sequence_sampled_parity():
    """One head of 2^20 + 37 tokens: byte offsets far past 2^24 inside the
    slice, 16385 key tiles with a ragged last one."""
    N = (1 << 20) + 37
    _say(f"case: long sequence B1 H1 N{N}")
    q, k, v = make_qkv(1, 1, N, 128, seed=31)
    o32 = dit.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out_fp32=True)
    torch.cuda.synchronize()
    rows = torch.unique(torch.cat([torch.tensor([0, 1, N // 2, N - 38, N - 37, N - 1]),
                                   torch.randint(0, N, (26,), generator=torch.Generator().manual_seed(32))]))
    ref, _ = oracle.attn(q, k, v, 1.0 / math.sqrt(128), rows=rows)
    e = errors(o32.reshape(-1, 128)[rows.to(DEV)].cpu(), ref)
    _say(f"fp32-out {e}")
    assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, e
