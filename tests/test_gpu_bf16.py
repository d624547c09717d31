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
from tests._rows import block_rows, nan_like_out, nan_lse
from workloads import WORKLOADS, make_qkv, make_workload_inputs

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


def _blockwise_parity(name, workspace: bool):
    """Every 384-row work-group of the launch is checked: its first, last and
    one random row against the oracle, after the outputs were pre-filled with
    NaN (a work-group that never stores its rows would leave NaN behind).
    With `workspace`, the launch is the one the benchmark times
    (dit_attn_fwd_ws: the last partial round split over key ranges, the
    workspace also pre-filled with NaN)."""
    w = WORKLOADS[name]
    B, H, N = w.batch, w.heads, w.seqlen
    _say(f"case: {w.describe()} blockwise, workspace={workspace}")
    q, k, v, _ = make_workload_inputs(w, seed=0)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    ws = None
    if workspace:
        ws = dit.fwd_workspace(qd)
        ws.view(torch.uint8).fill_(0xFF)
    o32 = dit.attn_fwd(qd, kd, vd, out_fp32=True, out=nan_like_out(B, H, N, True, DEV), workspace=ws)
    o16, lse = dit.attn_fwd(qd, kd, vd, return_lse=True, out=nan_like_out(B, H, N, False, DEV),
                            lse_out=nan_lse(B, H, N, DEV), workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o32).all()) and bool(torch.isfinite(o16).all())
    assert bool(torch.isfinite(lse).all())
    assert torch.equal(rne_bf16(o32).view(torch.int16), o16.view(torch.int16))
    rows = block_rows(B, H, N, 384, seed=0)
    ref, ref_lse = oracle.attn(q, k, v, w.scale, rows=rows)
    o32r = o32.reshape(-1, 128)[rows.to(DEV)].cpu()
    o16r = o16.reshape(-1, 128)[rows.to(DEV)].cpu()
    e32, e16 = errors(o32r, ref), errors(o16r, ref)
    _say(f"rows={rows.numel()} fp32-out {e32}  bf16-out {e16}")
    assert e32["max_abs"] <= BF16_MAX_ABS and e32["mean_abs"] <= BF16_MEAN_ABS, e32
    assert bf16_elementwise_ok(o16r, ref).all()
    assert e16["mean_abs"] <= BF16_MEAN_ABS
    lse_r = lse.reshape(-1)[rows.to(DEV)].cpu().double().numpy()
    assert np.max(np.abs(lse_r - ref_lse)) <= LSE_ABS


def test_img1024_full_parity():
    """Every one of the 110,592 output rows of the 1024^2 shape."""
    w = WORKLOADS["img1024"]
    B, H, N = w.batch, w.heads, w.seqlen
    _say(f"case: {w.describe()} all rows")
    q, k, v, _ = make_workload_inputs(w, seed=0)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    ws = dit.fwd_workspace(qd)
    for wsp in (None, ws):
        o32 = dit.attn_fwd(qd, kd, vd, out_fp32=True, out=nan_like_out(B, H, N, True, DEV), workspace=wsp)
        o16, lse = dit.attn_fwd(qd, kd, vd, return_lse=True, out=nan_like_out(B, H, N, False, DEV),
                                lse_out=nan_lse(B, H, N, DEV), workspace=wsp)
        torch.cuda.synchronize()
        assert torch.equal(rne_bf16(o32).view(torch.int16), o16.view(torch.int16))
        e32, e16 = _check_against(q, k, v, w.scale, o32, o16, lse)
        _say(f"workspace={wsp is not None}: fp32-out {e32}  bf16-out {e16}")


def _check_against(q, k, v, scale, o32, o16, lse):
    ref, ref_lse = oracle.attn(q, k, v, scale)
    e32 = errors(o32, ref)
    assert e32["max_abs"] <= BF16_MAX_ABS and e32["mean_abs"] <= BF16_MEAN_ABS, e32
    assert bf16_elementwise_ok(o16, ref).all()
    e16 = errors(o16, ref)
    assert e16["mean_abs"] <= BF16_MEAN_ABS, e16
    assert np.max(np.abs(to64(lse) - ref_lse)) <= LSE_ABS
    return e32, e16


@pytest.mark.parametrize("workspace", [False, True])
def test_img2048_cfg_pair_blockwise_parity(workspace):
    _blockwise_parity("img2048", workspace)


@pytest.mark.parametrize("workspace", [False, True])
def test_i2i2048_blockwise_parity(workspace):
    """Image-to-image joint sequence: text + target + reference latents."""
    _blockwise_parity("i2i2048", workspace)


# Rows whose logits ramp up over many 32-key tiles: the query row is a scaled
# basis vector e_r, so key j's logit for it is (nearly) K[j, r], which is set
# to slope * ln 2 * tile(j) for the tiles of the ramp -- a row max that grows
# by `slope` log2 units per tile -- and falls back to N(0, 1) afterwards.
# Slopes of 40 and 70 push a lane's weights past the 2^64 redo bound every
# one or two tiles, 10 stays under it, 0 is flat; other rows of the same
# waves see the ramps mixed into their own logits.
RAMP_ROWS = [(0, 40.0), (17, 70.0), (47, 10.0), (48, 0.0), (130, 100.0), (301, 64.0), (777, 40.0)]


def _ramp_inputs(N, seed, first_tile=1, last_tile=14, tile=32):
    q, k, v = make_qkv(1, 1, N, 128, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    for r, (i, slope) in enumerate(RAMP_ROWS):
        if i >= N:
            continue
        q[0, 0, i] = 0
        q[0, 0, i, r] = math.sqrt(128.0)
        for t in range(first_tile, last_tile + 1):
            j0, j1 = t * tile, min(N, (t + 1) * tile)
            if j0 >= N:
                break
            base = slope * math.log(2.0) * (t - first_tile + 1)
            k[0, 0, j0:j1, r] = (base + 0.5 * torch.randn(j1 - j0, generator=g)).to(torch.bfloat16)
    return q, k, v


@pytest.mark.parametrize("N", [1000, 4000])
def test_logit_ramp_over_many_tiles(N):
    """The lazy reference max: the weights are taken against a reference that
    may lag the row max, and the tile is redone (reference moved, O and l
    rescaled) only when a lane's weight sum passes 2^64.  Full parity on rows
    whose max climbs far beyond that bound over many tiles, for dit_attn_fwd,
    dit_attn_fwd_ws (here a small grid, so every block is split over key
    ranges and the partial results carry very different maxima into the
    merge) and the block-sparse kernel with every block kept."""
    _say(f"case: logit ramp N={N}")
    q, k, v = _ramp_inputs(N, seed=26)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    scale = 1.0 / math.sqrt(128)
    nb = (N + 127) // 128
    ones = torch.ones((nb, nb), dtype=torch.uint8, device=DEV)
    for label, fn in (("fwd", lambda **kw: dit.attn_fwd(qd, kd, vd, **kw)),
                      ("fwd_ws", lambda **kw: dit.attn_fwd(qd, kd, vd, workspace=dit.fwd_workspace(qd), **kw)),
                      ("sparse", lambda **kw: dit.attn_fwd_blocksparse(qd, kd, vd, ones, **kw))):
        o32 = fn(out_fp32=True)
        o16, lse = fn(return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(rne_bf16(o32).view(torch.int16), o16.view(torch.int16)), label
        e32, e16 = _check_against(q, k, v, scale, o32, o16, lse)
        _say(f"{label}: fp32-out {e32}")


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


def test_largest_row_stride():
    """Rows 2^22 elements apart, the largest stride the boundary accepts: the
    key tiles staged past the last row (up to 127 rows beyond N) sit at
    32-bit byte offsets near 2^30 that must read as zeros.  Dense (with and
    without the tail split) and block-sparse against the oracle."""
    N, S = 200, 1 << 22           # one (b, h) slice spans 1.7 GB, below the 2 GiB limit
    _say(f"case: row stride {S} elements, N={N}")
    base = torch.zeros((3, N, S), dtype=torch.bfloat16, device=DEV)   # 5 GB
    q, k, v = make_qkv(1, 1, N, 128, seed=131)
    for i, t in enumerate((q, k, v)):
        base[i, :, :128] = t[0, 0].to(DEV)
    qd, kd, vd = (base[i, :, :128].unsqueeze(0).unsqueeze(0) for i in range(3))
    assert qd.stride(2) == S
    ref, _ = oracle.attn(q, k, v, 1.0 / math.sqrt(128))
    outs = [dit.attn_fwd(qd, kd, vd, out_fp32=True),
            dit.attn_fwd(qd, kd, vd, out_fp32=True, workspace=dit.fwd_workspace(qd))]
    mask = torch.ones((2, 2), dtype=torch.uint8, device=DEV)
    outs.append(dit.attn_fwd_blocksparse(qd, kd, vd, mask, out_fp32=True))
    torch.cuda.synchronize()
    for o in outs:
        e = errors(o, ref)
        assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, e
    del base
