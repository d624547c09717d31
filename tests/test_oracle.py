"""Pins for the fp64 oracle: checked against things other than itself.

Nothing here touches the GPU or the HIP library.  Each test names what fixes
the expected value: a 60-digit mpmath brute force, a library routine
(torch's float64 CPU scaled_dot_product_attention, logsumexp, softmax, its
float8_e4m3fn cast), a closed form, or an invariant of softmax attention.
"""
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from workloads import make_block_mask, make_qkv

HERE = os.path.dirname(os.path.abspath(__file__))


def _sdpa64(q, k, v, scale, bool_mask=None):
    q, k, v = (t.to(torch.float64) for t in (q, k, v))
    return F.scaled_dot_product_attention(q, k, v, attn_mask=bool_mask, scale=scale)


def _expand_mask(mask, N, block=128):
    """Block mask [nb, nb] -> boolean token mask [N, N] (True = attend)."""
    idx = torch.arange(N) // block
    return mask.bool()[idx][:, idx]


# ----------------------------------------------------------------------------
# dense attention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("N,D", [(1, 8), (2, 8), (3, 5), (17, 8), (5, 128)])
def test_attn_vs_mpmath_bruteforce(N, D):
    """60-digit brute force: p_j = e^{s_j} / sum e^{s} with no max shift."""
    g = torch.Generator().manual_seed(100 + N * 7 + D)
    q, k, v = (torch.randn((1, 1, N, D), generator=g, dtype=torch.float64) for _ in range(3))
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attn(q, k, v, scale)
    mpmath.mp.dps = 60
    Q, K, V = (t[0, 0].tolist() for t in (q, k, v))
    for i in range(N):
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(Q[i][d]) * mpmath.mpf(K[j][d]) for d in range(D))
             for j in range(N)]
        e = [mpmath.exp(x) for x in s]
        z = mpmath.fsum(e)
        for d in range(D):
            ref = mpmath.fsum(e[j] * mpmath.mpf(V[j][d]) for j in range(N)) / z
            assert abs(o[0, 0, i, d] - float(ref)) <= 1e-13
        assert abs(lse[0, 0, i] - float(mpmath.log(z))) <= 1e-13


def test_attn_vs_torch_sdpa_tiny_workload():
    """Library routine: torch float64 CPU SDPA on the tiny joint workload
    (64 text + 256 image tokens, 2 heads), and torch.logsumexp for lse."""
    q, k, v = make_qkv(1, 2, 320, 128, seed=0)
    scale = 1.0 / math.sqrt(128)
    o, lse = oracle.attn(q, k, v, scale)
    ref = _sdpa64(q, k, v, scale).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12
    logits = scale * (q.double() @ k.double().transpose(-1, -2))
    ref_lse = torch.logsumexp(logits, dim=-1).numpy()
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


def test_attn_large_logits_stay_finite():
    """Logits of order 1e3 overflow a naive exp; the max shift must keep the
    result finite and equal to SDPA."""
    q, k, v = make_qkv(1, 1, 64, 128, seed=5)
    q = q.double() * 60.0
    scale = 1.0 / math.sqrt(128)
    o, lse = oracle.attn(q, k, v, scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    ref = _sdpa64(q, k, v, scale).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12


def test_attn_peaked_keys_vs_sdpa():
    """The x8 key rows of the 2048^2 workload, at a small N."""
    q, k, v = make_qkv(1, 2, 400, 128, seed=0, peaked_key_frac=0.01)
    scale = 1.0 / math.sqrt(128)
    o, _ = oracle.attn(q, k, v, scale)
    ref = _sdpa64(q, k, v, scale).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12


@pytest.mark.parametrize("N", [320, 257])
def test_block_mask_vs_sdpa(N):
    """Masked blocks are -inf logits: SDPA with the expanded boolean mask.
    The mask is asymmetric, so a transposed (key, query) lookup fails."""
    q, k, v = make_qkv(1, 2, N, 128, seed=3)
    nb = (N + 127) // 128
    mask = torch.zeros((nb, nb), dtype=torch.uint8)
    mask.fill_diagonal_(1)
    mask[0, nb - 1] = 1          # query block 0 also sees the ragged last block
    mask[nb - 1, 1] = 1 if nb > 2 else 0
    scale = 1.0 / math.sqrt(128)
    o, lse = oracle.attn(q, k, v, scale, mask=mask)
    bm = _expand_mask(mask, N)
    ref = _sdpa64(q, k, v, scale, bm).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12
    logits = scale * (q.double() @ k.double().transpose(-1, -2))
    ref_lse = torch.logsumexp(logits.masked_fill(~bm, -math.inf), dim=-1).numpy()
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


def test_block_mask_per_head_stride():
    """A different mask per (b, h) through mask_stride_bh."""
    N = 300
    q, k, v = make_qkv(1, 2, N, 128, seed=4)
    nb = 3
    m0 = make_block_mask(N, 0, 0.4, seed=1)
    m1 = make_block_mask(N, 0, 0.4, seed=2)
    masks = torch.stack([m0, m1])
    scale = 1.0 / math.sqrt(128)
    o, _ = oracle.attn(q, k, v, scale, mask=masks, mask_stride_bh=nb * nb)
    for h, m in enumerate((m0, m1)):
        ref = _sdpa64(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], scale, _expand_mask(m, N)).numpy()
        assert np.max(np.abs(o[:, h:h + 1] - ref)) <= 1e-12


def test_fully_masked_row_is_zero():
    q, k, v = make_qkv(1, 1, 256, 128, seed=6)
    mask = torch.tensor([[0, 0], [1, 1]], dtype=torch.uint8)
    o, lse = oracle.attn(q, k, v, 0.1, mask=mask)
    assert np.all(o[0, 0, :128] == 0.0)
    assert np.all(np.isneginf(lse[0, 0, :128]))
    assert np.all(np.isfinite(o[0, 0, 128:]))


def test_rows_of_p_sum_to_one_and_equal_softmax():
    """V = identity rows (N <= D) makes O the probability matrix itself."""
    N, D = 17, 128
    g = torch.Generator().manual_seed(11)
    q, k = (torch.randn((1, 1, N, D), generator=g, dtype=torch.float64) for _ in range(2))
    v = torch.zeros((1, 1, N, D), dtype=torch.float64)
    v[0, 0, torch.arange(N), torch.arange(N)] = 1.0
    scale = 1.0 / math.sqrt(D)
    o, _ = oracle.attn(q, k, v, scale)
    P = o[0, 0, :, :N]
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-12
    ref = scipy.special.softmax(scale * (q[0, 0].numpy() @ k[0, 0].numpy().T), axis=1)
    assert np.max(np.abs(P - ref)) <= 1e-14
    assert np.all(o[0, 0, :, N:] == 0.0)


def test_constant_v_returns_constant():
    q, k, _ = make_qkv(1, 2, 300, 128, seed=7)
    v = torch.full((1, 2, 300, 128), 0.375, dtype=torch.float64)
    v[:, :, :, 5] = -2.5
    o, _ = oracle.attn(q, k, v, 0.0883883)
    assert np.max(np.abs(o[..., :5] - 0.375)) <= 1e-14
    assert np.max(np.abs(o[..., 5] + 2.5)) <= 1e-14


def test_key_value_permutation_invariance_and_query_equivariance():
    q, k, v = make_qkv(1, 1, 200, 128, seed=8)
    scale = 1.0 / math.sqrt(128)
    o, lse = oracle.attn(q, k, v, scale)
    pk = torch.randperm(200, generator=torch.Generator().manual_seed(1))
    o2, lse2 = oracle.attn(q, k[:, :, pk], v[:, :, pk], scale)
    assert np.max(np.abs(o - o2)) <= 1e-13 and np.max(np.abs(lse - lse2)) <= 1e-13
    pq = torch.randperm(200, generator=torch.Generator().manual_seed(2))
    o3, _ = oracle.attn(q[:, :, pq], k, v, scale)
    assert np.max(np.abs(o3 - o[:, :, pq.numpy()])) <= 1e-13


def test_one_hot_dominant_key_selects_its_value_row():
    N, D = 64, 128
    q, k, v = make_qkv(1, 1, N, D, seed=9)
    q, k, v = q.double(), k.double(), v.double()
    i, j = 10, 37
    k[0, 0, j] = 30.0 * q[0, 0, i]          # logit gap of order 30 |q_i|^2 / sqrt(D) >> 50
    o, _ = oracle.attn(q, k, v, 1.0 / math.sqrt(D))
    assert np.max(np.abs(o[0, 0, i] - v[0, 0, j].numpy())) <= 1e-15


def test_single_token_and_zero_query():
    q, k, v = make_qkv(1, 1, 1, 128, seed=10)
    o, lse = oracle.attn(q, k, v, 0.1)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0].double().numpy())
    assert lse[0, 0, 0] == pytest.approx(0.1 * float((q.double() * k.double()).sum()), abs=1e-14)
    q, k, v = make_qkv(1, 1, 150, 128, seed=11)
    o, lse = oracle.attn(torch.zeros_like(q), k, v, 0.1)
    assert np.max(np.abs(o[0, 0] - v[0, 0].double().numpy().mean(axis=0))) <= 1e-14
    assert np.max(np.abs(lse - math.log(150))) <= 1e-14


def test_sampled_rows_match_full():
    q, k, v = make_qkv(1, 2, 330, 128, seed=12)
    o, lse = oracle.attn(q, k, v, 0.0883883)
    rows = np.array([0, 5, 329, 330, 659], dtype=np.int64)
    os_, ls_ = oracle.attn(q, k, v, 0.0883883, rows=rows)
    flat = o.reshape(-1, 128)
    assert np.array_equal(os_, flat[rows]) and np.array_equal(ls_, lse.reshape(-1)[rows])


# ----------------------------------------------------------------------------
# OCP E4M3 codec
# ----------------------------------------------------------------------------

def _torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_exhaustive_vs_torch():
    ref = _torch_decode_all()
    mine = np.array([oracle.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_e4m3_golden_points():
    path = os.path.join(HERE, "golden", "e4m3_points.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code_s, val_s = line.split()
        code, val = int(code_s, 16), float(val_s)
        got = oracle.e4m3_decode(code)
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val)
            assert oracle.e4m3_encode(val) == code
        n += 1
    assert n >= 10


def test_e4m3_encode_all_bf16_vs_torch():
    """Every finite bf16 bit pattern, clamped to +-448, encoded with RNE."""
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).to(torch.float32)
    fin = torch.isfinite(x)
    x = x[fin].clamp(-448.0, 448.0)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3_encode(float(t)) for t in x.tolist()], dtype=np.uint8)
    assert np.array_equal(mine, ref)


def test_e4m3_encode_ties_and_random_fp32_vs_torch():
    ref_vals = _torch_decode_all()
    fin = ref_vals[np.isfinite(ref_vals) & (ref_vals >= 0)]
    fin = np.unique(fin)
    mids = (fin[1:] + fin[:-1]) / 2.0        # exact ties between neighbours
    g = np.random.default_rng(0)
    rnd = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 0.05, 3.0, 150.0)])
    x = np.concatenate([mids, -mids, rnd]).astype(np.float32)
    x = np.clip(x, -448.0, 448.0)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3_encode(float(t)) for t in x], dtype=np.uint8)
    assert np.array_equal(mine, ref)


# ----------------------------------------------------------------------------
# fp8 quantiser and recipe
# ----------------------------------------------------------------------------

def test_fp8_quantize_properties():
    q, _, _ = make_qkv(1, 2, 300, 128, seed=13)
    q[0, 1, 128:256] = 0            # an all-zero block
    codes, scales = oracle.fp8_quantize(q)
    x = q.to(torch.float32).numpy()
    dec = oracle.e4m3_decode_array(codes)
    for h in range(2):
        for b, (j0, j1) in enumerate([(0, 128), (128, 256), (256, 300)]):
            blk = x[0, h, j0:j1]
            amax = np.float32(np.abs(blk).max())
            c = codes[0, h, j0:j1]
            if amax == 0:
                assert scales[0, h, b] == 1.0 and np.all(c == 0)
                continue
            assert scales[0, h, b] == np.float32(amax / np.float32(448.0))
            # the block maximum lands exactly on the largest code
            assert np.max(np.abs(dec[0, h, j0:j1])) == 448.0
            # dequantised values within half an e4m3 step (relative 2^-4) or
            # half the subnormal step
            y = blk.astype(np.float64) * float(np.float32(448.0) / amax)
            err = np.abs(dec[0, h, j0:j1] - y)
            assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 1e-12)


def test_fp8_quantize_vs_torch_cast():
    q, _, _ = make_qkv(1, 3, 260, 128, seed=14)
    codes, scales = oracle.fp8_quantize(q)
    x = q.to(torch.float32)
    for h in range(3):
        for b, (j0, j1) in enumerate([(0, 128), (128, 256), (256, 260)]):
            blk = x[0, h, j0:j1]
            amax = blk.abs().max()
            inv = torch.tensor(448.0, dtype=torch.float32) / amax
            ref = (blk * inv).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[0, h, j0:j1], ref)


def _quantized_inputs(N, seed, H=1, peaked=0.0):
    q, k, v = make_qkv(1, H, N, 128, seed=seed, peaked_key_frac=peaked)
    q8, sq = oracle.fp8_quantize(q)
    k8, sk = oracle.fp8_quantize(k)
    v8, sv = oracle.fp8_quantize(v)
    return (q, k, v), (q8, k8, v8, sq, sk, sv)


def _dequant(codes, scales, block=128):
    dec = oracle.e4m3_decode_array(codes)
    s = np.repeat(scales.astype(np.float64), block, axis=-1)[..., :codes.shape[2]]
    return dec * s[..., None]


@pytest.mark.parametrize("N", [128, 300, 700])
def test_fp8_recipe_without_p_quantisation_is_attention_on_dequantised_inputs(N):
    """With P kept exact the running-max recipe must reduce to the textbook
    definition on the dequantised Q, K, V (pins the block bookkeeping and
    where each scale is applied)."""
    _, (q8, k8, v8, sq, sk, sv) = _quantized_inputs(N, 15, H=2)
    scale = 1.0 / math.sqrt(128)
    o, lse = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale, quantize_p=False)
    qd, kd, vd = _dequant(q8, sq), _dequant(k8, sk), _dequant(v8, sv)
    ref, ref_lse = oracle.attn(qd, kd, vd, scale)
    sd = _sdpa64(*(torch.from_numpy(t) for t in (qd, kd, vd)), scale).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12
    assert np.max(np.abs(o - sd)) <= 1e-12
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


def test_fp8_recipe_one_hot_key_returns_dequantised_value_row():
    (q, k, v), _ = _quantized_inputs(200, 16)
    i, j = 3, 150
    k = k.clone()
    k[0, 0, j] = (20.0 * q[0, 0, i].float()).to(torch.bfloat16)
    q8, sq = oracle.fp8_quantize(q)
    k8, sk = oracle.fp8_quantize(k)
    v8, sv = oracle.fp8_quantize(v)
    o, _ = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, 1.0 / math.sqrt(128))
    vd = _dequant(v8, sv)
    # P8 = e4m3(448) = 448 for the dominant key, every other weight rounds to 0
    assert np.max(np.abs(o[0, 0, i] - vd[0, 0, j])) <= 1e-12


def test_fp8_recipe_single_block_closed_form():
    """N <= 128: one key block, so the running max is the row max and the
    recipe is O = sum_j p_j V_j / sum_j p_j with p_j = dec(e4m3(448 w_j)) / 448."""
    (q, k, v), (q8, k8, v8, sq, sk, sv) = _quantized_inputs(96, 17)
    scale = 1.0 / math.sqrt(128)
    o, _ = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale)
    qd, kd, vd = _dequant(q8, sq)[0, 0], _dequant(k8, sk)[0, 0], _dequant(v8, sv)[0, 0]
    t = scale * (qd @ kd.T)
    w = np.exp(t - t.max(axis=1, keepdims=True))
    p8 = torch.from_numpy((w.astype(np.float32) * np.float32(448.0))).to(torch.float8_e4m3fn)
    p = p8.to(torch.float64).numpy() / 448.0
    ref = (p @ vd) / p.sum(axis=1, keepdims=True)
    assert np.max(np.abs(o[0, 0] - ref)) <= 1e-12


def test_fp8_recipe_error_band_vs_unquantised_oracle():
    """Four e4m3-rounded operands: the recipe's error against the exact
    attention on the bf16 inputs is a few percent (relative L2) with cosine
    well above 0.99, and is zero-mean noise rather than a bias."""
    (q, k, v), (q8, k8, v8, sq, sk, sv) = _quantized_inputs(1024, 18, H=2)
    scale = 1.0 / math.sqrt(128)
    o8, _ = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale)
    ref, _ = oracle.attn(q, k, v, scale)
    a, b = o8.ravel(), ref.ravel()
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
    assert 0.02 <= rel <= 0.09, rel
    assert cos >= 0.99
    assert abs(np.mean(a - b)) <= 0.05 * np.sqrt(np.mean((a - b) ** 2))


def _torch_dec(codes):
    """e4m3 codes -> float64 through torch's own float8_e4m3fn decoder."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e4m3(x32):
    """float32 values in [0, 448] -> e4m3 codes by torch's cast (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _recipe_rows_numpy(q8, k8, v8, sq, sk, sv, scale, i, final_max=False, block=128):
    """Row i of (0, 0) of the fp8 recipe restated with numpy, torch's e4m3
    codec and no shared code: key blocks in order; each block's P8 is rounded
    against the running max m_kb (or, for the negative control, against the
    row's final max); accumulator and row sum carried with exp(m_old - m_new)."""
    N = q8.shape[2]
    nb = (N + block - 1) // block
    qd = _torch_dec(q8[0, 0, i])
    kd, vd = _torch_dec(k8[0, 0]), _torch_dec(v8[0, 0])
    qb = i // block
    t = np.concatenate([scale * float(sq[0, 0, qb]) * float(sk[0, 0, kb]) *
                        (kd[kb * block:(kb + 1) * block] @ qd) for kb in range(nb)])
    m_final = t.max()
    m, l, acc, ms = -np.inf, 0.0, np.zeros(q8.shape[3]), []
    for kb in range(nb):
        tb = t[kb * block:(kb + 1) * block]
        mnew = max(m, tb.max())
        alpha = 0.0 if m == -np.inf else math.exp(m - mnew)
        ref = m_final if final_max else mnew
        w = np.exp(tb - ref)
        p = _torch_dec(_torch_e4m3(w.astype(np.float32) * np.float32(448.0))) / 448.0
        if final_max:
            l += p.sum()
            acc += float(sv[0, 0, kb]) * (p @ vd[kb * block:(kb + 1) * block])
        else:
            l = alpha * l + p.sum()
            acc = alpha * acc + float(sv[0, 0, kb]) * (p @ vd[kb * block:(kb + 1) * block])
        m = mnew
        ms.append(mnew)
    return acc / l, ms


@pytest.mark.parametrize("N,gaps", [(256, (2.3,)), (384, (1.7, 3.1))])
def test_fp8_recipe_running_max_across_key_blocks(N, gaps):
    """The running max moves between key blocks: block b (b >= 1) holds one
    key whose logit is gaps[b-1] above every earlier logit of the row, so
    each block's weights are rounded to e4m3 against a different max.  The
    oracle must equal a numpy / torch-codec restatement of that schedule, and
    must differ clearly from the variant that rounds every block against the
    row's final max (a plausible mistake no other pin catches)."""
    q, k, v = make_qkv(1, 1, N, 128, seed=19)
    i = 5
    scale = 1.0 / math.sqrt(128)
    qi = q[0, 0, i].double()
    base = float((k[0, 0, :128].double() @ qi).max()) * scale
    for b, gap in enumerate(gaps, start=1):
        target = base + sum(gaps[:b])          # logit of the planted key of block b
        k[0, 0, 128 * b + 7] = (target / (scale * float(qi @ qi)) * qi).to(torch.bfloat16)
    q8, sq = oracle.fp8_quantize(q)
    k8, sk = oracle.fp8_quantize(k)
    v8, sv = oracle.fp8_quantize(v)
    o, _ = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale, rows=np.array([i]))
    ref, ms = _recipe_rows_numpy(q8, k8, v8, sq, sk, sv, scale, i)
    wrong, _ = _recipe_rows_numpy(q8, k8, v8, sq, sk, sv, scale, i, final_max=True)
    # the set-up really moves the max at every block boundary
    assert all(b - a > 1.0 for a, b in zip(ms, ms[1:])), ms
    assert np.max(np.abs(o[0] - ref)) <= 1e-12
    assert np.max(np.abs(o[0] - wrong)) >= 1e-4


def _recipe_one_range_per_block_numpy(q8, k8, v8, sq, sk, sv, scale, i, block=128):
    """Row i of (0, 0) with every key block its own range, restated with numpy
    and torch's e4m3 codec: each block's P8 rounded against that block's own
    max, then the blocks merged with exp(m_b - M)."""
    N = q8.shape[2]
    nb = (N + block - 1) // block
    qd = _torch_dec(q8[0, 0, i])
    kd, vd = _torch_dec(k8[0, 0]), _torch_dec(v8[0, 0])
    qb = i // block
    parts = []
    for kb in range(nb):
        tb = scale * float(sq[0, 0, qb]) * float(sk[0, 0, kb]) * (kd[kb * block:(kb + 1) * block] @ qd)
        mb = tb.max()
        p = _torch_dec(_torch_e4m3(np.exp(tb - mb).astype(np.float32) * np.float32(448.0))) / 448.0
        parts.append((mb, p.sum(), float(sv[0, 0, kb]) * (p @ vd[kb * block:(kb + 1) * block])))
    M = max(m for m, _, _ in parts)
    l = sum(math.exp(m - M) * lp for m, lp, _ in parts)
    acc = sum(math.exp(m - M) * a for m, _, a in parts)
    return acc / l, M + math.log(l)


def test_fp8_recipe_split_into_key_ranges():
    """The recipe with each row's key blocks cut into ranges, each from a
    fresh running max, merged exactly: one range is the recipe; without P
    quantisation any cut gives the textbook attention on the dequantised
    inputs (the merge is exact); one range per block matches an independent
    restatement; with P quantisation a cut changes the result (each range
    rounds P against its own max) by about the e4m3 step."""
    N = 700                                   # 6 key blocks, the last ragged
    _, (q8, k8, v8, sq, sk, sv) = _quantized_inputs(N, 21, H=2)
    scale = 1.0 / math.sqrt(128)
    o1, l1 = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale)
    o1s, l1s = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale, nsplit=1)
    assert np.array_equal(o1, o1s) and np.array_equal(l1, l1s)
    o3, l3 = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale, quantize_p=False, nsplit=3)
    qd, kd, vd = _dequant(q8, sq), _dequant(k8, sk), _dequant(v8, sv)
    ref, ref_lse = oracle.attn(qd, kd, vd, scale)
    assert np.max(np.abs(o3 - ref)) <= 1e-12
    assert np.max(np.abs(l3 - ref_lse)) <= 1e-12
    o6, l6 = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale, nsplit=6)
    for i in (0, 5, 300, 699):
        want, want_lse = _recipe_one_range_per_block_numpy(q8, k8, v8, sq, sk, sv, scale, i)
        assert np.max(np.abs(o6[0, 0, i] - want)) <= 1e-12
        assert abs(l6[0, 0, i] - want_lse) <= 1e-12
    o3q, _ = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale, nsplit=3)
    diff = o3q - o1
    assert np.max(np.abs(diff)) >= 1e-5
    assert np.linalg.norm(diff) / np.linalg.norm(o1) <= 0.05
    with pytest.raises(ValueError):
        oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, scale, nsplit=7)   # more ranges than blocks


def test_fp8_quantize_tiny_block_is_a_zero_block():
    """448 / absmax overflows fp32 for absmax below 448 / FLT_MAX (~1.3e-36):
    such a block is stored like an all-zero one (scale 1, codes +0), also when
    it holds negative zeros; just above the bound it is quantised normally
    (absmax lands on code 448)."""
    x = torch.zeros((1, 3, 384, 128), dtype=torch.float32)
    g = torch.Generator().manual_seed(20)
    x[0, 0, 0:128] = torch.randn((128, 128), generator=g) * 1e-37    # absmax ~4e-37
    x[0, 0, 128:256] = -0.0
    x[0, 0, 256:384] = torch.randn((128, 128), generator=g)
    big = 4.0 * 448.0 / float(np.finfo(np.float32).max)                 # absmax above the bound
    x[0, 1, 0:128] = torch.randn((128, 128), generator=g) * (big / 4.0)
    x[0, 1, 0, 0] = big
    xb = x.to(torch.bfloat16)
    amax0 = np.float32(xb[0, 0, :128].float().abs().max())
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(448.0) / amax0)            # the block really is below the bound
    codes, scales = oracle.fp8_quantize(xb)
    assert scales[0, 0, 0] == 1.0 and np.all(codes[0, 0, 0:128] == 0)
    assert scales[0, 0, 1] == 1.0 and np.all(codes[0, 0, 128:256] == 0)
    amax1 = np.float32(xb[0, 1, :128].float().abs().max())
    assert np.isfinite(np.float32(448.0) / amax1)
    assert scales[0, 1, 0] == amax1 / np.float32(448.0)
    assert np.max(np.abs(oracle.e4m3_decode_array(codes[0, 1, :128]))) == 448.0


# ----------------------------------------------------------------------------
# block-mask selection (tau rule)
# ----------------------------------------------------------------------------

def _library_select(q, k, scale, tau, text_tokens, block=128):
    """The rule from library steps: block means by torch's avg_pool1d (the
    ragged last block through its own call), scipy's softmax, the threshold
    and the forced blocks."""
    B, H, N, D = q.shape
    nb = (N + block - 1) // block

    def pool(x):
        x = x.to(torch.float64).reshape(B * H, N, D).transpose(1, 2)      # [BH, D, N]
        full = (N // block) * block
        parts = []
        if full:
            parts.append(F.avg_pool1d(x[:, :, :full], block))
        if N > full:
            parts.append(F.avg_pool1d(x[:, :, full:], N - full))
        return torch.cat(parts, dim=2).transpose(1, 2).numpy()           # [BH, nb, D]

    qm, km = pool(q), pool(k)
    s = scale * np.einsum("bid,bjd->bij", qm, km)
    p = scipy.special.softmax(s, axis=-1)
    tb = (text_tokens + block - 1) // block
    idx = np.arange(nb)
    forced = (idx[:, None] == idx[None, :]) | (idx[:, None] < tb) | (idx[None, :] < tb)
    mask = ((p >= tau / nb) | forced[None]).astype(np.uint8)
    return mask.reshape(B, H, nb, nb), p.reshape(B, H, nb, nb)


@pytest.mark.parametrize("N,tau,text", [(640, 1.0, 128), (700, 1.05, 0), (1000, 1.6, 64)])
def test_select_blocks_vs_library_pooling_and_softmax(N, tau, text):
    g = torch.Generator().manual_seed(200 + N)
    q, k = (torch.randn((1, 2, N, 128), generator=g) * 3).to(torch.bfloat16), \
        (torch.randn((1, 2, N, 128), generator=g) * 3).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(128)
    mask, share = oracle.select_blocks(q, k, scale, tau, text)
    ref_mask, ref_share = _library_select(q, k, scale, tau, text)
    assert np.max(np.abs(share - ref_share)) <= 1e-13
    assert np.allclose(share.sum(-1), 1.0, atol=1e-13)
    near = np.abs(ref_share - tau / ref_share.shape[-1]) <= 1e-9 * tau / ref_share.shape[-1]
    assert np.array_equal(mask[~near], ref_mask[~near])
    # the rule thins: fewer kept blocks than the dense count, more than the forced ones
    assert 0 < int(mask.sum()) < mask.size


def test_select_blocks_invariants():
    """Shifting every key by one vector shifts a row's logits by a constant
    (softmax unchanged); permuting whole key blocks permutes the shares'
    columns; tau = 0 keeps everything."""
    N, scale = 768, 1.0 / math.sqrt(128)
    g = torch.Generator().manual_seed(210)
    q = (torch.randn((1, 1, N, 128), generator=g) * 2).to(torch.bfloat16)
    k = (torch.randn((1, 1, N, 128), generator=g) * 2).to(torch.bfloat16)
    _, share = oracle.select_blocks(q, k, scale, 1.0, 0)
    shift = torch.randn(128, generator=g).to(torch.bfloat16)
    _, share_s = oracle.select_blocks(q, (k.double() + shift.double()), scale, 1.0, 0)
    assert np.max(np.abs(share - share_s)) <= 1e-12
    perm = torch.tensor([3, 0, 5, 1, 4, 2])
    kp = k.reshape(1, 1, 6, 128, 128)[:, :, perm].reshape(1, 1, N, 128)
    _, share_p = oracle.select_blocks(q, kp, scale, 1.0, 0)
    assert np.max(np.abs(share_p - share[..., perm.numpy()])) <= 1e-13
    mask0, _ = oracle.select_blocks(q, k, scale, 0.0, 0)
    assert mask0.all()


def test_select_blocks_identical_key_blocks_and_planted_block():
    """Every key block with the same mean: every share is exactly 1 / nb, so
    tau just below 1 keeps everything and just above keeps only the forced
    blocks.  A key block aligned with a query block's mean takes almost all
    of its mass and is the only unforced block kept at tau = 1."""
    nb, scale = 5, 1.0 / math.sqrt(128)
    g = torch.Generator().manual_seed(220)
    q = torch.randn((1, 1, nb * 128, 128), generator=g).to(torch.bfloat16)
    blockk = torch.randn((1, 1, 128, 128), generator=g).to(torch.bfloat16)
    k = blockk.repeat(1, 1, nb, 1)
    m_lo, share = oracle.select_blocks(q, k, scale, 0.999, 0)
    assert np.array_equal(share, np.full_like(share, 1.0 / nb))
    assert m_lo.all()
    m_hi, _ = oracle.select_blocks(q, k, scale, 1.001, 128)
    idx = np.arange(nb)
    forced = (idx[:, None] == idx[None, :]) | (idx[:, None] < 1) | (idx[None, :] < 1)
    assert np.array_equal(m_hi[0, 0], forced.astype(np.uint8))
    # planted: key block 3 = 20 x the mean of query block 1, tokens otherwise noise
    k2 = (torch.randn((1, 1, nb * 128, 128), generator=g) * 0.1).to(torch.bfloat16)
    qmean = q[0, 0, 128:256].double().mean(0)
    k2[0, 0, 384:512] = (20 * qmean).to(torch.bfloat16)
    m2, share2 = oracle.select_blocks(q, k2, scale, 1.0, 0)
    assert share2[0, 0, 1, 3] > 0.5
    kept_unforced = [j for j in range(nb) if m2[0, 0, 1, j] and j != 1]
    assert kept_unforced == [3]
