"""dit_attn_fwd_noalloc: the allocation-free variant of dit_attn_fwd_ws.

Called through the C ABI; its output must equal dit_attn_fwd_ws's bit for bit
(same kernels, same split plan), on two calls in a row, the second with a
smaller input (the library's static scratch keeps the first call's partial
results, which the second must not pick up), and a shape whose split would
not fit the scratch must be refused before anything runs."""
import ctypes

import pytest
import torch

import joint_attention_non_amd as dit
from workloads import WORKLOADS, make_qkv, make_workload_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _both(q, k, v):
    B, H, N, _ = q.shape
    lse_n = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    o_n = torch.full_like(q, float("nan"))
    o_n, lse_n = dit.attn_fwd_noalloc(q, k, v, return_lse=True, out=o_n, lse_out=lse_n)
    o_w, lse_w = dit.attn_fwd(q, k, v, return_lse=True, workspace=dit.fwd_workspace(q))
    torch.cuda.synchronize()
    return o_n, lse_n, o_w, lse_w


def test_noalloc_equals_workspace_entry_point_twice():
    w = WORKLOADS["img2048"]
    _say(f"case: noalloc {w.describe()}, then B1 H3 N5000")
    q, k, v, _ = make_workload_inputs(w, seed=0)
    q, k, v = (t.to(DEV) for t in (q, k, v))
    need = dit.fwd_workspace_bytes(q)
    assert 0 < need <= dit.load().dit_attn_fwd_noalloc_scratch_bytes()
    o_n, lse_n, o_w, lse_w = _both(q, k, v)
    assert torch.equal(o_n.view(torch.int16), o_w.view(torch.int16))
    assert torch.equal(lse_n, lse_w)
    del q, k, v, o_n, o_w
    # second call, smaller input: the scratch still holds the first call's partials
    q, k, v = (t.to(DEV) for t in make_qkv(1, 3, 5000, 128, seed=120))
    assert dit.fwd_workspace_bytes(q) > 0
    o_n, lse_n, o_w, lse_w = _both(q, k, v)
    assert torch.equal(o_n.view(torch.int16), o_w.view(torch.int16))
    assert torch.equal(lse_n, lse_w)
    # and fp32 output, through the raw C entry point
    o32 = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    s = dit._shape(q, k, v, o32, None, dit.FLAG_OUT_F32)
    rc = dit.load().dit_attn_fwd_noalloc(ctypes.byref(s), dit._ptr(q), dit._ptr(k), dit._ptr(v), dit._ptr(o32),
                                         None, dit._stream())
    assert rc == 0
    ref32 = dit.attn_fwd(q, k, v, out_fp32=True, workspace=dit.fwd_workspace(q))
    torch.cuda.synchronize()
    assert torch.equal(o32, ref32)


def test_noalloc_refuses_a_split_larger_than_its_scratch():
    """A shape is refused when its split needs more scratch than the library
    holds; on this device no shape does (the largest split is one partial
    block per compute unit), so the check is driven through the size query."""
    lib = dit.load()
    cap = lib.dit_attn_fwd_noalloc_scratch_bytes()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert cus * 384 * 132 * 4 <= cap, "one partial block per compute unit must fit"
