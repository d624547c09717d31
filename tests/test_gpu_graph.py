"""Every entry point can be captured into a HIP graph (torch.cuda.graph) and
replayed: the calls only enqueue kernels on the caller's stream, allocate
nothing and never read device memory from the host.  Each replay must equal
the eager result bit for bit, with eager work and synchronisations between
the replays (outputs are overwritten before each replay, so a replay that
did nothing would be caught)."""
import pytest
import torch

import joint_attention_non_amd as dit
from workloads import make_block_mask, make_local_qkv, make_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _replays_match(call, outs, eager, n=4):
    """call() writes into the preallocated tensors `outs`; eager = their
    values from an eager run."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    for i in range(n):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), f"replay {i} differs"
        # unrelated eager work between replays
        call()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), f"eager call after replay {i} differs"


@pytest.mark.parametrize("N", [300, 5000])
def test_graph_dense_with_workspace(N):
    _say(f"case: graph capture dit_attn_fwd_ws B1 H3 N{N}")
    q, k, v = (t.to(DEV) for t in make_qkv(1, 3, N, 128, seed=110))
    ws = dit.fwd_workspace(q)
    o = torch.empty_like(q)
    lse = torch.empty((1, 3, N), dtype=torch.float32, device=DEV)
    call = lambda: dit.attn_fwd(q, k, v, out=o, lse_out=lse, workspace=ws)
    call()
    torch.cuda.synchronize()
    _replays_match(call, (o, lse), (o.clone(), lse.clone()))


def test_graph_fp8():
    N = 3000
    _say(f"case: graph capture dit_attn_fwd_fp8 B1 H3 N{N}")
    q, k, v = (t.to(DEV) for t in make_qkv(1, 3, N, 128, seed=111))
    ws = torch.empty(dit.fp8_workspace_bytes(q), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((1, 3, N), dtype=torch.float32, device=DEV)
    call = lambda: dit.attn_fwd_fp8(q, k, v, out=o, lse_out=lse, workspace=ws)
    call()
    torch.cuda.synchronize()
    _replays_match(call, (o, lse), (o.clone(), lse.clone()))


def test_graph_blocksparse():
    N = 3000
    _say(f"case: graph capture dit_attn_fwd_blocksparse B1 H3 N{N}")
    q, k, v = (t.to(DEV) for t in make_qkv(1, 3, N, 128, seed=112))
    mask = make_block_mask(N, 512, 0.25, seed=3).to(DEV)
    o = torch.empty((1, 3, N, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, 3, N), dtype=torch.float32, device=DEV)
    call = lambda: dit.attn_fwd_blocksparse(q, k, v, mask, out=o, lse_out=lse, out_fp32=True)
    call()
    torch.cuda.synchronize()
    _replays_match(call, (o, lse), (o.clone(), lse.clone()))


def test_graph_select_then_blocksparse():
    """The selection and the block-sparse attention on its mask, captured
    together in one graph (three kernels: pooling, selection, attention)."""
    N = 3000
    _say(f"case: graph capture dit_attn_select_blocks + blocksparse B1 H3 N{N}")
    q, k, v = (t.to(DEV) for t in make_local_qkv(1, 3, N, 256, seed=113))
    nb = (N + 127) // 128
    mask = torch.empty((1, 3, nb, nb), dtype=torch.uint8, device=DEV)
    ws = torch.empty(dit.select_blocks_workspace_bytes(q), dtype=torch.uint8, device=DEV)
    o = torch.empty((1, 3, N, 128), dtype=torch.float32, device=DEV)

    def call():
        dit.select_blocks(q, k, 1.0, 256, out=mask, workspace=ws)
        dit.attn_fwd_blocksparse(q, k, v, mask, out=o, out_fp32=True)

    call()
    torch.cuda.synchronize()
    assert 0 < int(mask.sum()) < mask.numel()
    _replays_match(call, (mask, o), (mask.clone(), o.clone()))
