"""Every entry point captured into a HIP graph and replayed.

The library enqueues kernels only (no allocation, no memset, no host
synchronisation), so a caller may capture its calls.  Each case captures one
call with static buffers, then replays the graph several times with the
program's own eager work and synchronisations in between; before every replay
the outputs are overwritten with garbage, and after it they must equal the
eager call's outputs bit for bit.
"""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import assert_bitwise, banner, dev, host, weight_t

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def bi():
    import deterministic_persistent_gemm_amd as m
    return m


def replay_and_check(torch, call, outs, what):
    """call() writes into the tensors of `outs` (a list); returns nothing."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    eager = [host(o).copy() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 16, device="cuda")
    for r in range(REPLAYS):
        for o in outs:
            if o.dtype in (torch.float32, torch.bfloat16):
                o.fill_(float("nan"))
            else:
                o.fill_(-7)
        # unrelated eager work between replays
        scratch = torch.sin(scratch) * 1.5 + scratch.sum() * 1e-9
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert_bitwise(host(o), eager[i], f"{what}: replay {r}, output {i}")
    del g


@pytest.mark.parametrize("M", [1, 17, 128, 1024])
def test_graph_linear_f32(bi, M):
    import torch
    banner(f"graph replay bi_linear_f32 router M={M}")
    w = wl.router_weights(0)
    wd, bd = dev(w.w), dev(w.b)
    x = dev(wl.router_batch(M, w).x)
    out = torch.empty((M, 256), dtype=torch.float32, device="cuda")
    replay_and_check(torch, lambda: bi.bi_linear_f32(x, weight_t(wd), bd, out=out), [out], f"router M={M}")


@pytest.mark.parametrize("M", [1, 33, 256])
def test_graph_linear_bf16(bi, M):
    import torch
    banner(f"graph replay bi_linear_bf16 dense M={M}")
    w = wl.dense_bf16_weights(0)
    wd = dev(w.w)
    x = dev(wl.dense_bf16_batch(M, w).x)
    out = torch.empty((M, w.w.shape[0]), dtype=torch.bfloat16, device="cuda")
    replay_and_check(torch, lambda: bi.bi_linear_bf16(x, weight_t(wd), None, out=out), [out], f"bf16 M={M}")


@pytest.mark.parametrize("M", [1, 16, 64])
def test_graph_moe(bi, M):
    import torch
    banner(f"graph replay bi_moe_grouped_gemm M={M}")
    mw = wl.moe_weights(0)
    x = dev(wl.moe_batch(M, mw).x)
    wr, w13, w2 = dev(mw.w_router), dev(mw.w13), dev(mw.w2)
    k = wl.MOE_TOPK
    y = torch.empty((M, wl.MOE_H), dtype=torch.float32, device="cuda")
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    probs = torch.empty((M, k), dtype=torch.float32, device="cuda")

    def call():
        yy, ii, pp = bi.bi_moe_grouped_gemm(x, wr, None, w13, w2, k)
        y.copy_(yy)
        ids.copy_(ii.to(torch.int32))
        probs.copy_(pp)

    replay_and_check(torch, call, [y, ids, probs], f"MoE M={M}")


@pytest.mark.parametrize("rows", [1, 64])
def test_graph_indexer_topk(bi, rows):
    import torch
    banner(f"graph replay bi_indexer_topk rows={rows}")
    b = wl.indexer_decode(rows)
    s = dev(b.scores)
    rs, re = dev(b.row_start), dev(b.row_end)
    out = torch.empty((rows, 2048), dtype=torch.int32, device="cuda")
    replay_and_check(torch, lambda: bi.bi_indexer_topk(s, 2048, rs, re, out=out), [out], f"top-k rows={rows}")



def test_cached_workspace_outlives_a_graph_that_captured_it(bi):
    # capture a call at M=1 (it uses the stream's cached workspace), then grow
    # that cache with an eager call at M=128 on the same stream; the captured
    # graph still writes into the first workspace on replay, so that memory
    # must not be handed to another tensor.  A sentinel allocated after the
    # growth must survive the replays, and the replays keep their bits.
    import torch
    banner("graph replay after the cached workspace grew")
    w = wl.router_weights(0)
    wd, bd = dev(w.w), dev(w.b)
    stream = torch.cuda.Stream()
    x1 = dev(wl.router_batch(1, w).x)
    x128 = dev(wl.router_batch(128, w).x)
    y1 = torch.empty((1, 256), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(stream):
        bi.bi_linear_f32(x1, weight_t(wd), bd, out=y1)
    torch.cuda.synchronize()
    ref = host(y1).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        bi.bi_linear_f32(x1, weight_t(wd), bd, out=y1)
    torch.cuda.synchronize()
    key = (torch.cuda.current_device(), stream.cuda_stream)
    before = bi._ws_cache[key].data_ptr()
    with torch.cuda.stream(stream):
        big = bi.bi_linear_f32(x128, weight_t(wd), bd)
    torch.cuda.synchronize()
    assert bi._ws_cache[key].data_ptr() != before or \
        bi._ws_cache[key].numel() >= bi.lib().bi_linear_workspace_size(bi.BI_F32, 128, 256, 4096)
    big_ref = host(big).copy()
    sentinels = [torch.full((1 << 18,), 3.25, dtype=torch.float32, device="cuda") for _ in range(8)]
    for r in range(REPLAYS):
        y1.fill_(float("nan"))
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert_bitwise(host(y1), ref, f"replay {r} after the workspace grew")
        for s in sentinels:
            assert bool((s == 3.25).all()), "a tensor allocated after the growth was overwritten"
    with torch.cuda.stream(stream):
        again = bi.bi_linear_f32(x128, weight_t(wd), bd)
    torch.cuda.synchronize()
    assert_bitwise(host(again), big_ref, "M=128 after the replays")
    del g


def test_workspace_growth_inside_a_capture_is_refused(bi):
    # a call whose workspace would have to grow during a capture raises
    # instead of allocating memory the graph would then depend on
    import torch
    w = wl.router_weights(0)
    wd, bd = dev(w.w), dev(w.b)
    stream = torch.cuda.Stream()
    x = dev(wl.router_batch(16, w).x)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="graph capture"):
        with torch.cuda.graph(g, stream=stream):
            bi.bi_linear_f32(x, weight_t(wd), bd)
    torch.cuda.synchronize()
