"""The XCD hand-over decode (one launch) against the two-launch decode, the
persistent kernel and the oracle.

Every wave of an output tile runs on one XCD; the last wave to arrive at the
tile's counter folds the k tile partials in ascending order.  These tests
check that the dispatcher really puts workgroups whose linear ids agree
modulo 8 on one XCD, that the hand-over reproduces the other paths bit for
bit at every decode batch size (GateLinear page, "Tests": bitwise equality
across batch sizes), that the counters it leaves behind are zero, and that
it survives graph replays.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import F32_ATOL, F32_RTOL, assert_bitwise, assert_close, banner, dev, host, weight_t

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bi():
    import deterministic_persistent_gemm_amd as m
    return m


@pytest.fixture(scope="module")
def router():
    w = wl.router_weights(0)
    return w, dev(w.w), dev(w.b)


@pytest.mark.parametrize("gx,gy", [(512, 1), (512, 4), (4096, 1), (8, 64)])
def test_workgroups_agreeing_mod_8_share_an_xcd(bi, gx, gy):
    banner(f"XCD ids of a {gx}x{gy} grid")
    ids = host(bi.bi_lab_xcc_ids(gx, gy)).reshape(-1)
    lin = np.arange(ids.size)
    per_class = [np.unique(ids[lin % 8 == r]) for r in range(8)]
    assert all(len(u) == 1 for u in per_class), per_class
    assert len({int(u[0]) for u in per_class}) == 8, per_class


@pytest.mark.parametrize("M", [1, 2, 4, 8, 15, 16, 17, 32, 33, 64, 128, 200, 512])
def test_router_xcd_decode_bitwise(bi, router, M):
    w, wd, bd = router
    banner(f"router fp32 M={M} XCD hand-over vs two-launch vs persistent")
    batch = wl.router_batch(M, w)
    x = dev(batch.x)
    h = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_DECODE_XCD))
    d = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_DECODE))
    p = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_PERSISTENT))
    assert_bitwise(h, d, f"XCD hand-over vs two-launch at M={M}")
    assert_bitwise(h, p, f"XCD hand-over vs persistent at M={M}")
    sample = np.unique(np.r_[sum(batch.probes.values(), []), 0, M - 1]).astype(int)
    assert_close(h[sample], oracle.linear_f32(batch.x[sample], w.w, w.b), F32_ATOL, F32_RTOL, f"oracle M={M}")


@pytest.mark.parametrize("N,K,block_k", [(128, 2048, 128), (128, 320, 32), (128, 4096, 64), (256, 512, 256),
                                         (384, 1024, 128)])
def test_xcd_decode_other_tile_counts(bi, N, K, block_k):
    # 16, 10, 64 and 2 tile partials (more than one batch of partial loads
    # at 64), N tiles 8, 16 and 24
    g = np.random.default_rng(N * 7 + K + block_k)
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    b = (g.standard_normal(N) * 0.01).astype(np.float32)
    r = bi.bi_describe_recipe(bi.BI_F32, N, K)
    r.block_k = block_k
    wd, bd = dev(w), dev(b)
    for M in (1, 19, 40):
        banner(f"fp32 N={N} K={K} block_k={block_k} M={M} XCD hand-over")
        x = g.standard_normal((M, K)).astype(np.float32)
        xd = dev(x)
        h = host(bi.bi_lab_linear(xd, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_DECODE_XCD))
        d = host(bi.bi_lab_linear(xd, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_DECODE))
        assert_bitwise(h, d, "XCD hand-over vs two-launch")
        assert_close(h, oracle.linear_f32(x, w, b), F32_ATOL, F32_RTOL, "oracle")


def test_xcd_decode_rejects_what_it_cannot_serve(bi):
    import torch
    # N/16 not a multiple of 8: the waves of one output tile would span XCDs
    x = torch.zeros((4, 256), dtype=torch.float32, device="cuda")
    w = torch.zeros((32, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(bi.BIError) as e:
        bi.bi_lab_linear(x, weight_t(w), None, path=bi.BI_PATH_DECODE_XCD)
    assert e.value.status == bi.BI_EUNSUPPORTED


def test_counters_return_to_zero_and_calls_alternate(bi, router):
    # alternate batch sizes through one workspace; the counter region must
    # read zero after every call and every result keep its bits
    import torch
    w, wd, bd = router
    seq = (1, 33, 128, 16, 1, 200, 17, 128, 2)
    need = max(bi.lib().bi_lab_workspace_size(bi.bi_describe_recipe(bi.BI_F32, 256, 4096), bi.BI_PATH_DECODE_XCD,
                                              M, 256, 4096) for M in seq)
    ws = bi.alloc_workspace(need, "cuda")
    # the partial region may hold anything: poison it
    ws[bi.WS_COUNTER_BYTES:] = 0xFF
    refs = {}
    for i, M in enumerate(seq):
        banner(f"XCD hand-over shared workspace call {i}: M={M}")
        x = dev(wl.router_batch(M, w).x)
        y = torch.empty((M, 256), dtype=torch.float32, device="cuda")
        st = _abi_lab(bi, x, wd, bd, y, ws, bi.BI_PATH_DECODE_XCD)
        assert st == bi.BI_OK
        torch.cuda.synchronize()
        assert int(ws[:bi.WS_COUNTER_BYTES].count_nonzero()) == 0, f"counters left non-zero after call {i}"
        got = host(y)
        if M not in refs:
            refs[M] = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_DECODE))
        assert_bitwise(got, refs[M], f"call {i} M={M}")


def _abi_lab(bi, x, wd, bd, y, ws, path):
    import ctypes
    import torch
    M, K = x.shape
    N = wd.shape[0]
    r = bi.bi_describe_recipe(bi.BI_F32, N, K)
    return bi.lib().bi_lab_linear(ctypes.c_void_p(x.data_ptr()), K, ctypes.c_void_p(wd.data_ptr()), K,
                                  ctypes.c_void_p(bd.data_ptr()), ctypes.c_void_p(y.data_ptr()), bi.BI_F32, N,
                                  M, N, K, ctypes.byref(r), path, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_xcd_decode_graph_replays(bi, router):
    # a captured graph of hand-over calls replayed several times, with eager
    # calls and synchronisations in between, keeps every result's bits
    import torch
    w, wd, bd = router
    Ms = (1, 16, 33, 128)
    xs = {M: dev(wl.router_batch(M, w).x) for M in Ms}
    outs = {M: torch.empty((M, 256), dtype=torch.float32, device="cuda") for M in Ms}
    ref = {M: host(bi.bi_lab_linear(xs[M], weight_t(wd), bd, path=bi.BI_PATH_DECODE)) for M in Ms}
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for M in Ms:
            bi.bi_lab_linear(xs[M], weight_t(wd), bd, path=bi.BI_PATH_DECODE_XCD, out=outs[M])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for M in Ms:
            bi.bi_lab_linear(xs[M], weight_t(wd), bd, path=bi.BI_PATH_DECODE_XCD, out=outs[M])
    torch.cuda.synchronize()
    for rep in range(4):
        banner(f"XCD hand-over graph replay {rep}")
        for M in Ms:
            outs[M].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for M in Ms:
            assert_bitwise(host(outs[M]), ref[M], f"replay {rep} M={M}")
        # eager work between replays
        bi.bi_lab_linear(xs[33], weight_t(wd), bd, path=bi.BI_PATH_DECODE_XCD)
        torch.cuda.synchronize()
