"""The ring-fed fp32 tiles with their k tiles split over several workgroups
(tile codes 28: 32x32, 29: 64x32).

Every part of an output tile runs on one XCD; part 0 folds its k tiles into a
prefix, the later parts store each k tile's partial, and the part that
arrives last at the tile's counter finishes the fold in ascending k tile
order.  These tests check that the split really happens (the plan asks for a
workspace), that the result is the same bits as the unsplit register-staged
tile and every other path (GateLinear page, "Tests": bitwise equality across
batch sizes), that it meets the oracle, that the counters read back zero, and
that it survives graph replays.
"""
import ctypes

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


def _lab(bi, x, wd, bd, y, ws, recipe, path):
    import torch
    M, K = x.shape
    N = wd.shape[0]
    return bi.lib().bi_lab_linear(ctypes.c_void_p(x.data_ptr()), K, ctypes.c_void_p(wd.data_ptr()), K,
                                  None if bd is None else ctypes.c_void_p(bd.data_ptr()),
                                  ctypes.c_void_p(y.data_ptr()), bi.BI_F32, N, M, N, K, ctypes.byref(recipe),
                                  path, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("M,N,K,block_k,code", [
    (33, 256, 4096, 128, 28),     # 16 tiles, sixteen parts of two k tiles (ragged M)
    (90, 256, 4096, 128, 28),     # 24 tiles, eight parts of four k tiles
    (128, 256, 4096, 128, 28),    # 32 tiles, eight parts
    (200, 256, 4096, 128, 28),    # ragged M, 56 tiles, four parts
    (512, 256, 4096, 128, 28),    # 128 tiles, two parts
    (256, 256, 4096, 128, 29),    # 64x32: 32 tiles, eight parts
    (1000, 256, 4096, 128, 29),   # 64x32: 128 tiles, two parts, ragged M
    (300, 256, 7168, 256, 28),    # 28 k tiles: two parts of fourteen, two at a time
    (190, 128, 2048, 128, 28),    # N 128: 24 tiles, eight parts of two k tiles
    (96, 256, 4096, 256, 29),     # 16 k tiles of 256: eight parts of two
])
def test_split_ring_tiles_bitwise(bi, M, N, K, block_k, code):
    import torch
    g = np.random.default_rng(M * 31 + N + K + code)
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    b = (g.standard_normal(N) * 0.01).astype(np.float32)
    xh = g.standard_normal((M, K)).astype(np.float32)
    x, wd, bd = dev(xh), dev(w), dev(b)
    r = bi.bi_describe_recipe(bi.BI_F32, N, K)
    r.block_k = block_k
    path = bi.BI_PATH_PERSISTENT | (code << 8)
    need = bi.lib().bi_lab_workspace_size(ctypes.byref(r), path, M, N, K)
    assert need > bi.WS_COUNTER_BYTES, "the plan did not split the k tiles"
    banner(f"fp32 split ring tile code {code} M={M} N={N} K={K} block_k={block_k}")
    ws = bi.alloc_workspace(need, "cuda")
    ws[bi.WS_COUNTER_BYTES:] = 0xFF          # partial slots may hold anything (NaN)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    for rep in range(2):
        assert _lab(bi, x, wd, bd, y, ws, r, path) == bi.BI_OK
        torch.cuda.synchronize()
        assert int(ws[:bi.WS_COUNTER_BYTES].count_nonzero()) == 0, "counters left non-zero"
        got = host(y)
        ref3 = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_PERSISTENT | (3 << 8)))
        assert_bitwise(got, ref3, f"split code {code} vs register-staged 32x32 (call {rep})")
    dec = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_DECODE))
    assert_bitwise(got, dec, "split vs two-launch decode")
    rows = np.unique(np.r_[0, 1, 15, 16, 17, 31, 32, 33, M // 2, M - 1].clip(0, M - 1))
    assert_close(got[rows], oracle.linear_f32(xh[rows], w, b), F32_ATOL, F32_RTOL, "oracle")


def test_split_ring_rows_keep_their_bits_across_batch_sizes(bi, router):
    # the router with probe rows planted at tile-straddling positions: every
    # batch size, on the split tiles or not, gives each probe row its solo bits
    w, wd, bd = router
    banner("router fp32 probe rows alone")
    solo = host(bi.bi_linear_f32(dev(w.probes), weight_t(wd), bd))
    for M in (1, 64, 128, 200, 256, 512, 1000, 1024):
        batch = wl.router_batch(M, w)
        x = dev(batch.x)
        for code in (28, 29):
            banner(f"router M={M} split tile code {code}: probe rows")
            y = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_PERSISTENT | (code << 8)))
            for pid, rows in batch.probes.items():
                for rr in rows:
                    assert_bitwise(y[rr], solo[pid], f"probe {pid} row {rr} at M={M} code {code}")


def test_split_ring_graph_replays_and_shared_workspace(bi, router):
    # split calls of several sizes and hand-over decodes share one workspace
    # (and its counter region) inside a graph replayed several times, with
    # eager calls between the replays
    import torch
    w, wd, bd = router
    Ms = (64, 1, 256, 16, 1000)
    r = bi.bi_describe_recipe(bi.BI_F32, 256, 4096)
    paths = {64: bi.BI_PATH_PERSISTENT | (28 << 8), 1: bi.BI_PATH_DECODE_XCD, 256: bi.BI_PATH_PERSISTENT | (28 << 8),
             16: bi.BI_PATH_DECODE_XCD, 1000: bi.BI_PATH_PERSISTENT | (29 << 8)}
    need = max(bi.lib().bi_lab_workspace_size(ctypes.byref(r), paths[M], M, 256, 4096) for M in Ms)
    ws = bi.alloc_workspace(need, "cuda")
    xs = {M: dev(wl.router_batch(M, w).x) for M in Ms}
    outs = {M: torch.empty((M, 256), dtype=torch.float32, device="cuda") for M in Ms}
    ref = {M: host(bi.bi_lab_linear(xs[M], weight_t(wd), bd, path=bi.BI_PATH_PERSISTENT | (3 << 8))) for M in Ms}
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for M in Ms:
            assert _lab(bi, xs[M], wd, bd, outs[M], ws, r, paths[M]) == bi.BI_OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for M in Ms:
            _lab(bi, xs[M], wd, bd, outs[M], ws, r, paths[M])
    torch.cuda.synchronize()
    for rep in range(4):
        banner(f"split ring graph replay {rep}")
        for M in Ms:
            outs[M].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert int(ws[:bi.WS_COUNTER_BYTES].count_nonzero()) == 0, f"counters left non-zero, replay {rep}"
        for M in Ms:
            assert_bitwise(host(outs[M]), ref[M], f"replay {rep} M={M}")
        bi.bi_lab_linear(xs[256], weight_t(wd), bd, path=bi.BI_PATH_PERSISTENT | (28 << 8))
        torch.cuda.synchronize()


def test_no_alloc_entry_runs_split_plans_unsplit_when_they_do_not_fit(bi, router):
    # the static scratch holds 16 MiB of partials; a split plan that needs
    # more runs its tiles unsplit there -- the same bits
    import torch
    w, wd, bd = router
    M = 1024
    r = bi.bi_describe_recipe(bi.BI_F32, 256, 4096)
    need = bi.lib().bi_lab_workspace_size(ctypes.byref(r), bi.BI_PATH_PERSISTENT | (29 << 8), M, 256, 4096)
    assert need > (16 << 20) + bi.WS_COUNTER_BYTES
    x = dev(wl.router_batch(M, w).x)
    y = torch.empty((M, 256), dtype=torch.float32, device="cuda")
    banner("no-allocation entry at M=1024")
    st = bi.lib().bi_linear_f32_noalloc(ctypes.c_void_p(x.data_ptr()), 4096, ctypes.c_void_p(wd.data_ptr()), 4096,
                                        ctypes.c_void_p(bd.data_ptr()), ctypes.c_void_p(y.data_ptr()), 256, M,
                                        256, 4096, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == bi.BI_OK
    assert_bitwise(host(y), host(bi.bi_linear_f32(x, weight_t(wd), bd)), "no-allocation entry vs bi_linear_f32")


def test_split_ring_without_bias_strided_rows_and_bf16_output(bi):
    # no bias term (nothing added, -0.0 kept), an X row pitch wider than K,
    # and bf16 output: each equal to the unsplit tile's result in the same form
    import torch
    g = np.random.default_rng(4242)
    M, N, K = 200, 256, 4096
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    xh = g.standard_normal((M, K + 64)).astype(np.float32)
    xw = dev(xh)
    x = xw[:, :K]                                   # row pitch K + 64
    wd = dev(w)
    r = bi.bi_describe_recipe(bi.BI_F32, N, K)
    split = bi.BI_PATH_PERSISTENT | (28 << 8)
    assert bi.lib().bi_lab_workspace_size(ctypes.byref(r), split, M, N, K) > bi.WS_COUNTER_BYTES
    for out_dtype in (torch.float32, torch.bfloat16):
        banner(f"split ring M={M} no bias, strided X, out {out_dtype}")
        y = bi.bi_lab_linear(x, weight_t(wd), None, recipe=r, path=split, out_dtype=out_dtype)
        ref = bi.bi_lab_linear(x, weight_t(wd), None, recipe=r, path=bi.BI_PATH_PERSISTENT | (3 << 8),
                               out_dtype=out_dtype)
        assert torch.equal(y.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           ref.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32)), out_dtype
    y = host(bi.bi_lab_linear(x, weight_t(wd), None, recipe=r, path=split))
    assert_close(y[:8], oracle.linear_f32(xh[:8, :K].copy(), w, None), F32_ATOL, F32_RTOL, "oracle, no bias")
