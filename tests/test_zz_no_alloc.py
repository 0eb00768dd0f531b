"""bi_linear_f32_noalloc through the C ABI against bi_linear_f32.

The allocation-free entry point runs the same plan and kernels as
bi_linear_f32 with the library's static scratch in place of a workspace, so
its output must equal bi_linear_f32's bit for bit (fp32 bar of the GateLinear
page, "Tests", met exactly), call after call: a large input, then a smaller
one, then more in a row (the scratch keeps the last call's contents; its
counters must be back at zero and its partials rewritten each time), and
replayed from a HIP graph.
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


def noalloc(bi, x, wd, bd, y):
    import torch
    M, K = x.shape
    N = wd.shape[0]
    return bi.lib().bi_linear_f32_noalloc(ctypes.c_void_p(x.data_ptr()), K, ctypes.c_void_p(wd.data_ptr()), K,
                                          None if bd is None else ctypes.c_void_p(bd.data_ptr()),
                                          ctypes.c_void_p(y.data_ptr()), N, M, N, K,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_equals_the_workspace_entry_call_after_call(bi):
    import torch
    w = wl.router_weights(0)
    wd, bd = dev(w.w), dev(w.b)
    # two calls in a row, the second smaller (two-launch partials at M=128,
    # then the hand-over's counters at M=16), then more sizes and repeats
    for i, M in enumerate((128, 16, 1, 64, 512, 33, 1024, 2, 128, 16)):
        banner(f"noalloc call {i}: router fp32 M={M}")
        batch = wl.router_batch(M, w)
        x = dev(batch.x)
        ref = host(bi.bi_linear_f32(x, weight_t(wd), bd))
        y = torch.full((M, 256), float("nan"), dtype=torch.float32, device="cuda")
        assert noalloc(bi, x, wd, bd, y) == bi.BI_OK
        got = host(y)
        assert_bitwise(got, ref, f"noalloc vs bi_linear_f32 at M={M} (call {i})")
        rows = np.unique([0, M // 2, M - 1])
        assert_close(got[rows], oracle.linear_f32(batch.x[rows], w.w, w.b), F32_ATOL, F32_RTOL, f"oracle M={M}")


def test_noalloc_other_keys_and_no_bias(bi):
    import torch
    for N, K, M in ((128, 2048, 200), (128, 2048, 7), (32, 256, 17), (256, 7168, 64)):
        banner(f"noalloc fp32 N={N} K={K} M={M}")
        g = np.random.default_rng(N + K + M)
        w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
        x = g.standard_normal((M, K)).astype(np.float32)
        xd, wd = dev(x), dev(w)
        ref = host(bi.bi_linear_f32(xd, weight_t(wd), None))
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        assert noalloc(bi, xd, wd, None, y) == bi.BI_OK
        assert_bitwise(host(y), ref, f"noalloc N={N} K={K} M={M}")


def test_noalloc_rejects_what_its_scratch_cannot_hold(bi):
    import torch
    # an unlisted fp32 key decodes with 8 M tiles x 256 N tiles x 32 k tiles
    # of 1 KiB partials at M = 128: 64 MiB, beyond the 16 MiB scratch
    x = torch.zeros((128, 4096), dtype=torch.float32, device="cuda")
    w = torch.zeros((4096, 4096), dtype=torch.float32, device="cuda")
    y = torch.full((128, 4096), 7.0, dtype=torch.float32, device="cuda")
    assert noalloc(bi, x, w, None, y) == bi.BI_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a rejected call wrote its output"


def test_noalloc_graph_replays(bi):
    # captured with no workspace allocated anywhere; replayed with eager
    # calls of other sizes between the replays
    import torch
    w = wl.router_weights(0)
    wd, bd = dev(w.w), dev(w.b)
    xs = {M: dev(wl.router_batch(M, w).x) for M in (1, 16, 128)}
    ys = {M: torch.empty((M, 256), dtype=torch.float32, device="cuda") for M in xs}
    ref = {M: host(bi.bi_linear_f32(xs[M], weight_t(wd), bd)) for M in xs}
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for M in xs:
            assert noalloc(bi, xs[M], wd, bd, ys[M]) == bi.BI_OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for M in xs:
            noalloc(bi, xs[M], wd, bd, ys[M])
    torch.cuda.synchronize()
    for r in range(4):
        banner(f"noalloc graph replay {r}")
        for M in xs:
            ys[M].fill_(float("nan"))
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for M in xs:
            assert_bitwise(host(ys[M]), ref[M], f"replay {r} M={M}")
        y33 = torch.empty((33, 256), dtype=torch.float32, device="cuda")
        assert noalloc(bi, dev(wl.router_batch(33, w).x), wd, bd, y33) == bi.BI_OK
        torch.cuda.synchronize()
    del g
