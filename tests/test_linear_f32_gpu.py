"""fp32 batch-invariant linear on the GPU against the oracle, through the C ABI.

Workloads: the tiny fp32 layer and the DeepSeek-V4-shaped router (decode and
prefill batch sizes); see workloads.py.  Bars: oracle agreement at atol 2e-3 /
rtol 1e-4 (GateLinear page, "Tests"), and bitwise equality of every probe row
across every batch size, batch position and kernel path.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import (F32_ATOL, F32_RTOL, assert_bitwise, assert_close, banner, dev, host,
                            weight_t)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bi():
    import deterministic_persistent_gemm_amd as m
    return m


@pytest.fixture(scope="module")
def router():
    w = wl.router_weights(0)
    return w, dev(w.w), dev(w.b)


def run(bi, x_np, w_dev, b_dev, **kw):
    return host(bi.bi_linear_f32(dev(x_np), weight_t(w_dev), b_dev, **kw))


# ----------------------------------------------------------------- tiny fp32


def test_tiny_layer_against_oracle_and_invariant(bi):
    w = wl.tiny_weights(0)
    wd, bd = dev(w.w), dev(w.b)
    rows = {}
    for M in wl.TINY_M_SWEEP:
        banner(f"tiny fp32 M={M} bi_linear_f32")
        batch = wl.tiny_batch(M, w)
        y = run(bi, batch.x, wd, bd)
        assert_close(y, oracle.linear_f32(batch.x, w.w, w.b), F32_ATOL, F32_RTOL, f"tiny M={M}")
        rows[M] = y[0]
    for M in wl.TINY_M_SWEEP:
        assert_bitwise(rows[M], rows[1], f"tiny probe row, M={M} vs M=1")


# ------------------------------------------------------------ router decode


def test_router_decode_sweep(bi, router):
    w, wd, bd = router
    probe_out = {}
    worst = 0.0
    for M in wl.ROUTER_DECODE_M:
        banner(f"router fp32 decode M={M} bi_linear_f32")
        batch = wl.router_batch(M, w)
        y = run(bi, batch.x, wd, bd)
        ref = oracle.linear_f32(batch.x, w.w, w.b)
        worst = max(worst, assert_close(y, ref, F32_ATOL, F32_RTOL, f"router M={M}"))
        for pid, pos in batch.probes.items():
            for p in pos:
                probe_out.setdefault(pid, []).append((M, p, y[p]))
    for pid, outs in probe_out.items():
        for M, p, row in outs:
            assert_bitwise(row, outs[0][2], f"probe {pid} at M={M} row {p} vs M={outs[0][0]} row {outs[0][1]}")
    # the fp64 reference differs from any fp32 order by far less than the bar
    assert worst < 1e-4, worst


def test_router_prefill_rows_match_decode(bi, router):
    w, wd, bd = router
    banner("router fp32 M=1 reference row")
    solo = run(bi, w.probes, wd, bd)
    for M in wl.ROUTER_PREFILL_M:
        banner(f"router fp32 prefill M={M} bi_linear_f32")
        batch = wl.router_batch(M, w, copies=8)
        y = run(bi, batch.x, wd, bd)
        for pid, pos in batch.probes.items():
            assert len(pos) >= 8
            for p in pos:
                assert_bitwise(y[p], solo[pid], f"M={M} probe {pid} at row {p}")
        sample = np.unique(np.concatenate([np.arange(0, M, M // 48), [M - 1], np.arange(60, 70)]))
        ref = oracle.linear_f32(batch.x[sample], w.w, w.b)
        assert_close(y[sample], ref, F32_ATOL, F32_RTOL, f"router M={M} sampled rows")


def test_both_kernel_paths_agree_bitwise(bi, router):
    w, wd, bd = router
    for M in (1, 17, 64, 128, 200):
        banner(f"router fp32 M={M} decode vs persistent (bi_lab_linear)")
        batch = wl.router_batch(M, w)
        x = dev(batch.x)
        a = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_DECODE))
        b = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_PERSISTENT))
        c = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_DECODE_WG))
        h = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_DECODE_XCD))
        assert_bitwise(a, b, f"decode vs persistent at M={M}")
        assert_bitwise(c, b, f"one-launch decode vs persistent at M={M}")
        assert_bitwise(h, b, f"XCD hand-over decode vs persistent at M={M}")


@pytest.mark.parametrize("K,block_k", [(320, 32), (4096, 64), (2048, 128), (512, 256)])
def test_one_launch_decode_uneven_tile_counts(bi, K, block_k):
    # 10, 64, 16 and 2 tile partials: waves of the one-launch decode kernel
    # take unequal numbers of partials, or one each, or the LDS maximum
    g = np.random.default_rng(K + block_k)
    N = 48
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    b = (g.standard_normal(N) * 0.01).astype(np.float32)
    r = bi.bi_describe_recipe(bi.BI_F32, N, K)
    r.block_k = block_k
    for M in (1, 19, 40):
        banner(f"fp32 N={N} K={K} block_k={block_k} M={M} decode paths")
        x = g.standard_normal((M, K)).astype(np.float32)
        xd, wd, bd = dev(x), dev(w), dev(b)
        a = host(bi.bi_lab_linear(xd, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_DECODE))
        c = host(bi.bi_lab_linear(xd, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_DECODE_WG))
        p = host(bi.bi_lab_linear(xd, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_PERSISTENT))
        assert_bitwise(c, a, "one-launch vs two-launch decode")
        assert_bitwise(c, p, "one-launch decode vs persistent")
        assert_close(c, oracle.linear_f32(x, w, b), F32_ATOL, F32_RTOL, "oracle")


def test_every_persistent_tile_shape_gives_the_same_bits(bi, router):
    # tiling is not part of the recipe: every persistent tile shape must
    # reproduce the automatic choice bit for bit (ragged M and N tails too)
    w, wd, bd = router
    batch = wl.router_batch(300, w)
    x = dev(batch.x)
    ref = host(bi.bi_linear_f32(x, weight_t(wd), bd))
    for code in (*range(1, 11), 23, 24, 28, 29):
        banner(f"router fp32 M=300 persistent tile code {code}")
        y = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_PERSISTENT | (code << 8)))
        assert_bitwise(y, ref, f"tile code {code}")
    # a narrow N that no tile divides evenly
    banner("fp32 N=48 K=320 tile codes")
    g = np.random.default_rng(77)
    w2 = g.standard_normal((48, 320)).astype(np.float32)
    x2 = dev(g.standard_normal((70, 320)).astype(np.float32))
    ref2 = host(bi.bi_linear_f32(x2, weight_t(dev(w2)), None))
    assert_close(ref2, oracle.linear_f32(host(x2), w2, None), F32_ATOL, F32_RTOL, "N=48 K=320")
    for code in (*range(1, 11), 23, 24, 28, 29):
        y = host(bi.bi_lab_linear(x2, weight_t(dev(w2)), None, path=bi.BI_PATH_PERSISTENT | (code << 8)))
        assert_bitwise(y, ref2, f"N=48 tile code {code}")


@pytest.mark.parametrize("M,N,K,block_k", [
    (1000, 256, 7168, 256),    # 28 k tiles: the 32x32 ring works on four at a time
    (300, 96, 768, 128),       # 6 k tiles: two at a time
    (2047, 208, 4096, 64),     # k tiles of two blocks: the 64x32 ring only (ragged N)
    (4100, 48, 1024, 256),     # more 32x32 tiles than compute units
    (9000, 32, 512, 128),      # more tiles than compute units, one step per k tile group
    (64, 32, 4096, 4096),      # one k tile: both fall back
    (500, 64, 1536, 192),      # k tiles of six blocks: the step's place in its k tile known at run time only
    (700, 128, 4096, 512),     # k tiles of sixteen blocks: likewise
])
def test_ring_fed_fp32_tiles(bi, M, N, K, block_k):
    # the ring-fed fp32 shapes (32x32 on four or two k tiles at a time, 64x32
    # on two) hand tile partials between waves and fold them in k tile order:
    # bit for bit the 32x32 register-staged shape, which itself meets the oracle
    g = np.random.default_rng(M + N + K)
    w = g.standard_normal((N, K)).astype(np.float32) * 0.02
    b = (g.standard_normal(N) * 0.01).astype(np.float32)
    xh = g.standard_normal((M, K)).astype(np.float32)
    x, wd, bd = dev(xh), dev(w), dev(b)
    r = bi.bi_describe_recipe(bi.BI_F32, N, K)
    r.block_k = block_k
    banner(f"fp32 ring tiles M={M} N={N} K={K} block_k={block_k}")
    y3 = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_PERSISTENT | (3 << 8)))
    if M * K <= 300 * 768:
        assert_close(y3, oracle.linear_f32(xh, w, b), F32_ATOL, F32_RTOL, "oracle")
    for code in (23, 24, 28, 29):
        y = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_PERSISTENT | (code << 8)))
        assert_bitwise(y, y3, f"tile code {code} vs 3")


def test_repeat_determinism_with_workspace_reuse(bi, router):
    # alternate two different batches through the same workspace: a stale
    # partial or a counter left non-zero would change the second result
    w, wd, bd = router
    xa = dev(wl.router_batch(16, w).x)
    xb = dev(wl.router_batch(32, w).x)
    banner("router fp32 repeat-determinism x10")
    ya0 = host(bi.bi_linear_f32(xa, weight_t(wd), bd))
    yb0 = host(bi.bi_linear_f32(xb, weight_t(wd), bd))
    for i in range(10):
        assert_bitwise(host(bi.bi_linear_f32(xa, weight_t(wd), bd)), ya0, f"repeat {i} batch a")
        assert_bitwise(host(bi.bi_linear_f32(xb, weight_t(wd), bd)), yb0, f"repeat {i} batch b")


def test_poisoned_tail_rows_and_guard_bands(bi, router):
    import torch
    w, wd, bd = router
    M = 33
    batch = wl.router_batch(M, w)
    x_big = np.full((M + 16, wl.ROUTER_K), np.nan, np.float32)
    x_big[:M] = batch.x
    xd = dev(x_big)[:M]                        # rows past M hold NaN
    out_big = torch.full((M + 4, 256 + 32), 12345.0, dtype=torch.float32, device="cuda")
    out = out_big[2:M + 2, 16:16 + 256]       # strided window with canaries around it
    banner("router fp32 poisoned tail + guard bands")
    bi.bi_linear_f32(xd, weight_t(wd), bd, out=out)
    big = host(out_big)
    assert np.all(big[:2] == 12345.0) and np.all(big[M + 2:] == 12345.0)
    assert np.all(big[:, :16] == 12345.0) and np.all(big[:, 16 + 256:] == 12345.0)
    assert_bitwise(big[2:M + 2, 16:16 + 256], run(bi, batch.x, wd, bd), "strided out vs contiguous")


def test_poisoned_workspace(bi, router):
    # beyond its zeroed counter region the workspace needs no initialisation:
    # every partial is written before it is read in the same call, so NaN
    # left there must not leak into the result.  Uses its own workspace
    # through the C ABI.
    import ctypes
    import torch
    w, wd, bd = router
    M, N, K = 17, 256, 4096
    batch = wl.router_batch(M, w)
    ref = run(bi, batch.x, wd, bd)
    L = bi.lib()
    need = L.bi_linear_workspace_size(bi.BI_F32, M, N, K)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # 0xFFFFFFFF is a NaN
    ws[:bi.WS_COUNTER_BYTES] = 0           # the counter region starts at zero, by contract
    x = dev(batch.x)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    banner("router fp32 NaN-poisoned workspace (direct C ABI)")
    for _ in range(2):
        st = L.bi_linear_f32(ctypes.c_void_p(x.data_ptr()), K, ctypes.c_void_p(wd.data_ptr()), K,
                             ctypes.c_void_p(bd.data_ptr()), ctypes.c_void_p(y.data_ptr()), N, M, N, K,
                             ctypes.c_void_p(ws.data_ptr()), need, ctypes.c_void_p(s.cuda_stream))
        assert st == bi.BI_OK
        assert_bitwise(host(y), ref, "after poisoning the workspace")


def _abi_f32(bi, x, wd, bd, y, ws):
    import ctypes
    import torch
    M, K = x.shape
    N = wd.shape[0]
    return bi.lib().bi_linear_f32(ctypes.c_void_p(x.data_ptr()), K, ctypes.c_void_p(wd.data_ptr()), K,
                                  ctypes.c_void_p(bd.data_ptr()), ctypes.c_void_p(y.data_ptr()), N, M, N, K,
                                  ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_one_workspace_serves_every_shape_in_sequence(bi, router):
    # calls of different shapes in sequence through one workspace (an early
    # layout let a small-M call leave data a larger-M call misread)
    import torch
    w, wd, bd = router
    seq = (64, 128, 17, 128, 1, 64, 33, 128)
    need = max(bi.lib().bi_linear_workspace_size(bi.BI_F32, M, 256, 4096) for M in seq)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, M in enumerate(seq):
        banner(f"shared workspace call {i}: M={M}")
        batch = wl.router_batch(M, w)
        x = dev(batch.x)
        y = torch.empty((M, 256), dtype=torch.float32, device="cuda")
        fresh = torch.zeros_like(ws)
        y_ref = torch.empty_like(y)
        assert _abi_f32(bi, x, wd, bd, y_ref, fresh) == bi.BI_OK
        assert _abi_f32(bi, x, wd, bd, y, ws) == bi.BI_OK
        assert_bitwise(host(y), host(y_ref), f"shared workspace, call {i} (M={M})")


# ------------------------------------------------------------- closed forms


def test_closed_forms_bitwise(bi):
    g = np.random.default_rng(31)
    K = 256
    x = g.standard_normal((40, K)).astype(np.float32)
    b = g.standard_normal(K).astype(np.float32)
    banner("fp32 identity weight")
    y = run(bi, x, dev(np.eye(K, dtype=np.float32)), dev(b))
    assert_bitwise(y, x + b, "W = I")
    perm = g.permutation(K)[:64]
    wh = np.zeros((64, K), np.float32)
    wh[np.arange(64), perm] = 1.0
    banner("fp32 one-hot weight")
    assert_bitwise(run(bi, x, dev(wh), dev(b[:64])), x[:, perm] + b[:64], "one-hot W")
    banner("fp32 zero weight")
    assert_bitwise(run(bi, x, dev(np.zeros((32, K), np.float32)), dev(b[:32])),
                   np.broadcast_to(b[:32], (40, 32)), "W = 0")
    xi = g.integers(-8, 9, (70, 512)).astype(np.float32)
    wi = g.integers(-8, 9, (48, 512)).astype(np.float32)
    banner("fp32 small-integer exact")
    assert_bitwise(run(bi, xi, dev(wi), None), (xi.astype(np.int64) @ wi.astype(np.int64).T).astype(np.float32),
                   "small integers")


def test_power_of_two_scaling_bitwise(bi, router):
    import torch
    w, wd, bd = router
    x = wl.router_batch(8, w).x
    banner("router fp32 power-of-two scaling")
    y = run(bi, x, wd, bd)
    y8 = host(bi.bi_linear_f32(dev(x * np.float32(8)), weight_t(wd), bd * 8))
    assert_bitwise(y8, y * np.float32(8), "y(8x, 8b) == 8 y(x, b)")


# --------------------------------------------------------- recipe controls


def test_negative_control_breaks_invariance(bi, router):
    # the same machinery with an M-dependent BLOCK_K must change the probe row
    # between batch sizes on either side of its switch (GateLinear page,
    # "Tests": a negative control that actually fails)
    w, wd, bd = router
    rows = {}
    for M in (1, 8, 32, 64, 128):
        banner(f"negative control M={M}")
        batch = wl.router_batch(M, w)
        y = host(bi.bi_negctl_linear_f32(dev(batch.x), weight_t(wd), bd))
        rows[M] = y[M - 1]                  # probe 2 sits at M-1 for every M
        assert_close(y, oracle.linear_f32(batch.x, w.w, w.b), F32_ATOL, F32_RTOL, "negctl still accurate")
    assert np.array_equal(rows[1].view(np.uint32), rows[32].view(np.uint32))
    assert not np.array_equal(rows[32].view(np.uint32), rows[64].view(np.uint32)), \
        "negative control failed to break invariance"


def test_block_k_is_part_of_the_recipe(bi, router):
    # tile-partial recipes with different BLOCK_K round differently: the width
    # is load-bearing and has to stay in the key (GateLinear page, "A
    # correction to why the key excludes M").  Both stay within the bar.
    w, wd, bd = router
    batch = wl.router_batch(64, w)
    x = dev(batch.x)
    ref = oracle.linear_f32(batch.x, w.w, w.b)
    outs = {}
    for bk in (128, 256, 4096):
        r = bi.bi_describe_recipe(bi.BI_F32, 256, 4096)
        r.block_k = bk
        banner(f"router fp32 lab block_k={bk}")
        outs[bk] = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r))
        assert_close(outs[bk], ref, F32_ATOL, F32_RTOL, f"block_k={bk}")
        dec = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_DECODE))
        per = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_PERSISTENT))
        assert_bitwise(dec, per, f"paths agree at block_k={bk}")
        if bk < 4096:
            wg = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_DECODE_WG))
            assert_bitwise(wg, per, f"one-launch decode agrees at block_k={bk}")
    assert not np.array_equal(outs[128].view(np.uint32), outs[256].view(np.uint32))
    assert not np.array_equal(outs[128].view(np.uint32), outs[4096].view(np.uint32))


def test_bf16_roundtrip_control_fails_tolerance(bi, router):
    # GateLinear page, "What": routing through bf16 must fail the fp32 bar
    import torch
    w, wd, bd = router
    batch = wl.router_batch(128, w)
    banner("router bf16 round-trip control")
    xb = dev(batch.x).to(torch.bfloat16)
    wb = wd.to(torch.bfloat16)
    y = host(bi.bi_linear_bf16(xb, weight_t(wb), bd, out_dtype=torch.bfloat16).float())
    ref = oracle.linear_f32(batch.x, w.w, w.b)
    ratio = np.max(np.abs(y - ref) / (F32_ATOL + F32_RTOL * np.abs(ref)))
    print(f"bf16 round-trip error / fp32 tolerance = {ratio:.1f}x")
    assert ratio > 1.0


@pytest.mark.parametrize("K,block_k", [(4096, 64), (4096, 128), (4096, 256), (4096, 1024), (3072, 1024), (384, 128)])
def test_tile_partial_widths_agree_across_shapes(bi, K, block_k):
    # for several tile-partial widths (an odd number of k tiles, 3072 / 1024,
    # and a short K included) the 32x32 and 64x64 persistent shapes and the
    # decode path give the same bits
    g = np.random.default_rng(K + block_k)
    N, M = 96, 200
    w = g.standard_normal((N, K)).astype(np.float32) * 0.02
    b = (g.standard_normal(N) * 0.01).astype(np.float32)
    x = dev(g.standard_normal((M, K)).astype(np.float32))
    wd, bd = dev(w), dev(b)
    r = bi.bi_describe_recipe(bi.BI_F32, N, K)
    r.block_k = block_k
    banner(f"fp32 M={M} N={N} K={K} block_k={block_k} tile 3 vs 1")
    y3 = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_PERSISTENT | (3 << 8)))
    y1 = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_PERSISTENT | (1 << 8)))
    assert_bitwise(y3, y1, f"32x32 vs 64x64 K={K} block_k={block_k}")
    yd = host(bi.bi_lab_linear(x, weight_t(wd), bd, recipe=r, path=bi.BI_PATH_DECODE))
    assert_bitwise(y3, yd, f"32x32 vs decode K={K} block_k={block_k}")
