"""Every output tile is computed once, whatever order the persistent kernels
walk the tiles in.

The persistent kernels hand each XCD (workgroup w runs on XCD w % 8) one
block of the tile grid, in one round when the grid has a workgroup per tile
and over several rounds when it loops.  A mistake in that mapping would skip
some tiles and compute others twice.  Each case below fills the output with
NaN first and compares the result bit for bit with the decode path, which
walks no tile order at all, so a skipped tile cannot hide behind an earlier
call's values left in a reused buffer.
"""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import assert_bitwise, banner, dev, host, weight_t

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bi():
    import deterministic_persistent_gemm_amd as m
    return m


@pytest.fixture(scope="module")
def router():
    w = wl.router_weights(0)
    return w, dev(w.w), dev(w.b)


@pytest.fixture(scope="module")
def dense():
    w = wl.dense_bf16_weights(0)
    return w, dev(w.w)


def run_nan_prefilled(bi, torch, x, wt, bias, code, out_dtype, N):
    out = torch.full((x.shape[0], N), float("nan"), dtype=out_dtype, device="cuda")
    bi.bi_lab_linear(x, wt, bias, path=bi.BI_PATH_PERSISTENT | (code << 8), out=out)
    return host(out)


# (M, tile code): 32x32 over 1024 tiles on a 512-workgroup grid (two rounds),
# 32x32 with one workgroup per tile, 64x64 on 8 waves at 128 and 256 tiles,
# 64x64 on 4 waves at 64 tiles, and a tile count that is not a multiple of 8
@pytest.mark.parametrize("M,code", [(4096, 3), (4096, 7), (1024, 3), (2048, 10), (4096, 10), (1000, 1), (33, 10)])
def test_router_tile_order(bi, router, M, code):
    import torch
    w, wd, bd = router
    x = dev(wl.router_batch(M, w).x)
    banner(f"tile order fp32 router M={M} code {code}")
    ref = host(bi.bi_lab_linear(x, weight_t(wd), bd, path=bi.BI_PATH_DECODE))
    got = run_nan_prefilled(bi, torch, x, weight_t(wd), bd, code, torch.float32, wl.ROUTER_N)
    assert not np.isnan(got).any(), f"M={M} code {code}: tiles left unwritten"
    assert_bitwise(got, ref, f"M={M} code {code}")


# the streaming 64x64 kernel at 2 and 4 tile rows, the 256x256 tiles (one
# round), and 64x64 tiles over 4096 tiles on a 512-workgroup grid
@pytest.mark.parametrize("M,code", [(100, 20), (256, 20), (4096, 19), (4096, 12)])
def test_dense_tile_order(bi, dense, M, code):
    import torch
    w, wd = dense
    x = dev(wl.dense_bf16_batch(M, w).x)
    N = w.w.shape[0]
    banner(f"tile order bf16 dense M={M} code {code}")
    ref = host(bi.bi_lab_linear(x, weight_t(wd), None, path=bi.BI_PATH_DECODE))
    got = run_nan_prefilled(bi, torch, x, weight_t(wd), None, code, torch.bfloat16, N)
    as_f = got.astype(np.uint32) << 16
    assert not np.isnan(as_f.view(np.float32)).any(), f"M={M} code {code}: tiles left unwritten"
    assert_bitwise(got, ref, f"M={M} code {code}")
