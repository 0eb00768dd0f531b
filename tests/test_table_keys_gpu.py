"""Every key of the compiled recipe table, across every path boundary the
table sets for it.

The recipe is a function of (dtype, N, K) alone; M only chooses the kernel
path (the XCD hand-over decode up to m_xcd_max, another decode form up to
m_decode_max, then up to three persistent tile shapes split at m_a and m_b).  For each key, two probe rows are planted at the first
and last position of batches whose sizes sit on both sides of every one of
those boundaries; the probe rows must keep their bits at every M, and agree
with the oracle (fp32 keys within atol 2e-3 / rtol 1e-4, GateLinear page,
"Tests"; bf16 keys with fp32 output within the fp32-accumulation error of a
K-term sum).
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from deterministic_persistent_gemm_amd import sweep
from tests.gpu_util import F32_ATOL, F32_RTOL, assert_bitwise, assert_close, banner, dev, host, weight_t

pytestmark = pytest.mark.gpu

TABLE_ROWS = sweep.parse_table(open(sweep.TABLE).read())

def boundary_ms(row):
    ms = {1, 2, 17}
    for m in (row["m_decode_max"], row["m_a"], row["m_b"], row["m_xcd_max"]):
        if m > 0:
            ms.update({m, m + 1})
    return sorted(ms)

@pytest.fixture(scope="module")
def bi():
    import deterministic_persistent_gemm_amd as m
    return m

@pytest.mark.parametrize("row", TABLE_ROWS, ids=lambda r: f"{r['dtype']}-{r['N']}-{r['K']}")
def test_key_rows_keep_their_bits_across_path_boundaries(bi, row):
    import torch
    N, K = row["N"], row["K"]
    is_f32 = row["dtype"] == "BI_F32"
    g = np.random.default_rng(N * 7 + K)
    if is_f32:
        w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
        probes = g.standard_normal((2, K)).astype(np.float32)
    else:
        w = wl.normal_bf16(g, (N, K), 0.02)
        probes = wl.normal_bf16(g, (2, K), 1.0)
    b = (g.standard_normal(N) * 0.01).astype(np.float32)
    wd, bd = dev(w), dev(b)
    if is_f32:
        ref = oracle.linear_f32(probes, w, b)
    else:
        ref = oracle.linear_bf16(probes, w, b, out="f32")
    bits = [None, None]
    for M in boundary_ms(row):
        banner(f"table key {row['dtype']} N={N} K={K} M={M}")
        gm = np.random.default_rng(M)
        if is_f32:
            x = gm.standard_normal((M, K)).astype(np.float32)
        else:
            x = wl.normal_bf16(gm, (M, K), 1.0)
        x[0] = probes[0]
        if M > 1:
            x[M - 1] = probes[1]
        xd = dev(x)
        if is_f32:
            y = host(bi.bi_linear_f32(xd, weight_t(wd), bd))
        else:
            y = host(bi.bi_linear_bf16(xd, weight_t(wd), bd, out_dtype=torch.float32))
        seen = {0: y[0]} if M == 1 else {0: y[0], 1: y[M - 1]}
        for p, v in seen.items():
            if bits[p] is None:
                bits[p] = v
                if is_f32:
                    assert_close(v, ref[p], F32_ATOL, F32_RTOL, f"{N}x{K} probe {p} vs oracle")
                else:
                    assert_close(v, ref[p], 1e-5, 1e-4, f"{N}x{K} probe {p} vs oracle")
            else:
                assert_bitwise(v, bits[p], f"{row['dtype']} N={N} K={K} probe {p} at M={M}")
