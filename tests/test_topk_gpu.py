"""Deterministic indexer top-k on the GPU against the oracle, through the C ABI.

Bar: bit-exact (integer indices) against oracle.topk_rows on every row --
random plateau-heavy rows with ragged windows, every class of special fp32
bit pattern, strided and odd row pitches, and the full decode and prefill
indexer workloads (8192 columns, top-k 512/1024/2048).
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import banner, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bi():
    import deterministic_persistent_gemm_amd as m
    return m


def gpu_topk(bi, scores, topk, rs=None, re=None, pitch=None):
    import torch
    rows, cols = scores.shape
    if pitch is None or pitch == cols:
        s = dev(scores)
    else:
        buf = torch.full((rows, pitch), float("nan"), dtype=torch.float32, device="cuda")
        buf[:, :cols] = dev(scores)
        s = buf[:, :cols]
    r0 = None if rs is None else dev(np.asarray(rs, np.int64))
    r1 = None if re is None else dev(np.asarray(re, np.int64))
    return host(bi.bi_indexer_topk(s, topk, r0, r1))


def check(bi, scores, topk, rs=None, re=None, pitch=None, what=""):
    got = gpu_topk(bi, scores, topk, rs, re, pitch)
    want = oracle.topk_rows(scores, topk, None if rs is None else np.asarray(rs, np.int64),
                            None if re is None else np.asarray(re, np.int64))
    bad = np.argwhere((got != want).any(axis=1)).ravel()
    assert bad.size == 0, f"{what}: rows {bad[:5].tolist()} differ; first row got {got[bad[0]][:12]} want {want[bad[0]][:12]}"
    return got


@pytest.mark.parametrize("cols", [1, 31, 32, 33, 300, 2049, 8191, 8192])
def test_random_rows_ragged_windows(bi, cols):
    g = np.random.default_rng(cols)
    rows = 40
    s = np.maximum(g.standard_normal((rows, cols)), 0.0)
    s = (np.round(s * 8) / 8).astype(np.float32)
    s[g.random((rows, cols)) < 0.05] = -0.0
    s[g.random((rows, cols)) < 0.05] *= -1
    rs = g.integers(-3, cols + 3, rows)
    re = g.integers(-3, cols + 3, rows)
    re[::4] = cols
    rs[::5] = 0
    for topk in (1, 17, 512, 2048):
        banner(f"topk cols={cols} topk={topk} ragged windows")
        check(bi, s, topk, rs, re, what=f"cols={cols} topk={topk}")
    banner(f"topk cols={cols} no windows")
    check(bi, s, 64, what=f"cols={cols} full rows")


@pytest.mark.parametrize("pitch_extra", [1, 3, 4, 37])
def test_strided_and_odd_row_pitch(bi, pitch_extra):
    # pitches not a multiple of 4 take the scalar load path; padding holds NaN
    g = np.random.default_rng(pitch_extra)
    rows, cols = 9, 1000
    s = np.maximum(g.standard_normal((rows, cols)), 0).astype(np.float32)
    rs = g.integers(0, 500, rows)
    re = rs + g.integers(0, 600, rows)
    banner(f"topk strided pitch={cols + pitch_extra}")
    check(bi, s, 512, rs, re, pitch=cols + pitch_extra, what="strided")


# every special class, as the Sparse-MLA page's bit-pattern matrix names them
SPECIALS = [0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001,
            0xFF800001, 0x00000001, 0x807FFFFF, 0x007FFFFF, 0x80000001, 0x7F7FFFFF, 0xFF7FFFFF,
            0xFFFFFFFF, 0xFFFFFFFE, 0x7FFFFFFF, 0x3F800000]


def special_matrix(seed, copies=1):
    """Rows dominated by each special pattern in three window shapes, the
    whole set repeated `copies` times with fresh random fill."""
    g = np.random.default_rng(seed)
    cols = 8192
    rows = len(SPECIALS) * 3 * copies
    bits = g.integers(0, 2**32, (rows, cols), dtype=np.uint64).astype(np.uint32)
    rs = np.zeros(rows, np.int64)
    re = np.full(rows, cols, np.int64)
    for c in range(copies):
        for i, b in enumerate(SPECIALS):
            for w in range(3):
                r = (c * len(SPECIALS) + i) * 3 + w
                # a plateau of the special pattern, wide enough that the cut lands in it
                mask = g.random(cols) < 0.6
                bits[r, mask] = b
                if w == 1:                      # window narrower than top-k inside a wider row
                    rs[r], re[r] = 1, 31
                elif w == 2:                    # window wide enough to truncate at every top-k
                    rs[r], re[r] = 700, 3300
    return bits.view(np.float32), rs, re


@pytest.mark.parametrize("topk", [512, 1024, 2048])
def test_special_bit_pattern_matrix(bi, topk):
    s, rs, re = special_matrix(topk)
    banner(f"topk special bit patterns topk={topk}")
    check(bi, s, topk, rs, re, what="special patterns")


# From 1024 rows the kernel runs its 512-thread form (16 columns per thread,
# halved histogram copies); the inputs below reach it with every special
# pattern, the scalar load path and each top-k size.
@pytest.mark.parametrize("topk", [512, 1024, 2048])
def test_special_bit_pattern_matrix_wide_form(bi, topk):
    s, rs, re = special_matrix(topk + 1, copies=19)          # 1026 rows
    assert s.shape[0] >= 1024
    banner(f"topk special bit patterns, 512-thread form, topk={topk}")
    check(bi, s, topk, rs, re, what="special patterns, wide form")


@pytest.mark.parametrize("pitch_extra", [1, 37])
def test_odd_row_pitch_wide_form(bi, pitch_extra):
    g = np.random.default_rng(100 + pitch_extra)
    rows, cols = 1030, 1000
    s = np.maximum(g.standard_normal((rows, cols)), 0).astype(np.float32)
    rs = g.integers(0, 500, rows)
    re = rs + g.integers(0, 600, rows)
    banner(f"topk strided pitch={cols + pitch_extra}, 512-thread form")
    check(bi, s, 512, rs, re, pitch=cols + pitch_extra, what="strided, wide form")


def test_both_forms_select_the_same_rows(bi):
    # the same rows in a 1023-row batch (1024-thread form) and a 1024-row
    # batch (512-thread form) give the same selection
    g = np.random.default_rng(4)
    cols = 8192
    s = np.where(g.random((1024, cols)) < 0.5, 0.0, g.standard_normal((1024, cols))).astype(np.float32)
    s = (s.view(np.uint32) & 0xFFFF0000).view(np.float32)           # bf16-rounded ties, as the indexer has
    rs = g.integers(-5, 4000, 1024)
    re = rs + g.integers(0, 8000, 1024)
    for topk in wl.INDEXER_TOPK:
        banner(f"topk 1023 vs 1024 rows topk={topk}")
        a = gpu_topk(bi, s[:1023], topk, rs[:1023], re[:1023])
        b = gpu_topk(bi, s, topk, rs, re)
        assert np.array_equal(a, b[:1023]), f"the two forms differ at topk={topk}"
    want = oracle.topk_rows(s, 2048, rs.astype(np.int64), re.astype(np.int64))
    assert np.array_equal(b, want)


def test_window_offset_invariance_and_degenerate_rows(bi):
    g = np.random.default_rng(3)
    L = 2600
    logical = np.where(g.random(L) < 0.7, 0.0, g.standard_normal(L)).astype(np.float32)
    offs = (0, 1, 5, 64, 1000, 5000)
    cols = 8192
    s = np.full((len(offs), cols), np.inf, np.float32)
    s[:, ::2] = np.float32(np.nan)
    for i, o in enumerate(offs):
        s[i, o:o + L] = logical
    rs = np.array(offs, np.int64)
    re = rs + L
    for topk in (512, 1024, 2048):
        banner(f"topk window offsets topk={topk}")
        got = check(bi, s, topk, rs, re, what="offsets")
        assert (got == got[0]).all(), "a row's selection moved with its window"
    # all equal, all -inf, empty windows, bounds beyond int32
    d = np.stack([np.full(cols, 0.5, np.float32), np.full(cols, -np.inf, np.float32),
                  np.full(cols, -0.0, np.float32), np.zeros(cols, np.float32)])
    big = 1 << 40
    banner("topk degenerate rows")
    got = check(bi, d, 2048, [0, -big, 9000, 100], [cols, big, 9100, 100], what="degenerate")
    assert got[0].tolist() == list(range(2048)) and got[1].tolist() == list(range(2048))
    assert (got[2:] == -1).all()


def test_repeat_determinism_and_row_independence(bi):
    b = wl.indexer_decode(64)
    banner("topk decode 64 rows repeat")
    a1 = gpu_topk(bi, b.scores, 2048, b.row_start, b.row_end)
    a2 = gpu_topk(bi, b.scores, 2048, b.row_start, b.row_end)
    assert np.array_equal(a1, a2)
    solo = gpu_topk(bi, b.scores[17:18], 2048, b.row_start[17:18], b.row_end[17:18])
    assert np.array_equal(solo[0], a1[17])


@pytest.mark.parametrize("rows", wl.INDEXER_DECODE_ROWS)
def test_decode_workload_all_rows(bi, rows):
    b = wl.indexer_decode(rows)
    for topk in wl.INDEXER_TOPK:
        banner(f"topk decode rows={rows} topk={topk}")
        check(bi, b.scores, topk, b.row_start, b.row_end, what=f"decode rows={rows} topk={topk}")


def test_prefill_workload_all_rows(bi):
    b = wl.indexer_prefill(wl.INDEXER_PREFILL_ROWS)
    banner(f"topk prefill rows={wl.INDEXER_PREFILL_ROWS} topk=2048")
    check(bi, b.scores, 2048, b.row_start, b.row_end, what="prefill")
