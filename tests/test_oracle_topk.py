"""Pins for the oracle's indexer top-k (Sparse-MLA page, deterministic
per-row top-k commit notes).

The oracle ranks lanes by (inside the window first, larger int32 key, lower
column) with one library sort.  These tests hold it to facts fixed without it:
a pure-Python selection on finite rows that compares floats directly, the key
order of special fp32 bit patterns as the notes describe it, and the
invariants the notes test for (a row's result does not depend on where its
window sits, empty and all-equal rows, int64 bounds).
"""
import numpy as np
import pytest

import oracle


def brute(row, topk, rs, re):
    """Plain definition on finite values: sort the window's columns by
    (-score, column) with Python float comparison (-0.0 == +0.0), keep the
    first topk, emit ascending and row-local, pad with -1."""
    cols = len(row)
    rs = min(max(rs, 0), cols)
    re = min(max(re, 0), cols)
    cand = sorted(range(rs, max(re, rs)), key=lambda c: (-float(row[c]), c))
    sel = sorted(cand[:topk])
    return [c - rs for c in sel] + [-1] * (topk - len(sel))


def f32_from_bits(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


@pytest.mark.parametrize("seed", range(6))
def test_against_plain_python_selection(seed):
    g = np.random.default_rng(seed)
    rows, cols = 12, int(g.integers(1, 300))
    # quantised relu-like scores: many exact zeros and repeated values, both zeros
    s = np.maximum(g.standard_normal((rows, cols)), 0.0)
    s = (np.round(s * 4) / 4).astype(np.float32)
    s[g.random((rows, cols)) < 0.1] = -0.0
    s[g.random((rows, cols)) < 0.05] *= -1
    rs = g.integers(-5, cols + 5, rows)
    re = g.integers(-5, cols + 5, rows)
    re[::3] = cols + 100                       # windows running past the row
    for topk in (1, 7, max(1, cols // 3), cols + 3):
        got = oracle.topk_rows(s, topk, rs, re)
        for r in range(rows):
            assert got[r].tolist() == brute(s[r], topk, int(rs[r]), int(re[r])), (seed, topk, r)


# Special fp32 bit patterns, listed from the highest key to the lowest as the
# notes define the key: -0.0 is canonicalised to +0.0 (so the two tie and the
# lower column wins), positive NaNs sit above +inf ordered by their bits,
# negative NaNs below -inf, 0xfffffffe just above 0xffffffff = INT32_MIN.
RANKED = [
    0x7FFFFFFF,   # largest positive NaN pattern
    0x7FC00000,   # quiet NaN
    0x7F800001,   # signalling NaN
    0x7F800000,   # +inf
    0x7F7FFFFF,   # largest finite
    0x3F800000,   # 1.0
    0x00800000,   # smallest normal
    0x007FFFFF,   # largest denormal
    0x00000001,   # smallest denormal
    "ZEROS",      # +0.0 and -0.0, tied
    0x80000001,   # -smallest denormal
    0x807FFFFF,   # -largest denormal
    0xBF800000,   # -1.0
    0xFF7FFFFF,   # -largest finite
    0xFF800000,   # -inf
    0xFF800001,   # negative signalling NaN
    0xFFC00000,   # negative quiet NaN
    0xFFFFFFFE,   # key INT32_MIN + 1
    0xFFFFFFFF,   # key INT32_MIN
]


def special_row(perm):
    """The patterns above in a permuted column order; returns (bits, rank of
    each column), with the two zeros sharing a rank."""
    items = []
    for rank, b in enumerate(RANKED):
        if b == "ZEROS":
            items += [(0x00000000, rank), (0x80000000, rank)]
        else:
            items.append((b, rank))
    items = [items[i] for i in perm]
    return [b for b, _ in items], [r for _, r in items]


@pytest.mark.parametrize("seed", range(4))
def test_special_bit_patterns_rank_as_the_key_says(seed):
    g = np.random.default_rng(seed)
    n = len(RANKED) + 1
    bits, rank = special_row(g.permutation(n))
    order = sorted(range(n), key=lambda c: (rank[c], c))   # ties (the zeros) by column
    s = f32_from_bits(bits)[None, :]
    for k in range(1, n + 2):
        want = sorted(order[:k]) + [-1] * max(0, k - n)
        assert oracle.topk_rows(s, k).tolist()[0] == want, (seed, k)


def test_window_position_does_not_change_the_selection():
    # the same logical row placed at several offsets, surrounded by lanes that
    # would win if they were ranked inside the window (NaN, +inf, big values)
    # and by lanes tied with the window's plateau (masked lanes must not spend
    # the tie budget)
    g = np.random.default_rng(11)
    L = 700
    logical = np.where(g.random(L) < 0.6, 0.0, g.standard_normal(L)).astype(np.float32)
    ref = {}
    for off in (0, 1, 5, 64, 333, 1000):
        cols = off + L + 37
        row = np.zeros(cols, np.float32)
        row[:off] = np.where(np.arange(off) % 3 == 0, np.inf, np.nan if off % 2 else 0.0)
        row[off + L:] = f32_from_bits([0xFFFFFFFF] * 37)
        row[off:off + L] = logical
        for topk in (512, 1024, 2048):
            got = oracle.topk_rows(row[None, :], topk, np.array([off]), np.array([off + L]))[0]
            assert np.array_equal(got, ref.setdefault(topk, got)), (off, topk)
    # 60% zeros: the 512 cut falls inside the zero plateau, so the budget matters
    assert (ref[512] >= 0).sum() == 512 and (ref[1024] >= 0).sum() == L


def test_all_equal_all_minus_inf_and_empty_rows():
    cols = 100
    s = np.stack([np.full(cols, 0.25, np.float32), np.full(cols, -np.inf, np.float32),
                  np.full(cols, -0.0, np.float32), np.zeros(cols, np.float32)])
    got = oracle.topk_rows(s, 10)
    for r in range(3):
        assert got[r].tolist() == list(range(10))
    # empty windows: start at or past the end, start past the row, negative end
    rs = np.array([0, 50, cols + 5, -10], np.int64)
    re = np.array([cols, 50, cols + 9, -1], np.int64)
    got = oracle.topk_rows(s, 10, rs, re)
    assert got[0].tolist() == list(range(10))
    assert all(v == -1 for v in got[1:].ravel())


def test_int64_bounds_clamp_before_narrowing():
    cols = 64
    s = np.arange(cols, dtype=np.float32)[None, :].repeat(3, 0)
    big = np.int64(1) << 40
    rs = np.array([-big, 60, -(1 << 33)], np.int64)
    re = np.array([big, big, 3], np.int64)
    got = oracle.topk_rows(s, 4, rs, re)
    assert got[0].tolist() == [60, 61, 62, 63]       # whole row, largest four
    assert got[1].tolist() == [0, 1, 2, 3]            # window 60..63, row-local
    assert got[2].tolist() == [0, 1, 2, -1]           # window 0..2


def test_selection_is_the_topk_under_the_rank_order():
    # independent check of the cut: every selected lane outranks every
    # unselected in-window lane, on a large plateau-heavy row
    g = np.random.default_rng(5)
    cols = 8192
    row = np.maximum(g.standard_normal(cols), 0).astype(np.float32)
    row[g.random(cols) < 0.2] = -0.0
    for topk in (512, 1024, 2048):
        got = oracle.topk_rows(row[None, :], topk)[0]
        sel = set(got.tolist())
        assert len(sel) == topk and got.tolist() == sorted(sel)
        v = row.astype(np.float64)            # -0.0 == 0.0 in float comparison
        worst = min((v[c], -c) for c in sel)
        best_out = max(((v[c], -c) for c in range(cols) if c not in sel), default=None)
        assert best_out < worst
