"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each pin is chosen so that a plausible slip in the oracle -- a dropped bias,
a transposed weight, a wrong rounding mode, a swapped gate/up half, a
probability applied twice, a reversed tie rule -- fails at least one test:

* brute force with exact rationals (``fractions.Fraction``) on tiny shapes,
* closed forms (identity, one-hot, zero and small-integer weights),
* invariants (power-of-two scaling, row-locality, column permutation),
* an independent library computation (numpy float64 matmul) within the
  binary64 error bound,
* top-k against Python's stable sort, and MoE closed forms.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl
from tests import exact as ex

# --------------------------------------------------------------- linear f32


@pytest.mark.parametrize("M,N,K,bias", [(1, 1, 1, False), (3, 5, 7, True), (4, 8, 16, True),
                                        (2, 3, 16, False), (4, 6, 9, True)])
def test_linear_f32_brute_force(M, N, K, bias):
    g = np.random.default_rng(100 + M * 31 + N * 7 + K)
    x = (g.standard_normal((M, K)) * 2.0 ** g.integers(-8, 8, (M, K))).astype(np.float32)
    w = g.standard_normal((N, K)).astype(np.float32)
    b = g.standard_normal(N).astype(np.float32) if bias else None
    y = oracle.linear_f32(x, w, b)
    for m in range(M):
        for n in range(N):
            q = sum((ex.exact(x[m, k]) * ex.exact(w[n, k]) for k in range(K)), Fraction(0))
            if bias:
                q += ex.exact(b[n])
            assert y[m, n] == ex.to_f32(q), (m, n)


@pytest.mark.parametrize("M,N,K,bias,out", [(2, 3, 16, True, "bf16"), (3, 4, 8, False, "bf16"),
                                            (4, 5, 12, True, "f32"), (1, 8, 32, False, "f32")])
def test_linear_bf16_brute_force(M, N, K, bias, out):
    g = np.random.default_rng(200 + M + N + K)
    x = wl.normal_bf16(g, (M, K), 1.0)
    w = wl.normal_bf16(g, (N, K), 1.0)
    b = g.standard_normal(N).astype(np.float32) if bias else None
    y = oracle.linear_bf16(x, w, b, out=out)
    for m in range(M):
        for n in range(N):
            q = sum((ex.bf16_value(x[m, k]) * ex.bf16_value(w[n, k]) for k in range(K)), Fraction(0))
            if bias:
                q += ex.exact(b[n])
            want = ex.to_bf16_bits(q) if out == "bf16" else ex.to_f32(q)
            assert y[m, n] == want, (m, n)


def test_bf16_rounding_ties_and_ranges():
    # hand-picked: exact ties go to the even neighbour, subnormals, overflow
    vals = [1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, -2.5, 2 ** -133, 1.5 * 2 ** -133,
            2.5 * 2 ** -133, 3.0e38, 3.4e38, -0.0, 0.0]
    got = oracle.f64_to_bf16(np.array(vals))
    want = [ex.to_bf16_bits(Fraction(v)) if math.isfinite(v) and v != 0 else None for v in vals]
    for v, gbits, w in zip(vals, got, want):
        if w is None:
            continue
        assert gbits == w, (v, hex(gbits), hex(w))
    assert got[-2] == 0x8000 and got[-1] == 0x0000
    assert got[0] == 0x3F80 and got[1] == 0x3F80 and got[2] == 0x3F82 and got[3] == 0x3F81


def test_bf16_rounding_matches_torch_on_float_inputs():
    # torch's float32 -> bfloat16 conversion is round-to-nearest-even; for
    # values that are already float32 there is no double rounding to worry about.
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(5)
    f = (g.standard_normal(20000) * 2.0 ** g.integers(-60, 60, 20000)).astype(np.float32)
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32)
    f = np.concatenate([f, ties, -ties])
    ours = oracle.f64_to_bf16(f.astype(np.float64))
    theirs = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)


def test_identity_weight_closed_form():
    g = np.random.default_rng(11)
    K = 64
    x = g.standard_normal((5, K)).astype(np.float32)
    b = g.standard_normal(K).astype(np.float32)
    y = oracle.linear_f32(x, np.eye(K, dtype=np.float32), b)
    np.testing.assert_array_equal(y, x + b)           # one IEEE fp32 add
    np.testing.assert_array_equal(oracle.linear_f32(x, np.eye(K, dtype=np.float32)), x)


def test_one_hot_weight_closed_form():
    g = np.random.default_rng(12)
    N, K = 24, 40
    perm = g.permutation(K)[:N]
    w = np.zeros((N, K), np.float32)
    w[np.arange(N), perm] = 1.0
    x = g.standard_normal((7, K)).astype(np.float32)
    b = g.standard_normal(N).astype(np.float32)
    np.testing.assert_array_equal(oracle.linear_f32(x, w, b), x[:, perm] + b)


def test_zero_weight_is_bias():
    x = np.random.default_rng(13).standard_normal((3, 16)).astype(np.float32)
    b = np.arange(8, dtype=np.float32) - 3.5
    np.testing.assert_array_equal(oracle.linear_f32(x, np.zeros((8, 16), np.float32), b),
                                  np.broadcast_to(b, (3, 8)))


def test_small_integer_inputs_exact():
    g = np.random.default_rng(14)
    xi = g.integers(-8, 9, (9, 300))
    wi = g.integers(-8, 9, (20, 300))
    bi = g.integers(-100, 100, 20)
    y = oracle.linear_f32(xi.astype(np.float32), wi.astype(np.float32), bi.astype(np.float32))
    np.testing.assert_array_equal(y, (xi @ wi.T + bi).astype(np.float32))
    # bf16 operands: |v| <= 4 is exact in bf16; the bf16 result is RN_bf16(exact)
    xb = g.integers(-4, 5, (6, 128))
    wb = g.integers(-4, 5, (10, 128))
    yb = oracle.linear_bf16(wl.f32_to_bf16_bits(xb.astype(np.float32)),
                            wl.f32_to_bf16_bits(wb.astype(np.float32)), None, out="bf16")
    exact_int = xb @ wb.T
    want = np.array([[ex.to_bf16_bits(Fraction(int(v))) for v in row] for row in exact_int], np.uint16)
    np.testing.assert_array_equal(yb, want)


def test_power_of_two_scaling():
    w = wl.router_weights(0)
    x = wl.router_batch(5, w).x
    y = oracle.linear_f32(x, w.w, w.b)
    y8 = oracle.linear_f32(x * np.float32(8.0), w.w, w.b * np.float32(8.0))
    np.testing.assert_array_equal(y8, y * np.float32(8.0))


def test_row_locality_and_column_permutation():
    w = wl.tiny_weights(0)
    x = wl.tiny_batch(17, w).x
    y = oracle.linear_f32(x, w.w, w.b)
    for m in (0, 5, 16):
        np.testing.assert_array_equal(oracle.linear_f32(x[m:m + 1], w.w, w.b)[0], y[m])
    perm = np.random.default_rng(3).permutation(w.w.shape[0])
    np.testing.assert_array_equal(oracle.linear_f32(x, w.w[perm], w.b[perm]), y[:, perm])


def test_router_shape_against_float64_blas():
    # An independent implementation (BLAS, its own summation order) agrees
    # within the binary64 error bound K * 2^-53 * sum|x w|; then both round to
    # the same fp32 value except at a rounding boundary, which we allow.
    w = wl.router_weights(0)
    x = wl.router_batch(8, w).x
    y, y64 = oracle.linear_f32(x, w.w, w.b, want_f64=True)
    ref = x.astype(np.float64) @ w.w.astype(np.float64).T + w.b.astype(np.float64)
    bound = (x.shape[1] + 1) * 2.0 ** -53 * (np.abs(x.astype(np.float64)) @ np.abs(w.w.astype(np.float64)).T
                                             + np.abs(w.b))
    assert np.all(np.abs(y64 - ref) <= 2 * bound)
    assert np.mean(y == ref.astype(np.float32)) > 0.999


def test_bf16_roundtrip_fails_the_fp32_tolerance_at_router_shape():
    # GateLinear page, "What": the fp32 router must not round through bf16; a
    # bf16 round-trip fails the fp32 correctness tolerance.  The margin at this
    # synthetic shape is measured, not tuned (reported by the test output).
    w = wl.router_weights(0)
    x = wl.router_batch(128, w).x
    y = oracle.linear_f32(x, w.w, w.b)
    xb = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x))
    wb = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(w.w))
    y_rt = oracle.linear_f32(xb, wb, w.b)
    ratio = np.max(np.abs(y_rt - y) / (2e-3 + 1e-4 * np.abs(y)))
    assert ratio > 1.0, ratio


# -------------------------------------------------------------------- top-k


def _topk_sorted(row, k):
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]


def test_topk_against_stable_sort():
    g = np.random.default_rng(21)
    s = g.standard_normal((50, 128)).astype(np.float32)
    s[:, 5] = s[:, 9]                      # planted exact ties
    s[:10] = np.round(s[:10])              # heavy tie plateaus
    ids = oracle.topk(s, 8)
    for m in range(50):
        assert list(ids[m]) == _topk_sorted(s[m], 8), m


def test_topk_ties_lowest_index_and_signed_zero():
    s = np.zeros((3, 16), np.float32)
    np.testing.assert_array_equal(oracle.topk(s, 8)[0], np.arange(8))
    s[1, :] = -1.0
    s[1, 3] = -0.0
    s[1, 1] = 0.0
    s[1, 10] = 2.0
    np.testing.assert_array_equal(oracle.topk(s, 3)[1], [10, 1, 3])   # +0 and -0 tie -> index order
    s[2, :] = -np.inf
    s[2, 15] = np.inf
    np.testing.assert_array_equal(oracle.topk(s, 4)[2], [15, 0, 1, 2])
    with pytest.raises(ValueError):
        oracle.topk(np.array([[np.nan, 1.0]], np.float32), 1)


# ---------------------------------------------------------------------- MoE


def _tiny_moe(seed, H=16, E=8, I=4):
    return wl.moe_weights(seed, H=H, E=E, I=I)


def test_moe_zero_router_closed_form():
    w = _tiny_moe(1)
    w.w_router[:] = 0.0
    x = wl.moe_batch(5, w).x
    y, ids, probs, logits = oracle.moe(x, w.w_router, None, w.w13, w.w2, topk=3)
    np.testing.assert_array_equal(ids, np.tile(np.arange(3), (5, 1)))
    assert np.all(probs == 1.0 / 8.0) and np.all(logits == 0.0)


def test_moe_zero_down_projection():
    w = _tiny_moe(2)
    w.w2[:] = 0
    x = wl.moe_batch(4, w).x
    y, *_ = oracle.moe(x, w.w_router, None, w.w13, w.w2, topk=2)
    assert np.all(y == 0.0)


def test_moe_swiglu_closed_form():
    # one-hot token x = e_0; gate rows read g = 1, up rows read u = 2; router
    # W = 0 so p = 1/E on slots 0..k-1; w2 = identity on the first I outputs.
    # Then y[c] = RN_f32(k * RN_bf16(1 * sigma(1) * 2 * p)) for c < I, else 0.
    # Swapping gate and up would give 2*sigma(2) instead; dropping p, the
    # sigmoid, or the slot sum changes the value.
    H, E, I, k = 12, 4, 5, 3
    one = wl.f32_to_bf16_bits(np.float32(1.0))
    two = wl.f32_to_bf16_bits(np.float32(2.0))
    x = np.zeros((2, H), np.uint16)
    x[:, 0] = one
    w13 = np.zeros((E, 2 * I, H), np.uint16)
    w13[:, :I, 0] = one
    w13[:, I:, 0] = two
    w2 = np.zeros((E, H, I), np.uint16)
    for i in range(I):
        w2[:, i, i] = one
    y, ids, probs, _ = oracle.moe(x, np.zeros((E, H), np.float32), None, w13, w2, topk=k)
    sig1 = Fraction(1.0 / (1.0 + math.exp(-1.0)))
    a = ex.bf16_value(ex.to_bf16_bits(sig1 * 2 * Fraction(1, E)))
    want = np.zeros(H, np.float32)
    want[:I] = ex.to_f32(k * a)
    np.testing.assert_array_equal(y[0], want)
    np.testing.assert_array_equal(y[1], want)
    # swapped halves would not match
    sig2 = Fraction(1.0 / (1.0 + math.exp(-2.0)))
    assert ex.to_f32(k * ex.bf16_value(ex.to_bf16_bits(sig2 * 2 * Fraction(1, E)))) != want[0]


def _moe_dense_numpy(x, wr, w13, w2, k):
    """Independent dense formulation: every expert on every token, masked by
    the chosen set, with numpy float64 matmuls and torch-free rounding."""
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    logits = (xf @ wr.astype(np.float64).T).astype(np.float32)
    E = wr.shape[0]
    I = w2.shape[2]
    M = x.shape[0]
    out = np.zeros((M, w2.shape[1]))
    ids = np.array([_topk_sorted(logits[m], k) for m in range(M)])
    for m in range(M):
        l64 = logits[m].astype(np.float64)
        p_all = np.exp(l64 - l64.max()) / np.sum(np.exp(l64 - l64.max()))
        for j, e in enumerate(ids[m]):
            h = xf[m] @ wl.bf16_bits_to_f32(w13[e]).astype(np.float64).T
            h = np.array([float(ex.bf16_value(ex.to_bf16_bits(Fraction(v)))) for v in h])
            g, u = h[:I], h[I:]
            a = g / (1.0 + np.exp(-g)) * u * p_all[e]
            a = np.array([float(ex.bf16_value(ex.to_bf16_bits(Fraction(v)))) for v in a])
            out[m] += a @ wl.bf16_bits_to_f32(w2[e]).astype(np.float64).T
    return out.astype(np.float32), ids, logits


def test_moe_against_dense_formulation():
    w = _tiny_moe(3, H=32, E=8, I=6)
    x = wl.moe_batch(6, w).x
    y, ids, probs, logits = oracle.moe(x, w.w_router, None, w.w13, w.w2, topk=3)
    yd, idsd, logitsd = _moe_dense_numpy(x, w.w_router, w.w13, w.w2, 3)
    np.testing.assert_array_equal(ids, idsd)
    np.testing.assert_allclose(logits, logitsd, rtol=0, atol=1e-6)
    np.testing.assert_allclose(y, yd, rtol=1e-5, atol=1e-6)


def test_moe_row_locality_and_forced_ids():
    w = _tiny_moe(4)
    x = wl.moe_batch(7, w).x
    y, ids, probs, _ = oracle.moe(x, w.w_router, None, w.w13, w.w2, topk=2)
    y1, ids1, p1, _ = oracle.moe(x[3:4], w.w_router, None, w.w13, w.w2, topk=2)
    np.testing.assert_array_equal(y1[0], y[3])
    np.testing.assert_array_equal(ids1[0], ids[3])
    # forcing the ids the oracle chose reproduces it bit for bit; reversing the
    # slot order only permutes an fp64 sum of two terms (exact), same result
    yf, *_ = oracle.moe(x, w.w_router, None, w.w13, w.w2, topk=2, ids=ids)
    np.testing.assert_array_equal(yf, y)
    yr, idsr, pr, _ = oracle.moe(x, w.w_router, None, w.w13, w.w2, topk=2, ids=ids[:, ::-1].copy())
    np.testing.assert_array_equal(yr, y)
    np.testing.assert_array_equal(pr, probs[:, ::-1])


def test_moe_probabilities_are_softmax():
    w = _tiny_moe(5)
    x = wl.moe_batch(4, w).x
    _, ids, probs, logits = oracle.moe(x, w.w_router, None, w.w13, w.w2, topk=8)
    # all experts selected: probabilities sum to one and follow the logits
    np.testing.assert_allclose(probs.sum(axis=1), 1.0, rtol=1e-12)
    for m in range(4):
        l = logits[m].astype(np.float64)
        ref = np.exp(l - l.max()) / np.exp(l - l.max()).sum()
        np.testing.assert_allclose(probs[m], ref[ids[m]], rtol=1e-12)
        assert np.all(np.diff(probs[m]) <= 0)
