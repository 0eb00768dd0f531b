"""Pins for the oracle's MoE activation and combine options (CPU only).

Fused-MoE page: the batch-invariant MoE shipped a squared-ReLU activation
before gated SwiGLU was added, and its top-k sum has an (apply_weights,
acc_fp64) option matrix whose (false, false) point was found to apply the
routing weights anyway.  These tests pin the oracle's options to facts fixed
without it: exactly representable closed forms, a float32 re-computation of
the fp32 combine with numpy's IEEE arithmetic, an independent dense numpy
formulation, and the matrix properties themselves (unweighted results do not
depend on the router's probabilities).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl
from tests import exact as ex

SW, SQ = oracle.ACT_SWIGLU, oracle.ACT_SQRELU


def bf16(vals):
    return wl.f32_to_bf16_bits(np.asarray(vals, np.float32))


def sqrelu_layer(E=4, H=8, I=4, seed=0, M=5):
    """Small integers everywhere: h, a and every slot output are exact, so
    the only roundings left are the combine's."""
    g = np.random.default_rng(seed)
    w1 = bf16(g.integers(-1, 2, (E, I, H)))
    w2 = bf16(g.integers(-3, 4, (E, H, I)))
    wr = (g.standard_normal((E, H)) * 0.5).astype(np.float32)
    x = bf16(g.integers(-1, 2, (M, H)))
    return x, wr, w1, w2


def slot_outputs(x, w1, w2, ids):
    """Exact per-slot outputs of the squared-ReLU layer with integer data."""
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    out = np.zeros(ids.shape + (w2.shape[1],))
    for m in range(x.shape[0]):
        for j, e in enumerate(ids[m]):
            h = xf[m] @ wl.bf16_bits_to_f32(w1[e]).astype(np.float64).T
            a = np.maximum(h, 0.0) ** 2
            assert np.all(np.abs(a) < 256) and np.all(a == np.round(a))    # exact in bf16
            out[m, j] = a @ wl.bf16_bits_to_f32(w2[e]).astype(np.float64).T
    return out


@pytest.mark.parametrize("apply_weights", [False, True])
@pytest.mark.parametrize("acc_fp64", [False, True])
def test_sqrelu_combine_matrix_exact(apply_weights, acc_fp64):
    # three slots, so that an fp32 sum rounded once at the end (instead of
    # after every add) shows on some of the 40 tokens
    x, wr, w1, w2 = sqrelu_layer(M=40)
    k = 3
    y, ids, probs, _ = oracle.moe_ex(x, wr, None, w1, w2, k, act=SQ, probs_at_act=False,
                                     apply_weights=apply_weights, acc_fp64=acc_fp64)
    yj = slot_outputs(x, w1, w2, ids)
    if acc_fp64:
        want = np.zeros(yj.shape[::2])
        for m in range(x.shape[0]):
            s = [Fraction(0)] * yj.shape[2]
            for j in range(k):
                wj = Fraction(float(probs[m, j])) if apply_weights else Fraction(1)
                s = [s[c] + wj * Fraction(float(yj[m, j, c])) for c in range(yj.shape[2])]
            want[m] = [ex.to_f32(v) for v in s]
    else:
        # fp32 slot partials, fp32 products and fp32 adds in slot order (numpy float32 is IEEE RNE)
        want = np.zeros(yj.shape[::2], np.float32)
        for m in range(x.shape[0]):
            acc = np.zeros(yj.shape[2], np.float32)
            for j in range(k):
                t = yj[m, j].astype(np.float32)
                if apply_weights:
                    t = np.float32(probs[m, j]) * t
                acc = acc + t
            want[m] = acc
    np.testing.assert_array_equal(y, np.asarray(want, np.float32))


def test_unweighted_results_do_not_depend_on_the_probabilities():
    # the (false, false) point of the matrix applies no weights: two routers
    # with very different probabilities but the same forced ids give the same bits
    x, wr, w1, w2 = sqrelu_layer(seed=3)
    ids = np.array([[0, 2], [1, 3], [3, 0], [2, 1], [0, 1]], np.int32)
    for acc_fp64 in (False, True):
        ya, *_ = oracle.moe_ex(x, wr, None, w1, w2, 2, act=SQ, probs_at_act=False, apply_weights=False,
                               acc_fp64=acc_fp64, ids=ids)
        yb, *_ = oracle.moe_ex(x, wr * 7.0, None, w1, w2, 2, act=SQ, probs_at_act=False, apply_weights=False,
                               acc_fp64=acc_fp64, ids=ids)
        np.testing.assert_array_equal(ya, yb)
        yw, *_ = oracle.moe_ex(x, wr, None, w1, w2, 2, act=SQ, probs_at_act=False, apply_weights=True,
                               acc_fp64=acc_fp64, ids=ids)
        assert not np.array_equal(ya, yw)


def test_sqrelu_closed_form_and_negative_half():
    # one-hot token: h_i = w1[e, i, 0] exactly; squared-ReLU zeroes negatives
    E, H, I = 2, 8, 4
    w1 = np.zeros((E, I, H), np.float32)
    w1[:, :, 0] = [[1.5, -2.0, 3.0, 0.25], [-1.0, 2.5, 0.0, -0.5]]
    w2 = np.zeros((E, H, I), np.float32)
    for e in range(E):
        w2[e, :I, :] = np.eye(I)
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    ids = np.array([[0, 1]], np.int32)
    y, _, probs, _ = oracle.moe_ex(bf16(x), np.zeros((E, H), np.float32), None, bf16(w1), bf16(w2), 2,
                                   act=SQ, probs_at_act=False, apply_weights=False, acc_fp64=True, ids=ids)
    # unweighted: relu^2 of expert 0 plus relu^2 of expert 1
    np.testing.assert_array_equal(y[0, :I], np.float32([2.25 + 0, 0 + 6.25, 9.0 + 0, 0.0625 + 0]))
    assert np.all(y[0, I:] == 0)
    # probability at the activation instead: both probabilities are 1/2 (zero router)
    y2, *_ = oracle.moe_ex(bf16(x), np.zeros((E, H), np.float32), None, bf16(w1), bf16(w2), 2,
                           act=SQ, probs_at_act=True, apply_weights=False, acc_fp64=True, ids=ids)
    np.testing.assert_array_equal(y2[0, :I], np.float32([1.125, 3.125, 4.5, 0.03125]))


def _dense_variant(x, wr, w1, w2, k, act, probs_at_act, apply_weights):
    """Independent dense formulation with numpy float64 and exact rational
    bf16 rounding (binary64 combine)."""
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    logits = (xf @ wr.astype(np.float64).T).astype(np.float32)
    I = w2.shape[2]
    out = np.zeros((x.shape[0], w2.shape[1]))
    order = [sorted(range(wr.shape[0]), key=lambda e: (-float(logits[m, e]), e))[:k] for m in range(x.shape[0])]
    r16 = np.vectorize(lambda v: float(ex.bf16_value(ex.to_bf16_bits(Fraction(float(v))))))
    for m in range(x.shape[0]):
        l64 = logits[m].astype(np.float64)
        p_all = np.exp(l64 - l64.max()) / np.sum(np.exp(l64 - l64.max()))
        for e in order[m]:
            h = r16(xf[m] @ wl.bf16_bits_to_f32(w1[e]).astype(np.float64).T)
            if act == SW:
                g, u = h[:I], h[I:]
                v = g / (1.0 + np.exp(-g)) * u
            else:
                v = np.maximum(h, 0.0) ** 2
            a = r16(v * (p_all[e] if probs_at_act else 1.0))
            y = a @ wl.bf16_bits_to_f32(w2[e]).astype(np.float64).T
            out[m] += y * (p_all[e] if apply_weights else 1.0)
    return out.astype(np.float32), np.array(order, np.int32)


@pytest.mark.parametrize("act,pa,aw", [(SW, False, True), (SW, False, False), (SQ, False, True),
                                       (SQ, True, False), (SQ, False, False)])
def test_variants_against_dense_formulation(act, pa, aw):
    E, H, I, k = 8, 32, 6, 3
    g = np.random.default_rng(7)
    w1 = wl.normal_bf16(g, (E, 2 * I if act == SW else I, H), 0.2)
    w2 = wl.normal_bf16(g, (E, H, I), 0.2)
    wr = (g.standard_normal((E, H)) * 0.3).astype(np.float32)
    x = wl.normal_bf16(g, (6, H), 1.0)
    y, ids, _, _ = oracle.moe_ex(x, wr, None, w1, w2, k, act=act, probs_at_act=pa, apply_weights=aw,
                                 acc_fp64=True)
    yd, idsd = _dense_variant(x, wr, w1, w2, k, act, pa, aw)
    np.testing.assert_array_equal(ids, idsd)
    np.testing.assert_allclose(y, yd, rtol=1e-5, atol=1e-6)


def test_defaults_are_the_gated_layer():
    w = wl.moe_weights(2, H=16, E=8, I=4)
    x = wl.moe_batch(3, w).x
    a = oracle.moe(x, w.w_router, None, w.w13, w.w2, 2)
    b = oracle.moe_ex(x, w.w_router, None, w.w13, w.w2, 2)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
