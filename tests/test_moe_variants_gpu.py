"""MoE activation and top-k-sum options on the GPU against the oracle.

Fused-MoE page: squared-ReLU activation, and the (apply_weights, acc_fp64)
matrix of the top-k sum whose unweighted fp32 point must apply no weights.
Bars as in test_moe_gpu.py: ids bit-exact under the top-k rule on the GPU's
own logits, probabilities rtol 1e-5, outputs rtol 1e-2 with the measured
storage-point atol (tests/moe_bars.py) against the oracle run with the GPU ids, and rows
bitwise equal to the same rows computed alone.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import assert_bitwise, assert_close, banner, bf16_to_f32, dev, host, weight_t
from tests.moe_bars import RTOL, moe_atol

pytestmark = pytest.mark.gpu

SW, SQ = 0, 1          # bi_activation_t
VARIANTS = [  # (activation, probs_at_activation, apply_weights, acc_fp64)
    (SW, True, False, True), (SW, False, True, True), (SW, False, True, False), (SW, False, False, False),
    (SQ, False, True, False), (SQ, False, True, True), (SQ, False, False, False), (SQ, True, False, True),
]


@pytest.fixture(scope="module")
def bi():
    import deterministic_persistent_gemm_amd as m
    return m


def first_weight(w, act):
    # squared-ReLU experts use the gate half of the gated layer's first weight
    return w.w13 if act == SW else np.ascontiguousarray(w.w13[:, : w.w2.shape[2], :])


def run(bi, x, d, topk, v, b=None):
    act, pa, aw, f64 = v
    y, ids, probs = bi.bi_moe_grouped_gemm_ex(dev(x), d["wr"], b, d["w1"][act], d["w2"], topk, activation=act,
                                              probs_at_activation=pa, apply_weights=aw, acc_fp64=f64)
    return host(y), host(ids), host(probs)


def ora(x, w, b, topk, v, ids):
    act, pa, aw, f64 = v
    return oracle.moe_ex(x, w.w_router, b, first_weight(w, act), w.w2, topk,
                         act=oracle.ACT_SWIGLU if act == SW else oracle.ACT_SQRELU,
                         probs_at_act=pa, apply_weights=aw, acc_fp64=f64, ids=ids)


@pytest.mark.parametrize("v", VARIANTS, ids=lambda v: f"act{v[0]}-pa{int(v[1])}-aw{int(v[2])}-f64{int(v[3])}")
def test_small_layer_every_variant(bi, v):
    E, H, I, topk = 32, 256, 64, 4
    w = wl.moe_weights(5, H=H, E=E, I=I)
    b = (np.random.default_rng(9).standard_normal(E) * 0.05).astype(np.float32)
    d = dict(wr=dev(w.w_router), w2=dev(w.w2), w1={SW: dev(w.w13), SQ: dev(first_weight(w, SQ))})
    bd = dev(b)
    solo = None
    for M in (1, 5, 70, 200):
        banner(f"moe variant {v} small H=256 E=32 I=64 top-4 M={M}")
        x = wl.moe_batch(M, w).x
        x[M - 1] = wl.moe_batch(1, w).x[0]             # the same token at every M
        y, ids, probs = run(bi, x, d, topk, v, bd)
        lg = host(bi.bi_linear_f32(dev(bf16_to_f32(x)), weight_t(d["wr"]), bd))
        np.testing.assert_array_equal(oracle.topk(lg, topk), ids)
        yf, _, pf, _ = ora(x, w, b, topk, v, ids)
        assert_close(probs, pf, 0.0, 1e-5, f"probs M={M}")
        rms = float(np.sqrt(np.mean(yf.astype(np.float64) ** 2)))
        assert_close(y, yf, moe_atol(rms, H), RTOL, f"variant {v} M={M}")
        if solo is None:
            solo = (y[M - 1], ids[M - 1], probs[M - 1])
        assert_bitwise(y[M - 1], solo[0], f"token bits at M={M}")
        np.testing.assert_array_equal(ids[M - 1], solo[1])


def test_unweighted_points_ignore_the_probabilities(bi):
    # doubling the router weights doubles every logit exactly: the same experts
    # are chosen with different probabilities; unweighted results keep their
    # bits, weighted ones change
    E, H, I, topk = 32, 256, 64, 4
    w = wl.moe_weights(6, H=H, E=E, I=I)
    x = wl.moe_batch(40, w).x
    d1 = dict(wr=dev(w.w_router), w2=dev(w.w2), w1={SW: dev(w.w13), SQ: dev(first_weight(w, SQ))})
    d2 = dict(d1, wr=dev(w.w_router * np.float32(2.0)))
    for v in [(SQ, False, False, False), (SQ, False, False, True), (SW, False, False, False)]:
        banner(f"moe unweighted {v}")
        ya, ia, pa_ = run(bi, x, d1, topk, v)
        yb, ib, pb = run(bi, x, d2, topk, v)
        np.testing.assert_array_equal(ia, ib)
        assert not np.array_equal(pa_, pb)
        assert_bitwise(ya, yb, f"unweighted {v}")
    for v in [(SQ, False, True, False), (SQ, False, True, True)]:
        ya, _, _ = run(bi, x, d1, topk, v)
        yb, _, _ = run(bi, x, d2, topk, v)
        assert not np.array_equal(ya, yb), f"weighted {v} ignored the probabilities"


@pytest.mark.parametrize("v", [(SQ, False, True, False), (SQ, False, False, True)])
def test_qwen_shape_squared_relu(bi, v):
    w = wl.moe_weights(0)
    d = dict(wr=dev(w.w_router), w2=dev(w.w2), w1={SQ: dev(first_weight(w, SQ))})
    for M in (1, 16, 64):
        banner(f"moe Qwen shape squared-ReLU {v} M={M}")
        batch = wl.moe_batch(M, w)
        y, ids, probs = run(bi, batch.x, d, wl.MOE_TOPK, v)
        rows = np.unique(np.r_[0:min(M, 12), M - 1])
        yf, _, _, _ = ora(batch.x[rows], w, None, wl.MOE_TOPK, v, ids[rows])
        rms = float(np.sqrt(np.mean(yf.astype(np.float64) ** 2)))
        assert_close(y[rows], yf, moe_atol(rms, wl.MOE_H), RTOL, f"Qwen squared-ReLU M={M}")
