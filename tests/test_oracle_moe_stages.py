"""Pins for the MoE oracle's storage-point outputs (CPU).

The stage outputs must be the values the layer's own definition produces at
each storage point (fused-MoE page, "What's included": bf16 first projection,
bf16 activation with the probability applied, per-slot down projection, and
the top-k sum in slot order):
* h of every (token, slot) is the batch-invariant bf16 linear of the token's
  row with the chosen expert's first weight (pinned itself by exact rationals);
* each slot's part is the binary64 down projection of that slot's a (the bf16
  linear in binary64);
* the layer output is the fp32 rounding of the binary64 slot-order sum of the
  parts (unweighted configuration), and equal to moe()'s output bit for bit.
"""
import numpy as np

import oracle
import workloads as wl


def _layer():
    w = wl.moe_weights(3, H=128, E=16, I=32)
    x = wl.moe_batch(6, w).x
    return w, x


def test_stage_h_is_the_bf16_linear_of_the_chosen_expert():
    w, x = _layer()
    y, ids, probs, logits, h, a, part = oracle.moe_stages(x, w.w_router, None, w.w13, w.w2, 4)
    for m in range(x.shape[0]):
        for j in range(4):
            e = ids[m, j]
            ref = oracle.linear_bf16(x[m:m + 1], w.w13[e], out="bf16")[0]
            assert np.array_equal(h[m, j], ref), (m, j)


def test_stage_part_is_the_down_projection_of_a():
    w, x = _layer()
    y, ids, probs, logits, h, a, part = oracle.moe_stages(x, w.w_router, None, w.w13, w.w2, 4)
    for m in range(x.shape[0]):
        for j in range(4):
            _, y64 = oracle.linear_bf16(a[m, j][None, :], w.w2[ids[m, j]], out="f32", want_f64=True)
            assert np.array_equal(part[m, j], y64[0]), (m, j)


def test_output_is_the_slot_order_sum_of_parts_and_matches_moe():
    w, x = _layer()
    y, ids, probs, logits, h, a, part = oracle.moe_stages(x, w.w_router, None, w.w13, w.w2, 4)
    acc = np.zeros(part.shape[::2], np.float64)          # [M, H]
    for j in range(4):
        acc = acc + part[:, j, :]
    assert np.array_equal(y, acc.astype(np.float32))
    y2, ids2, probs2, logits2 = oracle.moe(x, w.w_router, None, w.w13, w.w2, 4)
    assert np.array_equal(y, y2) and np.array_equal(ids, ids2) and np.array_equal(probs, probs2)


def test_probability_lands_in_a_not_in_part_weights():
    # doubling the probability only through the activation: with the
    # probability applied at the activation, a depends on p; with it off
    # (unweighted sum) a does not, and h never does
    w, x = _layer()
    on = oracle.moe_stages(x, w.w_router, None, w.w13, w.w2, 4, probs_at_act=True)
    off = oracle.moe_stages(x, w.w_router, None, w.w13, w.w2, 4, probs_at_act=False)
    assert np.array_equal(on[4], off[4])
    assert not np.array_equal(on[5], off[5])
    w2x = wl.moe_weights(3, H=128, E=16, I=32)
    off2 = oracle.moe_stages(x, w2x.w_router * 2, None, w.w13, w.w2, 4, probs_at_act=False)
    same = off2[1] == off[1]
    assert np.array_equal(off2[5][same.all(axis=1)], off[5][same.all(axis=1)])


def test_activation_and_combine_steps_alone_reproduce_the_layer():
    # the separately callable steps are the layer's own: fed the layer's h
    # and p they return its a, fed its parts and p they return its output,
    # for every activation / weighting / sum option
    w, x = _layer()
    I = w.w2.shape[2]
    for act, w1 in ((oracle.ACT_SWIGLU, w.w13), (oracle.ACT_SQRELU, np.ascontiguousarray(w.w13[:, :I, :]))):
        for pa, aw, f64 in ((True, False, True), (False, True, True), (False, True, False), (False, False, False)):
            y, ids, probs, logits, h, a, part = oracle.moe_stages(x, w.w_router, None, w1, w.w2, 4, act=act,
                                                                 probs_at_act=pa, apply_weights=aw, acc_fp64=f64)
            M = x.shape[0]
            a2 = oracle.moe_activation(h.reshape(M * 4, -1), probs.reshape(-1), act=act, probs_at_act=pa)
            assert np.array_equal(a2, a.reshape(M * 4, I)), (act, pa, aw, f64)
            assert np.array_equal(oracle.moe_combine(part, probs, apply_weights=aw, acc_fp64=f64), y), \
                (act, pa, aw, f64)


def test_activation_closed_forms():
    # SwiGLU of g = 0 is 0 whatever u; squared-ReLU of a negative h is 0 and
    # of h = 2 is 4 (times p = 0.5: 2), exactly representable in bf16
    one, two, neg = 0x3F80, 0x4000, 0xC000
    h = np.array([[0x0000, one], [one, 0x0000]], np.uint16)           # SwiGLU rows, I = 1: [g | u]
    a = oracle.moe_activation(h, np.array([1.0, 1.0]), act=oracle.ACT_SWIGLU)
    assert a.tolist() == [[0], [0]]
    hs = np.array([[two], [neg]], np.uint16)
    a = oracle.moe_activation(hs, np.array([0.5, 0.5]), act=oracle.ACT_SQRELU, probs_at_act=True)
    assert a.tolist() == [[0x4000], [0]]
