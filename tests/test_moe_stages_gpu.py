"""Stage-wise parity of the MoE layer: the GPU's storage points against the
oracle's, read from the layer's own workspace after a call.

Fused-MoE page, "What's included" and the strict-review summary: the layer's
storage points are the bf16 first projection h, the bf16 activation a (the
routing probability applied there, one rounding) and the per-slot fp32 down
projection y_j; the top-k sum runs in slot order.  With the oracle run on
the GPU's own expert ids, every stage is checked on its own inputs:

* h: the expert GEMM carries out the recipe of its (bf16, rows, H) key, so
  the GPU's h is the library's bf16 linear of the token's row with the
  expert's weight.  The GPU rounds an fp32 sum, the oracle the exact one:
  |h_gpu - exact| <= (H-1) u sum|x w| + half a bf16 ulp of h_gpu, and
  >= 99 % of the values equal (a sum that cancels to near zero can differ
  by several bf16 ulps and still be right).
* a: the GPU's activation against the oracle's activation step applied to
  the GPU's own h and probability: one rounding apart at most, >= 99 % equal.
  (End to end a flip in h can move a by several ulps -- SiLU's relative
  slope grows like |g| for negative g -- so a is only held to >= 99 % equal
  against the oracle's own a.)
* y_j: the GPU's fp32 partial against the exact down projection of the
  GPU's own a: within (I-1) u sum|a w2| (u = 2^-24, the rounding bound of an
  I-term fp32 sum in any order; bf16 x bf16 products are exact in fp32),
  and within the fp32 linear bar atol 2e-3 / rtol 1e-4.
* y: the oracle's top-k-sum step applied to the GPU's own partials and
  probabilities reproduces the GPU output bit for bit; and end to end,
  |y_gpu - y_oracle| <= sum_j [ sum_i |a_gpu - a_oracle|_i |w2|_i
  + (I-1) u sum_i |a_gpu w2|_i ] (+ probability and final roundings),
  per output element from the measured a differences.

The test prints the flip statistics the scalar output bars of the other MoE
tests are set from (tests/moe_bars.py).
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import banner, dev, host

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def bi():
    import deterministic_persistent_gemm_amd as m
    return m


def bf16_ordered(b):
    """Monotone integer image of bf16 bit patterns (finite values): adjacent
    representable values differ by 1."""
    b = np.asarray(b, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_stages(bi, w, x, topk, b_router=None, act=None, probs_at_act=True, apply_weights=False, acc_fp64=True):
    import torch
    M, H = x.shape
    E = w.w_router.shape[0]
    I = w.w2.shape[2]
    sq = act == "sqrelu"
    w1 = np.ascontiguousarray(w.w13[:, :I, :]) if sq else w.w13
    L = bi.moe_layout(M, H, E, I, topk)
    ws = bi.alloc_workspace(L["total"], "cuda")
    xd, wr, w1d, w2d = dev(x), dev(w.w_router), dev(w1), dev(w.w2)
    bd = None if b_router is None else dev(b_router)
    if act is None:
        y, ids, probs = bi.bi_moe_grouped_gemm(xd, wr, bd, w1d, w2d, topk, ws=ws)
    else:
        y, ids, probs = bi.bi_moe_grouped_gemm_ex(xd, wr, bd, w1d, w2d, topk,
                                                  activation=bi.BI_ACT_SQRELU if sq else bi.BI_ACT_SWIGLU,
                                                  probs_at_activation=probs_at_act, apply_weights=apply_weights,
                                                  acc_fp64=acc_fp64, ws=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    P = M * topk
    srt = raw[L["sorted"]:L["sorted"] + 4 * P].view(np.int32)
    act_sorted = raw[L["act"]:L["act"] + 2 * P * I].view(np.uint16).reshape(P, I)
    part = raw[L["part"]:L["part"] + 4 * P * H].view(np.float32).reshape(P, H)
    assert np.array_equal(np.sort(srt), np.arange(P)), "sorted pair list is not a permutation"
    a_gpu = np.empty((P, I), np.uint16)
    a_gpu[srt] = act_sorted
    ids = host(ids)
    # the GPU's first projection: the library's bf16 linear of each token's
    # row with the chosen expert's weight (same key, same recipe)
    R1 = w1.shape[1]
    h_gpu = np.empty((P, R1), np.uint16)
    h_exact = np.empty((P, R1))
    h_abs = np.empty((P, R1))
    flat = ids.reshape(P)
    xf = bf16_f64(x)
    for e in np.unique(flat):
        pairs = np.nonzero(flat == e)[0]
        he = bi.bi_linear_bf16(xd[torch.from_numpy(pairs // topk).cuda()].contiguous(), w1d[int(e)].t())
        h_gpu[pairs] = host(he)
        w1e = bf16_f64(w1[e])
        h_exact[pairs] = xf[pairs // topk] @ w1e.T
        h_abs[pairs] = np.abs(xf[pairs // topk]) @ np.abs(w1e).T
    yo, _, po, _, ho, ao, parto = oracle.moe_stages(
        x, w.w_router, b_router, w1, w.w2, topk, act=oracle.ACT_SQRELU if sq else oracle.ACT_SWIGLU,
        probs_at_act=probs_at_act, apply_weights=apply_weights, acc_fp64=acc_fp64, ids=ids)
    return dict(y=host(y), ids=ids, probs=host(probs), a_gpu=a_gpu, h_gpu=h_gpu, h_exact=h_exact, h_abs=h_abs,
                K1=H, part=part, yo=yo, po=po,
                ao=ao.reshape(P, I), ho=ho.reshape(P, R1), parto=parto.reshape(P, H), M=M, H=H, I=I,
                topk=topk, act=oracle.ACT_SQRELU if sq else oracle.ACT_SWIGLU, probs_at_act=probs_at_act,
                apply_weights=apply_weights, acc_fp64=acc_fp64)


def check_stages(w, r, label, weighted=False, fp32_sum=False):
    M, H, I, topk = r["M"], r["H"], r["I"], r["topk"]
    P = M * topk
    a_gpu, ao = r["a_gpu"], r["ao"]
    p_gpu = r["probs"].reshape(P).astype(np.float64)
    # 1. first projection: the GPU's h against the exact sum and the oracle's h
    dh = np.abs(bf16_ordered(r["h_gpu"]) - bf16_ordered(r["ho"]))
    assert (dh != 0).sum() <= 0.01 * dh.size, f"{label}: {(dh != 0).sum()} of {dh.size} h values differ"
    hx, hb = r["h_exact"], r["h_abs"]
    hg = bf16_f64(r["h_gpu"])
    half_ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(hg), 1e-38))[1] - 9)
    hbound = (r["K1"] - 1) * U32 * hb * 1.0001 + half_ulp
    assert np.all(np.abs(hg - hx) <= hbound), \
        f"{label}: h outside the fp32-sum bound ({float((np.abs(hg - hx) / hbound).max()):.3f}x)"
    # 2. activation on the GPU's own h and probability: one rounding apart
    a_iso = oracle.moe_activation(r["h_gpu"], p_gpu, act=r["act"], probs_at_act=r["probs_at_act"])
    di = np.abs(bf16_ordered(a_gpu) - bf16_ordered(a_iso))
    assert di.max() <= 1, f"{label}: activation more than one bf16 ulp from the step on the GPU's h ({di.max()})"
    assert (di != 0).sum() <= 0.01 * di.size, f"{label}: {(di != 0).sum()} of {di.size} activations differ"
    # end to end against the oracle's own a
    d = np.abs(bf16_ordered(a_gpu) - bf16_ordered(ao))
    flips = d != 0
    n_flip = int(flips.sum())
    assert n_flip <= 0.01 * a_gpu.size, f"{label}: {n_flip} of {a_gpu.size} activations differ"
    # 2. slot partials against the exact projection of the GPU's own a
    ag = bf16_f64(a_gpu)
    dA = np.abs(ag - bf16_f64(ao))
    e_of = r["ids"].reshape(P)
    exact = np.empty((P, H))
    absum = np.empty((P, H))
    dsum = np.empty((P, H))
    for e in np.unique(e_of):
        rows = np.nonzero(e_of == e)[0]
        w2e = bf16_f64(w.w2[e])                                  # [H, I]
        exact[rows] = ag[rows] @ w2e.T
        absum[rows] = np.abs(ag[rows]) @ np.abs(w2e).T
        dsum[rows] = dA[rows] @ np.abs(w2e).T
    part_bound = (I - 1) * U32 * absum * 1.0001 + 1e-300
    perr = np.abs(r["part"].astype(np.float64) - exact)
    assert np.all(perr <= part_bound), f"{label}: slot partial outside the fp32 sum bound " \
                                       f"(worst {float((perr / part_bound).max()):.3f}x)"
    assert np.all(perr <= 2e-3 + 1e-4 * np.abs(exact)), label
    # 4. the top-k sum of the GPU's own partials and probabilities
    y_iso = oracle.moe_combine(r["part"].astype(np.float64).reshape(M, topk, H), p_gpu.reshape(M, topk),
                               apply_weights=r["apply_weights"], acc_fp64=r["acc_fp64"])
    assert np.array_equal(r["y"].view(np.uint32), y_iso.view(np.uint32)), \
        f"{label}: output differs from the top-k sum of the GPU's own partials"
    # 5. end to end, bounded per element by what the measured a
    # differences and the partials' rounding can move it
    wj = r["po"].reshape(P) if weighted else np.ones(P)
    per_pair = (dsum + part_bound) * np.abs(wj)[:, None]
    bound = per_pair.reshape(M, topk, H).sum(axis=1)
    yo = r["yo"].astype(np.float64)
    if weighted:
        # the GPU weights with its fp32 probability, the oracle with binary64
        pdiff = np.abs(r["probs"].reshape(P).astype(np.float64) - r["po"].reshape(P))
        bound = bound + (np.abs(exact) * pdiff[:, None]).reshape(M, topk, H).sum(axis=1)
    if fp32_sum:
        # fp32 slot-order sum of fp32 terms: one rounding per add and per
        # weighted product, on both sides
        mag = (np.abs(exact) * np.abs(wj)[:, None]).reshape(M, topk, H).sum(axis=1)
        bound = bound + 2 * (2 * topk + 1) * U32 * (mag + bound)
    bound = bound + U32 * (np.abs(yo) + np.abs(r["y"].astype(np.float64))) + 1e-30
    yerr = np.abs(r["y"].astype(np.float64) - yo)
    worst = float((yerr / bound).max())
    assert np.all(yerr <= bound), f"{label}: output outside the stage-derived bound ({worst:.3f}x)"
    rms = float(np.sqrt(np.mean(yo ** 2)))
    flips_per_pair = flips.sum(axis=1)
    flips_per_token = flips.reshape(M, topk, I).sum(axis=(1, 2))
    stat = {"pairs": P, "activations": int(a_gpu.size), "h_flips": int((dh != 0).sum()), "h_max_ulps": int(dh.max()),
            "a_flips_isolated": int((di != 0).sum()), "flips": n_flip, "max_ulps": int(d.max()),
            "flip_rate": n_flip / a_gpu.size, "max_flips_pair": int(flips_per_pair.max()),
            "max_flips_token": int(flips_per_token.max()),
            "max_err_over_rms": float(yerr.max() / rms) if rms > 0 else 0.0,
            "max_flip_shift_over_rms": float((dsum * np.abs(wj)[:, None]).reshape(M, topk, H).sum(axis=1).max() / rms)
            if rms > 0 else 0.0,
            "worst_bound_use": worst}
    print(f"{label}: {stat}")
    return stat


@pytest.mark.parametrize("M", wl.MOE_M_SWEEP)
def test_qwen_shape_storage_points(bi, M):
    w = wl.moe_weights(0)
    banner(f"moe stages Qwen3 shape M={M}")
    x = wl.moe_batch(M, w).x
    r = run_stages(bi, w, x, wl.MOE_TOPK)
    check_stages(w, r, f"qwen M={M}")


@pytest.mark.parametrize("E,topk", [(32, 4), (256, 8), (1024, 6)])
@pytest.mark.parametrize("M", [1, 5, 70, 200])
def test_small_shape_storage_points(bi, M, E, topk):
    w = wl.moe_weights(5, H=256, E=E, I=64)
    b = (np.random.default_rng(9).standard_normal(E) * 0.05).astype(np.float32)
    banner(f"moe stages small shape E={E} top-{topk} M={M}")
    x = wl.moe_batch(M, w).x
    r = run_stages(bi, w, x, topk, b_router=b)
    check_stages(w, r, f"small E={E} top-{topk} M={M}")


@pytest.mark.parametrize("v", [("sqrelu", False, True, False), ("sqrelu", False, False, True)])
@pytest.mark.parametrize("M", [1, 16, 64, 256])
def test_qwen_shape_squared_relu_storage_points(bi, M, v):
    act, pa, aw, f64 = v
    w = wl.moe_weights(0)
    banner(f"moe stages Qwen3 shape squared-ReLU {v} M={M}")
    x = wl.moe_batch(M, w).x
    r = run_stages(bi, w, x, wl.MOE_TOPK, act=act, probs_at_act=pa, apply_weights=aw, acc_fp64=f64)
    check_stages(w, r, f"qwen sqrelu aw={aw} f64={f64} M={M}", weighted=aw, fp32_sum=not f64)


@pytest.mark.parametrize("act,pa,aw,f64", [("sqrelu", True, False, True), ("sqrelu", False, True, False),
                                           ("swiglu", False, True, True), ("swiglu", False, False, False)])
def test_variant_storage_points(bi, act, pa, aw, f64):
    w = wl.moe_weights(5, H=256, E=32, I=64)
    banner(f"moe stages variant {act} probs_at_act={pa} apply_weights={aw} acc_fp64={f64}")
    x = wl.moe_batch(70, w).x
    r = run_stages(bi, w, x, 4, act=act, probs_at_act=pa, apply_weights=aw, acc_fp64=f64)
    check_stages(w, r, f"{act} pa={pa} aw={aw} f64={f64}", weighted=aw, fp32_sum=not f64)
