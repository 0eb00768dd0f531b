"""The C ABI on the host: exports, validation, error codes, recipe purity.

All checks here run before the library touches the GPU, so they need none.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bi.h")

bi = pytest.importorskip("deterministic_persistent_gemm_amd")
L = bi.lib()

FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced by validation
NULL = None


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(bi_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"bi_linear_f32", "bi_linear_bf16", "bi_moe_grouped_gemm", "bi_describe_recipe",
            "bi_linear_workspace_size", "bi_moe_workspace_size", "bi_status_str",
            "bi_lab_linear", "bi_negctl_linear_f32"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in bi.h but not exported"


def test_describe_recipe_takes_no_m():
    src = open(HEADER).read()
    m = re.search(r"bi_status_t bi_describe_recipe\(([^)]*)\)", src)
    params = [p.strip() for p in m.group(1).split(",")]
    assert len(params) == 4 and not any(re.search(r"\bM\b", p) for p in params)


def test_recipe_is_a_function_of_the_key():
    r1 = bi.bi_describe_recipe(bi.BI_F32, 256, 4096).as_dict()
    r2 = bi.bi_describe_recipe(bi.BI_F32, 256, 4096).as_dict()
    assert r1 == r2
    assert r1["mfma"] == bi.BI_MFMA_F32_16X16X4_F32 and r1["block_k"] == 128 and r1["bias_last"] == 1
    rb = bi.bi_describe_recipe(bi.BI_BF16, 4096, 4096).as_dict()
    assert rb["mfma"] == bi.BI_MFMA_F32_16X16X32_BF16 and rb["block_k"] == 4096   # fully chained
    # keys whose K is not a multiple of the tile width fall back to one chain
    assert bi.bi_describe_recipe(bi.BI_BF16, 2048, 768).block_k == 768
    # narrower bf16 keys (the MoE gate|up projection) use 512-k tile partials
    assert bi.bi_describe_recipe(bi.BI_BF16, 1536, 2048).block_k == 512
    assert bi.bi_describe_recipe(bi.BI_F32, 32, 256).block_k == 128


@pytest.mark.parametrize("N,K", [(0, 256), (15, 256), (32, 48), (32, 0), (17, 4096)])
def test_unsupported_keys(N, K):
    r = bi.Recipe()
    assert L.bi_describe_recipe(bi.BI_F32, N, K, ctypes.byref(r)) == bi.BI_EUNSUPPORTED


def test_unknown_dtype_and_null_out():
    r = bi.Recipe()
    assert L.bi_describe_recipe(7, 256, 4096, ctypes.byref(r)) == bi.BI_EINVAL
    assert L.bi_describe_recipe(bi.BI_F32, 256, 4096, None) == bi.BI_EINVAL


def call_f32(x=FAKE, ldx=4096, w=FAKE, ldw=4096, b=NULL, y=FAKE, ldy=256, M=1, N=256, K=4096,
             ws=NULL, ws_bytes=0):
    return L.bi_linear_f32(x, ldx, w, ldw, b, y, ldy, M, N, K, ws, ws_bytes, None)


def test_m_zero_is_ok_and_enqueues_nothing():
    assert call_f32(M=0) == bi.BI_OK
    assert call_f32(M=0, x=NULL, w=NULL, y=NULL) == bi.BI_OK


@pytest.mark.parametrize("kw", [dict(x=NULL), dict(w=NULL), dict(y=NULL), dict(M=-1),
                                dict(ldx=100), dict(ldw=4095), dict(ldy=100),
                                dict(x=ctypes.c_void_p(0x10004)), dict(w=ctypes.c_void_p(0x10008)),
                                dict(ldx=4097)])
def test_invalid_arguments(kw):
    assert call_f32(**kw) == bi.BI_EINVAL


def test_unsupported_shape_is_an_error_not_a_fallback():
    assert call_f32(N=250, ldy=256) == bi.BI_EUNSUPPORTED
    assert call_f32(K=4001, ldx=4096, ldw=4096) == bi.BI_EUNSUPPORTED


def lab_call(path, ws=NULL, ws_bytes=0, M=1):
    r = bi.bi_describe_recipe(bi.BI_F32, 256, 4096)
    return L.bi_lab_linear(FAKE, 4096, FAKE, 4096, None, FAKE, bi.BI_F32, 256, M, 256, 4096,
                           ctypes.byref(r), path, ws, ws_bytes, None)


def lab_ws(path, M):
    r = bi.bi_describe_recipe(bi.BI_F32, 256, 4096)
    return L.bi_lab_workspace_size(ctypes.byref(r), path, M, 256, 4096)


def test_workspace_required_and_sized():
    # the two-launch decode path keeps its tile partials in the workspace
    need = lab_ws(bi.BI_PATH_DECODE, 1)
    # the counter region every workspace starts with, then N tiles x k tiles
    # x 64 lanes x f32x4
    assert need == bi.WS_COUNTER_BYTES + 16 * 32 * 64 * 16
    # the XCD hand-over decode keeps the same partials and its counters in
    # that region
    assert lab_ws(bi.BI_PATH_DECODE_XCD, 1) == need
    assert lab_call(bi.BI_PATH_DECODE_XCD) == bi.BI_EWORKSPACE
    assert lab_call(bi.BI_PATH_DECODE_XCD, ws=FAKE, ws_bytes=need - 1) == bi.BI_EWORKSPACE
    assert lab_call(bi.BI_PATH_DECODE) == bi.BI_EWORKSPACE
    assert lab_call(bi.BI_PATH_DECODE, ws=FAKE, ws_bytes=need - 1) == bi.BI_EWORKSPACE
    # ... growing with M
    sizes = [lab_ws(bi.BI_PATH_DECODE, m) for m in (1, 16, 17, 64, 128)]
    assert sizes == sorted(sizes) and sizes[0] < sizes[-1]
    # the one-launch decode path folds in LDS and the persistent path keeps
    # its accumulators in registers: neither needs a workspace
    assert lab_ws(bi.BI_PATH_DECODE_WG, 1) == 0 and lab_ws(bi.BI_PATH_PERSISTENT, 1) == 0
    assert L.bi_linear_workspace_size(bi.BI_F32, 4096, 256, 4096) == 0
    # what the production entry asks for is what it checks
    for m in (1, 17, 128, 129):
        need = L.bi_linear_workspace_size(bi.BI_F32, m, 256, 4096)
        if need:
            assert call_f32(M=m, ws=FAKE, ws_bytes=need - 1) == bi.BI_EWORKSPACE


def test_bf16_entry_validation():
    f = L.bi_linear_bf16
    assert f(FAKE, 4096, FAKE, 4096, None, FAKE, 5, 4096, 1, 4096, 4096, None, 0, None) == bi.BI_EINVAL
    assert f(FAKE, 4100, FAKE, 4096, None, FAKE, bi.BI_BF16, 4096, 1, 4096, 4096, None, 0, None) == bi.BI_EINVAL
    assert f(FAKE, 4096, FAKE, 4096, None, FAKE, bi.BI_BF16, 4096, 0, 4096, 4096, None, 0, None) == bi.BI_OK


def test_lab_recipe_validation():
    r = bi.bi_describe_recipe(bi.BI_F32, 256, 4096)
    r.block_k = 96                      # does not divide K
    f = L.bi_lab_linear
    args = (FAKE, 4096, FAKE, 4096, None, FAKE, bi.BI_F32, 256, 1, 256, 4096)
    assert f(*args, ctypes.byref(r), bi.BI_PATH_AUTO, None, 0, None) == bi.BI_EUNSUPPORTED
    r = bi.bi_describe_recipe(bi.BI_F32, 256, 4096)
    r.mfma = bi.BI_MFMA_F32_16X16X32_BF16   # instruction must match the operand type
    assert f(*args, ctypes.byref(r), bi.BI_PATH_AUTO, None, 0, None) == bi.BI_EUNSUPPORTED
    r = bi.bi_describe_recipe(bi.BI_F32, 256, 4096)
    assert f(*args, ctypes.byref(r), 9, None, 0, None) == bi.BI_EINVAL
    # the one-launch decode keeps at most 64 tile partials in LDS, and needs two
    r.block_k = 32                      # 128 tile partials
    assert f(*args, ctypes.byref(r), bi.BI_PATH_DECODE_WG, None, 0, None) == bi.BI_EUNSUPPORTED
    r.block_k = 4096                    # fully chained: nothing to fold
    assert f(*args, ctypes.byref(r), bi.BI_PATH_DECODE_WG, None, 0, None) == bi.BI_EUNSUPPORTED
    # tile shapes go with the persistent path only
    assert f(*args, ctypes.byref(r), bi.BI_PATH_DECODE | (3 << 8), None, 0, None) == bi.BI_EINVAL


def test_status_strings():
    for s in range(5):
        assert L.bi_status_str(s).startswith(b"BI_")


def test_indexer_topk_validation():
    f = L.bi_indexer_topk
    args = dict(s=FAKE, ld=8192, rows=4, cols=8192, rs=None, re=None, k=2048, out=FAKE, ldo=2048)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["s"], a["ld"], a["rows"], a["cols"], a["rs"], a["re"], a["k"], a["out"], a["ldo"], None)

    assert call(rows=0) == bi.BI_OK
    assert call(cols=8193, ld=8193) == bi.BI_EUNSUPPORTED      # past the one-workgroup row envelope
    for kw in (dict(k=0), dict(ld=100), dict(ldo=100), dict(rows=-1), dict(out=None),
               dict(s=None), dict(s=ctypes.c_void_p(0x10002)), dict(rs=ctypes.c_void_p(0x10004))):
        assert call(**kw) == bi.BI_EINVAL, kw


def test_moe_options_validation():
    f = L.bi_moe_grouped_gemm_ex
    def call(opt):
        return f(FAKE, FAKE, None, FAKE, FAKE, 4, 256, 32, 64, 4, ctypes.byref(opt), FAKE, FAKE, FAKE, FAKE,
                 1 << 30, None)
    O = bi.MoEOptions
    assert call(O(0, 1, 1, 1)) == bi.BI_EINVAL        # probability applied twice
    assert call(O(2, 1, 0, 1)) == bi.BI_EINVAL        # unknown activation
    assert call(O(1, 0, 2, 1)) == bi.BI_EINVAL        # flags are 0 or 1
    assert call(O(1, 0, 1, -1)) == bi.BI_EINVAL


def test_direct_to_lds_decode_scope():
    # chained bf16 recipes only, up to 64 rows, K a multiple of the phase
    f = L.bi_lab_linear
    def call(dtype, N, K, M, block_k=None):
        r = bi.bi_describe_recipe(dtype, N, K)
        if block_k:
            r.block_k = block_k
        return f(FAKE, K, FAKE, K, None, FAKE, bi.BI_F32, N, M, N, K, ctypes.byref(r), bi.BI_PATH_DECODE_DMA,
                 None, 0, None)
    assert call(bi.BI_F32, 256, 4096, 1, block_k=4096) == bi.BI_EUNSUPPORTED      # fp32
    assert call(bi.BI_BF16, 1536, 2048, 1) == bi.BI_EUNSUPPORTED                  # 512-k tile partials
    assert call(bi.BI_BF16, 4096, 4096, 65) == bi.BI_EUNSUPPORTED                 # more than 4 M tiles
    assert call(bi.BI_BF16, 64, 480, 1, block_k=480) == bi.BI_EUNSUPPORTED        # K not a phase multiple


def test_noalloc_entry_rejects_on_the_host():
    # validation and the scratch-size check come before any HIP call: an
    # unlisted fp32 key whose decode partials (8 M tiles x 256 N tiles x 32 k
    # tiles x 1 KiB at M = 128) exceed the 16 MiB static scratch, bad
    # pointers and pitches; M = 0 is a no-op
    f = L.bi_linear_f32_noalloc
    assert f(FAKE, 4096, FAKE, 4096, None, FAKE, 4096, 128, 4096, 4096, None) == bi.BI_EWORKSPACE
    assert f(None, 4096, FAKE, 4096, None, FAKE, 256, 1, 256, 4096, None) == bi.BI_EINVAL
    assert f(FAKE, 4095, FAKE, 4096, None, FAKE, 256, 1, 256, 4096, None) == bi.BI_EINVAL
    assert f(FAKE, 4096, FAKE, 4096, None, FAKE, 256, 0, 256, 4096, None) == bi.BI_OK


def test_l2_read_probe_rejects_on_the_host():
    # the region must be a power of two from 32 KiB to 2 MiB (one full round
    # of the probe's loads, small enough to stay in one XCD's L2)
    f = L.bi_lab_l2_read
    assert f(FAKE, 3 << 20, 1, FAKE, 256, None) == bi.BI_EINVAL
    assert f(FAKE, 4 << 20, 1, FAKE, 256, None) == bi.BI_EINVAL
    assert f(FAKE, 16 << 10, 1, FAKE, 256, None) == bi.BI_EINVAL
    assert f(FAKE, 1 << 20, 0, FAKE, 256, None) == bi.BI_EINVAL
    assert f(FAKE, 1 << 20, 1, FAKE, 0, None) == bi.BI_EINVAL
    assert f(None, 1 << 20, 1, FAKE, 256, None) == bi.BI_EINVAL
    assert f(FAKE, 1 << 20, 1, None, 256, None) == bi.BI_EINVAL


def test_mfma_rate_probe_rejects_on_the_host():
    # one, two, four or eight accumulator chains per wave; a recipe dtype; an
    # 8-byte aligned output
    f = L.bi_lab_mfma_rate
    for chains in (0, 3, 16, -1):
        assert f(FAKE, bi.BI_F32, chains, 256, 10, None) == bi.BI_EINVAL, chains
    assert f(FAKE, 7, 8, 256, 10, None) == bi.BI_EINVAL
    assert f(FAKE, bi.BI_BF16, 8, 0, 10, None) == bi.BI_EINVAL
    assert f(FAKE, bi.BI_BF16, 8, 256, 0, None) == bi.BI_EINVAL
    assert f(None, bi.BI_F32, 8, 256, 10, None) == bi.BI_EINVAL
    assert f(ctypes.c_void_p(FAKE.value + 4), bi.BI_F32, 8, 256, 10, None) == bi.BI_EINVAL


def _split_ws_model(M, N, K, block_k, code, cus=256):
    # the k split of the ring-fed fp32 tiles as a plain function: the largest
    # power of two S >= 2 with tiles x S <= cus whose parts each hold a whole
    # number of k tile groups (four or two k tiles at a time for 32-row tiles,
    # two for 64-row tiles), a tile count that is a multiple of 8 and at most
    # 128; workspace = counters + tiles x (k tiles - k tiles per part + 1)
    # partial tiles of BM x 32 fp32
    bm = 32 if code == 28 else 64
    tiles = -(-M // bm) * -(-N // 32)
    T, kbpt = K // block_k, block_k // 32
    spt = kbpt // 2
    if tiles % 8 or tiles > 128 or K % 64 or kbpt % 2 or kbpt < (4 if bm == 32 else 2):
        return 0
    best, ks = 0, 2
    while tiles * ks <= cus and ks <= T:
        if T % ks == 0:
            kts = T // ks
            for par in ((4, 2) if bm == 32 else (2,)):
                if kts >= par and kts % par == 0 and ((kts // par) * spt) % 2 == 0:
                    best = ks
                    break
        ks *= 2
    return 0 if not best else bi.WS_COUNTER_BYTES + tiles * (T - T // best + 1) * (bm // 8) * 64 * 16


@pytest.mark.parametrize("N,K,block_k", [(256, 4096, 128), (256, 7168, 256), (128, 4096, 256), (128, 2048, 128),
                                         (96, 1024, 64), (256, 4096, 4096), (512, 3072, 192)])
def test_k_split_plan_and_workspace(N, K, block_k):
    # the planner's k split of tile codes 28 and 29 and the workspace it asks
    # for, against the plain model above, over a range of M (no GPU: 256
    # compute units are assumed, the MI355X count)
    r = bi.bi_describe_recipe(bi.BI_F32, N, K)
    r.block_k = block_k
    split_seen = 0
    for code in (28, 29):
        for M in (1, 5, 16, 31, 32, 33, 64, 96, 100, 128, 200, 256, 300, 512, 777, 1000, 1024, 2048):
            got = L.bi_lab_workspace_size(ctypes.byref(r), bi.BI_PATH_PERSISTENT | (code << 8), M, N, K)
            want = _split_ws_model(M, N, K, block_k, code)
            assert got == want, (code, M, got, want)
            split_seen += want > 0
    if (N, K, block_k) == (256, 4096, 128):
        assert split_seen >= 20
