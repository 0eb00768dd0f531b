// bi_plan.cpp -- the (dtype, N, K) recipe table and the launch planner.
//
// GateLinear page, sections "What" and "A correction to why the key excludes
// M": the persistent-matmul config is keyed on (dtype, N[, K]) and never on M,
// so one config serves every batch size.  Here the key fixes the whole
// numeric recipe; M only chooses between two kernel shapes that carry out the
// same recipe bit for bit.
#include "bi_plan.h"

#include <atomic>

#include <hip/hip_runtime_api.h>

namespace bi {

namespace {

// fp32: tile partials of 128 k (32 instructions of 16x16x4 per partial chain)
// keep the decode kernel's dependent chain short enough to stream the weight
// at HBM speed; the persistent kernel pays one fp32 add per 128 k.
constexpr int kF32BlockK = 128;

// Keys measured by the offline sweeper.  GateLinear page, "Perf" and "Update:
// is the M=4096 cost avoidable?": the config of a key comes from a sweep in
// the production weight.t() layout, keyed on (dtype, N, K) only.
const KeyEntry kTable[] = {
#include "bi_table.inc"
    {-1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0}   // end marker
};
constexpr int kTableSize = (int)(sizeof(kTable) / sizeof(kTable[0])) - 1;

}  // namespace

const KeyEntry* table_lookup(int32_t dtype, int64_t N, int64_t K)
{
    for (int i = 0; i < kTableSize; ++i)
        if (kTable[i].dtype == dtype && kTable[i].N == N && kTable[i].K == K)
            return &kTable[i];
    return nullptr;
}

int table_size() { return kTableSize; }

const KeyEntry* table_entry(int i) { return (i >= 0 && i < kTableSize) ? &kTable[i] : nullptr; }

bi_status_t recipe_for(int32_t dtype, int64_t N, int64_t K, bi_recipe_t* out)
{
    if (!out)
        return BI_EINVAL;
    if (dtype != BI_F32 && dtype != BI_BF16)
        return BI_EINVAL;
    if (N <= 0 || K <= 0)
        return BI_EUNSUPPORTED;
    if (N % 16 != 0 || K % 32 != 0 || N > (int64_t(1) << 30) || K > (int64_t(1) << 30))
        return BI_EUNSUPPORTED;
    bi_recipe_t r{};
    r.dtype = dtype;
    r.k_group = 8;
    r.reduce = BI_R2_TILE_PARTIAL;
    r.bias_last = 1;
    if (dtype == BI_F32) {
        r.mfma = BI_MFMA_F32_16X16X4_F32;
        r.block_k = (K % kF32BlockK == 0) ? kF32BlockK : (int32_t)K;
        r.m_decode_max = 128;
    } else {
        // bf16: one 16x16x32 instruction covers 32 k, so even K = 4096 is a
        // chain of only 128 instructions.  When the N tiles alone fill the
        // chip (N/16 >= 256) the recipe is fully chained: measured on MI355X
        // for (bf16, 4096, 4096) it matches 512-k tile partials at decode
        // (13.7 vs 13.5 us at M=1, one launch instead of two, no workspace)
        // and frees the partial registers large persistent tiles need.  With
        // fewer N tiles (the MoE expert GEMMs) 512-k tile partials let the
        // k reduction spread over more waves.
        r.mfma = BI_MFMA_F32_16X16X32_BF16;
        r.block_k = (N >= 4096 || K % 512 != 0) ? (int32_t)K : 512;
        r.m_decode_max = 64;
    }
    // a measured entry replaces the rule's choices (its block_k must be one
    // the kernels can carry out; an entry that is not is ignored)
    if (const KeyEntry* e = table_lookup(dtype, N, K)) {
        if (e->block_k > 0 && e->block_k % 32 == 0 && K % e->block_k == 0 && e->m_decode_max >= 0) {
            r.block_k = e->block_k;
            r.m_decode_max = e->m_decode_max;
        }
    }
    *out = r;
    return BI_OK;
}

bi_status_t recipe_valid(const bi_recipe_t& r, int64_t N, int64_t K)
{
    if (r.dtype != BI_F32 && r.dtype != BI_BF16)
        return BI_EINVAL;
    const int want_mfma = r.dtype == BI_F32 ? BI_MFMA_F32_16X16X4_F32 : BI_MFMA_F32_16X16X32_BF16;
    if (r.mfma != want_mfma || r.k_group != 8 || r.reduce != BI_R2_TILE_PARTIAL || r.bias_last != 1)
        return BI_EUNSUPPORTED;
    if (N <= 0 || K <= 0 || N % 16 != 0 || K % 32 != 0)
        return BI_EUNSUPPORTED;
    if (r.block_k <= 0 || r.block_k % 32 != 0 || K % r.block_k != 0)
        return BI_EUNSUPPORTED;
    if (r.m_decode_max < 0)
        return BI_EINVAL;
    return BI_OK;
}

int device_cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 256;
    if (dev < 64) {
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0)
            return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev < 64)
        cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

int xcd_m_per_wave(const Plan& p)
{
    if (p.m_per_wave > 0)
        return p.m_per_wave;
    if ((int64_t)p.mtiles * p.ntiles <= kDecodeMaxCounters)
        return 1;
    return decode_m_per_wave(p);
}

bool decode_xcd_ok(const Plan& p)
{
    if (p.tiles_k < 2 || p.ntiles % 8 != 0)
        return false;
    const int mw = xcd_m_per_wave(p);
    const int groups = (p.mtiles + mw - 1) / mw;
    return (int64_t)groups * p.ntiles <= kDecodeMaxCounters;
}

bool tile_code_valid(int dtype, int code)
{
    if (dtype == BI_F32)
        return (code >= 1 && code <= 10) || code == 23 || code == 24 || code == 28 || code == 29;
    return code >= 11 && code <= 22;
}

static Tiling persistent_tiling(const bi_recipe_t& r)
{
    (void)r;
    return Tiling{64, 64, 2, 2};
}

bi_status_t make_plan(const bi_recipe_t& r, int32_t path_req, int64_t M, int64_t N, int64_t K,
                      Plan* plan)
{
    bi_status_t st = recipe_valid(r, N, K);
    if (st != BI_OK)
        return st;
    if (M < 0 || M > (int64_t(1) << 30))
        return BI_EINVAL;
    Plan p{};
    p.recipe = r;
    p.kbpt = r.block_k / 32;
    p.tiles_k = (int)(K / r.block_k);
    p.mtiles = (int)((M + 15) / 16);
    p.ntiles = (int)(N / 16);
    p.tiling = persistent_tiling(r);
    // bits 8..15: a persistent tile shape, or the M tiles per wave of the
    // k-tile-parallel decode paths (experiments only; never the numerics)
    const bool no_split = (path_req & kPathNoSplit) != 0;
    const int tile_code = (path_req >> 8) & 0xff;
    path_req &= 0xff;
    if (tile_code != 0) {
        if (path_req == BI_PATH_PERSISTENT) {
            if (!tile_code_valid(r.dtype, tile_code))
                return BI_EINVAL;
            p.tile_code = tile_code;
        } else if (path_req == BI_PATH_DECODE || path_req == BI_PATH_DECODE_XCD) {
            if (tile_code != 1 && tile_code != 2 && tile_code != 4)
                return BI_EINVAL;
            p.m_per_wave = tile_code;
        } else
            return BI_EINVAL;
    }
    const bool wg_ok = p.tiles_k >= 2 && p.tiles_k <= kDecodeWgMaxTiles;
    if (path_req == BI_PATH_DECODE)
        p.path = kPathDecode;
    else if (path_req == BI_PATH_DECODE_WG) {
        if (!wg_ok)
            return BI_EUNSUPPORTED;
        p.path = kPathDecodeWg;
    } else if (path_req == BI_PATH_DECODE_DMA) {
        if (!decode_dma_ok(p, K))
            return BI_EUNSUPPORTED;
        p.path = kPathDecodeDma;
    } else if (path_req == BI_PATH_DECODE_XCD) {
        if (!decode_xcd_ok(p))
            return BI_EUNSUPPORTED;
        p.path = kPathDecodeXcd;
    } else if (path_req == BI_PATH_PERSISTENT)
        p.path = kPathPersistent;
    else if (path_req == BI_PATH_AUTO) {
        const KeyEntry* e = table_lookup(r.dtype, N, K);
        // The one-launch decode puts a whole output tile's k reduction on one
        // compute unit, which then streams 16 rows x K of W by itself; a
        // compute unit sustains only ~20 GB/s of such loads (measured on
        // MI355X), so it pays only while that slab is small.  Measured per
        // call, cold W: (bf16, 1536, 2048) M=1 6.9 vs 9.1 us two-launch;
        // (fp32, 256, 4096) M=1 13.8 vs 9.6 us.
        const int64_t slab = K * (r.dtype == BI_F32 ? 4 : 2);
        // A fully chained bf16 recipe streams its weight through LDS with
        // direct-to-LDS loads for one chain wave: (bf16, 4096, 4096) M=1
        // 10.8 us against 14.1 us for one wave per N tile.
        const bool dma_ok = decode_dma_ok(p, K);
        if (M > r.m_decode_max)
            p.path = kPathPersistent;
        else if (e && M <= e->m_xcd_max && decode_xcd_ok(p))
            p.path = kPathDecodeXcd;
        else if (e && e->decode_path == BI_PATH_DECODE)
            p.path = kPathDecode;
        else if (e && e->decode_path == BI_PATH_DECODE_WG && wg_ok)
            p.path = kPathDecodeWg;
        else if (e && e->decode_path == BI_PATH_DECODE_DMA && dma_ok)
            p.path = kPathDecodeDma;
        else
            p.path = (wg_ok && slab <= 4096) ? kPathDecodeWg : dma_ok ? kPathDecodeDma : kPathDecode;
        if (p.path == kPathPersistent && e) {
            const int code = M <= e->m_a ? e->tile_a : (M <= e->m_b ? e->tile_b : e->tile_c);
            if (tile_code_valid(r.dtype, code))
                p.tile_code = code;
        }
    }
    else
        return BI_EINVAL;
    // tile partials follow the counter region every workspace starts with
    p.ws_bytes = 0;
    if ((p.path == kPathDecode || p.path == kPathDecodeXcd) && p.tiles_k > 1)
        p.ws_bytes = kDecodeCounterBytes + (size_t)p.mtiles * (size_t)p.ntiles * (size_t)p.tiles_k * 64 * 16;
    // the k-split ring tiles (fp32 operands): the parts' partials
    if (p.path == kPathPersistent && r.dtype == BI_F32 && (p.tile_code == 28 || p.tile_code == 29)) {
        if (no_split) {
            p.tile_code = p.tile_code == 28 ? 23 : 24;
        } else {
            const RingSplit rs = ring_split_plan(p, M, N, K, p.tile_code);
            p.ksplit = rs.ksplit;
            p.ws_bytes = rs.ws_bytes;
        }
    }
    *plan = p;
    return BI_OK;
}

}  // namespace bi
