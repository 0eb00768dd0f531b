// bi_topk.hip -- deterministic per-row top-k of indexer scores, gfx950.
//
// Sparse-MLA page, commit notes of the deterministic per-row top-k: the
// selected set and its order must not depend on timing (no tie resolution by
// atomics), so the k-th largest score is found exactly on an integer key and
// ties are handed out in ascending column order.
//
//  * Ranking key: -0.0 becomes +0.0, then the fp32 bit pattern b maps to the
//    unsigned value (b has its sign bit set ? ~b : b | 0x80000000).  Unsigned
//    order of this value is the order of the page's monotone int32 key, so
//    every fp32 bit pattern (NaNs included) has a rank.
//  * Validity first: only columns inside the row's window [rs, re) (bounds
//    clamped to [0, cols]) take part; out-of-window lanes never count, never
//    spend the tie budget and are never emitted.
//  * k_eff = min(topk, re - rs).  The k_eff-th largest key T is found by a
//    three-pass radix select over digits of 11, 11 and 10 bits, most
//    significant first: each pass builds a histogram in LDS of the digit of
//    the lanes still matching the digits chosen so far, and keeps the digit
//    where the running rank lands.  Histogram bins are integer counts, so the
//    order in which the LDS atomics land cannot change T (the page's concern
//    is atomics that decide WHICH tied lane wins; here none does).  Each bin
//    has 4 (last pass: 2) copies, picked by lane, so a plateau of equal
//    scores does not serialise a wave's increments on one address.  The three
//    histograms (72 KiB) are cleared once while the row's loads are in
//    flight, and 72 KiB leaves room for two rows per compute unit.
//  * Emission: every lane with key > T and the first `budget` lanes (in
//    column order) with key == T, where budget = k_eff - #(key > T).  A
//    lane's output slot is #(key > T before it) + min(#(key == T before it),
//    budget), from one exclusive scan, so the output is ascending in column
//    and row-local (column - rs); slots k_eff .. topk-1 get -1.
//
// One workgroup of 1024 threads per row; thread t owns the 8 consecutive
// columns [8t, 8t + 8), which bounds a row at 8192 columns (the envelope the
// page's fast path is gated to).
#include <hip/hip_runtime.h>

#include "bi_device.h"
#include "bi_topk.h"

namespace bi {

namespace {

constexpr int kThreads = 1024;
constexpr int kPerThread = 8;
constexpr int kWaves = kThreads / 64;
static_assert(kThreads * kPerThread == kTopkMaxCols, "row envelope");

// Radix digits (most significant first) and LDS copies of each histogram.
constexpr int kShift0 = 21, kBins0 = 2048, kCopies0 = 4;   // key bits 31..21
constexpr int kShift1 = 10, kBins1 = 2048, kCopies1 = 4;   // key bits 20..10
constexpr int kShift2 = 0, kBins2 = 1024, kCopies2 = 2;    // key bits 9..0

__device__ __forceinline__ uint32_t rank_bits(float v)
{
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u)
        b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}


// Inclusive prefix sum over the workgroup's threads in thread order.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum, int lane, int wave)
{
    v = wave_incl_scan(v, lane);
    if (lane == 63)
        wsum[wave] = v;
    __syncthreads();
    const uint4* w4 = reinterpret_cast<const uint4*>(wsum);
    uint32_t base = 0;
#pragma unroll
    for (int q = 0; q < kWaves / 4; ++q) {
        const uint4 t = w4[q];
        base += (4 * q + 0 < wave ? t.x : 0u) + (4 * q + 1 < wave ? t.y : 0u) + (4 * q + 2 < wave ? t.z : 0u) +
                (4 * q + 3 < wave ? t.w : 0u);
    }
    return base + v;
}

template <int COPIES>
__device__ __forceinline__ uint32_t bin_count(const uint32_t* hist, int bin)
{
    if constexpr (COPIES == 8) {
        const uint4 a = reinterpret_cast<const uint4*>(hist)[2 * bin];
        const uint4 b = reinterpret_cast<const uint4*>(hist)[2 * bin + 1];
        return a.x + a.y + a.z + a.w + b.x + b.y + b.z + b.w;
    } else if constexpr (COPIES == 4) {
        const uint4 h = reinterpret_cast<const uint4*>(hist)[bin];
        return h.x + h.y + h.z + h.w;
    } else {
        const uint2 h = reinterpret_cast<const uint2*>(hist)[bin];
        return h.x + h.y;
    }
}

// One radix pass.  Counts the digit (key >> SHIFT) % BINS of the active lanes
// into `hist` (COPIES copies per bin, by lane), finds the digit d holding the
// rem-th largest active key (#(digit > d) < rem <= #(digit >= d)) with one
// block-wide scan over the bins in descending order, and returns the updated
// prefix and rank through LDS.
template <int SHIFT, int BINS, int COPIES>
__device__ __forceinline__ void radix_pass(uint32_t* hist, uint32_t* wsum, uint32_t* sel,
                                           const uint32_t (&key)[kPerThread], uint32_t& active, uint32_t& prefix,
                                           uint32_t& rem, int tid, int lane, int wave)
{
    constexpr uint32_t kMask = BINS - 1;
    constexpr int kPer = BINS / kThreads;     // bins per thread in the scan: 1 or 2
    static_assert(kPer == 1 || kPer == 2, "bins per thread");
    const int copy = lane & (COPIES - 1);
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
        if ((active >> j) & 1u)
            atomicAdd(&hist[((key[j] >> SHIFT) & kMask) * COPIES + copy], 1u);
    __syncthreads();
    // descending digit order: thread t holds bins BINS-1-kPer*t ... (high first)
    const int bh = BINS - 1 - kPer * tid;
    const uint32_t ch = bin_count<COPIES>(hist, bh);
    const uint32_t cl = kPer == 2 ? bin_count<COPIES>(hist, bh - 1) : 0u;
    const uint32_t ge_l = block_incl_scan(ch + cl, wsum, lane, wave);   // #(digit >= lowest bin held)
    const uint32_t ge_h = ge_l - cl;                                     // #(digit >= bh)
    if (ge_h - ch < rem && rem <= ge_h) {
        sel[0] = prefix | ((uint32_t)bh << SHIFT);
        sel[1] = rem - (ge_h - ch);
    } else if (kPer == 2 && ge_h < rem && rem <= ge_l) {
        sel[0] = prefix | ((uint32_t)(bh - 1) << SHIFT);
        sel[1] = rem - ge_h;
    }
    __syncthreads();
    prefix = sel[0];
    rem = sel[1];
    const uint32_t dsel = (prefix >> SHIFT) & kMask;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
        if (((key[j] >> SHIFT) & kMask) != dsel)
            active &= ~(1u << j);
}

__global__ __launch_bounds__(kThreads) void k_topk_rows(const float* __restrict__ scores, int64_t ld, int cols,
                                                        int vec_ok, const int64_t* __restrict__ row_start,
                                                        const int64_t* __restrict__ row_end, int topk,
                                                        int32_t* __restrict__ out, int64_t ld_out)
{
    // one histogram per pass, all cleared once while the row is in flight
    __shared__ __attribute__((aligned(16))) uint32_t hist0[kBins0 * kCopies0];
    __shared__ __attribute__((aligned(16))) uint32_t hist1[kBins1 * kCopies1];
    __shared__ __attribute__((aligned(16))) uint32_t hist2[kBins2 * kCopies2];
    __shared__ __attribute__((aligned(16))) uint32_t wsum[4][kWaves];
    __shared__ uint32_t sel[2];

    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t s64 = row_start ? row_start[r] : 0;
    const int64_t e64 = row_end ? row_end[r] : cols;
    const int rs = (int)min<int64_t>(max<int64_t>(s64, 0), cols);
    const int re = (int)min<int64_t>(max<int64_t>(e64, 0), cols);
    const int keff = min(topk, max(re - rs, 0));
    int32_t* orow = out + (int64_t)r * ld_out;

    // this thread's window columns [lo, hi) within [c0, c0 + 8)
    const int c0 = tid * kPerThread;
    const int lo = max(c0, rs), hi = min(c0 + kPerThread, re);
    float v[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
        v[j] = 0.f;
    if (lo < hi) {
        const float* p = scores + (int64_t)r * ld + c0;
        if (vec_ok && c0 + kPerThread <= cols) {
            const float4 a = reinterpret_cast<const float4*>(p)[0];
            const float4 b = reinterpret_cast<const float4*>(p)[1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int j = 0; j < kPerThread; ++j)
                if (c0 + j >= lo && c0 + j < hi)
                    v[j] = p[j];
        }
    }
    const uint32_t valid = lo < hi ? ((1u << (hi - c0)) - 1u) ^ ((1u << (lo - c0)) - 1u) : 0u;

    if (keff > 0) {
        {
            uint4* h0 = reinterpret_cast<uint4*>(hist0);
            uint4* h1 = reinterpret_cast<uint4*>(hist1);
            uint4* h2 = reinterpret_cast<uint4*>(hist2);
#pragma unroll
            for (int i = 0; i < kBins0 * kCopies0 / 4 / kThreads; ++i)
                h0[tid + i * kThreads] = uint4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < kBins1 * kCopies1 / 4 / kThreads; ++i)
                h1[tid + i * kThreads] = uint4{0u, 0u, 0u, 0u};
            if (tid < kBins2 * kCopies2 / 4)
                h2[tid] = uint4{0u, 0u, 0u, 0u};
        }
        uint32_t key[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread; ++j)
            key[j] = rank_bits(v[j]);
        __syncthreads();

        // ---- radix select of the keff-th largest key
        uint32_t prefix = 0, rem = (uint32_t)keff, active = valid;
        radix_pass<kShift0, kBins0, kCopies0>(hist0, wsum[0], sel, key, active, prefix, rem, tid, lane, wave);
        radix_pass<kShift1, kBins1, kCopies1>(hist1, wsum[1], sel, key, active, prefix, rem, tid, lane, wave);
        radix_pass<kShift2, kBins2, kCopies2>(hist2, wsum[2], sel, key, active, prefix, rem, tid, lane, wave);
        const uint32_t T = prefix, budget = rem;

        // ---- emission in ascending column order
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j)
            if ((valid >> j) & 1u) {
                ngt += key[j] > T ? 1u : 0u;
                neq += key[j] == T ? 1u : 0u;
            }
        const uint32_t packed = ngt | (neq << 16);
        const uint32_t excl = block_incl_scan(packed, wsum[3], lane, wave) - packed;
        uint32_t gt_before = excl & 0xFFFFu, eq_before = excl >> 16;
        // the selection is gathered in LDS (the first histogram is no longer
        // needed) and then written to the row with contiguous stores
        uint32_t* stage = hist0;
        static_assert(kBins0 * kCopies0 >= kTopkMaxCols, "staging fits the first histogram");
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            if (!((valid >> j) & 1u))
                continue;
            // slots are < keff by construction; the bound only keeps a
            // broken count from writing outside the staging area
            const uint32_t local = (uint32_t)(c0 + j - rs);
            if (key[j] > T) {
                const uint32_t slot = gt_before + min(eq_before, budget);
                if (slot < (uint32_t)keff)
                    stage[slot] = local;
                ++gt_before;
            } else if (key[j] == T) {
                const uint32_t slot = gt_before + eq_before;
                if (eq_before < budget && slot < (uint32_t)keff)
                    stage[slot] = local;
                ++eq_before;
            }
        }
        __syncthreads();
        for (int i = tid; i < keff; i += kThreads)
            orow[i] = (int32_t)stage[i];
    }
    for (int i = keff + tid; i < topk; i += kThreads)
        orow[i] = -1;
}

}  // namespace

hipError_t launch_topk_rows(const float* scores, int64_t ld, int64_t rows, int64_t cols,
                            const int64_t* row_start, const int64_t* row_end, int64_t topk, int32_t* out,
                            int64_t ld_out, hipStream_t stream)
{
    const int vec_ok = ((reinterpret_cast<uintptr_t>(scores) & 15u) == 0 && ld % 4 == 0) ? 1 : 0;
    k_topk_rows<<<dim3((unsigned)rows), kThreads, 0, stream>>>(scores, ld, (int)cols, vec_ok, row_start, row_end,
                                                               (int)topk, out, ld_out);
    return hipGetLastError();
}

}  // namespace bi
