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
//    has several copies, picked by lane, so a plateau of equal scores does
//    not serialise a wave's increments on one address.  The three histograms
//    are cleared once while the row's loads are in flight.
//  * Emission: every lane with key > T and the first `budget` lanes (in
//    column order) with key == T, where budget = k_eff - #(key > T).  A
//    lane's output slot is #(key > T before it) + min(#(key == T before it),
//    budget), from one exclusive scan, so the output is ascending in column
//    and row-local (column - rs); slots k_eff .. topk-1 get -1.
//
// One workgroup per row; thread t owns PT consecutive columns [PT t, PT t +
// PT), NT x PT = 8192 columns (the envelope the page's fast path is gated
// to).  Two forms carry out the same selection: 1024 threads with 8 columns
// each and 4/4/2 histogram copies (72 KiB of LDS, two rows per compute unit:
// the shortest time per row, for decode batches), and 512 threads with 16
// columns each and 2/2/1 copies (36 KiB, four rows per compute unit: more
// rows in flight, for prefill batches).
#include <hip/hip_runtime.h>

#include "bi_device.h"
#include "bi_topk.h"

namespace bi {

namespace {

template <int NT>
struct TopkCfg;
template <>
struct TopkCfg<1024> {
    static constexpr int kC0 = 4, kC1 = 4, kC2 = 2;
};
template <>
struct TopkCfg<512> {
    static constexpr int kC0 = 2, kC1 = 2, kC2 = 1;
};

constexpr int kShift0 = 21, kBins0 = 2048;   // key bits 31..21
constexpr int kShift1 = 10, kBins1 = 2048;   // key bits 20..10
constexpr int kShift2 = 0, kBins2 = 1024;    // key bits 9..0

__device__ __forceinline__ uint32_t rank_bits(float v)
{
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u)
        b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive scan over the workgroup: the wave scan (wave_incl_scan), then the
// wave totals of the lower waves added from LDS.
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum, int lane, int wave)
{
    constexpr int kWaves = NT / 64;
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
    if constexpr (COPIES == 4) {
        const uint4 h = reinterpret_cast<const uint4*>(hist)[bin];
        return h.x + h.y + h.z + h.w;
    } else if constexpr (COPIES == 2) {
        const uint2 h = reinterpret_cast<const uint2*>(hist)[bin];
        return h.x + h.y;
    } else {
        return hist[bin];
    }
}

// One radix pass.  Counts the digit (key >> SHIFT) % BINS of the active lanes
// into `hist` (COPIES copies per bin, by lane), finds the digit d holding the
// rem-th largest active key (#(digit > d) < rem <= #(digit >= d)) with one
// block-wide scan over the bins in descending order (thread t holds the
// BINS/NT bins just below BINS - BINS/NT * t), and returns the updated prefix
// and rank through LDS.
template <int NT, int PT, int SHIFT, int BINS, int COPIES>
__device__ __forceinline__ void radix_pass(uint32_t* hist, uint32_t* wsum, uint32_t* sel, const uint32_t (&key)[PT],
                                           uint32_t& active, uint32_t& prefix, uint32_t& rem, int tid, int lane,
                                           int wave)
{
    constexpr uint32_t kMask = BINS - 1;
    constexpr int kPer = BINS / NT;           // bins per thread in the scan
    static_assert(kPer >= 1 && kPer * NT == BINS, "bins per thread");
    const int copy = lane & (COPIES - 1);
#pragma unroll
    for (int j = 0; j < PT; ++j)
        if ((active >> j) & 1u)
            atomicAdd(&hist[((key[j] >> SHIFT) & kMask) * COPIES + copy], 1u);
    __syncthreads();
    const int bh = BINS - 1 - kPer * tid;     // highest bin held, then bh-1, ...
    uint32_t c[kPer], total = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        c[i] = bin_count<COPIES>(hist, bh - i);
        total += c[i];
    }
    // #(digit >= bh - i) = #(digit > bh) + c[0] + ... + c[i]
    uint32_t ge = block_incl_scan<NT>(total, wsum, lane, wave) - total;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const uint32_t ge_i = ge + c[i];
        if (ge < rem && rem <= ge_i) {
            sel[0] = prefix | ((uint32_t)(bh - i) << SHIFT);
            sel[1] = rem - ge;
        }
        ge = ge_i;
    }
    __syncthreads();
    prefix = sel[0];
    rem = sel[1];
    const uint32_t dsel = (prefix >> SHIFT) & kMask;
#pragma unroll
    for (int j = 0; j < PT; ++j)
        if (((key[j] >> SHIFT) & kMask) != dsel)
            active &= ~(1u << j);
}

template <int NT>
__global__ __launch_bounds__(NT) void k_topk_rows(const float* __restrict__ scores, int64_t ld, int cols, int vec_ok,
                                                  const int64_t* __restrict__ row_start,
                                                  const int64_t* __restrict__ row_end, int topk,
                                                  int32_t* __restrict__ out, int64_t ld_out)
{
    constexpr int PT = kTopkMaxCols / NT;     // columns per thread
    constexpr int C0 = TopkCfg<NT>::kC0, C1 = TopkCfg<NT>::kC1, C2 = TopkCfg<NT>::kC2;
    static_assert(NT * PT == kTopkMaxCols && PT <= 16 && PT % 4 == 0, "row envelope");
    // one histogram per pass, all cleared once while the row is in flight;
    // the first two are one array, which later stages the selection
    constexpr int kH0 = kBins0 * C0, kH1 = kBins1 * C1, kH2 = kBins2 * C2;
    static_assert(kH0 + kH1 >= kTopkMaxCols, "staging fits the first two histograms");
    __shared__ __attribute__((aligned(16))) uint32_t hist01[kH0 + kH1];
    __shared__ __attribute__((aligned(16))) uint32_t hist2[kH2];
    __shared__ __attribute__((aligned(16))) uint32_t wsum[4][NT / 64];
    __shared__ uint32_t sel[2];
    uint32_t* hist0 = hist01;
    uint32_t* hist1 = hist01 + kH0;

    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t s64 = row_start ? row_start[r] : 0;
    const int64_t e64 = row_end ? row_end[r] : cols;
    const int rs = (int)min<int64_t>(max<int64_t>(s64, 0), cols);
    const int re = (int)min<int64_t>(max<int64_t>(e64, 0), cols);
    const int keff = min(topk, max(re - rs, 0));
    int32_t* orow = out + (int64_t)r * ld_out;

    // this thread's window columns [lo, hi) within [c0, c0 + PT)
    const int c0 = tid * PT;
    const int lo = max(c0, rs), hi = min(c0 + PT, re);
    float v[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j)
        v[j] = 0.f;
    if (lo < hi) {
        const float* p = scores + (int64_t)r * ld + c0;
        if (vec_ok && c0 + PT <= cols) {
#pragma unroll
            for (int q = 0; q < PT / 4; ++q) {
                const float4 a = reinterpret_cast<const float4*>(p)[q];
                v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < PT; ++j)
                if (c0 + j >= lo && c0 + j < hi)
                    v[j] = p[j];
        }
    }
    const uint32_t valid = lo < hi ? ((1u << (hi - c0)) - 1u) ^ ((1u << (lo - c0)) - 1u) : 0u;

    if (keff > 0) {
        {
            uint4* h01 = reinterpret_cast<uint4*>(hist01);
            uint4* h2 = reinterpret_cast<uint4*>(hist2);
#pragma unroll
            for (int i = 0; i < (kH0 + kH1) / 4 / NT; ++i)
                h01[tid + i * NT] = uint4{0u, 0u, 0u, 0u};
            if (tid < kH2 / 4)
                h2[tid] = uint4{0u, 0u, 0u, 0u};
        }
        uint32_t key[PT];
#pragma unroll
        for (int j = 0; j < PT; ++j)
            key[j] = rank_bits(v[j]);
        __syncthreads();

        // ---- radix select of the keff-th largest key
        uint32_t prefix = 0, rem = (uint32_t)keff, active = valid;
        radix_pass<NT, PT, kShift0, kBins0, C0>(hist0, wsum[0], sel, key, active, prefix, rem, tid, lane, wave);
        radix_pass<NT, PT, kShift1, kBins1, C1>(hist1, wsum[1], sel, key, active, prefix, rem, tid, lane, wave);
        radix_pass<NT, PT, kShift2, kBins2, C2>(hist2, wsum[2], sel, key, active, prefix, rem, tid, lane, wave);
        const uint32_t T = prefix, budget = rem;

        // ---- emission in ascending column order
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int j = 0; j < PT; ++j)
            if ((valid >> j) & 1u) {
                ngt += key[j] > T ? 1u : 0u;
                neq += key[j] == T ? 1u : 0u;
            }
        const uint32_t packed = ngt | (neq << 16);
        const uint32_t excl = block_incl_scan<NT>(packed, wsum[3], lane, wave) - packed;
        uint32_t gt_before = excl & 0xFFFFu, eq_before = excl >> 16;
        // the selection is gathered in LDS (the first two histograms are no
        // longer needed) and then written to the row with contiguous stores
        uint32_t* stage = hist01;
#pragma unroll
        for (int j = 0; j < PT; ++j) {
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
        for (int i = tid; i < keff; i += NT)
            orow[i] = (int32_t)stage[i];
    }
    for (int i = keff + tid; i < topk; i += NT)
        orow[i] = -1;
}

}  // namespace

hipError_t launch_topk_rows(const float* scores, int64_t ld, int64_t rows, int64_t cols,
                            const int64_t* row_start, const int64_t* row_end, int64_t topk, int32_t* out,
                            int64_t ld_out, hipStream_t stream)
{
    const int vec_ok = ((reinterpret_cast<uintptr_t>(scores) & 15u) == 0 && ld % 4 == 0) ? 1 : 0;
    if (rows >= kTopkWideRows)
        k_topk_rows<512><<<dim3((unsigned)rows), 512, 0, stream>>>(scores, ld, (int)cols, vec_ok, row_start,
                                                                   row_end, (int)topk, out, ld_out);
    else
        k_topk_rows<1024><<<dim3((unsigned)rows), 1024, 0, stream>>>(scores, ld, (int)cols, vec_ok, row_start,
                                                                     row_end, (int)topk, out, ld_out);
    return hipGetLastError();
}

}  // namespace bi
