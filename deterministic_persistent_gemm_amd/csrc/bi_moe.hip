// bi_moe.hip -- batch-invariant MoE layer with gated SwiGLU experts, gfx950.
//
// Fused-MoE page, "What's included" and the strict-review summary: the expert
// GEMMs pin their k reduction (fp32 accumulate, no batch-dependent split, a
// fixed k tile width), routing probabilities are applied at the activation
// with fp32 math and one final bf16 rounding (gate|up half-split), and the
// top-k outputs are added with unit weights in fp64 in a fixed slot order.
// The number of rows routed to each expert never leaves the device.
//
// Pipeline (one stream):
//   router   logits[M,E] = fp32(x) . w_router^T (+b)   linear kernels, key (fp32, E, H)
//   route    softmax over E and top-k per token          one wave per token
//   dispatch stable counting sort of (token, slot) pairs by expert, and the
//            list of 16-row work units                   one workgroup
//   gemm1    act = bf16(silu(bf16(x.Wg^T)) * bf16(x.Wu^T) * p)   key (bf16, 2I, H)
//            or, squared-ReLU, act = bf16(relu(bf16(x.W1^T))^2 [* p]) key (bf16, I, H)
//   gemm2    part[pair] = act . W2^T (fp32)                       key (bf16, H, I)
//   combine  y[m] = fp32(sum_j (double) part[m*topk + j]), or the weighted
//            and/or fp32 forms of the top-k sum
//
// Every row of every GEMM is computed by the same per-element operation
// sequence as the dense linear kernels for that key, so a token's bits do
// not depend on which other tokens share the batch or an expert.
#include <hip/hip_runtime.h>

#include "bi_device.h"
#include "bi_launch.h"
#include "bi_moe.h"
#include "bi_plan.h"

namespace bi {

namespace {

constexpr int kTileRows = 16;     // rows of one MFMA output tile
constexpr int kActNone = 0, kActSwiGLU = 1, kActSqReLU = 2;   // grouped-GEMM epilogues
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 32;

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Workspace layout of one MoE call (offsets in bytes).
struct MoELayout {
    size_t router_ws, logits, offsets, unit_expert, unit_row, nunits, sorted, act, part, total;
    int64_t max_units;
};

// Rows per grouped-GEMM work unit: 32 (two M tiles per wave, each weight
// fragment used twice) once experts average 16 rows or more, else 16.
int unit_rows_for(int64_t M, int64_t E, int64_t topk) { return M * topk >= 16 * E ? 32 : 16; }

MoELayout moe_layout(int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk, size_t router_ws_bytes)
{
    MoELayout L{};
    const int64_t P = M * topk;
    const int64_t U = unit_rows_for(M, E, topk);
    L.max_units = (P + U - 1) / U + (P < E ? P : E);
    size_t o = 0;
    // the router's workspace (counter region, then its tile partials) comes
    // first, so the counter region is the MoE workspace's own
    L.router_ws = o;   o = align256(o + (router_ws_bytes > kDecodeCounterBytes ? router_ws_bytes : kDecodeCounterBytes));
    L.logits = o;      o = align256(o + (size_t)M * E * sizeof(float));
    L.offsets = o;     o = align256(o + (size_t)(E + 1) * sizeof(int32_t));
    L.unit_expert = o; o = align256(o + (size_t)L.max_units * sizeof(int32_t));
    L.unit_row = o;    o = align256(o + (size_t)L.max_units * sizeof(int32_t));
    L.nunits = o;      o = align256(o + sizeof(int32_t));
    L.sorted = o;      o = align256(o + (size_t)P * sizeof(int32_t));
    L.act = o;         o = align256(o + (size_t)P * I * sizeof(uint16_t));
    L.part = o;        o = align256(o + (size_t)P * H * sizeof(float));
    L.total = o;
    return L;
}

}  // namespace

// ------------------------------------------------------------------ dispatch

// Stable counting sort of the M*topk (token, slot) pairs by expert, tokens
// ascending within an expert, and the work units (unit_rows rows each).  One workgroup of
// 1024 threads.  A token selects an expert at most once, so within a chunk
// of 64 tokens a pair's rank among the expert's pairs is a popcount of the
// chunk's per-expert token mask below it.
__device__ __forceinline__ void dispatch_body(const int32_t* ids, int M, int E, int topk, int unit_rows,
                                              int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                                              int32_t* __restrict__ unit_expert, int32_t* __restrict__ unit_row,
                                              int32_t* __restrict__ nunits)
{
    __shared__ int cnt[kMaxExperts];
    __shared__ int cursor[kMaxExperts];
    __shared__ int ustart[kMaxExperts];
    __shared__ unsigned long long mask[kMaxExperts];
    __shared__ int scan_tmp[2][kMaxExperts];
    const int tid = threadIdx.x;
    const int P = M * topk;
    for (int e = tid; e < E; e += blockDim.x)
        cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += blockDim.x)
        atomicAdd(&cnt[ids[p]], 1);
    __syncthreads();
    // inclusive scans of the counts and of the unit counts (Hillis-Steele)
    for (int e = tid; e < E; e += blockDim.x) {
        scan_tmp[0][e] = cnt[e];
        scan_tmp[1][e] = (cnt[e] + unit_rows - 1) / unit_rows;
    }
    __syncthreads();
    for (int off = 1; off < E; off <<= 1) {
        int a = 0, b = 0;
        if (tid < E) {
            a = scan_tmp[0][tid] + (tid >= off ? scan_tmp[0][tid - off] : 0);
            b = scan_tmp[1][tid] + (tid >= off ? scan_tmp[1][tid - off] : 0);
        }
        __syncthreads();
        if (tid < E) {
            scan_tmp[0][tid] = a;
            scan_tmp[1][tid] = b;
        }
        __syncthreads();
    }
    for (int e = tid; e < E; e += blockDim.x) {
        const int start = scan_tmp[0][e] - cnt[e];
        cursor[e] = start;
        offsets[e] = start;
        ustart[e] = scan_tmp[1][e] - (cnt[e] + unit_rows - 1) / unit_rows;
    }
    if (tid == 0) {
        offsets[E] = P;
        nunits[0] = scan_tmp[1][E - 1];
    }
    __syncthreads();
    // work units: expert e owns units ustart[e] .. covering its rows
    for (int e = tid; e < E; e += blockDim.x) {
        const int nu = (cnt[e] + unit_rows - 1) / unit_rows;
        for (int u = 0; u < nu; ++u) {
            unit_expert[ustart[e] + u] = e;
            unit_row[ustart[e] + u] = cursor[e] + u * unit_rows;
        }
    }
    // stable placement, 64 tokens at a time
    for (int m0 = 0; m0 < M; m0 += 64) {
        for (int e = tid; e < E; e += blockDim.x)
            mask[e] = 0ull;
        __syncthreads();
        const int chunk_pairs = min(64, M - m0) * topk;
        for (int i = tid; i < chunk_pairs; i += blockDim.x) {
            const int p = m0 * topk + i;
            atomicOr(&mask[ids[p]], 1ull << (i / topk));
        }
        __syncthreads();
        for (int i = tid; i < chunk_pairs; i += blockDim.x) {
            const int p = m0 * topk + i;
            const int e = ids[p];
            const unsigned long long below = (1ull << (i / topk)) - 1ull;
            sorted[cursor[e] + __popcll(mask[e] & below)] = p;
        }
        __syncthreads();
        for (int e = tid; e < E; e += blockDim.x)
            cursor[e] += __popcll(mask[e]);
        __syncthreads();
    }
}

__global__ __launch_bounds__(1024) void k_dispatch(const int32_t* __restrict__ ids, int M, int E, int topk,
                                                   int unit_rows,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ sorted,
                                                   int32_t* __restrict__ unit_expert,
                                                   int32_t* __restrict__ unit_row,
                                                   int32_t* __restrict__ nunits)
{
    dispatch_body(ids, M, E, topk, unit_rows, offsets, sorted, unit_expert, unit_row, nunits);
}

// The same dispatch done by one wave, for the routing kernel when it serves
// every token (M <= kRouteTokens, so a token set fits a 16-bit mask): the
// per-expert counts and token masks by LDS atomics, the prefix sums of the
// counts and of the unit counts by a wave scan over contiguous runs of
// experts per lane, then the stable placement by popcount.  No barriers.

__device__ __forceinline__ void dispatch_wave(const int32_t* sids, int M, int E, int topk, int unit_rows, int lane,
                                              int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                                              int32_t* __restrict__ unit_expert, int32_t* __restrict__ unit_row,
                                              int32_t* __restrict__ nunits)
{
    __shared__ int cnt[kMaxExperts];
    __shared__ uint32_t tmask[kMaxExperts];
    const int P = M * topk;
    for (int e = lane; e < E; e += 64) {
        cnt[e] = 0;
        tmask[e] = 0u;
    }
    __builtin_amdgcn_wave_barrier();
    for (int p = lane; p < P; p += 64) {
        const int e = sids[p];
        atomicAdd(&cnt[e], 1);
        atomicOr(&tmask[e], 1u << (p / topk));
    }
    __builtin_amdgcn_wave_barrier();
    // lane l owns experts l*per .. l*per + per - 1
    const int per = (E + 63) / 64;
    const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
    uint32_t c_run = 0, u_run = 0;
    for (int e = e0; e < e1; ++e) {
        const int c = cnt[e];
        c_run += (uint32_t)c;
        u_run += (uint32_t)((c + unit_rows - 1) / unit_rows);
    }
    const uint32_t c_incl = wave_incl_scan(c_run, lane), u_incl = wave_incl_scan(u_run, lane);
    int start = (int)(c_incl - c_run), ustart = (int)(u_incl - u_run);
    for (int e = e0; e < e1; ++e) {
        const int c = cnt[e];
        offsets[e] = start;
        const int nu = (c + unit_rows - 1) / unit_rows;
        for (int u = 0; u < nu; ++u) {
            unit_expert[ustart + u] = e;
            unit_row[ustart + u] = start + u * unit_rows;
        }
        cnt[e] = start;                  // from here on: the expert's first position
        start += c;
        ustart += nu;
    }
    if (lane == 63) {
        offsets[E] = P;
        nunits[0] = (int)u_incl;
    }
    __builtin_amdgcn_wave_barrier();
    for (int p = lane; p < P; p += 64) {
        const int e = sids[p];
        const uint32_t below = (1u << (p / topk)) - 1u;
        sorted[cnt[e] + __popc(tmask[e] & below)] = p;
    }
}

// ------------------------------------------------------------------- routing

constexpr int kRouteTokens = 16;   // tokens per routing workgroup, one wave each

// Outputs of the dispatch step when it runs inside the routing kernel.
struct DispatchOut {
    int unit_rows;
    int32_t* offsets;
    int32_t* sorted;
    int32_t* unit_expert;
    int32_t* unit_row;
    int32_t* nunits;
};

// Ordering key of a logit for the expert choice: NaN ranks like -inf.
__device__ __forceinline__ float rank_key(float v) { return (v != v) ? -INFINITY : v; }

// Unsigned integer whose order is the order of the (non-NaN) float; -0.0
// maps like +0.0.
__device__ __forceinline__ uint32_t order_bits(float v)
{
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u)
        b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Maximum over the wave's 64 lanes (wave-uniform result): within each row of
// 16 lanes by DPP exchanges (neighbours, pairs, half-row mirror, row mirror),
// then over the four rows through lane reads.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
#define BI_DPP_MAX_STEP(CTRL)                                                                     \
    {                                                                                             \
        const uint32_t ohi = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, CTRL, 0xF, 0xF, false);   \
        const uint32_t olo = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, CTRL, 0xF, 0xF, false);   \
        const bool take = ohi > hi || (ohi == hi && olo > lo);                                    \
        hi = take ? ohi : hi;                                                                     \
        lo = take ? olo : lo;                                                                     \
    }
    BI_DPP_MAX_STEP(0xB1)     // quad_perm 1,0,3,2
    BI_DPP_MAX_STEP(0x4E)     // quad_perm 2,3,0,1
    BI_DPP_MAX_STEP(0x141)    // row_half_mirror
    BI_DPP_MAX_STEP(0x140)    // row_mirror
#undef BI_DPP_MAX_STEP
    uint64_t best = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint64_t c = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
        best = c > best ? c : best;
    }
    return best;
}

// Butterfly over the wave with the partner order xor 1, 2, 4, 8, 16, 32
// (at step k lane i combines its value with lane i ^ k's): DPP inside each
// row of 16 lanes, lane reads across the four rows.  The half-row and row
// mirrors pair a lane with another lane of the xor partner's group, whose
// value is the same by then, and a + b == b + a exactly, so every lane ends
// with the bits of the shuffle butterfly: ((r0 + r1) + (r2 + r3)) over the
// row values r.
template <typename Op>
__device__ __forceinline__ float wave_butterfly(float v, Op op)
{
    v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));   // xor 1
    v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));   // xor 2
    v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));  // ~xor 4
    v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));  // ~xor 8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return op(op(r0, r1), op(r2, r3));
}

// Softmax and top-k of one token (one wave): see k_route.
template <int kPer, bool FUSE>
__device__ __forceinline__ void route_token(const float* l, int lane, int m, int E, int topk,
                                            int32_t* __restrict__ ids, float* __restrict__ probs, int32_t* sid)
{
    float v[kPer];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? l[e] : -INFINITY;
        mx = fmaxf(mx, v[i]);
    }
    mx = wave_butterfly(mx, [](float a, float b) { return fmaxf(a, b); });
    float ex[kPer];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        ex[i] = e < E ? expf(v[i] - mx) : 0.f;
        sum = sum + ex[i];
    }
    sum = wave_butterfly(sum, [](float a, float b) { return a + b; });

    // Top-k by repeated arg-max over unique 64-bit keys: high word the
    // logit's order key (NaN as -inf, -0.0 as +0.0), low word ~e, so the
    // larger logit wins and equal logits go to the lower expert index.
    uint64_t key[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? ((uint64_t)order_bits(rank_key(v[i])) << 32) | (uint32_t)~(uint32_t)e : 0ull;
    }
    for (int j = 0; j < topk; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < kPer; ++i)
            best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (key[i] == best) {          // exactly one lane holds the winner
                const int e = lane + 64 * i;
                ids[(int64_t)m * topk + j] = e;
                probs[(int64_t)m * topk + j] = ex[i] / sum;
                if (FUSE)
                    sid[j] = e;
                key[i] = 0ull;
            }
    }
}

// One workgroup per 16 tokens, one wave per token.
//  1. Logits of the 16 tokens into LDS: either read from `logits` [M,E], or
//     folded here from the router's k tile partials in ascending tile order
//     (acc = P0; acc = acc + P1; ...; + bias) -- the linear fold, same bits.
//  2. Softmax over all E: max (exact), exp, a sum in a fixed order (each
//     lane ascending over its experts, then a fixed butterfly), p = e / sum.
//  3. Top-k: slot j receives the j-th largest logit, equal logits in
//     ascending expert order, -0.0 equal to +0.0 (repeated wave arg-max
//     over unique keys).
//  4. FUSE (a single workgroup, M <= 16): the dispatch of the next step runs
//     in the same workgroup on the ids just chosen (one wave, no barriers),
//     saving a launch.
template <int kPer, bool FUSE>   // experts per lane: E <= 64 * kPer
__global__ __launch_bounds__(kRouteTokens * 64) void k_route(const float* __restrict__ logits,
                                                             const f32x4* __restrict__ partials,
                                                             const float* __restrict__ bias, int tiles_k,
                                                             int M, int E, int topk,
                                                             int32_t* __restrict__ ids,
                                                             float* __restrict__ probs, DispatchOut d)
{
    __shared__ float lg[kRouteTokens][kMaxExperts];
    __shared__ int32_t sids[FUSE ? kRouteTokens * kMaxTopk : 1];
    const int mt = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (partials) {
        const int ntiles = E >> 4;
        for (int pi = tid; pi < ntiles * 64; pi += kRouteTokens * 64) {
            const int nt = pi >> 6, ln = pi & 63;
            const f32x4* p = partials + ((int64_t)mt * ntiles + nt) * tiles_k * 64 + ln;
            // up to 16 partials are requested before the first add, so the
            // ordered fold costs one memory round trip per 16 k tiles
            constexpr int kBatch = 16;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int u0 = 0; u0 < tiles_k; u0 += kBatch) {
                const int n = min(kBatch, tiles_k - u0);
                f32x4 v[kBatch];
#pragma unroll
                for (int i = 0; i < kBatch; ++i)
                    if (i < n)
                        v[i] = p[(int64_t)(u0 + i) * 64];
#pragma unroll
                for (int i = 0; i < kBatch; ++i)
                    if (i < n)
                        acc = (u0 + i == 0) ? v[i] : acc + v[i];
            }
            const int col = nt * 16 + acc_col(ln);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v = acc[q];
                if (bias)
                    v = v + bias[col];
                lg[acc_row(ln, q)][col] = v;
            }
        }
    } else {
        for (int i = tid; i < kRouteTokens * E; i += kRouteTokens * 64) {
            const int r = i / E, e = i % E;
            const int m = mt * kRouteTokens + r;
            lg[r][e] = m < M ? logits[(int64_t)m * E + e] : 0.f;
        }
    }
    __syncthreads();
    const int m = mt * kRouteTokens + wave;
    if (m < M)
        route_token<kPer, FUSE>(lg[wave], lane, m, E, topk, ids, probs, sids + wave * topk);
    if constexpr (FUSE) {
        __syncthreads();
        if (wave == 0)
            dispatch_wave(sids, M, E, topk, d.unit_rows, lane, d.offsets, d.sorted, d.unit_expert, d.unit_row,
                          d.nunits);
    }
}


// ------------------------------------------------------------ grouped GEMMs

struct GroupedArgs {
    const uint16_t* a;        // GEMM1: x [M, K] (rows gathered by token); GEMM2: act [P, K] by position
    int64_t lda;
    int a_by_token;           // 1: a row = token of the pair at that position
    const uint16_t* w;        // expert weights, expert e at w + e * w_stride, [rows, K] row-major
    int64_t w_stride, ldw;
    int n_out;                // GEMM1: I (gate/up pairs); GEMM2: H
    int up_offset;            // GEMM1: I (row offset of the up half); GEMM2: 0
    int K, kbpt, tiles_k;
    const int32_t* offsets;
    const int32_t* sorted;
    const int32_t* unit_expert;
    const int32_t* unit_row;
    const int32_t* nunits;
    const float* probs;       // [P] routing probabilities by pair
    int act_probs;            // GEMM1: 1 = multiply the activation by the pair's probability
    int topk;
    uint16_t* act;            // GEMM1 output [P, I] by position
    float* part;              // GEMM2 output [P, H] by pair
    // GEMM2 with the top-k sum folded in (small M): arrival counters, one
    // per column block, in the workspace's counter region (nullptr: the sum
    // runs as its own kernel), the layer output and the sum's options
    uint32_t* comb_counters;
    float* y;
    int tokens, comb_apply, comb_fp64;
};

// Counters of the folded top-k sum: 128 bytes apart, after the first 64 of
// the counter region.
constexpr int kCombCounterStride = (int)(kDecodeCounterBytes / 4 / kDecodeMaxCounters);
constexpr int kCombCounterFirst = 64;
constexpr int kCombMaxBlocks = kDecodeMaxCounters - kCombCounterFirst;
// up to this many tokens the sum is folded into the down projection: its
// last workgroup per column block (256 threads, 64 columns) then sums one
// (token, column) per thread in one round of loads (measured on the
// Qwen3-shaped layer: M=1 33.0 -> 31.8 us; at M=16, four sums per thread
// one after another, 150.9 -> 158.4)
constexpr int64_t kCombMaxTokens = 4;

// The top-k sum of token t at column c, in slot order j = 0..topk-1
// (fused-MoE page: fixed slot order; the (apply_weights, acc_fp64) options
// honoured independently, so the unweighted fp32 point applies no weights):
//   acc_fp64:  fp32( sum_j w_j * (double) part_j ),  w_j = p_j or 1, in binary64
//   fp32:      acc = +0; acc = acc + t_j,  t_j = p_j * part_j (fp32) or part_j
template <bool APPLY, bool FP64>
__device__ __forceinline__ float topk_sum(const float* __restrict__ part, const float* __restrict__ probs,
                                          int64_t t, int64_t c, int H, int topk)
{
    const float* p = part + (t * topk) * (int64_t)H + c;
    if (FP64) {
        double s = 0.0;
        for (int j = 0; j < topk; ++j) {
            const double v = (double)p[(int64_t)j * H];
            s += APPLY ? (double)probs[t * topk + j] * v : v;
        }
        return (float)s;
    } else {
        float s = 0.0f;
        for (int j = 0; j < topk; ++j) {
            const float v = p[(int64_t)j * H];
            s = s + (APPLY ? probs[t * topk + j] * v : v);
        }
        return s;
    }
}

// Workgroup = TW x NW waves: TW waves split the k tile partials of one
// output tile (folded in ascending order through LDS), NW waves take NW
// neighbouring groups of NT 16-column tiles.  A work unit is MT tiles of 16
// rows of one expert; each wave runs MT x NB x NT independent chains, its
// activation fragments shared by the NT column tiles.  ACT (kActNone: GEMM2,
// fp32 partial per pair; kActSwiGLU: a gate block and the matching up block
// per column tile; kActSqReLU: one block) applies the activation in the
// epilogue.
template <int TW, int NW, int MT, int ACT, int CH, int NT>
__global__ __launch_bounds__(TW * NW * 64) void k_grouped(GroupedArgs g)
{
    constexpr int NB = ACT == kActSwiGLU ? 2 : 1;       // output blocks per column tile
    constexpr int NBT = NB * NT;                        // weight blocks per wave: b * NT + j
    __shared__ f32x4 lds[(TW > 1) ? TW * NW * MT * NBT * 64 : 1];
    const int u = blockIdx.y;
    if (u >= g.nunits[0])
        return;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int tw = wid % TW, nw = wid / TW;
    const int r = lane & 15, gslot = lane >> 4;
    const int nt = (blockIdx.x * NW + nw) * NT;        // first column tile of the wave
    const bool nt_ok = nt * 16 < g.n_out;
    const int e = g.unit_expert[u];
    const int row0 = g.unit_row[u];
    const int row_end = g.offsets[e + 1];

    // this lane's operand rows (rows past the expert's last read its last row)
    const uint16_t* ap[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int pos = min(row0 + m * kTileRows + r, row_end - 1);
        const int arow = g.a_by_token ? g.sorted[pos] / g.topk : pos;
        ap[m] = g.a + (int64_t)arow * g.lda + kSlotLen * gslot;
    }
    const uint16_t* we = g.w + (int64_t)e * g.w_stride;
    const uint16_t* wp[NBT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        // column tiles past n_out read tile 0 and are never stored
        const int ntc = (nt + j) * 16 < g.n_out ? nt + j : 0;
        wp[j] = we + (int64_t)(ntc * 16 + r) * g.ldw + kSlotLen * gslot;
        if (ACT == kActSwiGLU)
            wp[NT + j] = we + (int64_t)(g.up_offset + ntc * 16 + r) * g.ldw + kSlotLen * gslot;
    }

    f32x4 acc[MT][NBT];
    for (int t = tw; t < g.tiles_k; t += TW) {
        f32x4 P[MT][NBT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int b = 0; b < NBT; ++b)
                P[m][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int64_t k0 = (int64_t)t * g.kbpt * kKBlock;
        // chunks of CH k blocks, the next chunk's loads in flight while the
        // current one feeds the chains (two fragment buffers)
        Frag<false> af0[CH][MT], af1[CH][MT];
        Frag<false> bf0[CH][NBT], bf1[CH][NBT];
        auto load_chunk = [&](Frag<false> (&af)[CH][MT], Frag<false> (&bf)[CH][NBT], int c) {
#pragma unroll
            for (int i = 0; i < CH; ++i) {
#pragma unroll
                for (int b = 0; b < NBT; ++b)
                    load_frag<BF16>(bf[i][b], wp[b] + k0 + (int64_t)(c + i) * kKBlock);
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    load_frag<BF16>(af[i][m], ap[m] + k0 + (int64_t)(c + i) * kKBlock);
            }
        };
        auto run_chunk = [&](Frag<false> (&af)[CH][MT], Frag<false> (&bf)[CH][NBT]) {
#pragma unroll
            for (int i = 0; i < CH; ++i)
                mfma_tiles<MT, NBT>(af[i], bf[i], P);
        };
        chunk_pipeline<CH>(
            g.kbpt, [&](int c) { load_chunk(af0, bf0, c); }, [&](int c) { load_chunk(af1, bf1, c); },
            [&](int) { run_chunk(af0, bf0); }, [&](int) { run_chunk(af1, bf1); });
        if (TW == 1) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int b = 0; b < NBT; ++b)
                    acc[m][b] = (t == 0) ? P[m][b] : acc[m][b] + P[m][b];
        } else {
            // one tile per wave (TW == tiles_k); stage it for the ordered fold
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int b = 0; b < NBT; ++b)
                    lds[(((t * NW + nw) * MT + m) * NBT + b) * 64 + lane] = P[m][b];
        }
    }
    if (TW > 1) {
        __syncthreads();
        if (tw != 0)
            return;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int b = 0; b < NBT; ++b) {
                acc[m][b] = lds[(((0 * NW + nw) * MT + m) * NBT + b) * 64 + lane];
                for (int t = 1; t < g.tiles_k; ++t)
                    acc[m][b] = acc[m][b] + lds[(((t * NW + nw) * MT + m) * NBT + b) * 64 + lane];
            }
    }
    if (ACT != kActNone && !nt_ok)
        return;

#pragma unroll
    for (int j = 0; j < NT; ++j) {
    const int col = (nt + j) * 16 + acc_col(lane);
    const bool col_ok = (nt + j) * 16 < g.n_out;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int p = row0 + m * kTileRows + acc_row(lane, q);
            if (p >= row_end || !col_ok)
                continue;
            if (ACT == kActSwiGLU) {
                // storage point of the gate/up projection, then the activation
                // in fp32 (with the routing probability if asked), one
                // rounding to bf16
                const float hg = bf16_to_f32(f32_to_bf16_rne(acc[m][j][q]));
                const float hu = bf16_to_f32(f32_to_bf16_rne(acc[m][NT + j][q]));
                const float sg = 1.0f / (1.0f + expf(-hg));
                float av = (hg * sg) * hu;
                if (g.act_probs)
                    av = av * g.probs[g.sorted[p]];
                g.act[(int64_t)p * g.n_out + col] = f32_to_bf16_rne(av);
            } else if (ACT == kActSqReLU) {
                // squared ReLU of the bf16 storage point (exact in fp32: an
                // 8-bit significand squared), then the optional probability
                const float h = bf16_to_f32(f32_to_bf16_rne(acc[m][j][q]));
                const float rl = h > 0.f ? h : 0.f;
                float av = rl * rl;
                if (g.act_probs)
                    av = av * g.probs[g.sorted[p]];
                g.act[(int64_t)p * g.n_out + col] = f32_to_bf16_rne(av);
            } else {
                g.part[(int64_t)g.sorted[p] * g.n_out + col] = acc[m][j][q];
            }
        }
    }
    if constexpr (ACT == kActNone && TW == 1 && NT == 1) {
        // The top-k sum in the same launch (small M).  Every workgroup of
        // column block bx runs on XCD bx mod 8 (workgroups go to the XCDs
        // round-robin and the grid's row is a multiple of 8 blocks), so the
        // partials of the block's columns, written by the workgroups of all
        // work units, meet in that XCD's L2.  A workgroup's stores are
        // complete there before it counts itself in; the workgroup that
        // arrives last drops its L1 and sums the block's columns for every
        // token.  The counter wraps to zero at the last arrival.
        if (g.comb_counters) {
            __shared__ uint32_t last;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0) {
                const uint32_t n = (uint32_t)g.nunits[0];
                const uint32_t prev = __builtin_amdgcn_atomic_inc32(g.comb_counters + blockIdx.x * kCombCounterStride,
                                                                    n - 1, __ATOMIC_RELAXED, "workgroup");
                last = prev == n - 1;
            }
            __syncthreads();
            if (!last)
                return;
            asm volatile("buffer_inv sc0" ::: "memory");
            const int c0 = blockIdx.x * NW * 16;
            const int ncol = min(NW * 16, g.n_out - c0);
            for (int i = tid; i < g.tokens * ncol; i += NW * 64) {
                const int64_t t = i / ncol, c = c0 + i % ncol;
                float v;
                if (g.comb_apply && g.comb_fp64)
                    v = topk_sum<true, true>(g.part, g.probs, t, c, g.n_out, g.topk);
                else if (g.comb_apply)
                    v = topk_sum<true, false>(g.part, g.probs, t, c, g.n_out, g.topk);
                else if (g.comb_fp64)
                    v = topk_sum<false, true>(g.part, g.probs, t, c, g.n_out, g.topk);
                else
                    v = topk_sum<false, false>(g.part, g.probs, t, c, g.n_out, g.topk);
                g.y[t * g.n_out + c] = v;
            }
        }
    }
}

// ------------------------------------------------------------------- combine

// Top-k sum as its own kernel (larger M): topk_sum for every (token, column).
template <bool APPLY, bool FP64>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ part, const float* __restrict__ probs,
                                                 int M, int H, int topk, float* __restrict__ y)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)M * H)
        return;
    y[i] = topk_sum<APPLY, FP64>(part, probs, i / H, i % H, H, topk);
}

// ------------------------------------------------------------------ host side

static int pick_ch(int kbpt)
{
    for (int c = 16; c >= 1; c >>= 1)
        if (kbpt % c == 0)
            return c;
    return 1;
}

template <int TW, int NW, int MT, int ACT, int NT>
static hipError_t launch_grouped_tw(const GroupedArgs& g, int64_t max_units, hipStream_t s)
{
    const int ntiles = (g.n_out / 16 + NW * NT - 1) / (NW * NT);
    dim3 grid((unsigned)ntiles, (unsigned)max_units);
    // two buffers of CH k blocks of MT activation and NB weight fragments.
    // Short chunks keep the registers per wave low, and more waves per SIMD
    // keep more weight bytes in flight than long chunks do (measured on
    // MI355X, Qwen3-30B-A3B-shaped layer: CH 4 for 16-row units, 2 for 32-row
    // units gave M=16 153.7 us (was 162.6 with CH 8), M=64 230.4 (253.7) and
    // M=256 305.9 (366.7 with CH 4 / 8))
    int ch = pick_ch(g.kbpt);
    const int ch_max = MT == 1 ? 4 : 2;
    if (ch > ch_max)
        ch = ch_max;
    switch (ch) {
    case 4:  k_grouped<TW, NW, MT, ACT, 4, NT><<<grid, TW * NW * 64, 0, s>>>(g); break;
    case 2:  k_grouped<TW, NW, MT, ACT, 2, NT><<<grid, TW * NW * 64, 0, s>>>(g); break;
    default: k_grouped<TW, NW, MT, ACT, 1, NT><<<grid, TW * NW * 64, 0, s>>>(g); break;
    }
    return hipGetLastError();
}

// Column tiles per wave for 32-row work units of kernels with one weight
// block per tile (the down projection, squared ReLU): the wave's activation
// fragments serve both tiles, which halves the activation rows streamed per
// weight byte (measured on MI355X, Qwen3-30B-A3B-shaped layer at M=256:
// squared ReLU 245.6 -> 218.4 us, SwiGLU 306.7 -> 300.6; four tiles, or two
// for the SwiGLU gate/up kernel with its gate and up blocks, cost more in
// registers than they save)
constexpr int kUnit32Tiles = 2;

template <int MT, int ACT>
static hipError_t launch_grouped_mt(const GroupedArgs& g, int64_t max_units, hipStream_t s)
{
    // k tile partials of one output tile are spread over the workgroup's
    // waves when there are 2 or 4; otherwise the waves take more columns
    constexpr int NT = (MT == 2 && ACT != kActSwiGLU) ? kUnit32Tiles : 1;
    if (g.tiles_k == 4)
        return launch_grouped_tw<4, 1, MT, ACT, NT>(g, max_units, s);
    if (g.tiles_k == 2)
        return launch_grouped_tw<2, 2, MT, ACT, NT>(g, max_units, s);
    return launch_grouped_tw<1, 4, MT, ACT, NT>(g, max_units, s);
}

template <int ACT>
static hipError_t launch_grouped(const GroupedArgs& g, int unit_rows, int64_t max_units, hipStream_t s)
{
    return unit_rows == 32 ? launch_grouped_mt<2, ACT>(g, max_units, s)
                           : launch_grouped_mt<1, ACT>(g, max_units, s);
}

// The router's plan: the linear layer's own choice, except that at small M
// the two-launch decode form is used and the routing kernel folds the
// router's tile partials itself (saving the fold launch).
static bi_status_t router_plan(const bi_recipe_t& r, int64_t M, int64_t E, int64_t H, Plan* p)
{
    // on a decode path the routing kernel folds the router's tile partials
    // itself, so the router runs the two-launch decode's first kernel alone
    bi_status_t st = make_plan(r, BI_PATH_AUTO, M, E, H, p);
    if (st == BI_OK && (p->path == kPathDecodeWg || p->path == kPathDecodeXcd))
        st = make_plan(r, BI_PATH_DECODE, M, E, H, p);
    return st;
}

size_t moe_workspace_size(int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk)
{
    if (M <= 0 || H <= 0 || E <= 0 || I <= 0 || topk <= 0)
        return 0;
    bi_recipe_t r;
    if (recipe_for(BI_F32, E, H, &r) != BI_OK)
        return 0;
    Plan p;
    if (router_plan(r, M, E, H, &p) != BI_OK)
        return 0;
    return moe_layout(M, H, E, I, topk, p.ws_bytes).total;
}

bi_status_t moe_layout_offsets(int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk, int64_t* out)
{
    if (!out || M <= 0 || H <= 0 || E <= 0 || I <= 0 || topk <= 0)
        return BI_EINVAL;
    bi_recipe_t r;
    bi_status_t st = recipe_for(BI_F32, E, H, &r);
    if (st != BI_OK)
        return st;
    Plan p;
    if ((st = router_plan(r, M, E, H, &p)) != BI_OK)
        return st;
    const MoELayout L = moe_layout(M, H, E, I, topk, p.ws_bytes);
    out[0] = (int64_t)L.sorted;
    out[1] = (int64_t)L.act;
    out[2] = (int64_t)L.part;
    out[3] = (int64_t)L.total;
    return BI_OK;
}

bi_status_t moe_run(const uint16_t* x, const float* w_router, const float* b_router, const uint16_t* w13,
                    const uint16_t* w2, int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk,
                    const bi_moe_options_t& opt,
                    int32_t* topk_ids, float* topk_probs, float* y, void* ws, size_t ws_bytes,
                    hipStream_t stream)
{
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (M < 0 || H <= 0 || E <= 0 || I <= 0 || topk <= 0)
        return BI_EINVAL;
    if (M == 0)
        return BI_OK;
    if (!x || !w_router || !w13 || !w2 || !topk_ids || !topk_probs || !y)
        return BI_EINVAL;
    if (!al16(x) || !al16(w_router) || !al16(w13) || !al16(w2) || (b_router && !al16(b_router)))
        return BI_EINVAL;
    if (E > kMaxExperts || topk > kMaxTopk || topk > E || M > (1 << 24) / topk)
        return BI_EUNSUPPORTED;
    if (H % 32 != 0 || I % 32 != 0 || E % 16 != 0)
        return BI_EUNSUPPORTED;
    if (opt.activation != BI_ACT_SWIGLU && opt.activation != BI_ACT_SQRELU)
        return BI_EINVAL;
    if ((opt.probs_at_activation != 0 && opt.probs_at_activation != 1) ||
        (opt.apply_weights != 0 && opt.apply_weights != 1) || (opt.acc_fp64 != 0 && opt.acc_fp64 != 1))
        return BI_EINVAL;
    // the probability applied at the activation and again as a weight of the
    // top-k sum would count it twice
    if (opt.probs_at_activation && opt.apply_weights)
        return BI_EINVAL;
    const bool gated = opt.activation == BI_ACT_SWIGLU;

    bi_recipe_t r_router, r_g1, r_g2;
    bi_status_t st;
    if ((st = recipe_for(BI_F32, E, H, &r_router)) != BI_OK)
        return st;
    if ((st = recipe_for(BI_BF16, gated ? 2 * I : I, H, &r_g1)) != BI_OK)
        return st;
    if ((st = recipe_for(BI_BF16, H, I, &r_g2)) != BI_OK)
        return st;
    Plan pr;
    if ((st = router_plan(r_router, M, E, H, &pr)) != BI_OK)
        return st;
    const MoELayout L = moe_layout(M, H, E, I, topk, pr.ws_bytes);
    if (!ws || ws_bytes < L.total || !al16(ws))
        return BI_EWORKSPACE;
    char* base = reinterpret_cast<char*>(ws);
    float* logits = reinterpret_cast<float*>(base + L.logits);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    int32_t* unit_expert = reinterpret_cast<int32_t*>(base + L.unit_expert);
    int32_t* unit_row = reinterpret_cast<int32_t*>(base + L.unit_row);
    int32_t* nunits = reinterpret_cast<int32_t*>(base + L.nunits);
    int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
    uint16_t* act = reinterpret_cast<uint16_t*>(base + L.act);
    float* part = reinterpret_cast<float*>(base + L.part);

    // router: the batch-invariant fp32 linear layer on the widened bf16 rows;
    // on the decode path its k tile partials are folded by the routing kernel
    LinearArgs ra{x, H, w_router, H, b_router, logits, 0, E, (int)M, (int)E, (int)H};
    const bool fused_fold = pr.path == kPathDecode && pr.tiles_k > 1;
    if (launch_linear(kXBF16Widen, ra, pr, base + L.router_ws, stream, !fused_fold) != hipSuccess)
        return BI_EHIP;
    const unsigned route_groups = (unsigned)((M + kRouteTokens - 1) / kRouteTokens);
    const float* lsrc = fused_fold ? nullptr : logits;
    const f32x4* psrc = fused_fold ? reinterpret_cast<const f32x4*>(base + L.router_ws + kDecodeCounterBytes) : nullptr;
    const int unit_rows = unit_rows_for(M, E, topk);
    const DispatchOut dout{unit_rows, offsets, sorted, unit_expert, unit_row, nunits};
    // one routing workgroup (M <= 16): the dispatch runs inside it
    const bool fuse = route_groups == 1;
#define BI_ROUTE(KPER)                                                                                      \
    do {                                                                                                    \
        if (fuse)                                                                                           \
            k_route<KPER, true><<<1, kRouteTokens * 64, 0, stream>>>(lsrc, psrc, b_router, pr.tiles_k,      \
                                                                     (int)M, (int)E, (int)topk, topk_ids,  \
                                                                     topk_probs, dout);                    \
        else                                                                                                \
            k_route<KPER, false><<<route_groups, kRouteTokens * 64, 0, stream>>>(                           \
                lsrc, psrc, b_router, pr.tiles_k, (int)M, (int)E, (int)topk, topk_ids, topk_probs, dout);   \
    } while (0)
    if (E <= 128)
        BI_ROUTE(2);
    else if (E <= 256)
        BI_ROUTE(4);
    else if (E <= 512)
        BI_ROUTE(8);
    else
        BI_ROUTE(16);
#undef BI_ROUTE
    if (!fuse)
        k_dispatch<<<1, 1024, 0, stream>>>(topk_ids, (int)M, (int)E, (int)topk, unit_rows, offsets, sorted,
                                           unit_expert, unit_row, nunits);
    if (hipGetLastError() != hipSuccess)
        return BI_EHIP;

    GroupedArgs g1{};
    g1.a = x;
    g1.lda = H;
    g1.a_by_token = 1;
    g1.w = w13;
    g1.w_stride = (gated ? 2 * I : I) * H;
    g1.ldw = H;
    g1.n_out = (int)I;
    g1.up_offset = gated ? (int)I : 0;
    g1.K = (int)H;
    g1.kbpt = r_g1.block_k / 32;
    g1.tiles_k = (int)(H / r_g1.block_k);
    g1.offsets = offsets;
    g1.sorted = sorted;
    g1.unit_expert = unit_expert;
    g1.unit_row = unit_row;
    g1.nunits = nunits;
    g1.probs = topk_probs;
    g1.act_probs = opt.probs_at_activation;
    g1.topk = (int)topk;
    g1.act = act;
    const hipError_t e1 = gated ? launch_grouped<kActSwiGLU>(g1, unit_rows, L.max_units, stream)
                                : launch_grouped<kActSqReLU>(g1, unit_rows, L.max_units, stream);
    if (e1 != hipSuccess)
        return BI_EHIP;

    GroupedArgs g2 = g1;
    g2.a = act;
    g2.lda = I;
    g2.a_by_token = 0;
    g2.w = w2;
    g2.w_stride = H * I;
    g2.ldw = I;
    g2.n_out = (int)H;
    g2.up_offset = 0;
    g2.K = (int)I;
    g2.kbpt = r_g2.block_k / 32;
    g2.tiles_k = (int)(I / r_g2.block_k);
    g2.act = nullptr;
    g2.part = part;
    g2.act_probs = 0;
    // small M: the top-k sum runs in the down projection's launch (one
    // workgroup of four waves per 64 columns, TW == 1; the column blocks
    // must split evenly over the eight XCDs)
    const int64_t comb_blocks = (H / 16 + 3) / 4;
    const bool fold_sum = M <= kCombMaxTokens && g2.tiles_k != 2 && g2.tiles_k != 4 &&
                          comb_blocks % 8 == 0 && comb_blocks <= kCombMaxBlocks;
    if (fold_sum) {
        g2.comb_counters = reinterpret_cast<uint32_t*>(base + L.router_ws) + kCombCounterFirst * kCombCounterStride;
        g2.y = y;
        g2.tokens = (int)M;
        g2.comb_apply = opt.apply_weights;
        g2.comb_fp64 = opt.acc_fp64;
    }
    if (launch_grouped<kActNone>(g2, unit_rows, L.max_units, stream) != hipSuccess)
        return BI_EHIP;
    if (fold_sum)
        return BI_OK;

    const int64_t n = M * H;
    const unsigned cgrid = (unsigned)((n + 255) / 256);
    if (opt.apply_weights && opt.acc_fp64)
        k_combine<true, true><<<cgrid, 256, 0, stream>>>(part, topk_probs, (int)M, (int)H, (int)topk, y);
    else if (opt.apply_weights)
        k_combine<true, false><<<cgrid, 256, 0, stream>>>(part, topk_probs, (int)M, (int)H, (int)topk, y);
    else if (opt.acc_fp64)
        k_combine<false, true><<<cgrid, 256, 0, stream>>>(part, topk_probs, (int)M, (int)H, (int)topk, y);
    else
        k_combine<false, false><<<cgrid, 256, 0, stream>>>(part, topk_probs, (int)M, (int)H, (int)topk, y);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_EHIP;
}

}  // namespace bi
