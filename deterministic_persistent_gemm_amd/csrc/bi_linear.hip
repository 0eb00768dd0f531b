// bi_linear.hip -- batch-invariant linear layer kernels for gfx950.
//
// Two kernel shapes carry out one recipe (bi_device.h) bit for bit:
//
//  * k_decode (small M): one wave per (16-row M tile, 16-column N tile, k tile
//    partial).  The k tile partials of one output tile are computed on
//    different compute units, so the weight streams through the whole chip
//    and every weight element is fetched by exactly one wave (for M <= 16).
//    The last wave to finish an output tile -- elected with a device-scope
//    counter -- adds the partials in ascending tile order, adds the bias and
//    stores.  The counter is reset by that wave, so the workspace stays clean.
//
//  * k_persistent (large M): a grid of at most a few workgroups per compute
//    unit loops over BM x BN output tiles.  Each k block of X and W is staged
//    through LDS with coalesced 16-byte loads (rows padded by 16 bytes so the
//    lanes' fragment reads spread over the banks); the tile partials are
//    chained in registers and added in ascending order, exactly as above.
//
// GateLinear page, section "Update: is the M=4096 cost avoidable?": decode is
// latency-bound and wants many small pieces of work, while M=4096 wants few
// wide tiles so that X is not re-read once per N tile.  Keeping the recipe
// separate from the kernel shape lets each regime have its own shape.
#include <hip/hip_runtime.h>

#include "bi_device.h"
#include "bi_launch.h"

namespace bi {

// ------------------------------------------------------------------ epilogue

__device__ __forceinline__ void store_elem(const LinearArgs& a, int row, int col, float v)
{
    if (a.bias)
        v = v + a.bias[col];
    if (a.y_bf16)
        reinterpret_cast<uint16_t*>(a.y)[(int64_t)row * a.ldy + col] = f32_to_bf16_rne(v);
    else
        reinterpret_cast<float*>(a.y)[(int64_t)row * a.ldy + col] = v;
}

// acc holds rows row0 + q (q = 0..3) of column col.
__device__ __forceinline__ void store_acc(const LinearArgs& a, int row0, int col, f32x4 acc)
{
    if (col >= a.N)
        return;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (row0 + q < a.M)
            store_elem(a, row0 + q, col, acc[q]);
}

// -------------------------------------------------------------------- decode

template <typename OX, typename OW, int CH>
__global__ __launch_bounds__(64) void k_decode(LinearArgs a, int kbpt, int tiles_k,
                                               f32x4* __restrict__ partials,
                                               unsigned* __restrict__ counters)
{
    using EX = typename OX::elem;
    using EW = typename OW::elem;
    const int lane = threadIdx.x;
    const int r = lane & 15, g = lane >> 4;
    const int t = blockIdx.x % tiles_k;
    const int nt = blockIdx.x / tiles_k;
    const int mt = blockIdx.y;
    const int ntiles = a.N >> 4;

    const int64_t kbase = (int64_t)t * kbpt * kKBlock + kSlotLen * g;
    const EW* wp = reinterpret_cast<const EW*>(a.w) + (int64_t)(nt * 16 + r) * a.ldw + kbase;
    // rows past M read row M-1 (always valid); their results are never stored
    const int xrow = min(mt * 16 + r, a.M - 1);
    const EX* xp = reinterpret_cast<const EX*>(a.x) + (int64_t)xrow * a.ldx + kbase;

    f32x4 P = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < kbpt; c += CH) {
        FragOf<OW> wf[CH];
        FragOf<OX> xf[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i)
            load_frag<OW>(wf[i], wp + (int64_t)(c + i) * kKBlock);
#pragma unroll
        for (int i = 0; i < CH; ++i)
            load_frag<OX>(xf[i], xp + (int64_t)(c + i) * kKBlock);
        // every load of the chunk is in flight before the first instruction
        // of the chain waits on one (memory-level parallelism for streaming)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < CH; ++i)
            P = mfma_block(xf[i], wf[i], P);
    }

    const int row0 = mt * 16 + acc_row(lane, 0);
    const int col = nt * 16 + acc_col(lane);
    if (tiles_k == 1) {
        store_acc(a, row0, col, P);
        return;
    }

    // publish this tile partial, then count arrivals for the output tile
    const int64_t otile = (int64_t)mt * ntiles + nt;
    f32x4* base = partials + otile * tiles_k * 64;
    if (row0 < a.M)
        base[(int64_t)t * 64 + lane] = P;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    unsigned prev = 0;
    if (lane == 0)
        prev = __hip_atomic_fetch_add(&counters[otile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0);
    if (prev != (unsigned)(tiles_k - 1))
        return;

    // last arrival: ordered combine acc = P0; acc = acc + P1; ...
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (row0 < a.M) {
        acc = base[lane];
        for (int u = 1; u < tiles_k; ++u) {
            const f32x4 p = base[(int64_t)u * 64 + lane];
            acc = acc + p;
        }
    }
    if (lane == 0)
        __hip_atomic_store(&counters[otile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    store_acc(a, row0, col, acc);
}

// ---------------------------------------------------------------- persistent

// s-outer order across the FM x FN tiles keeps eight independent chains in
// flight; per output element the order is still s = 0..7 within the block.
template <int FM, int FN>
__device__ __forceinline__ void mfma_tiles(const Frag<true> (&xf)[FM], const Frag<true> (&wf)[FN],
                                           f32x4 (&part)[FM][FN])
{
#define BI_STEP(S)                                                            \
    _Pragma("unroll") for (int fm = 0; fm < FM; ++fm)                         \
        _Pragma("unroll") for (int fn = 0; fn < FN; ++fn)                     \
            part[fm][fn] = mfma_f32_step<S>(xf[fm], wf[fn], part[fm][fn]);
    BI_STEP(0) BI_STEP(1) BI_STEP(2) BI_STEP(3) BI_STEP(4) BI_STEP(5) BI_STEP(6) BI_STEP(7)
#undef BI_STEP
}

template <int FM, int FN>
__device__ __forceinline__ void mfma_tiles(const Frag<false> (&xf)[FM], const Frag<false> (&wf)[FN],
                                           f32x4 (&part)[FM][FN])
{
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            part[fm][fn] = mfma_block(xf[fm], wf[fn], part[fm][fn]);
}

// Stage rows [row0, row0 + ROWS) x one 32-wide k block into LDS with pitch
// PITCH elements; rows past `rows_valid` read the last valid row.
template <typename E, int ROWS, int PITCH, int NT>
__device__ __forceinline__ void stage_block(E* __restrict__ lds, const E* __restrict__ g, int64_t ld,
                                            int row0, int rows_valid, int64_t k0, int tid)
{
    constexpr int kPer16 = 16 / (int)sizeof(E);
    constexpr int kChunks = kKBlock / kPer16;           // 16-byte chunks per row
    constexpr int kTotal = ROWS * kChunks;
#pragma unroll
    for (int i = tid; i < kTotal; i += NT) {
        const int row = i / kChunks, c = i % kChunks;
        const int grow = min(row0 + row, rows_valid - 1);
        const u32x4 v = *reinterpret_cast<const u32x4*>(g + (int64_t)grow * ld + k0 + c * kPer16);
        *reinterpret_cast<u32x4*>(lds + row * PITCH + c * kPer16) = v;
    }
}

template <typename OX, typename OW, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void k_persistent(LinearArgs a, int kbpt, int tiles_m, int tiles_n)
{
    using EX = typename OX::elem;
    using EW = typename OW::elem;
    constexpr int NT = WM * WN * 64;
    constexpr int FM = BM / (WM * 16), FN = BN / (WN * 16);
    constexpr int XP = kKBlock + 16 / (int)sizeof(EX);   // pitch, elements (16 B pad)
    constexpr int WP = kKBlock + 16 / (int)sizeof(EW);
    __shared__ __attribute__((aligned(16))) EX sx[BM * XP];
    __shared__ __attribute__((aligned(16))) EW sw[BN * WP];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int r = lane & 15, g = lane >> 4;
    const int nkb = a.K / kKBlock;
    const EX* xg = reinterpret_cast<const EX*>(a.x);
    const EW* wg = reinterpret_cast<const EW*>(a.w);

    for (int tile = blockIdx.x; tile < tiles_m * tiles_n; tile += gridDim.x) {
        const int tm = tile / tiles_n, tn = tile % tiles_n;
        const int m0 = tm * BM, n0 = tn * BN;
        f32x4 acc[FM][FN], part[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int kb = 0; kb < nkb; ++kb) {
            if (kb % kbpt == 0) {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        part[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            const int64_t k0 = (int64_t)kb * kKBlock;
            stage_block<EX, BM, XP, NT>(sx, xg, a.ldx, m0, a.M, k0, tid);
            stage_block<EW, BN, WP, NT>(sw, wg, a.ldw, n0, a.N, k0, tid);
            __syncthreads();
            FragOf<OX> xf[FM];
            FragOf<OW> wf[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                load_frag<OX>(xf[fm], sx + (wm * FM * 16 + fm * 16 + r) * XP + kSlotLen * g);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                load_frag<OW>(wf[fn], sw + (wn * FN * 16 + fn * 16 + r) * WP + kSlotLen * g);
            __syncthreads();
            mfma_tiles<FM, FN>(xf, wf, part);
            if (kb % kbpt == kbpt - 1) {
                const bool first = kb < kbpt;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = first ? part[fm][fn] : acc[fm][fn] + part[fm][fn];
            }
        }

#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                store_acc(a, m0 + wm * FM * 16 + fm * 16 + acc_row(lane, 0),
                          n0 + wn * FN * 16 + fn * 16 + acc_col(lane), acc[fm][fn]);
    }
}

// ------------------------------------------------------------------ launcher

template <typename OX, typename OW>
static hipError_t launch_decode(const LinearArgs& a, const Plan& p, void* ws, hipStream_t s)
{
    unsigned* counters = reinterpret_cast<unsigned*>(ws);
    f32x4* partials = reinterpret_cast<f32x4*>(reinterpret_cast<char*>(ws) + p.ws_counter_bytes);
    dim3 grid((unsigned)(p.ntiles * p.tiles_k), (unsigned)p.mtiles);
    const int kbpt = p.kbpt;
    constexpr int kMaxCH = OX::f32_frag ? 8 : 16;   // register budget per chunk
    int ch = 1;
    for (int c = kMaxCH; c >= 1; c >>= 1)
        if (kbpt % c == 0) {
            ch = c;
            break;
        }
    switch (ch) {
    case 16: k_decode<OX, OW, 16><<<grid, 64, 0, s>>>(a, kbpt, p.tiles_k, partials, counters); break;
    case 8:  k_decode<OX, OW, 8><<<grid, 64, 0, s>>>(a, kbpt, p.tiles_k, partials, counters); break;
    case 4:  k_decode<OX, OW, 4><<<grid, 64, 0, s>>>(a, kbpt, p.tiles_k, partials, counters); break;
    case 2:  k_decode<OX, OW, 2><<<grid, 64, 0, s>>>(a, kbpt, p.tiles_k, partials, counters); break;
    default: k_decode<OX, OW, 1><<<grid, 64, 0, s>>>(a, kbpt, p.tiles_k, partials, counters); break;
    }
    return hipGetLastError();
}

template <typename OX, typename OW>
static hipError_t launch_persistent(const LinearArgs& a, const Plan& p, hipStream_t s)
{
    constexpr int BM = 64, BN = 64, WM = 2, WN = 2;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int grid = min(tiles, device_cu_count() * 2);
    k_persistent<OX, OW, BM, BN, WM, WN><<<grid, WM * WN * 64, 0, s>>>(a, p.kbpt, tiles_m, tiles_n);
    return hipGetLastError();
}

template <typename OX, typename OW>
static hipError_t launch_typed(const LinearArgs& a, const Plan& p, void* ws, hipStream_t s)
{
    if (p.path == kPathDecode)
        return launch_decode<OX, OW>(a, p, ws, s);
    return launch_persistent<OX, OW>(a, p, s);
}

hipError_t launch_linear(int xkind, const LinearArgs& a, const Plan& p, void* ws, hipStream_t s)
{
    if (p.recipe.dtype == BI_F32) {
        if (xkind == kXF32)
            return launch_typed<F32, F32>(a, p, ws, s);
        return launch_typed<BF16W, F32>(a, p, ws, s);
    }
    return launch_typed<BF16, BF16>(a, p, ws, s);
}

}  // namespace bi
