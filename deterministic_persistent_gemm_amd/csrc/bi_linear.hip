// bi_linear.hip -- batch-invariant linear layer kernels for gfx950.
//
// Five kernel shapes carry out one recipe (bi_device.h) bit for bit:
//
//  * k_decode + k_decode_fold (small M): one wave per (16-column N tile, k
//    tile partial, group of 16-row M tiles).  The k tile partials of one
//    output tile are computed on different compute units, so the weight
//    streams through the whole chip and every weight element is fetched from
//    HBM once.  A second launch adds the partials in ascending tile order,
//    adds the bias and stores; the kernel boundary is the only
//    synchronisation (no device-wide fences, no counters).
//
//  * k_decode_wg (small M, short K): one workgroup per 16x16 output tile;
//    its waves compute the tile partials and fold them through LDS in one
//    launch.
//
//  * k_decode_dma (small M, fully chained bf16 recipes): loader waves stream
//    a 16-column weight slab into an LDS ring with direct-to-LDS loads for
//    one wave that runs the chains.
//
//  * k_persistent (large M): a grid of at most two workgroups per compute
//    unit loops over BM x BN output tiles.  Stages of k blocks of X and W go
//    through LDS (16-byte loads along k, XOR-swizzled rows), the next stages
//    are prefetched into registers, and the tile partials are chained in
//    registers and added in ascending order, exactly as above.
//
//  * k_stream_bf16 (bf16, mid M): 64x64 tiles on eight waves fed by a deep
//    ring of LDS stages written by direct-to-LDS loads.
//
// The persistent kernels hand each XCD one block of the tile grid (xcd_tile).
// GateLinear page, section "Update: is the M=4096 cost avoidable?": decode is
// latency-bound and wants many small pieces of work, while M=4096 wants few
// wide tiles so that X is not re-read once per N tile.  Keeping the recipe
// separate from the kernel shape lets each regime have its own shape.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "bi_device.h"
#include "bi_launch.h"

namespace bi {

// ------------------------------------------------------------------ epilogue

__device__ __forceinline__ void store_elem(const LinearArgs& a, int row, int col, float v)
{
    if (a.y_bf16)
        reinterpret_cast<uint16_t*>(a.y)[(int64_t)row * a.ldy + col] = f32_to_bf16_rne(v);
    else
        reinterpret_cast<float*>(a.y)[(int64_t)row * a.ldy + col] = v;
}

// acc holds rows row0 + q (q = 0..3) of column col.  The bias is one fp32 add
// after the full reduction; without a bias nothing is added (adding +0.0
// would turn a -0.0 result into +0.0).  b is the bias element of col, loaded
// by the caller (load_bias), possibly long before.
__device__ __forceinline__ void store_acc(const LinearArgs& a, int row0, int col, f32x4 acc, float b)
{
    if (col >= a.N)
        return;
    const bool has_bias = a.bias != nullptr;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (row0 + q < a.M)
            store_elem(a, row0 + q, col, has_bias ? acc[q] + b : acc[q]);
}

__device__ __forceinline__ float load_bias(const LinearArgs& a, int col)
{
    return (a.bias && col < a.N) ? a.bias[col] : 0.f;
}

// The same with the bias element loaded here, once, before the rows.
__device__ __forceinline__ void store_acc(const LinearArgs& a, int row0, int col, f32x4 acc)
{
    store_acc(a, row0, col, acc, load_bias(a, col));
}

// -------------------------------------------------------------------- decode

// Arrival counters of the XCD hand-over decode: one 32-bit counter per
// 128-byte L2 line, at the start of the workspace.
constexpr int kCounterStride = kDecodeCounterBytes / 4 / kDecodeMaxCounters;

// The ordered fold of one output tile's partials, for the four accumulator
// rows of this lane: acc = P0; acc = acc + P1; ... (p points at this lane's
// entry of partial 0, partials 64 entries apart).  Up to 32 partials are
// requested at once, so the usual case is one memory round trip.  NQ rows are
// folded: where the M tile holds fewer than four rows (M < 4) the rows past M
// are never stored, so their loads and adds are skipped; the folded rows get
// exactly the same operations.
template <int NQ>
__device__ __forceinline__ f32x4 fold_partials_nq(const f32x4* __restrict__ p, int tiles_k)
{
    constexpr int kBatch = 32;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int u0 = 0; u0 < tiles_k; u0 += kBatch) {
        const int n = min(kBatch, tiles_k - u0);
        f32x4 v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (i < n) {
                const f32x4* q = p + (int64_t)(u0 + i) * 64;
                if constexpr (NQ == 4) {
                    v[i] = *q;
                } else if constexpr (NQ == 2) {
                    const float2 t = *reinterpret_cast<const float2*>(q);
                    v[i][0] = t.x;
                    v[i][1] = t.y;
                } else {
                    v[i][0] = *reinterpret_cast<const float*>(q);
                }
            }
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (i < n)
#pragma unroll
                for (int c = 0; c < NQ; ++c)
                    acc[c] = (u0 + i == 0) ? v[i][c] : acc[c] + v[i][c];
    }
    return acc;
}

// rows: the rows of the M tile that exist (M - 16 mt, wave-uniform).  Below
// four only the lanes of rows 0..3 store, and they hold that many rows.
__device__ __forceinline__ f32x4 fold_partials(const f32x4* __restrict__ p, int tiles_k, int rows)
{
    if (rows >= 3)
        return fold_partials_nq<4>(p, tiles_k);
    if (rows == 2)
        return fold_partials_nq<2>(p, tiles_k);
    return fold_partials_nq<1>(p, tiles_k);
}

// One wave per (16-column N tile, k tile partial, group of MT 16-row M tiles).
// The wave loads its slab of W once and runs MT independent chains over it,
// one per M tile.  With a single k tile (block_k == K) the wave finishes the
// output itself.  Otherwise it stores its tile partials and then either
//  * HANDOFF == false: k_decode_fold adds them up in ascending tile order in a
//    second launch (the kernel boundary makes the partials visible), or
//  * HANDOFF == true: the wave counts itself in at its output tile's arrival
//    counter, and the wave that arrives last adds every partial of the tile
//    in ascending tile order, adds the bias and stores -- one launch.
//
// The hand-over stays inside one XCD's L2.  Workgroups are dispatched
// to the XCDs round-robin (workgroup w runs on XCD w mod 8, as AMD documents
// for the MI300-family dispatcher), and the grid runs the N tile fastest with
// N/16 a multiple of 8, so every wave of an output tile runs on XCD nt mod 8
// and the L2 it shares is the coherence point of the hand-over: each wave's
// partial stores are acknowledged by that L2 before its counter increment
// (an atomic, also performed in that L2) is issued, and the last wave drops
// its L1 before reading the other partials.  No device-scope fence, no L2
// write-back, and no wave ever waits on another.  The counter wraps to zero
// at its last arrival (atomic increment modulo tiles_k), so every call
// leaves the counters as it found them: zero.
template <typename OX, typename OW, int CH, int MT, bool HANDOFF = false>
__global__ __launch_bounds__(64) void k_decode(LinearArgs a, int kbpt, int tiles_k, int mtiles,
                                               f32x4* __restrict__ partials,
                                               uint32_t* __restrict__ counters = nullptr)
{
    using EX = typename OX::elem;
    using EW = typename OW::elem;
    const int lane = threadIdx.x;
    const int r = lane & 15, g = lane >> 4;
    // N tile fastest: workgroup w runs on XCD w % 8, so (when N/16 is a
    // multiple of 8) XCD nt % 8 streams every k slab of N tile nt's W rows
    // and writes all its tile partials as one contiguous run.  Measured per
    // call on the router against k tile fastest: M=1 7.05 -> 6.67 us, M=128
    // 14.2 -> 13.1, although each XCD then fetches the X slabs of every
    // k tile (X read up to 8 times, mostly from the Infinity Cache); giving
    // each XCD a contiguous k range instead reads X once and is slower (7.15)
    const int ntiles = a.N >> 4;
    const int t = blockIdx.x / ntiles;
    const int nt = blockIdx.x % ntiles;
    const int mt0 = blockIdx.y * MT;
    // the wave that finishes an output tile adds the bias last; its element
    // is requested now so that the epilogue never waits on memory
    const float bcol = (tiles_k == 1 || HANDOFF) ? load_bias(a, nt * 16 + acc_col(lane)) : 0.f;

    const int64_t kbase = (int64_t)t * kbpt * kKBlock + kSlotLen * g;
    const EW* wp = reinterpret_cast<const EW*>(a.w) + (int64_t)(nt * 16 + r) * a.ldw + kbase;
    const EX* xp[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        // rows past M read row M-1 (always valid); their results are never stored
        const int xrow = min((mt0 + m) * 16 + r, a.M - 1);
        xp[m] = reinterpret_cast<const EX*>(a.x) + (int64_t)xrow * a.ldx + kbase;
    }

    f32x4 P[MT][1];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        P[m][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Chunks of CH k blocks; while one chunk feeds the chain the next one's
    // loads are in flight (two fragment buffers, loop unrolled by two).
    FragOf<OW> wf0[CH][1], wf1[CH][1];
    FragOf<OX> xf0[CH][MT], xf1[CH][MT];
    // block by block (weight, then its activation rows), so that the chain
    // can start on the first block while the later ones are still arriving
    auto load_chunk = [&](FragOf<OW> (&wf)[CH][1], FragOf<OX> (&xf)[CH][MT], int c) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            // the hand-over serves small M: every weight element is read by
            // exactly one wave, so it streams past the caches
            if constexpr (HANDOFF)
                load_frag_nt<OW>(wf[i][0], wp + (int64_t)(c + i) * kKBlock);
            else
                load_frag<OW>(wf[i][0], wp + (int64_t)(c + i) * kKBlock);
#pragma unroll
            for (int m = 0; m < MT; ++m)
                load_frag<OX>(xf[i][m], xp[m] + (int64_t)(c + i) * kKBlock);
            // keep the issue order: the scheduler would otherwise put the
            // first block's loads last and wait for all of them
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto run_chunk = [&](FragOf<OW> (&wf)[CH][1], FragOf<OX> (&xf)[CH][MT]) {
#pragma unroll
        for (int i = 0; i < CH; ++i)
            mfma_tiles<MT, 1>(xf[i], wf[i], P);
    };
    if (kbpt == CH) {
        // one chunk (the usual decode tile): straight-line code, so that each
        // block's instructions wait only for that block's loads
        load_chunk(wf0, xf0, 0);
        run_chunk(wf0, xf0);
    } else {
        chunk_pipeline<CH>(
            kbpt, [&](int c) { load_chunk(wf0, xf0, c); }, [&](int c) { load_chunk(wf1, xf1, c); },
            [&](int) { run_chunk(wf0, xf0); }, [&](int) { run_chunk(wf1, xf1); });
    }

    const int col = nt * 16 + acc_col(lane);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int mt = mt0 + m;
        const int row0 = mt * 16 + acc_row(lane, 0);
        if (mt >= mtiles || row0 >= a.M)
            continue;
        if (tiles_k == 1)
            store_acc(a, row0, col, P[m][0], bcol);
        else
            partials[(((int64_t)mt * ntiles + nt) * tiles_k + t) * 64 + lane] = P[m][0];
    }
    if constexpr (HANDOFF) {
        if (tiles_k == 1)
            return;
        // this wave's partial stores are complete in the XCD's L2
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        uint32_t prev = 0;
        if (lane == 0)
            prev = __builtin_amdgcn_atomic_inc32(counters + (blockIdx.y * ntiles + nt) * kCounterStride,
                                                 (uint32_t)(tiles_k - 1), __ATOMIC_RELAXED, "workgroup");
        prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
        if (prev != (uint32_t)(tiles_k - 1))
            return;
        // last arrival: every other partial of the tile is in L2; drop stale
        // L1 lines, then fold exactly as k_decode_fold does
        asm volatile("buffer_inv sc0" ::: "memory");
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int mt = mt0 + m;
            const int row0 = mt * 16 + acc_row(lane, 0);
            if (mt >= mtiles || row0 >= a.M)
                continue;
            // this wave's own partial is read back with the others
            const f32x4* p = partials + ((int64_t)mt * ntiles + nt) * tiles_k * 64 + lane;
            store_acc(a, row0, col, fold_partials(p, tiles_k, a.M - mt * 16), bcol);
        }
    }
}

// Ordered fold of the tile partials (fold_partials), then the bias.
__global__ __launch_bounds__(64) void k_decode_fold(LinearArgs a, int tiles_k,
                                                    const f32x4* __restrict__ partials)
{
    const int lane = threadIdx.x;
    const int nt = blockIdx.x, mt = blockIdx.y;
    const int ntiles = a.N >> 4;
    const int row0 = mt * 16 + acc_row(lane, 0);
    if (row0 >= a.M)
        return;
    const float b = load_bias(a, nt * 16 + acc_col(lane));
    const f32x4* p = partials + ((int64_t)mt * ntiles + nt) * tiles_k * 64 + lane;
    store_acc(a, row0, nt * 16 + acc_col(lane), fold_partials(p, tiles_k, a.M - mt * 16), b);
}

// One workgroup per (16-row M tile, 16-column N tile), NW waves.  Wave w
// computes the tile partials t = w, w + NW, w + 2 NW, ... (each a chain from
// zero over its own k blocks) and leaves them in LDS; after one barrier wave 0
// adds them in ascending tile order, adds the bias and stores.  The whole
// reduction of an output tile stays inside one compute unit, so one launch
// does the work of k_decode + k_decode_fold with no workspace.  A wave walks
// its k blocks as one flattened sequence in chunks of CH (CH divides kbpt, so
// no chunk straddles two partials) with the next chunk's loads in flight.
template <typename OX, typename OW, int CH, int NW>
__global__ __launch_bounds__(NW * 64) void k_decode_wg(LinearArgs a, int kbpt, int tiles_k)
{
    using EX = typename OX::elem;
    using EW = typename OW::elem;
    extern __shared__ f32x4 lds_part[];   // [tiles_k][64]
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int nt = blockIdx.x, mt = blockIdx.y;
    const int nblk = (tiles_k > w ? (tiles_k - w + NW - 1) / NW : 0) * kbpt;

    const EW* wp = reinterpret_cast<const EW*>(a.w) + (int64_t)(nt * 16 + r) * a.ldw + kSlotLen * g;
    // rows past M read row M-1 (always valid); their results are never stored
    const int xrow = min(mt * 16 + r, a.M - 1);
    const EX* xp = reinterpret_cast<const EX*>(a.x) + (int64_t)xrow * a.ldx + kSlotLen * g;
    // k offset of the c-th block of this wave's sequence
    auto koff = [&](int c) {
        const int j = c / kbpt;
        return (int64_t)((w + j * NW) * kbpt + (c - j * kbpt)) * kKBlock;
    };

    f32x4 P[1][1];
    FragOf<OW> wf0[CH][1], wf1[CH][1];
    FragOf<OX> xf0[CH][1], xf1[CH][1];
    auto load_chunk = [&](FragOf<OW> (&wf)[CH][1], FragOf<OX> (&xf)[CH][1], int c) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int64_t o = koff(c + i);
            load_frag<OW>(wf[i][0], wp + o);
            load_frag<OX>(xf[i][0], xp + o);
        }
    };
    auto run_chunk = [&](FragOf<OW> (&wf)[CH][1], FragOf<OX> (&xf)[CH][1], int c) {
        if (c % kbpt == 0)
            P[0][0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < CH; ++i)
            mfma_tiles<1, 1>(xf[i], wf[i], P);
        if ((c + CH) % kbpt == 0)
            lds_part[(w + (c / kbpt) * NW) * 64 + lane] = P[0][0];
    };
    if (nblk > 0)
        chunk_pipeline<CH>(
            nblk, [&](int c) { load_chunk(wf0, xf0, c); }, [&](int c) { load_chunk(wf1, xf1, c); },
            [&](int c) { run_chunk(wf0, xf0, c); }, [&](int c) { run_chunk(wf1, xf1, c); });
    __syncthreads();
    if (w != 0)
        return;
    const int row0 = mt * 16 + acc_row(lane, 0);
    f32x4 acc = lds_part[lane];
    for (int t = 1; t < tiles_k; ++t)
        acc = acc + lds_part[t * 64 + lane];
    store_acc(a, row0, nt * 16 + acc_col(lane), acc);
}

// Decode for a fully chained bf16 recipe (one tile partial): one workgroup
// per 16-column N tile and all M tiles (MT <= 4).  The chain itself is short
// (one 16x16x32 instruction per 32 k per M tile), so the wave that runs it
// would otherwise wait on its own loads; here kLoaders waves stream the
// weight slab and the activation rows into an LDS ring with direct-to-LDS
// loads (each k block of 16 rows lands as one 1 KiB chunk laid out exactly
// as the fragment lanes read it), several phases ahead, and MT chain waves
// only read LDS and issue the chains, one M tile each.  Phases are handed
// over with one barrier each; a loader waits for its own loads of a phase
// before the barrier.
constexpr int kDmaLoaders = 8;

// One 16-byte direct-to-LDS load per lane: lane i's bytes land at LDS byte
// address `lds` + 16 i (M0 holds the wave's base).  Written as inline
// assembly so that the compiler does not order every such load after the
// previous one (it would treat each as an aliasing LDS write and wait for
// all earlier ones); the waits are explicit below instead.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}

// The same with a wave-uniform 64-bit base in scalar registers and a 32-bit
// per-lane byte offset (one vector register per load stream instead of two).
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt with vmcnt <= N (N < 64), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vm()
{
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0), other counters untouched
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14)); }

// A workgroup barrier without the memory fence of __syncthreads (whose
// release would wait for every outstanding load); the callers wait for
// exactly what the other side needs first.
__device__ __forceinline__ void bar() { asm volatile("s_barrier" : : : "memory"); }

// vmcnt <= later * LW for a runtime later in [0, C]
template <int LW, int C>
__device__ __forceinline__ void wait_later(int later)
{
    if constexpr (C <= 0) {
        wait_vm<0>();
    } else {
        if (later >= C)
            wait_vm<C * LW>();
        else
            wait_later<LW, C - 1>(later);
    }
}

// MT M tiles, PB k blocks per phase, a ring of R phases in LDS.
// XR > 0 (MT = 1, M <= XR, K <= kDmaXMaxK): the first XR activation rows are
// loaded once into LDS at the start (16-byte chunks, row-major), so the ring
// holds the weight only and can run further ahead; rows past M are never
// stored, so lanes of those rows read row M-1.  XR = 0: each k block's
// activation tiles travel in the ring beside the weight.
constexpr int kDmaXMaxK = 4096;

template <int MT, int PB, int R, int XR>
__global__ __launch_bounds__((kDmaLoaders + MT) * 64) void k_decode_dma(LinearArgs a)
{
    static_assert(XR == 0 || MT == 1, "activation rows in LDS for one M tile");
    constexpr int IPB = XR ? 1 : 1 + MT;              // 1 KiB items per k block: W (then MT X tiles)
    constexpr int IT = XR ? 16 : PB * IPB;            // items per phase (XR: one weight row each)
    constexpr int LW = IT / kDmaLoaders;              // items per loader per phase
    static_assert(IT % kDmaLoaders == 0, "items split evenly");
    static_assert(R >= 2 && (R - 2) * LW < 64, "ring depth");
    static_assert(!XR || PB * 4 == 64, "a weight row of a phase is one 1 KiB load");
    // XR: row i of the 16-row weight slab at ring[.][i], its PB*32 k values
    // contiguous (1 KiB, one load), rows 1040 bytes apart so that the 16 rows
    // of a fragment read fall on different banks
    constexpr int kRowPitch = XR ? 65 : 64;
    __shared__ u32x4 ring[R][IT][kRowPitch];
    __shared__ u32x4 xs[XR ? XR * kDmaXMaxK / 8 : 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int nt = blockIdx.x;
    const int nblk = a.K / kKBlock;
    const int P = nblk / PB;
    const int kc = a.K / 8;                           // 16-byte chunks per activation row
    const uint16_t* xbase = reinterpret_cast<const uint16_t*>(a.x);

    if (wave >= MT) {
        const int ld = wave - MT;                     // loader index
        if constexpr (XR > 0) {
            // the activation rows, once: chunk c of row c / kc, 64 chunks per load
            const int nload = (XR * kc) / 64;
            for (int d = ld; d < nload; d += kDmaLoaders) {
                const int c = d * 64 + lane;
                const int row = min(c / kc, a.M - 1);
                dma16(xbase + (int64_t)row * a.ldx + (c % kc) * 8,
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(&xs[d * 64])));
            }
        }
        // loader: items i = ld + kDmaLoaders * t of every phase
        const uint16_t* wrow = reinterpret_cast<const uint16_t*>(a.w) + (int64_t)(nt * 16 + r) * a.ldw + kSlotLen * g;
        const uint16_t* wslab = reinterpret_cast<const uint16_t*>(a.w) + (int64_t)(nt * 16) * a.ldw + 8 * lane;
        auto issue = [&](int ph) {
            if constexpr (XR > 0) {
                // whole rows: lane l takes k = ph*PB*32 + 8l .. +7 of row i
#pragma unroll
                for (int t = 0; t < LW; ++t) {
                    const int i = ld + kDmaLoaders * t;
                    dma16(wslab + (int64_t)i * a.ldw + (int64_t)ph * PB * kKBlock,
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(&ring[ph % R][i][0])));
                }
                return;
            }
#pragma unroll
            for (int t = 0; t < LW; ++t) {
                const int i = ld + kDmaLoaders * t;
                const int j = i / IPB, kind = i % IPB;      // kind 0: W, m + 1: X tile m
                const int64_t k0 = (int64_t)(ph * PB + j) * kKBlock;
                // rows past M read row M-1 (always valid); their results are never stored
                const int xr = min((kind - 1) * 16 + r, a.M - 1);
                const uint16_t* src =
                    kind == 0 ? wrow + k0 : xbase + (int64_t)max(xr, 0) * a.ldx + kSlotLen * g + k0;
                dma16(src, (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(&ring[ph % R][i][0])));
            }
        };
        for (int ph = 0; ph < R - 1 && ph < P; ++ph)
            issue(ph);
        for (int ph = 0; ph < P; ++ph) {
            // this loader's loads up to phase ph (the activation rows first)
            // have landed once at most the later phases in flight,
            // min(R - 2, P - 1 - ph), are outstanding
            wait_later<LW, R - 2>(min(R - 2, P - 1 - ph));
            bar();
            if (ph + R - 1 < P)
                issue(ph + R - 1);
        }
        return;
    }

    // waves 0 .. MT-1: the chains, wave m the chain of M tile m (the weight
    // fragment of each k block is read by every chain wave; the chains run
    // on MT SIMDs side by side instead of one after another in one wave)
    const int m = wave;
    f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
    const int xrow = min(r, a.M - 1);
    for (int ph = 0; ph < P; ++ph) {
        wait_lgkm0();          // the previous phase's LDS reads are done before its slot is refilled
        bar();
        const u32x4(*slot)[kRowPitch] = ring[ph % R];
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            FragOf<BF16> wf[1], xf[1];
            if constexpr (XR > 0) {
                wf[0].v = slot[r][j * 4 + g];
                xf[0].v = xs[xrow * kc + (ph * PB + j) * 4 + g];
            } else {
                wf[0].v = slot[j * IPB][lane];
                xf[0].v = slot[j * IPB + 1 + m][lane];
            }
            mfma_tiles<1, 1>(xf, wf, acc);
        }
    }
    store_acc(a, m * 16 + acc_row(lane, 0), nt * 16 + acc_col(lane), acc[0][0]);
}

// One LDS stage holds KBS k blocks of BM rows of X and BN rows of W.  Each
// thread moves whole 16-byte chunks: consecutive threads take consecutive
// chunks of a row, so a row segment is read with coalesced 16-byte loads.
// In LDS the chunks of a row are permuted by an XOR with a key taken from
// the row (rows are not padded).  The LDS has 64 banks of 4 bytes, i.e. a
// 256-byte bank window; the key spreads the 16 rows a fragment read touches
// over distinct chunk positions of that window, which measured zero bank
// conflicts on gfx950 (SQ_LDS_BANK_CONFLICT) for both the stage stores and
// the fragment reads, against ~2 conflict cycles per instruction with
// 16-byte row padding.
template <typename E, int ROWS, int KS, int NT>
struct Stager {
    static constexpr int kPer16 = 16 / (int)sizeof(E);
    static constexpr int kChunks = KS / kPer16;          // 16-byte chunks per row
    static constexpr int kPitch = KS;                    // LDS row pitch, elements
    // rows of 64 bytes (four chunks) take their key from row / 2: measured
    // conflict-free, where row / 4 costs about three conflict cycles per
    // 16-row fragment read
    static constexpr int kRowsPerWindow = kChunks >= 16 ? 1 : kChunks == 4 ? 2 : 16 / kChunks;
    static constexpr int kKeyMask = (kChunks >= 16 ? 16 : kChunks) - 1;
    static constexpr int kTotal = ROWS * kChunks;
    static constexpr int kPerThread = (kTotal + NT - 1) / NT;

    __device__ __forceinline__ static int key(int row) { return (row / kRowsPerWindow) & kKeyMask; }

    // element offset of chunk c of row `row`
    __device__ __forceinline__ static int at(int row, int c) { return row * kPitch + (c ^ key(row)) * kPer16; }

    // rows past rows_valid read the last valid row (never stored)
    __device__ __forceinline__ static void load(u32x4 (&v)[kPerThread], const E* __restrict__ g, int64_t ld,
                                                int row0, int rows_valid, int64_t k0, int tid)
    {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int i = tid + j * NT;
            if (kTotal % NT != 0 && i >= kTotal)
                break;
            const int row = i / kChunks, c = i % kChunks;
            const int grow = min(row0 + row, rows_valid - 1);
            v[j] = *reinterpret_cast<const u32x4*>(g + (int64_t)grow * ld + k0 + c * kPer16);
        }
    }
    __device__ __forceinline__ static void store(E* __restrict__ lds, const u32x4 (&v)[kPerThread], int tid)
    {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int i = tid + j * NT;
            if (kTotal % NT != 0 && i >= kTotal)
                break;
            const int row = i / kChunks, c = i % kChunks;
            *reinterpret_cast<u32x4*>(lds + at(row, c)) = v[j];
        }
    }
    // one lane's slot of k block kbl: the eight elements kbl*32 + 8g .. +7
    template <typename Op>
    __device__ __forceinline__ static void frag(FragOf<Op>& f, const E* __restrict__ lds, int row, int kbl, int g)
    {
        if constexpr (sizeof(E) == 4) {
            const int c = kbl * 8 + 2 * g;
            f.lo = *reinterpret_cast<const f32x4*>(lds + at(row, c));
            f.hi = *reinterpret_cast<const f32x4*>(lds + at(row, c + 1));
        } else {
            load_frag<Op>(f, lds + at(row, kbl * 4 + g));
        }
    }
};

// Instruction order of one stage of the persistent kernel: the LDS reads of
// k block kbl+1 are spread one by one between the MFMAs of block kbl (NR
// reads and NM MFMAs per block), so each read has several MFMAs to land in.
template <int NR, int NM, int KBS>
__device__ __forceinline__ void interleave_stage()
{
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int kbl = 0; kbl < KBS; ++kbl) {
        if (kbl + 1 < KBS) {
            constexpr int pairs = NR < NM ? NR : NM;
#pragma unroll
            for (int i = 0; i < pairs; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if constexpr (NR > NM)
                __builtin_amdgcn_sched_group_barrier(0x100, NR - NM, 0);
            if constexpr (NM > NR)
                __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
        } else {
            __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
        }
    }
}

// Workgroup w runs on XCD w % 8, and with a grid that is a multiple of 8 so
// does every tile index it = w + r * grid it walks.  XCD x = it % 8 therefore
// owns the tiles it, it + 8, ...; they are mapped onto one xbm x xbn block of
// the tile grid (row-major inside the block), so the tiles that share rows
// of X or of W sit behind the same L2.  xbm == 0 keeps the row-major order.
__device__ __forceinline__ int xcd_tile(int it, int tiles_n, int xbm, int xbn)
{
    if (xbm == 0)
        return it;
    const int x = it & 7, j = it >> 3;
    const int bx = tiles_n / xbn;
    const int m = (x / bx) * xbm + j / xbn;
    const int n = (x % bx) * xbn + j % xbn;
    return m * tiles_n + n;
}

// The block shape of xcd_tile: of the xbm x xbn blocks that split the
// tiles_m x tiles_n grid into eight, the one whose L2 fetches the fewest
// operand rows (xbm * BM rows of X, xbn * BN rows of W); {0, 0} when the
// grid or the tile count is not a multiple of 8.
struct XcdBlock {
    int xbm, xbn;
};

static XcdBlock xcd_block(int tiles_m, int tiles_n, int BM, int BN, int grid)
{
    const int tiles = tiles_m * tiles_n;
    XcdBlock best{0, 0};
    if (grid % 8 != 0 || tiles % 8 != 0)
        return best;
    const int per = tiles / 8;
    long best_rows = 0;
    for (int bm = 1; bm <= tiles_m; ++bm) {
        if (tiles_m % bm != 0 || per % bm != 0 || tiles_n % (per / bm) != 0)
            continue;
        const long rows = (long)bm * BM + (long)(per / bm) * BN;
        if (best.xbm == 0 || rows < best_rows) {
            best = {bm, per / bm};
            best_rows = rows;
        }
    }
    return best;
}

// CHAINED: the recipe has a single k tile (block_k == K), so the chain runs
// straight into the accumulator and no partial registers are needed.
template <typename OX, typename OW, int BM, int BN, int WM, int WN, int KBS, int PD, bool CHAINED>
__global__ __launch_bounds__(WM * WN * 64) void k_persistent(LinearArgs a, int kbpt, int tiles_m, int tiles_n, int xbm, int xbn)
{
    using EX = typename OX::elem;
    using EW = typename OW::elem;
    constexpr int NT = WM * WN * 64;
    constexpr int FM = BM / (WM * 16), FN = BN / (WN * 16);
    constexpr int KS = KBS * kKBlock;
    using SX = Stager<EX, BM, KS, NT>;
    using SW = Stager<EW, BN, KS, NT>;
    __shared__ __attribute__((aligned(16))) EX sx[2][BM * SX::kPitch];
    __shared__ __attribute__((aligned(16))) EW sw[2][BN * SW::kPitch];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int r = lane & 15, g = lane >> 4;
    const int nstages = a.K / KS;
    const int tiles = tiles_m * tiles_n;
    const EX* xg = reinterpret_cast<const EX*>(a.x);
    const EW* wg = reinterpret_cast<const EW*>(a.w);

    for (int it = blockIdx.x; it < tiles; it += gridDim.x) {
        const int tile = xcd_tile(it, tiles_n, xbm, xbn);
        const int tm = tile / tiles_n, tn = tile % tiles_n;
        const int m0 = tm * BM, n0 = tn * BN;
        f32x4 acc[FM][FN], part[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
                part[fm][fn] = acc[fm][fn];
            }

        // The k loop keeps two stages in flight in registers (two register
        // sets, alternating by stage parity) while a third feeds the MFMAs
        // from LDS: a stage is loaded two iterations before it is stored.
        // Fragments of k block kbl+1 are read from LDS before the MFMAs of
        // block kbl are issued, so their latency hides behind those MFMAs.
        auto frags = [&](FragOf<OX> (&xf)[FM], FragOf<OW> (&wf)[FN], int buf, int kbl) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                SX::template frag<OX>(xf[fm], sx[buf], wm * FM * 16 + fm * 16 + r, kbl, g);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                SW::template frag<OW>(wf[fn], sw[buf], wn * FN * 16 + fn * 16 + r, kbl, g);
        };
        // A stage never straddles a k tile (block_k is a whole number of
        // stages), so the partial is cleared and folded only between stages
        // and the unrolled k blocks of a stage form one straight-line block.
        auto compute = [&](int buf, int st) {
            // a second fragment set only where the registers allow it (the
            // largest tiles would spill)
            constexpr int kFragRegs = (FM + FN) * (OX::f32_frag ? 8 : 4);
            constexpr bool kPrefetch = FM * FN * 4 * (CHAINED ? 1 : 2) + 2 * kFragRegs <= 160;
            constexpr int kSets = kPrefetch ? 2 : 1;
            FragOf<OX> xf[kSets][FM];
            FragOf<OW> wf[kSets][FN];
            if constexpr (kPrefetch)
                frags(xf[0], wf[0], buf, 0);
            if constexpr (!CHAINED) {
                if ((st * KBS) % kbpt == 0) {
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn)
                            part[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int kbl = 0; kbl < KBS; ++kbl) {
                const int cur = kPrefetch ? (kbl & 1) : 0;
                if constexpr (kPrefetch) {
                    if (kbl + 1 < KBS)
                        frags(xf[(kbl + 1) & 1], wf[(kbl + 1) & 1], buf, kbl + 1);
                } else {
                    frags(xf[0], wf[0], buf, kbl);
                }
                if constexpr (CHAINED)
                    mfma_tiles<FM, FN>(xf[cur], wf[cur], acc);
                else
                    mfma_tiles<FM, FN>(xf[cur], wf[cur], part);
            }
            if constexpr (kPrefetch)
                interleave_stage<(FM + FN) * (OX::f32_frag && !OX::widen ? 2 : 1),
                                 FM * FN * (OX::f32_frag ? 8 : 1), KBS>();
            if constexpr (!CHAINED) {
                const int kb_end = (st + 1) * KBS;
                if (kb_end % kbpt == 0) {
                    const bool first = kb_end == kbpt;
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn)
                            acc[fm][fn] = first ? part[fm][fn] : acc[fm][fn] + part[fm][fn];
                }
            }
        };
        if constexpr (PD == 2) {
        u32x4 rx0[SX::kPerThread], rw0[SW::kPerThread], rx1[SX::kPerThread], rw1[SW::kPerThread];
        SX::load(rx0, xg, a.ldx, m0, a.M, 0, tid);
        SW::load(rw0, wg, a.ldw, n0, a.N, 0, tid);
        if (nstages > 1) {
            SX::load(rx1, xg, a.ldx, m0, a.M, KS, tid);
            SW::load(rw1, wg, a.ldw, n0, a.N, KS, tid);
        }
        SX::store(sx[0], rx0, tid);
        SW::store(sw[0], rw0, tid);
        if (nstages > 2) {
            SX::load(rx0, xg, a.ldx, m0, a.M, (int64_t)2 * KS, tid);
            SW::load(rw0, wg, a.ldw, n0, a.N, (int64_t)2 * KS, tid);
        }
        __syncthreads();
        for (int st = 0; st < nstages; st += 2) {
            // even stage: set 1 holds stage st+1, set 0 holds stage st+2
            compute(0, st);
            if (st + 1 < nstages) {
                SX::store(sx[1], rx1, tid);
                SW::store(sw[1], rw1, tid);
            }
            if (st + 3 < nstages) {
                SX::load(rx1, xg, a.ldx, m0, a.M, (int64_t)(st + 3) * KS, tid);
                SW::load(rw1, wg, a.ldw, n0, a.N, (int64_t)(st + 3) * KS, tid);
            }
            __syncthreads();
            if (st + 1 >= nstages)
                break;
            // odd stage: set 0 holds stage st+2, set 1 holds stage st+3
            compute(1, st + 1);
            if (st + 2 < nstages) {
                SX::store(sx[0], rx0, tid);
                SW::store(sw[0], rw0, tid);
            }
            if (st + 4 < nstages) {
                SX::load(rx0, xg, a.ldx, m0, a.M, (int64_t)(st + 4) * KS, tid);
                SW::load(rw0, wg, a.ldw, n0, a.N, (int64_t)(st + 4) * KS, tid);
            }
            __syncthreads();
        }
        } else {
            // one stage in flight (shapes whose accumulators leave no room
            // for a second register set)
            u32x4 rx[SX::kPerThread], rw[SW::kPerThread];
            SX::load(rx, xg, a.ldx, m0, a.M, 0, tid);
            SW::load(rw, wg, a.ldw, n0, a.N, 0, tid);
            SX::store(sx[0], rx, tid);
            SW::store(sw[0], rw, tid);
            if (nstages > 1) {
                SX::load(rx, xg, a.ldx, m0, a.M, KS, tid);
                SW::load(rw, wg, a.ldw, n0, a.N, KS, tid);
            }
            __syncthreads();
            for (int st = 0; st < nstages; ++st) {
                const int buf = st & 1;
                compute(buf, st);
                if (st + 1 < nstages) {
                    SX::store(sx[buf ^ 1], rx, tid);
                    SW::store(sw[buf ^ 1], rw, tid);
                }
                if (st + 2 < nstages) {
                    SX::load(rx, xg, a.ldx, m0, a.M, (int64_t)(st + 2) * KS, tid);
                    SW::load(rw, wg, a.ldw, n0, a.N, (int64_t)(st + 2) * KS, tid);
                }
                __syncthreads();
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

// ------------------------------------- 64x64 bf16 tiles fed by a deep LDS ring

// bf16 recipes at mid-size M, where the work is bound by how fast each
// compute unit can stream its operand rows in (a register-staged kernel keeps
// too few bytes in flight per CU to cover the memory latency): one 64x64
// output tile per workgroup of eight waves (each a 16x32 slice, two waves
// per SIMD), X and W streamed into a ring of kStreamRing LDS stages of 64 k
// by direct-to-LDS loads issued kStreamRing - 1 stages ahead, i.e. about
// 112 KiB in flight per compute unit.  Direct-to-LDS loads issue at a rate
// per wave, so eight issuing waves stream faster than four (dense bf16
// M=256: 24.2 us against 26.1; deeper rings of 9 or 10 stages were slower).
// One barrier per stage; the next stage's fragments are read while the
// current stage's MFMAs issue.  The chains are the recipe's (one
// v_mfma_f32_16x16x32_bf16 per k block in ascending order, the usual lane
// slots; with several k tiles the partials are cleared and added in ascending
// order at tile boundaries, which fall between stages), so the bits equal
// every other path's.
//
// Stage layout: X rows 0..63 then W rows 0..63, 128 bytes (64 k) per row,
// chunk c of row q at position c ^ ((q / 2) & 7) -- the Stager layout for
// 64-k stages, which measured free of bank conflicts.  A direct-to-LDS load
// covers 8 rows (1 KiB); lane i lands at row i / 8, position i % 8 and so
// fetches chunk (i % 8) ^ key(row) of its row.
constexpr int kStreamTile = 64;
constexpr int kStreamRing = 8;
constexpr int kStreamWaves = 8;
constexpr int kStreamRowBytes = 2 * kKBlock * 2;                         // 64 k of bf16
constexpr int kStreamHalf = kStreamTile * kStreamRowBytes;               // 8 KiB
constexpr int kStreamStage = 2 * kStreamHalf;                            // 16 KiB

template <bool CHAINED>
__global__ __launch_bounds__(kStreamWaves * 64) void k_stream_bf16(LinearArgs a, int kbpt, int tiles_m, int tiles_n,
                                                                  int xbm, int xbn)
{
    __shared__ __attribute__((aligned(16))) unsigned char ring[kStreamRing * kStreamStage];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;                                   // rows 16 wm.., columns 32 wn..
    const int r = lane & 15, g = lane >> 4;
    const int ns = a.K / (2 * kKBlock);                                  // stages
    const int tiles = tiles_m * tiles_n;
    const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* wg = reinterpret_cast<const uint16_t*>(a.w);
    const uint32_t lds0 = lds_addr(ring);

    for (int it = blockIdx.x; it < tiles; it += gridDim.x) {
        const int tile = xcd_tile(it, tiles_n, xbm, xbn);
        const int m0 = (tile / tiles_n) * kStreamTile, n0 = (tile % tiles_n) * kStreamTile;
        // wave w loads rows 8 w .. 8 w + 7 of the X and of the W tile, one
        // load each; rows past M (N) read row M-1 (N-1), whose results are
        // never stored
        const int lrow = 8 * w + (lane >> 3);
        const int lchunk = (lane & 7) ^ ((lrow >> 1) & 7);
        const uint16_t* src[2] = {xg + (int64_t)min(m0 + lrow, a.M - 1) * a.ldx + lchunk * 8,
                                  wg + (int64_t)min(n0 + lrow, a.N - 1) * a.ldw + lchunk * 8};
        auto issue = [&](int s) {
            const uint32_t base = lds0 + (uint32_t)(s % kStreamRing) * kStreamStage + (8 * w) * kStreamRowBytes;
#pragma unroll
            for (int t = 0; t < 2; ++t)
                dma16(src[t] + (int64_t)s * 2 * kKBlock,
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + t * kStreamHalf)));
        };
        // fragment of k block b (0, 1) of stage s: X row wm*16 + r, W rows
        // wn*32 + 16 n + r; chunk 4 b + g of the row
        auto frag = [&](int s, int half, int row, int b) {
            const unsigned char* p = ring + (s % kStreamRing) * kStreamStage + half * kStreamHalf;
            return *reinterpret_cast<const u32x4*>(p + row * kStreamRowBytes + (((4 * b + g) ^ ((row >> 1) & 7)) << 4));
        };
        auto frags = [&](u32x4 (&x)[2], u32x4 (&wf)[2][2], int s) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                x[b] = frag(s, 0, wm * 16 + r, b);
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    wf[b][n] = frag(s, 1, wn * 32 + 16 * n + r, b);
            }
        };

        f32x4 acc[2], part[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
            part[n] = acc[n];
        }
        auto mfmas = [&](const u32x4 (&x)[2], const u32x4 (&wf)[2][2], int s) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int kb = 2 * s + b;
                if constexpr (!CHAINED) {
                    if (kb % kbpt == 0) {
#pragma unroll
                        for (int n = 0; n < 2; ++n)
                            part[n] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    f32x4& c = CHAINED ? acc[n] : part[n];
                    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x[b]),
                                                                __builtin_bit_cast(bf16x8, wf[b][n]), c, 0, 0, 0);
                }
                if constexpr (!CHAINED) {
                    if (kb % kbpt == kbpt - 1) {
                        const bool first = kb < kbpt;
#pragma unroll
                        for (int n = 0; n < 2; ++n)
                            acc[n] = first ? part[n] : acc[n] + part[n];
                    }
                }
            }
        };

        // the previous tile's fragment reads are done everywhere before the
        // ring is refilled
        wait_lgkm0();
        bar();
        for (int s = 0; s < kStreamRing - 1 && s < ns; ++s)
            issue(s);
        wait_later<2, kStreamRing - 2>(min(kStreamRing - 2, ns - 1));
        bar();
        u32x4 xa[2], wa[2][2], xb[2], wb[2][2];
        frags(xa, wa, 0);
        // stage s: make stage s+1 visible (this wave's loads of it waited
        // for, then the barrier, which also tells that every wave is done
        // with stage s-1, whose slot the load issued next refills), read its
        // fragments, then the MFMAs of stage s
        auto step = [&](int s, const u32x4 (&xc)[2], const u32x4 (&wc)[2][2], u32x4 (&xn)[2], u32x4 (&wnx)[2][2]) {
            if (s + 1 < ns) {
                wait_later<2, kStreamRing - 3>(min(kStreamRing - 3, ns - 2 - s));
                bar();
                if (s + kStreamRing - 1 < ns)
                    issue(s + kStreamRing - 1);
                frags(xn, wnx, s + 1);
            }
            mfmas(xc, wc, s);
        };
        for (int s = 0; s < ns; s += 2) {
            step(s, xa, wa, xb, wb);
            if (s + 1 < ns)
                step(s + 1, xb, wb, xa, wa);
        }

#pragma unroll
        for (int n = 0; n < 2; ++n)
            store_acc(a, m0 + wm * 16 + acc_row(lane, 0), n0 + wn * 32 + n * 16 + acc_col(lane), acc[n]);
    }
}

static hipError_t launch_stream_bf16(const LinearArgs& a, const Plan& p, hipStream_t s)
{
    // whole 64-k stages, and a k tile holds whole stages
    if (a.K % (2 * kKBlock) != 0 || (p.tiles_k != 1 && p.kbpt % 2 != 0))
        return hipErrorInvalidValue;
    const int tiles_m = (a.M + kStreamTile - 1) / kStreamTile;
    const int tiles_n = (a.N + kStreamTile - 1) / kStreamTile;
    const int grid = min(tiles_m * tiles_n, device_cu_count());
    const XcdBlock xb = xcd_block(tiles_m, tiles_n, kStreamTile, kStreamTile, grid);
    if (p.tiles_k == 1)
        k_stream_bf16<true><<<grid, kStreamWaves * 64, 0, s>>>(a, p.kbpt, tiles_m, tiles_n, xb.xbm, xb.xbn);
    else
        k_stream_bf16<false><<<grid, kStreamWaves * 64, 0, s>>>(a, p.kbpt, tiles_m, tiles_n, xb.xbm, xb.xbn);
    return hipGetLastError();
}

// ------------------------------- large bf16 tiles fed by a ring of 32-k stages

// Fully chained bf16 recipes at large M: one BM x BN output tile per
// workgroup of WM x WN waves (each an FM x FN block of 16x16 accumulators,
// two waves per SIMD), X and W streamed by direct-to-LDS loads into a ring
// of R stages of one 32-k block each, issued R - 1 blocks ahead.  A wave
// holds the fragments of two k blocks: while the MFMAs of block s issue, the
// fragments of block s + 1 are read -- the X fragments first, then one W
// fragment after each group of FM MFMAs that used block s's W fragment at
// that position, which is then free -- so the reads land behind the MFMAs
// and the loop waits only at its one barrier per block.  The chains are the
// recipe's fully chained ones (one v_mfma_f32_16x16x32_bf16 per k block, in
// ascending order), so the bits equal every other path's.
//
// Stage layout: X rows 0..BM-1 then W rows 0..BN-1, 64 bytes (32 k) per row,
// chunk c of row q at position c ^ ((q / 2) & 3), which measured free of
// bank conflicts for the 16-row fragment reads on gfx950 (the key (q / 4) & 3
// spreads the same reads over distinct 16-byte bank groups too, yet costs
// about three conflict cycles per read: SQ_LDS_BANK_CONFLICT).  A
// direct-to-LDS load covers 16 rows (1 KiB); lane i lands at row i / 4,
// position i % 4, and so fetches chunk (i % 4) ^ key(row) of its row.
// Epilogue of a wave's (16 FM) x (16 FN) block through LDS: the block is
// written to the wave's own LDS area in groups of 128 / sizeof(E) columns
// (one element per lane and row of each 16x16 accumulator, the same bias add
// and rounding as store_acc), then read back as 16-byte row chunks and stored
// with 16-byte global stores -- instead of one 2- or 4-byte store per element.
// Rows are padded by 16 bytes so that the element writes of the four row
// groups of a wave fall on distinct banks.  Caller: the whole block lies
// inside Y, and Y and its row pitch are 16-byte aligned.
constexpr int kEpiPitch = 128 + 16;                     // bytes per staged row
constexpr int kEpiBytes = 64 * kEpiPitch;                // one wave's area (64 rows)

template <typename E, int FM, int FN>
__device__ __forceinline__ void ring_epilogue(const LinearArgs& a, const f32x4 (&acc)[FM][FN], unsigned char* area,
                                              int row0, int col0, int lane)
{
    static_assert(FM * 16 == 64, "a wave's block is 64 rows");
    constexpr int CG = 128 / (int)sizeof(E);            // columns per group
    constexpr int TG = CG / 16;                         // accumulator columns per group
    constexpr int kChunks = 128 / 16;                   // 16-byte chunks per staged row
    const bool has_bias = a.bias != nullptr;
#pragma unroll
    for (int grp = 0; grp < FN / TG; ++grp) {
#pragma unroll
        for (int t = 0; t < TG; ++t) {
            const int fn = grp * TG + t;
            const float b = load_bias(a, col0 + fn * 16 + acc_col(lane));
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float v = has_bias ? acc[fm][fn][q] + b : acc[fm][fn][q];
                    E* dst = reinterpret_cast<E*>(area + (fm * 16 + acc_row(lane, q)) * kEpiPitch) + t * 16 + acc_col(lane);
                    if constexpr (sizeof(E) == 2)
                        *dst = f32_to_bf16_rne(v);
                    else
                        *dst = v;
                }
        }
        // the element writes and the chunk reads go through different types:
        // keep the compiler from moving one past the other (the LDS itself
        // executes a wave's accesses in order)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 64 * kChunks / 64; ++i) {
            const int c = lane + 64 * i;
            const int row = c / kChunks, ch = c % kChunks;
            const u32x4 v = *reinterpret_cast<const u32x4*>(area + row * kEpiPitch + ch * 16);
            E* y = reinterpret_cast<E*>(a.y) + (int64_t)(row0 + row) * a.ldy + col0 + grp * CG + ch * (16 / (int)sizeof(E));
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(y));
        }
        asm volatile("" ::: "memory");
    }
}

template <int BM, int BN, int WM, int WN, int R, int NL>
__global__ __launch_bounds__(WM * WN * 64) void k_ring_bf16(LinearArgs a, int tiles_m, int tiles_n, int xbm, int xbn)
{
    constexpr int NW = WM * WN;
    constexpr int FM = BM / (WM * 16), FN = BN / (WN * 16);
    constexpr int kRow = kKBlock * 2;                       // bytes of a row's 32-k slice
    constexpr int kFrag = 16 * kRow;                        // 16 rows: one fragment, one load
    constexpr int kXBytes = BM * kRow;
    constexpr int kStage = (BM + BN) * kRow;
    // the first NL waves issue the loads: LX + LW loads of 1 KiB per stage each
    constexpr int LX = BM / (16 * NL), LW = BN / (16 * NL);
    constexpr int LS = LX + LW;
    static_assert(NL <= NW && LX * 16 * NL == BM && LW * 16 * NL == BN, "stage rows split evenly over the loaders");
    static_assert(R >= 3 && (R - 2) * LS < 64, "a ring of at least three stages");
    __shared__ __attribute__((aligned(16))) unsigned char ring[R * kStage];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    const int r = lane & 15, g = lane >> 4;
    const int ns = a.K / kKBlock;
    const int tiles = tiles_m * tiles_n;
    const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* wg = reinterpret_cast<const uint16_t*>(a.w);
    const uint32_t lds0 = lds_addr(ring);
    // lane (r, g) reads chunk g of row r of a fragment's 16 rows; the key of
    // row 16 j + r is (r / 2) & 3 for every j
    const unsigned char* fbase = ring + r * kRow + ((g ^ ((r >> 1) & 3)) << 4);
    const int xf0 = wm * FM * kFrag, wf0 = kXBytes + wn * FN * kFrag;

    for (int it = blockIdx.x; it < tiles; it += gridDim.x) {
        const int tile = xcd_tile(it, tiles_n, xbm, xbn);
        const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
        // loading wave w loads rows 16 (w LX + t) .. +15 of the X tile and
        // 16 (w LW + t) .. +15 of the W tile; rows past M (N) read row M-1
        // (N-1), whose results are never stored.  Each load is a per-lane
        // byte offset from the tile's first row (a scalar base).
        const unsigned char* xt = reinterpret_cast<const unsigned char*>(xg + (int64_t)m0 * a.ldx);
        const unsigned char* wt = reinterpret_cast<const unsigned char*>(wg + (int64_t)n0 * a.ldw);
        uint32_t voff[LS];
        const int wl = w < NL ? w : 0;                     // waves past NL load nothing
#pragma unroll
        for (int t = 0; t < LS; ++t) {
            const int row = 16 * (t < LX ? wl * LX + t : wl * LW + t - LX) + (lane >> 2);
            const int chunk = (lane & 3) ^ ((row >> 1) & 3);
            voff[t] = t < LX ? (uint32_t)((int64_t)(min(m0 + row, a.M - 1) - m0) * a.ldx * 2 + chunk * 16)
                             : (uint32_t)((int64_t)(min(n0 + row, a.N - 1) - n0) * a.ldw * 2 + chunk * 16);
        }
        // block st into slot st % R; past the last block the loads re-read
        // the last block into a slot no later block uses (the slot of block
        // st - R, long consumed), so that every step of the loop is the same
        auto issue_one = [&](int st, int t) {
            const uint32_t base = lds0 + (uint32_t)(st % R) * kStage;
            const int64_t k0 = (int64_t)min(st, ns - 1) * kKBlock * 2;
            const uint32_t dst = t < LX ? base + (wl * LX + t) * kFrag : base + kXBytes + (wl * LW + t - LX) * kFrag;
            dma16s(voff[t], (t < LX ? xt : wt) + k0, (uint32_t)__builtin_amdgcn_readfirstlane((int)dst));
        };
        auto issue = [&](int st) {
            if (NL < NW && w >= NL)
                return;
#pragma unroll
            for (int t = 0; t < LS; ++t)
                issue_one(st, t);
        };
        auto fragx = [&](const unsigned char* sb, int fm) {
            return *reinterpret_cast<const u32x4*>(sb + xf0 + fm * kFrag);
        };
        auto fragw = [&](const unsigned char* sb, int fn) {
            return *reinterpret_cast<const u32x4*>(sb + wf0 + fn * kFrag);
        };

        f32x4 acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto mfma_col = [&](const u32x4 (&xc)[FM], const u32x4& wc, int fn) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xc[fm]),
                                                                      __builtin_bit_cast(bf16x8, wc), acc[fm][fn], 0, 0, 0);
        };

        // the previous tile's fragment reads are done everywhere before the
        // ring is refilled
        wait_lgkm0();
        bar();
#pragma unroll
        for (int st = 0; st < R - 1; ++st)
            issue(st);
        wait_vm<(R - 2) * LS>();
        bar();
        // X fragments of two blocks alternate between xa and xb; each W
        // fragment is replaced in place once its FM MFMAs have issued
        // (in the order the loop's own reads have -- X, then W by column --
        // so that the loop's first wait on a fragment is as loose as its
        // others)
        u32x4 xa[FM], xb[FM], wf[FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            xa[fm] = fragx(fbase, fm);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            wf[fn] = fragw(fbase, fn);
        __builtin_amdgcn_sched_group_barrier(0x100, FM, 0);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);

        // block st: make block st+1 visible (this wave's loads of it waited
        // for, then the barrier, which also tells that every wave is done
        // with block st-1, whose slot the loads of this step refill), then
        // the MFMAs of block st with block st+1's fragment reads between them
        // and, in the loading waves, the loads of block st+R-1 spread over the
        // same gaps (inline assembly, which the compiler keeps in place), so
        // that they issue while the matrix unit is busy.  The last step reads
        // a slot of re-read data that nothing uses.
        auto step = [&](auto loader, int st, const u32x4 (&xc)[FM], u32x4 (&xn)[FM]) {
            constexpr bool LD = decltype(loader)::value;
            wait_vm<(R - 3) * LS>();
            bar();
            const unsigned char* sb = fbase + ((st + 1) % R) * kStage;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                xn[fm] = fragx(sb, fm);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                mfma_col(xc, wf[fn], fn);
                wf[fn] = fragw(sb, fn);
                if constexpr (LD) {
                    // the loads split the code into scheduling regions; keep
                    // each region's order: (the X reads,) the MFMAs, the read
                    if (fn == 0)
                        __builtin_amdgcn_sched_group_barrier(0x100, FM, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                    for (int t = fn * LS / FN; t < (fn + 1) * LS / FN; ++t)
                        issue_one(st + R - 1, t);
                }
            }
            if constexpr (!LD) {
                // one W fragment read after each group of FM MFMAs
                __builtin_amdgcn_sched_group_barrier(0x100, FM, 0);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
        };
        if (NL == NW || w < NL) {
            for (int st = 0; st < ns; st += 2) {
                step(std::true_type{}, st, xa, xb);
                step(std::true_type{}, st + 1, xb, xa);
            }
        } else {
            for (int st = 0; st < ns; st += 2) {
                step(std::false_type{}, st, xa, xb);
                step(std::false_type{}, st + 1, xb, xa);
            }
        }
        // every load into the ring has landed and every wave is done with
        // it before the epilogue stages the output there
        wait_vm<0>();
        wait_lgkm0();
        bar();

        const bool inside = m0 + BM <= a.M && n0 + BN <= a.N;
        const int esz = a.y_bf16 ? 2 : 4;
        const bool aligned = ((uintptr_t)a.y & 15) == 0 && ((a.ldy * esz) & 15) == 0;
        if (inside && aligned) {
            if (a.y_bf16)
                ring_epilogue<uint16_t, FM, FN>(a, acc, ring + w * kEpiBytes, m0 + wm * FM * 16, n0 + wn * FN * 16, lane);
            else
                ring_epilogue<float, FM, FN>(a, acc, ring + w * kEpiBytes, m0 + wm * FM * 16, n0 + wn * FN * 16, lane);
        } else {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    store_acc(a, m0 + (wm * FM + fm) * 16 + acc_row(lane, 0), n0 + (wn * FN + fn) * 16 + acc_col(lane),
                              acc[fm][fn]);
        }
    }
}

// What the ring kernel needs: a fully chained recipe (no tile partials), an
// even number of 32-k blocks (the loop takes them in pairs), and byte offsets
// inside a tile's rows that fit 32 bits.
static bool ring_ok(const LinearArgs& a, const Plan& p, int BM, int BN)
{
    return p.tiles_k == 1 && a.K % (2 * kKBlock) == 0 &&
           (int64_t)(BM - 1) * a.ldx * 2 + (int64_t)a.K * 2 < (int64_t(1) << 32) &&
           (int64_t)(BN - 1) * a.ldw * 2 + (int64_t)a.K * 2 < (int64_t(1) << 32);
}

template <int BM, int BN, int WM, int WN, int R, int NL>
static hipError_t launch_ring_bf16(const LinearArgs& a, const Plan& p, hipStream_t s)
{
    if (!ring_ok(a, p, BM, BN))
        return hipErrorInvalidValue;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + BN - 1) / BN;
    const int grid = min(tiles_m * tiles_n, device_cu_count());
    const XcdBlock xb = xcd_block(tiles_m, tiles_n, BM, BN, grid);
    k_ring_bf16<BM, BN, WM, WN, R, NL><<<grid, WM * WN * 64, 0, s>>>(a, tiles_m, tiles_n, xb.xbm, xb.xbn);
    return hipGetLastError();
}

// ------------------------------------------------------------------ launcher

template <typename OX, typename OW, int MT, bool HANDOFF>
static hipError_t launch_decode_mt(const LinearArgs& a, const Plan& p, f32x4* partials, uint32_t* counters,
                                   hipStream_t s)
{
    dim3 grid((unsigned)(p.ntiles * p.tiles_k), (unsigned)((p.mtiles + MT - 1) / MT));
    const int kbpt = p.kbpt;
    // register budget per chunk of k blocks (two buffers of W fragments plus
    // MT X fragments)
    constexpr int kMaxCH = (OX::f32_frag ? 4 : 8) / (MT > 2 ? 2 : 1);
    int ch = 1;
    for (int c = kMaxCH; c >= 1; c >>= 1)
        if (kbpt % c == 0) {
            ch = c;
            break;
        }
    if constexpr (kMaxCH >= 16) {
        if (ch == 16) {
            k_decode<OX, OW, 16, MT, HANDOFF><<<grid, 64, 0, s>>>(a, kbpt, p.tiles_k, p.mtiles, partials, counters);
            return hipGetLastError();
        }
    }
    if constexpr (kMaxCH >= 8) {
        if (ch == 8) {
            k_decode<OX, OW, 8, MT, HANDOFF><<<grid, 64, 0, s>>>(a, kbpt, p.tiles_k, p.mtiles, partials, counters);
            return hipGetLastError();
        }
    }
    switch (ch) {
    case 4:  k_decode<OX, OW, 4, MT, HANDOFF><<<grid, 64, 0, s>>>(a, kbpt, p.tiles_k, p.mtiles, partials, counters); break;
    case 2:  k_decode<OX, OW, 2, MT, HANDOFF><<<grid, 64, 0, s>>>(a, kbpt, p.tiles_k, p.mtiles, partials, counters); break;
    default: k_decode<OX, OW, 1, MT, HANDOFF><<<grid, 64, 0, s>>>(a, kbpt, p.tiles_k, p.mtiles, partials, counters); break;
    }
    return hipGetLastError();
}

// M tiles per wave: a wave's W fragments serve 2 M tiles from 4 M tiles on
// and 4 from 12 on, while at least ~1000 waves remain (measured for the fp32
// router: M=64 11.0 -> 10.4 us, M=96 13.5 -> 12.2, M=192 18.5 -> 17.6; below
// 4 M tiles one M tile per wave is as fast)
int decode_m_per_wave(const Plan& p)
{
    if (p.m_per_wave > 0)
        return p.m_per_wave;
    const int waves1 = p.ntiles * p.tiles_k * p.mtiles;
    if (p.mtiles >= 12 && waves1 >= 6144)
        return 4;
    if (p.mtiles >= 4 && waves1 >= 2048)
        return 2;
    return 1;
}

template <typename OX, typename OW>
static hipError_t launch_decode(const LinearArgs& a, const Plan& p, void* ws, hipStream_t s, bool fold)
{
    const int mt = p.path == kPathDecodeXcd ? xcd_m_per_wave(p) : decode_m_per_wave(p);
    uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
    f32x4* partials = ws ? reinterpret_cast<f32x4*>(reinterpret_cast<char*>(ws) + kDecodeCounterBytes) : nullptr;
    if (p.path == kPathDecodeXcd) {
        if (mt == 4)
            return launch_decode_mt<OX, OW, 4, true>(a, p, partials, counters, s);
        if (mt == 2)
            return launch_decode_mt<OX, OW, 2, true>(a, p, partials, counters, s);
        return launch_decode_mt<OX, OW, 1, true>(a, p, partials, counters, s);
    }
    hipError_t e;
    if (mt == 4)
        e = launch_decode_mt<OX, OW, 4, false>(a, p, partials, nullptr, s);
    else if (mt == 2)
        e = launch_decode_mt<OX, OW, 2, false>(a, p, partials, nullptr, s);
    else
        e = launch_decode_mt<OX, OW, 1, false>(a, p, partials, nullptr, s);
    if (e != hipSuccess || p.tiles_k == 1 || !fold)
        return e;
    k_decode_fold<<<dim3((unsigned)p.ntiles, (unsigned)p.mtiles), 64, 0, s>>>(a, p.tiles_k, partials);
    return hipGetLastError();
}

template <typename OX, typename OW, int NW>
static hipError_t launch_decode_wg_nw(const LinearArgs& a, const Plan& p, hipStream_t s)
{
    const dim3 grid((unsigned)p.ntiles, (unsigned)p.mtiles);
    const size_t lds = (size_t)p.tiles_k * 64 * sizeof(f32x4);
    // CH k blocks per chunk, two chunks in flight; CH must divide kbpt.  The
    // register budget per wave shrinks as NW grows (NW / 4 waves per SIMD).
    constexpr int kMaxCH = (OX::f32_frag ? 2 : 4) * (NW <= 4 ? 2 : 1);
    int ch = 1;
    for (int c = kMaxCH; c >= 1; c >>= 1)
        if (p.kbpt % c == 0) {
            ch = c;
            break;
        }
    if constexpr (kMaxCH >= 8) {
        if (ch == 8) {
            k_decode_wg<OX, OW, 8, NW><<<grid, NW * 64, lds, s>>>(a, p.kbpt, p.tiles_k);
            return hipGetLastError();
        }
    }
    if constexpr (kMaxCH >= 4) {
        if (ch == 4) {
            k_decode_wg<OX, OW, 4, NW><<<grid, NW * 64, lds, s>>>(a, p.kbpt, p.tiles_k);
            return hipGetLastError();
        }
    }
    if (ch == 2)
        k_decode_wg<OX, OW, 2, NW><<<grid, NW * 64, lds, s>>>(a, p.kbpt, p.tiles_k);
    else
        k_decode_wg<OX, OW, 1, NW><<<grid, NW * 64, lds, s>>>(a, p.kbpt, p.tiles_k);
    return hipGetLastError();
}

// The direct-to-LDS decode serves chained bf16 recipes with M <= 64 and K a
// multiple of a phase (16 k blocks at MT = 1, 8 at MT = 2, 4 at MT = 4).
// k blocks per phase for MT M tiles (a phase holds PB x (1 + MT) KiB)
static int dma_phase_blocks(int mtiles) { return mtiles == 1 ? 16 : 8; }

bool decode_dma_ok(const Plan& p, int64_t K)
{
    if (p.recipe.dtype != BI_BF16 || p.tiles_k != 1 || p.mtiles < 1 || p.mtiles > 4)
        return false;
    return K % (dma_phase_blocks(p.mtiles) * kKBlock) == 0;
}

static hipError_t launch_decode_dma(const LinearArgs& a, const Plan& p, hipStream_t s)
{
    if (!decode_dma_ok(p, a.K))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.ntiles);
    // MT chain waves, then the loaders
    auto threads = [](int mt) { return (kDmaLoaders + mt) * 64; };
    // LDS: ring R x PB x (items per block) KiB, plus XR activation rows of
    // up to 8 KiB each
    if (p.mtiles == 1 && a.K <= kDmaXMaxK && a.M == 1)
        k_decode_dma<1, 16, 8, 1><<<grid, threads(1), 0, s>>>(a);      // 128 + 8 KiB
    else if (p.mtiles == 1 && a.K <= kDmaXMaxK && a.M <= 4)
        k_decode_dma<1, 16, 7, 4><<<grid, threads(1), 0, s>>>(a);      // 112 + 32 KiB
    else if (p.mtiles == 1 && a.K <= kDmaXMaxK && a.M <= 8)
        k_decode_dma<1, 16, 5, 8><<<grid, threads(1), 0, s>>>(a);      // 80 + 64 KiB
    else if (p.mtiles == 1)
        k_decode_dma<1, 16, 4, 0><<<grid, threads(1), 0, s>>>(a);      // 128 KiB, activation in the ring
    else if (p.mtiles == 2)
        k_decode_dma<2, 8, 4, 0><<<grid, threads(2), 0, s>>>(a);       // 96 KiB
    else
        k_decode_dma<4, 8, 3, 0><<<grid, threads(4), 0, s>>>(a);       // 120 KiB (3 M tiles read a clamped 4th)
    return hipGetLastError();
}

template <typename OX, typename OW>
static hipError_t launch_decode_wg(const LinearArgs& a, const Plan& p, hipStream_t s)
{
    if (p.tiles_k < 2 || p.tiles_k > kDecodeWgMaxTiles)
        return hipErrorInvalidValue;
    if (p.tiles_k >= 16)
        return launch_decode_wg_nw<OX, OW, 16>(a, p, s);
    if (p.tiles_k >= 8)
        return launch_decode_wg_nw<OX, OW, 8>(a, p, s);
    return launch_decode_wg_nw<OX, OW, 4>(a, p, s);
}

template <typename OX, typename OW, int BM, int BN, int WM, int WN, int KBS, int PD = 2, int PDC = PD>
static hipError_t launch_persistent_t(const LinearArgs& a, const Plan& p, hipStream_t s)
{
    // the k loop walks whole stages: K must be a multiple of the stage width
    if (a.K % (KBS * kKBlock) != 0)
        return hipErrorInvalidValue;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int grid = min(tiles, device_cu_count() * 2);
    const XcdBlock xb = xcd_block(tiles_m, tiles_n, BM, BN, grid);
    // a k tile must hold whole stages (the kernel folds between stages)
    if (p.tiles_k != 1 && p.kbpt % KBS != 0)
        return hipErrorInvalidValue;
    if (p.tiles_k == 1) {
        k_persistent<OX, OW, BM, BN, WM, WN, KBS, PDC, true><<<grid, WM * WN * 64, 0, s>>>(a, p.kbpt, tiles_m, tiles_n,
                                                                                           xb.xbm, xb.xbn);
    } else {
        // the largest tiles exist only in the chained form (the dispatcher
        // never selects them for a recipe with several k tiles)
        if constexpr (BM * BN >= 256 * 256)
            return hipErrorInvalidValue;
        else
            k_persistent<OX, OW, BM, BN, WM, WN, KBS, PD, false><<<grid, WM * WN * 64, 0, s>>>(a, p.kbpt, tiles_m,
                                                                                              tiles_n, xb.xbm, xb.xbn);
    }
    return hipGetLastError();
}

// ------------------------------- fp32 BMx32 tiles fed by a ring of 64-k stages

// fp32 recipes with tile partials at mid M (the router at M = 1024 and 2048:
// one tile per compute unit).  Every output element's tile partial is one
// chain of dependent MFMAs (the recipe's chain from +0 over the k tile's
// blocks, ascending), so a SIMD only keeps its matrix unit busy when it holds
// several independent chains.  Here the chains are the BM/16 x 2 sub-tiles of
// 16x16 times PAR k tiles worked on at once: eight waves, two per SIMD, wave
// w takes sub-tile w % S (S = BM/8) and the C = PAR S / 8 consecutive k tiles
// C (w / S) .. C (w / S) + C - 1 of every group of PAR k tiles.  At the end of
// each group the waves past the first hand their partials to the first
// through LDS, which adds the group's partials in ascending tile order
// (acc = P0; acc = acc + P1; ...) -- the same fold as every other path, then
// the bias once.
//
// X and W stream into a ring of R units by direct-to-LDS loads; a unit is one
// 64-k stage of one k tile (BM X rows, then 32 W rows, of 256 bytes), and a
// step consumes PAR units, one per k tile of the group.  At step j the loads
// of units PAR j + R .. PAR j + R + PAR - 1 are issued: each lands in the slot
// of a unit whose fragments were read during step j - 1 or earlier (the
// barrier that opens step j follows every wave's wait for its fragment
// reads), while the fragments of step j + 1 are read and step j's MFMAs
// issue.  Past the last step the loads re-read the last stage into slots no
// later step uses, so that every step is the same.
//
// Stage layout: chunk c of row q at position c ^ (q & 15), the layout of the
// register-staged fp32 kernels' 64-k stages (measured free of bank conflicts
// for the fragment reads; 128-byte rows of 32-k stages are not, with either
// key tried).  A direct-to-LDS load covers 4 rows (1 KiB); lane i lands at
// row i / 16, position i % 16, and so fetches chunk (i % 16) ^ (row & 15).
//
// SPLIT: the k tiles of one output tile are split evenly over ksplit
// workgroups (workgroup b takes tile b % tiles, part b / tiles), so that a
// grid of tiles x ksplit workgroups fills the chip when the tiles alone
// would not.  Part 0 folds its k tiles as above into a prefix (acc after
// its last k tile); a later part cannot add its partials to anything yet,
// so every one of its waves stores each k tile's partial as soon as the
// tile is done.  The tile count is a multiple of 8, so every part of a tile
// runs on the same XCD (workgroups go to the XCDs round-robin) and meets the
// others in that L2: a workgroup's stores are complete there before it
// counts itself in at the tile's counter, and the part that arrives last
// drops its L1 and finishes the fold in ascending k tile order -- the
// prefix, then each later partial -- then adds the bias: the same
// operations as one workgroup doing the whole k range, and no workgroup
// ever waits for another.  The counter wraps to zero at the last arrival.
//
// SPT: stages per k tile fixed at compile time (0: kbpt / 2 at run time).
// With it fixed the step loop is unrolled over whole k tiles and a chain's
// first MFMA takes a zero accumulator itself; a run-time choice between zero
// and the running sum is a select on the previous MFMA's result, which makes
// every step wait for the matrix pipe to drain (the same bits either way).
template <int BM, int PAR, int R, bool SPLIT = false, int SPT = 0>
__global__ __launch_bounds__(512) void k_ring_f32(LinearArgs a, int kbpt, int tiles_k, int tiles_m, int tiles_n,
                                                  int xbm, int xbn, int ksplit = 1,
                                                  f32x4* __restrict__ partials = nullptr,
                                                  uint32_t* __restrict__ counters = nullptr)
{
    constexpr int kRow = 256;                               // 64 k of fp32
    constexpr int kUnit = (BM + 32) * kRow;
    constexpr int S = BM / 8;                               // 16x16 sub-tiles
    constexpr int G = 8 / S;                                // wave groups
    constexpr int C = PAR / G;                              // chains per wave
    constexpr int LPU = (BM + 32) / 32;                     // 1 KiB loads per unit and wave
    static_assert((BM == 32 || BM == 64) && C >= 1 && C * G == PAR && R >= 2 * PAR, "ring shape");
    __shared__ __attribute__((aligned(16))) unsigned char ring[R * kUnit];
    __shared__ f32x4 hand[G > 1 ? (G - 1) * S * C : 1][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = w % S, grp = w / S;
    const int sm = sub >> 1, sn = sub & 1;
    const int r = lane & 15, g = lane >> 4;
    const int spt = SPT > 0 ? SPT : kbpt / 2;               // stages per k tile
    const int kts = tiles_k / ksplit;                       // k tiles of this workgroup
    const int nsteps = (kts / PAR) * spt;
    const int tiles = tiles_m * tiles_n;
    const int part = SPLIT ? (int)blockIdx.x / tiles : 0;
    const int kt0 = part * kts;                             // its first k tile
    const int st_end = (kt0 + kts) * spt;                   // one past its last stage
    // a later part stores its partials instead of folding them
    const bool stores = SPLIT && part > 0;
    const float* xg = reinterpret_cast<const float*>(a.x);
    const float* wg = reinterpret_cast<const float*>(a.w);
    const uint32_t lds0 = lds_addr(ring);
    // lane (r, g) of a fragment reads chunks 2g, 2g+1 of k block b of row
    // r of its sub-tile's X rows (W rows); the key of those rows is r
    const unsigned char* fx = ring + (sm * 16 + r) * kRow;
    const unsigned char* fw = ring + (BM + sn * 16 + r) * kRow;
    // the wave index is uniform; reading it through the scalar unit lets
    // the choice of X or W (whole 4-row groups) stay a scalar base
    const int wu = __builtin_amdgcn_readfirstlane(w);

    for (int it = SPLIT ? (int)blockIdx.x % tiles : (int)blockIdx.x; it < tiles; it += SPLIT ? tiles : gridDim.x) {
        const int tile = xcd_tile(it, tiles_n, xbm, xbn);
        const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * 32;
        // wave w loads the 4-row groups w LPU .. w LPU + LPU - 1 of each unit
        // (X rows 0..BM-1, then W rows); rows past M (N) read row M-1 (N-1),
        // whose results are never stored
        const unsigned char* xt = reinterpret_cast<const unsigned char*>(xg + (int64_t)m0 * a.ldx);
        const unsigned char* wt = reinterpret_cast<const unsigned char*>(wg + (int64_t)n0 * a.ldw);
        uint32_t voff[LPU];
        bool isx[LPU];
#pragma unroll
        for (int t = 0; t < LPU; ++t) {
            const int q = 4 * (wu * LPU + t) + (lane >> 4);
            const int chunk = (lane & 15) ^ (q & 15);
            isx[t] = wu * LPU + t < BM / 4;
            voff[t] = isx[t] ? (uint32_t)((int64_t)(min(m0 + q, a.M - 1) - m0) * a.ldx * 4 + chunk * 16)
                             : (uint32_t)((int64_t)(min(n0 + q - BM, a.N - 1) - n0) * a.ldw * 4 + chunk * 16);
        }
        // unit u = PAR j + h: stage j % spt of k tile PAR (j / spt) + h, in
        // slot u % R
        auto issue_unit = [&](int u) {
            const int j = u / PAR, h = u % PAR;
            const int st = min((kt0 + PAR * (j / spt) + h) * spt + j % spt, st_end - 1);
            const uint32_t slot = lds0 + (uint32_t)(u % R) * kUnit + wu * LPU * 1024;
#pragma unroll
            for (int t = 0; t < LPU; ++t)
                dma16s(voff[t], (isx[t] ? xt : wt) + (int64_t)st * 256,
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(slot + t * 1024)));
        };
        // the fragments of this wave's chains at step j
        auto frags = [&](Frag<true> (&A)[C][2], Frag<true> (&B)[C][2], int j) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int slot = (PAR * j + grp * C + c) % R;
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int c0 = b * 8 + 2 * g;
                    A[c][b].lo = *reinterpret_cast<const f32x4*>(fx + slot * kUnit + (((c0) ^ r) << 4));
                    A[c][b].hi = *reinterpret_cast<const f32x4*>(fx + slot * kUnit + (((c0 + 1) ^ r) << 4));
                    B[c][b].lo = *reinterpret_cast<const f32x4*>(fw + slot * kUnit + (((c0) ^ r) << 4));
                    B[c][b].hi = *reinterpret_cast<const f32x4*>(fw + slot * kUnit + (((c0 + 1) ^ r) << 4));
                }
            }
        };
        // workspace slot q of this tile (slot 0: part 0's prefix; slot
        // kt - kts + 1: the partial of k tile kt of a later part), this
        // wave's 16x16 sub-tile
        const int nslots = tiles_k - kts + 1;
        auto slot_ptr = [&](int q) {
            return partials + ((int64_t)(it * nslots + q) * S + sub) * 64 + lane;
        };
        // the group's partials in ascending k tile order, after the barrier
        // that follows the hand-over
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        f32x4 P[C];
        auto fold = [&](bool first) {
#pragma unroll
            for (int c = 0; c < C; ++c)
                acc = (first && c == 0) ? P[c] : acc + P[c];
#pragma unroll
            for (int q = 1; q < G; ++q)
#pragma unroll
                for (int c = 0; c < C; ++c)
                    acc = acc + hand[((q - 1) * S + sub) * C + c][lane];
        };

        // the previous tile's fragment and hand-over reads are done
        // everywhere before the ring is refilled
        wait_lgkm0();
        bar();
#pragma unroll
        for (int u = 0; u < R; ++u)
            issue_unit(u);
        // step 0 has landed
        wait_vm<(R - PAR) * LPU>();
        bar();
        Frag<true> Aa[C][2], Ba[C][2], Ab[C][2], Bb[C][2];
        frags(Aa, Ba, 0);

        // step j: step j + 1 is visible (this wave's loads of it waited for,
        // then the barrier); the next step's fragments are read while this
        // step's MFMAs issue, the chains interleaved block by block
        auto step = [&](int j, auto ph, const Frag<true> (&A)[C][2], const Frag<true> (&B)[C][2],
                        Frag<true> (&An)[C][2], Frag<true> (&Bn)[C][2]) {
            // the step's place in its k tile: fixed at compile time where the
            // loop is unrolled over whole k tiles, so that a chain's first
            // MFMA takes a zero accumulator without a select
            constexpr int PH = decltype(ph)::value, SP = SPT > 0 ? SPT : 1;
            const bool first = PH >= 0 ? PH % SP == 0 : j % spt == 0;
            const bool last = PH >= 0 ? PH % SP == SP - 1 : j % spt == spt - 1;
            wait_vm<(R - 2 * PAR) * LPU>();
            wait_lgkm0();
            bar();
            if (j > 0 && first && grp == 0 && !stores)
                fold(j == spt);
#pragma unroll
            for (int h = 0; h < PAR; ++h)
                issue_unit(PAR * j + R + h);
            frags(An, Bn, j + 1);
            if (first) {
#pragma unroll
                for (int c = 0; c < C; ++c)
                    P[c] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
#define BI_RING_STEP(SS)                                                      \
                for (int c = 0; c < C; ++c)                                   \
                    P[c] = mfma_f32_step<SS>(A[c][b], B[c][b], P[c]);
#pragma unroll
                BI_RING_STEP(0)
#pragma unroll
                BI_RING_STEP(1)
#pragma unroll
                BI_RING_STEP(2)
#pragma unroll
                BI_RING_STEP(3)
#pragma unroll
                BI_RING_STEP(4)
#pragma unroll
                BI_RING_STEP(5)
#pragma unroll
                BI_RING_STEP(6)
#pragma unroll
                BI_RING_STEP(7)
#undef BI_RING_STEP
            }
            if (stores) {
                // k tile kt0 + PAR (j / spt) + C grp + c is complete
                if (last) {
#pragma unroll
                    for (int c = 0; c < C; ++c)
                        *slot_ptr(kt0 - kts + PAR * (j / spt) + grp * C + c + 1) = P[c];
                }
            } else if (G > 1 && last && grp > 0) {
#pragma unroll
                for (int c = 0; c < C; ++c)
                    hand[((grp - 1) * S + sub) * C + c][lane] = P[c];
            }
        };
        using Run = std::integral_constant<int, -1>;
        if constexpr (SPT == 0) {
            for (int j = 0; j < nsteps; j += 2) {
                step(j, Run{}, Aa, Ba, Ab, Bb);
                step(j + 1, Run{}, Ab, Bb, Aa, Ba);
            }
        } else if constexpr (SPT <= 2) {
            for (int j = 0; j < nsteps; j += 2) {
                step(j, std::integral_constant<int, 0>{}, Aa, Ba, Ab, Bb);
                step(j + 1, std::integral_constant<int, 1>{}, Ab, Bb, Aa, Ba);
            }
        } else {
            static_assert(SPT == 4, "stages per k tile");
            for (int j = 0; j < nsteps; j += 4) {
                step(j, std::integral_constant<int, 0>{}, Aa, Ba, Ab, Bb);
                step(j + 1, std::integral_constant<int, 1>{}, Ab, Bb, Aa, Ba);
                step(j + 2, std::integral_constant<int, 2>{}, Aa, Ba, Ab, Bb);
                step(j + 3, std::integral_constant<int, 3>{}, Ab, Bb, Aa, Ba);
            }
        }
        // the last group: its hand-over is in LDS after one more barrier
        wait_vm<0>();
        wait_lgkm0();
        bar();
        if (grp == 0 && !stores)
            fold(nsteps == spt);
        const int row = m0 + sm * 16 + acc_row(lane, 0), col = n0 + sn * 16 + acc_col(lane);
        if constexpr (!SPLIT) {
            if (grp == 0)
                store_acc(a, row, col, acc);
        } else {
            if (part == 0 && grp == 0)
                *slot_ptr(0) = acc;
            // this workgroup's stores are complete in the XCD's L2 before
            // it counts itself in
            wait_vm<0>();
            __shared__ uint32_t last;
            __syncthreads();
            if (threadIdx.x == 0)
                last = __builtin_amdgcn_atomic_inc32(counters + it * kCounterStride, (uint32_t)(ksplit - 1),
                                                     __ATOMIC_RELAXED, "workgroup") == (uint32_t)(ksplit - 1);
            __syncthreads();
            if (!last)
                return;
            // last arrival: drop stale L1 lines, then the prefix and every
            // later partial in ascending k tile order, up to 32 per round trip
            asm volatile("buffer_inv sc0" ::: "memory");
            if (grp == 0) {
                f32x4 r = part == 0 ? acc : *slot_ptr(0);
                constexpr int kB = 16;
                for (int q0 = 1; q0 < nslots; q0 += kB) {
                    f32x4 v[kB];
#pragma unroll
                    for (int i = 0; i < kB; ++i)
                        if (q0 + i < nslots)
                            v[i] = *slot_ptr(q0 + i);
#pragma unroll
                    for (int i = 0; i < kB; ++i)
                        if (q0 + i < nslots)
                            r = r + v[i];
                }
                store_acc(a, row, col, r);
            }
        }
    }
}

// What the fp32 ring kernel needs: a number of k tiles that PAR divides, each
// an even number of 32-k blocks (at least four where partials are handed
// over, so that a hand-over slot is read before it is written again), an even
// number of steps, and byte offsets inside a tile's rows that fit 32 bits.
static bool ring_f32_ok(const LinearArgs& a, const Plan& p, int bm, int par)
{
    const int spt = p.kbpt / 2;
    const bool hands = bm == 32;
    return p.tiles_k >= par && p.tiles_k % par == 0 && p.kbpt >= (hands ? 4 : 2) && p.kbpt % 2 == 0 &&
           ((p.tiles_k / par) * spt) % 2 == 0 && a.K % 64 == 0 &&
           (int64_t)(bm - 1) * a.ldx * 4 + (int64_t)a.K * 4 < (int64_t(1) << 32) &&
           (int64_t)31 * a.ldw * 4 + (int64_t)a.K * 4 < (int64_t(1) << 32);
}

// k tiles of 4 or 8 32-k blocks (2 on the 64-row tile) run the step loop
// unrolled over whole k tiles, with each step's place in its k tile known at
// compile time; other even block counts keep it a run-time value
template <int BM, int PAR, int R, bool SPLIT>
static void ring_f32_kernel(int kbpt, int grid, hipStream_t s, const LinearArgs& a, int kb, int tiles_k,
                            int tiles_m, int tiles_n, int xbm, int xbn, int ks, f32x4* partials, uint32_t* counters)
{
    const dim3 g((unsigned)grid), b(512);
    if (BM == 64 && kbpt == 2)
        k_ring_f32<BM, PAR, R, SPLIT, 1><<<g, b, 0, s>>>(a, kb, tiles_k, tiles_m, tiles_n, xbm, xbn, ks, partials,
                                                          counters);
    else if (kbpt == 4)
        k_ring_f32<BM, PAR, R, SPLIT, 2><<<g, b, 0, s>>>(a, kb, tiles_k, tiles_m, tiles_n, xbm, xbn, ks, partials,
                                                          counters);
    else if (kbpt == 8)
        k_ring_f32<BM, PAR, R, SPLIT, 4><<<g, b, 0, s>>>(a, kb, tiles_k, tiles_m, tiles_n, xbm, xbn, ks, partials,
                                                          counters);
    else
        k_ring_f32<BM, PAR, R, SPLIT><<<g, b, 0, s>>>(a, kb, tiles_k, tiles_m, tiles_n, xbm, xbn, ks, partials,
                                                       counters);
}

template <int BM, int PAR, int R>
static hipError_t launch_ring_f32(const LinearArgs& a, const Plan& p, hipStream_t s)
{
    if (!ring_f32_ok(a, p, BM, PAR))
        return hipErrorInvalidValue;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + 31) / 32;
    const int grid = min(tiles_m * tiles_n, device_cu_count());
    const XcdBlock xb = xcd_block(tiles_m, tiles_n, BM, 32, grid);
    ring_f32_kernel<BM, PAR, R, false>(p.kbpt, grid, s, a, p.kbpt, p.tiles_k, tiles_m, tiles_n, xb.xbm, xb.xbn, 1,
                                       nullptr, nullptr);
    return hipGetLastError();
}

// The k split of the ring-fed tiles (tile codes 28: 32x32, 29: 64x32): the
// largest power of two S >= 2 for which tiles x S workgroups fit one per
// compute unit and every part holds a whole number of k tile groups, with
// the tile count a multiple of 8 (every part of a tile on one XCD) and at
// most one counter per tile; 0 where no split serves (the launcher then runs
// the unsplit ring tile of the same shape).
static bool ring_split_ok(const LinearArgs& a, const Plan& p, int bm, int par, int ks)
{
    if (p.tiles_k % ks != 0)
        return false;
    Plan q = p;
    q.tiles_k = p.tiles_k / ks;
    return ring_f32_ok(a, q, bm, par);
}

RingSplit ring_split_plan(const Plan& p, int64_t M, int64_t N, int64_t K, int code)
{
    RingSplit r{};
    if (code != 28 && code != 29)
        return r;
    const int bm = code == 28 ? 32 : 64;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + 31) / 32);
    if (tiles % 8 != 0 || tiles > kDecodeMaxCounters)
        return r;
    LinearArgs a{};
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.ldx = a.K;
    a.ldw = a.K;
    const int cus = device_cu_count();
    for (int ks = 2; tiles * ks <= cus && ks <= p.tiles_k; ks *= 2) {
        for (int par : {4, 2}) {
            if (bm == 64 && par == 4)
                continue;
            if (ring_split_ok(a, p, bm, par, ks)) {
                r.ksplit = ks;
                r.par = par;
                r.bm = bm;
                r.tiles = (int)tiles;
                break;
            }
        }
    }
    if (r.ksplit) {
        const int64_t nslots = p.tiles_k - p.tiles_k / r.ksplit + 1;
        r.ws_bytes = kDecodeCounterBytes + (size_t)tiles * (size_t)nslots * (size_t)(bm / 8) * 64 * 16;
    }
    return r;
}

template <int BM, int PAR, int R>
static hipError_t launch_ring_f32_split(const LinearArgs& a, const Plan& p, void* ws, hipStream_t s)
{
    const int ks = p.ksplit;
    if (!ws || ks < 2 || !ring_split_ok(a, p, BM, PAR, ks))
        return hipErrorInvalidValue;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + 31) / 32;
    const int tiles = tiles_m * tiles_n;
    if (tiles % 8 != 0 || tiles > kDecodeMaxCounters)
        return hipErrorInvalidValue;
    const XcdBlock xb = xcd_block(tiles_m, tiles_n, BM, 32, tiles);
    uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
    f32x4* partials = reinterpret_cast<f32x4*>(reinterpret_cast<char*>(ws) + kDecodeCounterBytes);
    ring_f32_kernel<BM, PAR, R, true>(p.kbpt, tiles * ks, s, a, p.kbpt, p.tiles_k, tiles_m, tiles_n, xb.xbm, xb.xbn,
                                      ks, partials, counters);
    return hipGetLastError();
}

// Persistent tile shapes (BM x BN, waves WM x WN, k blocks per LDS stage).
// Code 0 picks automatically: the largest tile that still gives every compute
// unit a tile.  Tiling never changes the numerics, only the speed.
template <typename OX, typename OW>
static hipError_t launch_persistent(const LinearArgs& a, const Plan& p, void* ws, hipStream_t s)
{
    const int cus = device_cu_count();
    auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
    int code = p.tile_code;
    // stage width of each shape, in k: shapes whose stage does not fit fall
    // back to the 32-k-stage shape of the same dtype
    auto stage_k = [](int c) {
        return (c == 7 || c == 8 || c == 17) ? 32 : (c == 9 || c == 10 || c == 13 || c == 16) ? 128 : 64;
    };
    // a stage must divide K and, with several k tiles, the k tile too
    auto stage_fits = [&](int c) {
        const int kbs = stage_k(c) / kKBlock;
        return a.K % stage_k(c) == 0 && (p.tiles_k == 1 || p.kbpt % kbs == 0);
    };
    if constexpr (OX::f32_frag) {
        // measured on MI355X for the (fp32, 256, 4096) router with cold
        // weights: the ring-fed 32x32 tile up to M = 1024 (28.6 us there;
        // register-staged 32x32: 36.8 us), the ring-fed 64x32 tile at
        // M = 2048 (44.6 us; 52.2 us), 64x64 on 8 waves from M = 4096
        // the ring-fed shapes stream fp32 rows as they are: operands widened
        // from bf16 (the MoE router's activations) take the register-staged
        // shapes
        constexpr bool rings = std::is_same<OX, F32>::value && std::is_same<OW, F32>::value;
        if (code == 0)
            code = tiles(64, 64) >= cus ? 4 : !rings ? 3 : tiles(64, 32) >= cus ? 24 : 23;
        if constexpr (rings) {
            // the ring-fed 32x32 tile works on four k tiles at once where
            // their number allows, else on two; the 64x32 tile on two
            // the k-split forms; the planner set p.ksplit (0: the tiles fill
            // the chip or no split serves, and the unsplit tile runs)
            if (code == 28 && p.ksplit >= 2 && ring_split_ok(a, p, 32, 4, p.ksplit))
                return launch_ring_f32_split<32, 4, 8>(a, p, ws, s);
            if (code == 28 && p.ksplit >= 2 && ring_split_ok(a, p, 32, 2, p.ksplit))
                return launch_ring_f32_split<32, 2, 8>(a, p, ws, s);
            if (code == 29 && p.ksplit >= 2 && ring_split_ok(a, p, 64, 2, p.ksplit))
                return launch_ring_f32_split<64, 2, 6>(a, p, ws, s);
            if (code == 28)
                code = 23;
            if (code == 29)
                code = 24;
            if (code == 23 && ring_f32_ok(a, p, 32, 4))
                return launch_ring_f32<32, 4, 8>(a, p, s);
            if (code == 23 && ring_f32_ok(a, p, 32, 2))
                return launch_ring_f32<32, 2, 8>(a, p, s);
            if (code == 24 && ring_f32_ok(a, p, 64, 2))
                return launch_ring_f32<64, 2, 6>(a, p, s);
        }
        if (code == 23 || code == 24 || code == 28 || code == 29)
            code = 3;
        if (!stage_fits(code))
            code = 7;
        switch (code) {
        case 1: return launch_persistent_t<OX, OW, 64, 64, 2, 2, 2>(a, p, s);
        case 2: return launch_persistent_t<OX, OW, 32, 64, 2, 2, 2>(a, p, s);
        case 3: return launch_persistent_t<OX, OW, 32, 32, 2, 2, 2>(a, p, s);
        case 4: return launch_persistent_t<OX, OW, 64, 64, 4, 2, 2>(a, p, s);
        case 5: return launch_persistent_t<OX, OW, 128, 64, 4, 2, 2>(a, p, s);
        case 6: return launch_persistent_t<OX, OW, 64, 128, 2, 4, 2>(a, p, s);
        case 8: return launch_persistent_t<OX, OW, 64, 256, 2, 4, 1>(a, p, s);
        case 9: return launch_persistent_t<OX, OW, 32, 64, 2, 2, 4>(a, p, s);
        case 10: return launch_persistent_t<OX, OW, 64, 64, 4, 2, 4>(a, p, s);
        default: return launch_persistent_t<OX, OW, 32, 32, 2, 2, 1>(a, p, s);
        }
    } else {
        // measured on MI355X for the (bf16, 4096, 4096) GEMM: 256x256 fed by
        // the 32-k ring at M=4096 (112-120 us; register-staged 256x256:
        // 134-140 us; 128x256: 161 us); 64x64 at M=256 (25 us)
        if (code == 0) {
            if (p.tiles_k == 1 && tiles(256, 256) >= cus)
                code = 21;
            else
                code = tiles(128, 256) >= cus ? 15 : 12;
        }
        if (!stage_fits(code))
            code = 17;
        // 256x256 tiles only fit the registers without tile partials
        if ((code == 18 || code == 19) && p.tiles_k != 1)
            code = 15;
        if (code == 20) {
            if (a.K % (2 * kKBlock) == 0 && (p.tiles_k == 1 || p.kbpt % 2 == 0))
                return launch_stream_bf16(a, p, s);
            code = 12;
        }
        if (code == 21 || code == 22) {
            if (ring_ok(a, p, 256, 256))
                return code == 21 ? launch_ring_bf16<256, 256, 4, 2, 4, 4>(a, p, s)
                                  : launch_ring_bf16<256, 256, 4, 2, 4, 8>(a, p, s);
            code = p.tiles_k == 1 ? 19 : 15;
        }
        switch (code) {
        case 11: return launch_persistent_t<OX, OW, 128, 128, 2, 2, 2>(a, p, s);
        case 12: return launch_persistent_t<OX, OW, 64, 64, 2, 2, 2>(a, p, s);
        case 13: return launch_persistent_t<OX, OW, 128, 128, 2, 2, 4>(a, p, s);
        case 14: return launch_persistent_t<OX, OW, 256, 128, 4, 2, 2, 1, 1>(a, p, s);
        case 15: return launch_persistent_t<OX, OW, 128, 256, 2, 4, 2, 1, 1>(a, p, s);
        case 18: return launch_persistent_t<OX, OW, 256, 256, 2, 4, 2, 1, 1>(a, p, s);
        case 19: return launch_persistent_t<OX, OW, 256, 256, 4, 2, 2, 1, 1>(a, p, s);
        case 16: return launch_persistent_t<OX, OW, 64, 128, 2, 2, 4>(a, p, s);
        default: return launch_persistent_t<OX, OW, 64, 64, 2, 2, 1>(a, p, s);
        }
    }
}

template <typename OX, typename OW>
static hipError_t launch_typed(const LinearArgs& a, const Plan& p, void* ws, hipStream_t s, bool fold)
{
    if (p.path == kPathDecodeWg && fold)
        return launch_decode_wg<OX, OW>(a, p, s);
    if constexpr (!OX::f32_frag) {
        if (p.path == kPathDecodeDma)
            return launch_decode_dma(a, p, s);
    }
    if (p.path == kPathDecode || p.path == kPathDecodeWg || p.path == kPathDecodeXcd)
        return launch_decode<OX, OW>(a, p, ws, s, fold);
    return launch_persistent<OX, OW>(a, p, ws, s);
}

hipError_t launch_linear(int xkind, const LinearArgs& a, const Plan& p, void* ws, hipStream_t s, bool fold)
{
    if (p.recipe.dtype == BI_F32) {
        if (xkind == kXF32)
            return launch_typed<F32, F32>(a, p, ws, s, fold);
        return launch_typed<BF16W, F32>(a, p, ws, s, fold);
    }
    return launch_typed<BF16, BF16>(a, p, ws, s, fold);
}

}  // namespace bi
