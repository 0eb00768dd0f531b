// bi_device.h -- device building blocks shared by every batch-invariant kernel.
//
// The numeric recipe lives here, in one place, so that every kernel path (the
// k-tile-parallel decode kernel, the persistent kernel, the grouped MoE
// kernels) performs the identical sequence of floating-point operations for
// each output element:
//
//   * K is walked in k blocks of 32.  In a block starting at k0, lane l of a
//     wave holds, for its tile row r = l % 16, the eight consecutive operand
//     values k0 + 8g .. k0 + 8g + 7 of slot g = l / 16.
//   * fp32 operands: eight v_mfma_f32_16x16x4_f32 per block, instruction s
//     (s = 0..7, ascending) taking element s of every slot, i.e. the four k
//     values k0+s, k0+8+s, k0+16+s, k0+24+s in slots 0..3.
//   * bf16 operands: one v_mfma_f32_16x16x32_bf16 per block taking all 32.
//   * A tile partial is the chain of these instructions over block_k/32
//     consecutive blocks, started from +0.0; tile partials are added in
//     ascending tile order (acc = P0; acc = acc + P1; ...); bias is added once
//     at the end.
//
// GateLinear page, "A correction to why the key excludes M": chunk
// independence of a chained dot product is a property of how a compiler
// lowers it, not a contract, so the instruction, the slot assignment and the
// tile width are fixed here explicitly rather than left to a lowering.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kKBlock = 32;   // k values per block
constexpr int kSlotLen = 8;   // consecutive k values per lane slot

// Operand kinds.  F32: fp32 in memory, fp32 instruction.  BF16: bf16 in
// memory, bf16 instruction.  BF16W: bf16 in memory, widened exactly to fp32
// and fed to the fp32 instruction (the MoE router reads bf16 activations).
struct F32   { using elem = float;    static constexpr bool f32_frag = true;  static constexpr bool widen = false; };
struct BF16  { using elem = uint16_t; static constexpr bool f32_frag = false; static constexpr bool widen = false; };
struct BF16W { using elem = uint16_t; static constexpr bool f32_frag = true;  static constexpr bool widen = true; };

// One lane's eight operand values of one k block, in instruction form.
template <bool F32Frag> struct Frag;
template <> struct Frag<true>  { f32x4 lo, hi; };   // fp32: elements 0..3, 4..7
template <> struct Frag<false> { u32x4 v; };        // bf16: 8 packed values

template <typename Op> using FragOf = Frag<Op::f32_frag>;

__device__ __forceinline__ f32x4 widen_lo(u32x4 v)
{
    f32x4 r;
    r[0] = __uint_as_float(v[0] << 16); r[1] = __uint_as_float(v[0] & 0xffff0000u);
    r[2] = __uint_as_float(v[1] << 16); r[3] = __uint_as_float(v[1] & 0xffff0000u);
    return r;
}
__device__ __forceinline__ f32x4 widen_hi(u32x4 v)
{
    f32x4 r;
    r[0] = __uint_as_float(v[2] << 16); r[1] = __uint_as_float(v[2] & 0xffff0000u);
    r[2] = __uint_as_float(v[3] << 16); r[3] = __uint_as_float(v[3] & 0xffff0000u);
    return r;
}

// Load one lane's slot (8 consecutive elements at p, 16-byte aligned).
template <typename Op>
__device__ __forceinline__ void load_frag(FragOf<Op>& f, const typename Op::elem* p)
{
    if constexpr (Op::f32_frag && !Op::widen) {
        f.lo = *reinterpret_cast<const f32x4*>(p);
        f.hi = *reinterpret_cast<const f32x4*>(p + 4);
    } else if constexpr (Op::widen) {
        u32x4 v = *reinterpret_cast<const u32x4*>(p);
        f.lo = widen_lo(v);
        f.hi = widen_hi(v);
    } else {
        f.v = *reinterpret_cast<const u32x4*>(p);
    }
}

// The same with a non-temporal hint for data read exactly once (a weight
// slab streamed by one wave): measured on the router's hand-over decode,
// M=1 5.55 -> 5.28 us per call with cold weights.  Widened and bf16
// operands keep the plain load.
template <typename Op>
__device__ __forceinline__ void load_frag_nt(FragOf<Op>& f, const typename Op::elem* p)
{
    if constexpr (Op::f32_frag && !Op::widen) {
        f.lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        f.hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
    } else {
        load_frag<Op>(f, p);
    }
}

template <typename Op>
__device__ __forceinline__ void zero_frag(FragOf<Op>& f)
{
    if constexpr (Op::f32_frag) {
        f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
        f.hi = f.lo;
    } else {
        f.v = u32x4{0u, 0u, 0u, 0u};
    }
}

// One fp32 instruction of a block: step s takes element s of the slot.
template <int S>
__device__ __forceinline__ f32x4 mfma_f32_step(const Frag<true>& a, const Frag<true>& b, f32x4 acc)
{
    const float av = S < 4 ? a.lo[S & 3] : a.hi[S & 3];
    const float bv = S < 4 ? b.lo[S & 3] : b.hi[S & 3];
    return __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
}

// The whole block for one 16x16 output tile, in recipe order.
__device__ __forceinline__ f32x4 mfma_block(const Frag<true>& a, const Frag<true>& b, f32x4 acc)
{
    acc = mfma_f32_step<0>(a, b, acc);
    acc = mfma_f32_step<1>(a, b, acc);
    acc = mfma_f32_step<2>(a, b, acc);
    acc = mfma_f32_step<3>(a, b, acc);
    acc = mfma_f32_step<4>(a, b, acc);
    acc = mfma_f32_step<5>(a, b, acc);
    acc = mfma_f32_step<6>(a, b, acc);
    acc = mfma_f32_step<7>(a, b, acc);
    return acc;
}

__device__ __forceinline__ f32x4 mfma_block(const Frag<false>& a, const Frag<false>& b, f32x4 acc)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                   __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}

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

// Double-buffered walk over nblk k blocks in chunks of CH blocks (CH divides
// nblk): while one buffer's chunk feeds the chains the other buffer's chunk
// is in flight.  load0/load1(c) issue the loads of the chunk starting at
// block c into buffer 0/1, run0/run1(c) feed that chunk to the chains.  The
// steady-state loop issues both of its loads unconditionally and the tail is
// peeled, so every chunk waits only for its own loads; with a load guarded
// by a branch inside the loop the compiler's wait at the join covers the
// loads just issued as well (a full wait before every chunk).
template <int CH, typename L0, typename L1, typename R0, typename R1>
__device__ __forceinline__ void chunk_pipeline(int nblk, L0&& load0, L1&& load1, R0&& run0, R1&& run1)
{
    load0(0);
    int c = 0;
    for (; c + 2 * CH < nblk; c += 2 * CH) {
        load1(c + CH);
        __builtin_amdgcn_sched_barrier(0);
        run0(c);
        load0(c + 2 * CH);
        __builtin_amdgcn_sched_barrier(0);
        run1(c + CH);
    }
    if (c + CH < nblk) {
        load1(c + CH);
        __builtin_amdgcn_sched_barrier(0);
        run0(c);
        run1(c + CH);
    } else {
        __builtin_amdgcn_sched_barrier(0);
        run0(c);
    }
}

// Inclusive prefix sum over the wave's lanes: a Hillis-Steele scan inside
// each row of 16 lanes with DPP row shifts (lanes whose source falls outside
// the row add 0), then the totals of the rows below are added.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Output element a lane owns in a 16x16 accumulator tile: register q of lane
// l is row 4*(l/16) + q, column l % 16.
__device__ __forceinline__ int acc_row(int lane, int q) { return 4 * (lane >> 4) + q; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

}  // namespace bi
