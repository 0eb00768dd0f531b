// bi_lab.hip -- diagnostic kernels behind the bi_lab_* entry points.
//
// None of them is on the batch-invariant path.  They measure what that path
// is up against on this part: where workgroups run (the XCD hand-over decode
// needs every wave of an output tile on one XCD), what one kernel launch
// costs with nothing in it, how fast the chip streams a cold buffer, the
// shader clock while every compute unit is busy, and the rates at which a
// compute unit reads its LDS and issues the recipe's MFMA instructions when
// nothing else is in the way.  GateLinear page, "Update:
// is the M=4096 cost avoidable?": a decode-sized kernel is judged by its
// device time against a launch floor, not by wall time.
#include <hip/hip_runtime.h>

#include "bi_device.h"
#include "bi_launch.h"

namespace bi {

// Workgroup (x, y) writes the id of the XCD it runs on.
__global__ __launch_bounds__(64) void k_xcc_ids(uint32_t* __restrict__ out)
{
    uint32_t v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    if (threadIdx.x == 0)
        out[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = v;
}

hipError_t launch_xcc_ids(uint32_t* out, int gx, int gy, hipStream_t s)
{
    k_xcc_ids<<<dim3((unsigned)gx, (unsigned)gy), 64, 0, s>>>(out);
    return hipGetLastError();
}

// A kernel with nothing in it: its device time is the floor every launch pays.
__global__ void k_empty() {}

hipError_t launch_empty(int grid, int threads, hipStream_t s)
{
    k_empty<<<(unsigned)grid, (unsigned)threads, 0, s>>>();
    return hipGetLastError();
}

// Reads n16 16-byte chunks once (grid-stride, four loads in flight per
// thread) and folds them into one word per workgroup so the loads are kept.
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride)
        acc ^= src[i];
    uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    __shared__ uint32_t red[256];
    red[threadIdx.x] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int j = 1; j < 256; ++j)
            v ^= red[j];
        sink[blockIdx.x] = v;
    }
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, hipStream_t s)
{
    k_stream_read<<<(unsigned)grid, 256, 0, s>>>(reinterpret_cast<const u32x4*>(src), bytes / 16, sink);
    return hipGetLastError();
}

// L2-to-compute-unit delivery rate.  Every workgroup reads the same region
// of n16 16-byte chunks (n16 a power of two, at most 2 MiB, so that after
// its first pass the region stays in each XCD's L2) `iters` times with
// 16-byte loads, eight in flight per lane; each workgroup starts at its own
// offset (and each pass one KiB further on) so that the workgroups of an XCD
// spread over the L2 channels and no pass repeats the previous one's
// addresses.
__global__ __launch_bounds__(256) void k_l2_read(const u32x4* __restrict__ src, int n16, int iters,
                                                 uint32_t* __restrict__ sink)
{
    const int mask = n16 - 1;
    const int rounds = n16 / (256 * 8);
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int it = 0; it < iters; ++it) {
        const int i0 = (int)(((uint32_t)blockIdx.x * 4099u + (uint32_t)it * 64u) & (uint32_t)mask) + threadIdx.x;
        for (int r = 0; r < rounds; ++r) {
            u32x4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = src[(i0 + (r * 8 + j) * 256) & mask];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc ^= v[j];
        }
    }
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    __shared__ uint32_t red[256];
    red[threadIdx.x] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int j = 1; j < 256; ++j)
            x ^= red[j];
        sink[blockIdx.x] = x;
    }
}

hipError_t launch_l2_read(const void* src, int64_t bytes, int iters, uint32_t* sink, int grid, hipStream_t s)
{
    k_l2_read<<<(unsigned)grid, 256, 0, s>>>(reinterpret_cast<const u32x4*>(src), (int)(bytes / 16), iters, sink);
    return hipGetLastError();
}

// Each workgroup's first wave runs `iters` rounds of a dependent chain of 64
// fp32 multiply-adds and records the shader-clock cycles (s_memtime) and the
// constant-rate wall-clock ticks (s_memrealtime) it took.
__global__ __launch_bounds__(64) void k_clock(uint64_t* __restrict__ out, int iters, float seed)
{
    const uint64_t c0 = __builtin_readcyclecounter();
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    float v = seed + (float)threadIdx.x;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 64; ++j)
            v = __builtin_fmaf(v, 0.999999f, 1e-7f);
    }
    const uint64_t c1 = __builtin_readcyclecounter();
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[3 * blockIdx.x] = c1 - c0;
        out[3 * blockIdx.x + 1] = t1 - t0;
        out[3 * blockIdx.x + 2] = __float_as_uint(v);
    }
}

hipError_t launch_clock(uint64_t* out, int grid, int iters, hipStream_t s)
{
    k_clock<<<(unsigned)grid, 64, 0, s>>>(out, iters, 1.0f);
    return hipGetLastError();
}

// LDS read rate.  One workgroup of 16 waves fills 64 KiB of LDS, then every
// lane reads 16-byte chunks `iters` x 4 times; the 64 lanes of a wave take 64
// consecutive chunks (one contiguous KiB, no bank conflicts) and the slice
// moves on by a KiB every round.  Every word read is folded with three-input
// adds (two vector ALU instructions per 16-byte load, which keeps the ALU far
// from limiting the rate); thread 0 records the shader cycles and wall ticks
// of the read loop (between two barriers), and the folded words feed a
// conditional store so that no read can be dropped.
__global__ __launch_bounds__(1024) void k_lds_read(uint64_t* __restrict__ out, int iters)
{
    __shared__ u32x4 buf[4096];
    const int tid = threadIdx.x;
    for (int i = tid; i < 4096; i += 1024)
        buf[i] = u32x4{(uint32_t)i, (uint32_t)i * 2654435761u, (uint32_t)blockIdx.x, 0x9E37u};
    __syncthreads();
    const uint64_t c0 = __builtin_readcyclecounter();
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    uint32_t a0 = 0, a1 = 0;
    int base = tid;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 v = buf[base + j * 1024];
            a0 = a0 + v[0] + v[1];
            a1 = a1 + v[2] + v[3];
        }
        base = (base + 64) & 1023;
    }
    __syncthreads();
    const uint64_t c1 = __builtin_readcyclecounter();
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    if (tid == 0) {
        out[3 * blockIdx.x] = c1 - c0;
        out[3 * blockIdx.x + 1] = t1 - t0;
    }
    if ((a0 ^ a1) == 0xFFFFFFFFu)
        out[3 * blockIdx.x + 2] = 1;
}

hipError_t launch_lds_read(uint64_t* out, int grid, int iters, hipStream_t s)
{
    k_lds_read<<<(unsigned)grid, 1024, 0, s>>>(out, iters);
    return hipGetLastError();
}

// MFMA issue rate on register operands: eight waves per workgroup, each
// running CH independent accumulator chains, eight MFMAs per round taking the
// chains in turn, so that each MFMA depends on the one CH before it (two A
// and four B operands,
// fixed pseudo-random values with random signs and mantissas, as switching
// data costs clock) of the recipe's instruction for `iters` rounds.  Thread
// 0 records shader cycles and wall ticks; the accumulators are folded into a
// conditional store.
__device__ __forceinline__ uint32_t lab_hash(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7FEB352Du;
    x ^= x >> 15;
    x *= 0x846CA68Bu;
    x ^= x >> 16;
    return x;
}

template <bool BF16, int CH>
__global__ __launch_bounds__(512) void k_mfma_rate(uint64_t* __restrict__ out, int iters)
{
    const int tid = threadIdx.x;
    const uint32_t seed = (uint32_t)tid * 0x9E3779B1u ^ (uint32_t)blockIdx.x * 0x85EBCA77u;
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
        acc[c] = f32x4{(float)c, (float)(c + 1), (float)(c + 2), (float)(c + 3)};
    const uint64_t c0 = __builtin_readcyclecounter();
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    if constexpr (BF16) {
        bf16x8 a[2], b[4];
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = (lab_hash(seed + 4u * i + e) & 0x807F807Fu) | 0x3F003F00u;   // +-[0.5, 1)
            if (i < 2)
                a[i] = __builtin_bit_cast(bf16x8, v);
            else
                b[i - 2] = __builtin_bit_cast(bf16x8, v);
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
                acc[c % CH] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c & 1], b[c >> 1], acc[c % CH], 0, 0, 0);
        }
    } else {
        float a[2], b[4];
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const float v = __uint_as_float((lab_hash(seed + i) & 0x807FFFFFu) | 0x3F000000u);
            if (i < 2)
                a[i] = v;
            else
                b[i - 2] = v;
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
                acc[c % CH] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c & 1], b[c >> 1], acc[c % CH], 0, 0, 0);
        }
    }
    __syncthreads();
    const uint64_t c1 = __builtin_readcyclecounter();
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    if (tid == 0) {
        out[3 * blockIdx.x] = c1 - c0;
        out[3 * blockIdx.x + 1] = t1 - t0;
    }
    uint32_t h = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c)
        h ^= __float_as_uint(acc[c][0]) ^ __float_as_uint(acc[c][1]) ^ __float_as_uint(acc[c][2]) ^
             __float_as_uint(acc[c][3]);
    if (h == 0xFFFFFFFFu)
        out[3 * blockIdx.x + 2] = 1;
}

template <bool BF16>
static void launch_mfma_chains(uint64_t* out, int chains, int grid, int iters, hipStream_t s)
{
    switch (chains) {
    case 1:  k_mfma_rate<BF16, 1><<<(unsigned)grid, 512, 0, s>>>(out, iters); break;
    case 2:  k_mfma_rate<BF16, 2><<<(unsigned)grid, 512, 0, s>>>(out, iters); break;
    case 4:  k_mfma_rate<BF16, 4><<<(unsigned)grid, 512, 0, s>>>(out, iters); break;
    default: k_mfma_rate<BF16, 8><<<(unsigned)grid, 512, 0, s>>>(out, iters); break;
    }
}

hipError_t launch_mfma_rate(uint64_t* out, bool bf16, int chains, int grid, int iters, hipStream_t s)
{
    if (bf16)
        launch_mfma_chains<true>(out, chains, grid, iters, s);
    else
        launch_mfma_chains<false>(out, chains, grid, iters, s);
    return hipGetLastError();
}

}  // namespace bi
