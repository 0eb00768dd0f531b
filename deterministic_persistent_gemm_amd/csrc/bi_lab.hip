// bi_lab.hip -- diagnostic kernels behind the bi_lab_* entry points.
//
// None of them is on the batch-invariant path.  They measure what that path
// is up against on this part: where workgroups run (the XCD hand-over decode
// needs every wave of an output tile on one XCD), what one kernel launch
// costs with nothing in it, how fast the chip streams a cold buffer, and the
// shader clock while every compute unit is busy.  GateLinear page, "Update:
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

}  // namespace bi
