// bi_noalloc.hip -- bi_linear_f32 for callers that cannot allocate.
//
// Some callers may not allocate device memory at all (code under HIP graph
// capture, tight serving loops, harnesses that forbid it) and so cannot hand
// the router a workspace.  bi_linear_f32_noalloc runs the same plan and the
// same kernels as bi_linear_f32, with the workspace replaced by `scratch`: a
// file-scope device array of kNoallocScratchBytes that each GPU the library
// runs on holds until the process ends.  Its first kDecodeCounterBytes are
// the decode's arrival counters, cleared once per device at set-up and left
// at zero by every call; the rest holds tile partials, which every call
// writes before it reads them.  All calls on one GPU share this array, so two
// calls that overlap on one GPU race; calls on different GPUs do not.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bi.h"
#include "bi_launch.h"
#include "bi_plan.h"

namespace bi {

// 16 MiB of tile partials: the largest decode workspace any fp32 key of the
// compiled table needs up to its decode limit (router (256, 7168) at M = 512:
// 14 MiB), plus the counter region.
constexpr size_t kNoallocScratchBytes = (size_t(16) << 20) + kDecodeCounterBytes;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];       // address of `scratch` on each device
hipError_t g_setup[kMaxDevices];    // result of each device's set-up

__global__ void k_zero_words(uint32_t* __restrict__ p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

// Once per device, with that device current: the device address of
// `scratch` (host code must never pass the array's name itself to a kernel)
// and a cleared counter region (a fill kernel, not a memset, so that a
// first call under graph capture records no memset node).
void setup(int dev, hipStream_t stream)
{
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e == hipSuccess && ptr == nullptr)
        e = hipErrorInvalidSymbol;
    if (e == hipSuccess) {
        const int words = (int)(kDecodeCounterBytes / 4);
        k_zero_words<<<(words + 255) / 256, 256, 0, stream>>>(reinterpret_cast<uint32_t*>(ptr), words);
        e = hipGetLastError();
    }
    g_scratch[dev] = e == hipSuccess ? ptr : nullptr;
    g_setup[dev] = e;
}

}  // namespace

}  // namespace bi

using namespace bi;

extern "C" bi_status_t bi_linear_f32_noalloc(const float* x, int64_t ldx, const float* w, int64_t ldw,
                                             const float* bias, float* y, int64_t ldy, int64_t M, int64_t N,
                                             int64_t K, hipStream_t stream)
{
    size_t need = 0;
    bi_status_t st = linear_f32_checked(x, ldx, w, ldw, bias, y, ldy, M, N, K, &need);
    if (st != BI_OK || M == 0)
        return st;
    // a k-split plan whose partials do not fit runs its tiles unsplit (the
    // same bits, no workspace)
    bool no_split = false;
    if (need > kNoallocScratchBytes) {
        size_t need_unsplit = 0;
        if (linear_f32_checked(x, ldx, w, ldw, bias, y, ldy, M, N, K, &need_unsplit, true) == BI_OK &&
            need_unsplit <= kNoallocScratchBytes) {
            need = need_unsplit;
            no_split = true;
        }
    }
    if (need > kNoallocScratchBytes)
        return BI_EWORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
            return BI_EHIP;
        std::call_once(g_once[dev], setup, dev, stream);
        if (g_setup[dev] != hipSuccess)
            return BI_EHIP;
        ws = g_scratch[dev];
    }
    return linear_f32_run(x, ldx, w, ldw, bias, y, ldy, M, N, K, ws, need, stream, no_split);
}
