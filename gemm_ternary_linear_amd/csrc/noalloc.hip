// ternary_linear_batch_noalloc: ternary_linear_batch for callers that cannot
// allocate (code under stream capture, tight serving loops, harnesses that
// forbid hipMalloc).  The only scratch the layer's kernels use, the fp32
// partial tiles of a split-K GEMM, lives in a static device array of this
// library instead of the per-stream workspace, so the call never allocates or
// frees.  Each GPU the library runs on holds its own copy of the array until
// the process ends; every call on a GPU shares it, so calls that overlap on
// one GPU (two streams, or two host threads) race.
#include <mutex>

#include "../../include/ternary.h"
#include "internal.h"

namespace ternary {

// The batch call of api.hip; `noalloc` selects the static scratch.
int linear_batch(const ternary_problem *problems, int count, int dtype, hipStream_t stream,
                 bool noalloc);

namespace {

constexpr size_t kScratchBytes = TERNARY_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of each device's `scratch`

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void **out)
{
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        // once per device, with that device current: the array's name in host
        // code is only a stand-in; its device address comes from the runtime
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace ternary

extern "C" int ternary_linear_batch_noalloc(const ternary_problem *problems, int count, int dtype,
                                            hipStream_t stream)
{
    return ternary::linear_batch(problems, count, dtype, stream, true);
}
