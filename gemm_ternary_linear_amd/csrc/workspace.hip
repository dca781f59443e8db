// Library-owned device workspaces: one per (device, stream), grown on demand.
//
// The split-K GEMM keeps its fp32 partial tiles here between its two
// kernels.  A workspace belongs to one stream, so work on other streams never
// shares it; calls on one stream run in order, so consecutive calls may reuse
// it.
#include <map>
#include <mutex>
#include <utility>

#include "internal.h"

namespace ternary {

namespace {

struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_pool;

}  // namespace

hipError_t stream_workspace(hipStream_t stream, size_t bytes, void **out)
{
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace &w = g_pool[{dev, stream}];
    if (w.bytes < bytes) {
        // no allocation (nor free) while the stream is being captured
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess)
            return e;
        if (cap != hipStreamCaptureStatusNone)
            return hipSuccess;
        if (w.ptr) {
            // earlier work on this stream may still read the old buffer
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess)
                return e;
            e = hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
            if (e != hipSuccess)
                return e;
        }
        // round up to 16 MiB so that slowly growing shapes do not reallocate
        const size_t want = (bytes + (size_t(16) << 20) - 1) & ~((size_t(16) << 20) - 1);
        e = hipMalloc(&w.ptr, want);
        if (e != hipSuccess) {
            w.ptr = nullptr;
            return e;
        }
        w.bytes = want;
    }
    *out = w.ptr;
    return hipSuccess;
}

hipError_t release_workspaces()
{
    std::lock_guard<std::mutex> lock(g_mu);
    hipError_t first = hipSuccess;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess)
        cur = -1;
    for (auto &kv : g_pool) {
        if (!kv.second.ptr)
            continue;
        hipError_t e = hipSetDevice(kv.first.first);
        if (e == hipSuccess)
            e = hipStreamSynchronize(kv.first.second);
        if (e == hipSuccess)
            e = hipFree(kv.second.ptr);
        if (e != hipSuccess && first == hipSuccess)
            first = e;
    }
    g_pool.clear();
    if (cur >= 0)
        (void)hipSetDevice(cur);
    return first;
}

}  // namespace ternary
