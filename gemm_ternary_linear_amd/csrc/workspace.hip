// Library-owned device workspaces: one per (device, stream), grown on demand.
//
// The split-K GEMM keeps its fp32 partial tiles here between its two
// kernels.  A workspace belongs to one stream, so work on other streams never
// shares it; calls on one stream run in order, so consecutive calls may reuse
// it.  A HIP graph captured on a stream keeps the workspace address it was
// captured with, so a workspace replaced by a larger one is retired, not
// freed: retired buffers live until ternary_shutdown().
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "internal.h"

namespace ternary {

namespace {

struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_pool;
std::vector<std::pair<int, void *>> g_retired;  // (device, buffer) replaced by larger ones

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
        // nothing is allocated while the stream is being captured: the
        // caller runs the same call once outside capture first
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess)
            return e;
        if (cap != hipStreamCaptureStatusNone)
            return kErrCaptureWorkspace;
        // round up to 16 MiB so that slowly growing shapes do not reallocate
        const size_t want = (bytes + (size_t(16) << 20) - 1) & ~((size_t(16) << 20) - 1);
        void *p = nullptr;
        e = hipMalloc(&p, want);
        if (e != hipSuccess)
            return e;
        if (w.ptr)
            g_retired.push_back({dev, w.ptr});  // work queued or captured earlier may use it
        w.ptr = p;
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
    std::vector<std::pair<int, void *>> all = g_retired;
    for (auto &kv : g_pool)
        if (kv.second.ptr)
            all.push_back({kv.first.first, kv.second.ptr});
    // wait for every device that holds a buffer (its streams may still use
    // them), then free them all
    std::vector<int> synced;
    for (auto &dp : all) {
        hipError_t e = hipSetDevice(dp.first);
        bool seen = false;
        for (int d : synced)
            seen = seen || d == dp.first;
        if (e == hipSuccess && !seen) {
            e = hipDeviceSynchronize();
            synced.push_back(dp.first);
        }
        if (e == hipSuccess)
            e = hipFree(dp.second);
        if (e != hipSuccess && first == hipSuccess)
            first = e;
    }
    g_pool.clear();
    g_retired.clear();
    if (cur >= 0)
        (void)hipSetDevice(cur);
    return first;
}

}  // namespace ternary
