// Measurement probes (include/ternary_probe.h): kernels of known traffic or
// flop count that show what plain code reaches on this device, beside the
// published HBM and MFMA peaks.  None of them is used by the layer.
#include <stdint.h>

#include "../../include/ternary_probe.h"
#include "common.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// One 16-byte load, plain or non-temporal (the `nt` cache-policy bit).
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4 *p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    if constexpr (NT) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

// Grid-stride read of n 16-byte words, four loads in flight per lane.
template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const uint4 *__restrict__ src,
                                                              int64_t n, uint32_t *sink)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = load16<NT>(src + i), b = load16<NT>(src + i + stride),
                    c = load16<NT>(src + i + 2 * stride), d = load16<NT>(src + i + 3 * stride);
        acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
    }
    for (; i < n; i += stride)
        acc ^= fold(load16<NT>(src + i));
    // A store that depends on every load keeps them live; it almost never runs.
    if (acc == 0x9e3779b9u)
        sink[0] = acc;
}

// Grid-stride copy of n 16-byte words, four loads then four stores per lane.
__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const uint4 *__restrict__ src,
                                                              uint4 *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride],
                    d = src[i + 3 * stride];
        dst[i] = a;
        dst[i + stride] = b;
        dst[i + 2 * stride] = c;
        dst[i + 3 * stride] = d;
    }
    for (; i < n; i += stride)
        dst[i] = src[i];
}

// Four independent bf16 MFMA chains per wave on register operands.  The
// operands are bf16 values 2^-7 * (1 + j/8), j in 0..7, so every product is
// at most 2^-12 and the accumulators stay below 2^13 for iters <= 2^20.
__global__ __launch_bounds__(kThreads) void probe_mfma_kernel(int iters, float *out)
{
    const uint32_t lane = threadIdx.x & 63;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = 0x3c00u | (((lane + 2 * e) & 7u) << 4);
        const uint32_t hi = 0x3c00u | (((lane + 2 * e + 1) & 7u) << 4);
        w[e] = lo | hi << 16;
    }
    const ternary::bf16x8_t a =
        __builtin_bit_cast(ternary::bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
    const ternary::bf16x8_t b =
        __builtin_bit_cast(ternary::bf16x8_t, make_uint4(w[3], w[2], w[1], w[0]));
    ternary::f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    // distinct registers for the four chains (their equal starting values
    // would otherwise be merged, and the loop would copy accumulators)
    asm volatile("" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        s += c0[r] + c1[r] + c2[r] + c3[r];
    out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool bad_grid(int32_t workgroups) { return workgroups < 1 || workgroups > TERNARY_PROBE_MAX_WORKGROUPS; }

int launched() { return hipGetLastError() == hipSuccess ? TERNARY_OK : TERNARY_ERR_HIP; }

template <bool NT>
int probe_read(const void *src, int64_t bytes, int32_t workgroups, uint32_t *sink,
               hipStream_t stream)
{
    if (bytes < 0 || bytes % 16 != 0 || bad_grid(workgroups))
        return TERNARY_ERR_SHAPE;
    if (bytes == 0)
        return TERNARY_OK;
    if (!src || !sink)
        return TERNARY_ERR_NULL;
    if (!aligned(src, 16) || !aligned(sink, 4))
        return TERNARY_ERR_ALIGN;
    hipLaunchKernelGGL(probe_read_kernel<NT>, dim3(workgroups), dim3(kThreads), 0, stream,
                       (const uint4 *)src, bytes / 16, sink);
    return launched();
}

}  // namespace

extern "C" {

int ternary_probe_read(const void *src, int64_t bytes, int32_t workgroups, uint32_t *sink,
                       hipStream_t stream)
{
    return probe_read<false>(src, bytes, workgroups, sink, stream);
}

int ternary_probe_read_nt(const void *src, int64_t bytes, int32_t workgroups, uint32_t *sink,
                          hipStream_t stream)
{
    return probe_read<true>(src, bytes, workgroups, sink, stream);
}

int ternary_probe_copy(const void *src, void *dst, int64_t bytes, int32_t workgroups,
                       hipStream_t stream)
{
    if (bytes < 0 || bytes % 16 != 0 || bad_grid(workgroups))
        return TERNARY_ERR_SHAPE;
    if (bytes == 0)
        return TERNARY_OK;
    if (!src || !dst)
        return TERNARY_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16))
        return TERNARY_ERR_ALIGN;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes)
        return TERNARY_ERR_ALIAS;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(workgroups), dim3(kThreads), 0, stream,
                       (const uint4 *)src, (uint4 *)dst, bytes / 16);
    return launched();
}

int ternary_probe_mfma(int32_t workgroups, int32_t iters, float *out, hipStream_t stream)
{
    if (bad_grid(workgroups) || iters < 1 || iters > (1 << 20))
        return TERNARY_ERR_SHAPE;
    if (!out)
        return TERNARY_ERR_NULL;
    if (!aligned(out, 4))
        return TERNARY_ERR_ALIGN;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(workgroups), dim3(kThreads), 0, stream, iters,
                       out);
    return launched();
}

}  // extern "C"
