// Ternary quantizer on gfx950: 16-bit weights -> 2-bit codes + fp16 scales,
// the step before the layer (its inputs are what this writes).
//
// Rule: the symmetric linear quantizer of the yangyitao.com vLLM book,
// chapter 13, §13.1.3 (w_q = round(w / s), s = max|w| / (largest code)),
// with the ternary code range {-1, 0, +1}, so s = max|w| over the group (one
// output channel, or g consecutive K weights of it).  s is stored as fp16
// (nearest even) and the codes are rounded against that stored s, so that
// q * s reproduces w within s/2 (§13.1.4).  round(w/s) is +-1 exactly when
// |w| > s/2 (ties go to the even code, 0), and both sides of that comparison
// are exact in fp32: no division.  A group whose s is 0 gets codes 0.
// Codes are written in the layer's format ([trdm] trdm.cn
// "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1): +1 -> 01,
// -1 -> 10, 0 -> 00, four per byte, the first weight in the lowest bits.
//
// One workgroup per row (rows beyond 65536 workgroups are walked grid-stride); a lane takes 4 weights (8 bytes) and writes their
// code byte.  A group spans g/4 consecutive lanes of one wave, whose maximum
// is a butterfly of lane shuffles; a per-channel row takes a first pass for
// its maximum (block reduction through LDS) and a second for the codes.
// HBM-bound: 2 bytes read and a quarter byte written per weight.
#include "common.h"
#include "internal.h"

namespace ternary {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRowBlocks = 65536;

template <bool FP16>
__device__ __forceinline__ float widen16(uint32_t b)
{
    if constexpr (FP16)
        return f16_bits_to_f32((uint16_t)b);
    else
        return __builtin_bit_cast(float, b << 16);
}

// The four 16-bit weights of one 8-byte piece.
template <bool FP16>
__device__ __forceinline__ void load4(const uint16_t *p, float v[4])
{
    const uint2 d = *reinterpret_cast<const uint2 *>(p);
    v[0] = widen16<FP16>(d.x & 0xffffu);
    v[1] = widen16<FP16>(d.x >> 16);
    v[2] = widen16<FP16>(d.y & 0xffffu);
    v[3] = widen16<FP16>(d.y >> 16);
}

__device__ __forceinline__ float absmax4(const float v[4])
{
    return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}

// Code byte of four weights against scale s (fp32 value of the fp16 scale).
__device__ __forceinline__ uint8_t codes4(const float v[4], float s)
{
    const float half = 0.5f * s;  // exact: s is a normal or subnormal fp16 value
    uint32_t b = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool nz = s > 0.f && fabsf(v[i]) > half;
        const uint32_t c = nz ? (v[i] < 0.f ? 2u : 1u) : 0u;
        b |= c << (2 * i);
    }
    return (uint8_t)b;
}

// glog: log2 of the group size, or 0 for one scale per row.
template <bool FP16>
__device__ __forceinline__ void quantize_row(const uint16_t *__restrict__ w, int K, int glog,
                                             uint8_t *__restrict__ packed,
                                             uint16_t *__restrict__ scale, int64_t row)
{
    const int tid = threadIdx.x;
    const int nu = K >> 2;  // 4-weight units of the row
    const uint16_t *wr = w + row * K;
    uint8_t *pr = packed + row * nu;

    if (glog == 0) {
        __shared__ float wmax[kThreads / 64];
        float m = 0.f;
        for (int u = tid; u < nu; u += kThreads) {
            float v[4];
            load4<FP16>(wr + 4 * u, v);
            m = fmaxf(m, absmax4(v));
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            m = fmaxf(m, __shfl_xor(m, o));
        if ((tid & 63) == 0)
            wmax[tid >> 6] = m;
        __syncthreads();
        m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        __syncthreads();  // wmax is rewritten by the workgroup's next row
        const uint16_t sb = f32_to_f16_rne(m);
        const float s = f16_bits_to_f32(sb);
        if (tid == 0)
            scale[row] = sb;
        for (int u = tid; u < nu; u += kThreads) {
            float v[4];
            load4<FP16>(wr + 4 * u, v);
            pr[u] = codes4(v, s);
        }
        return;
    }

    // Groups of g = 2^glog weights: g/4 lanes each, aligned within a wave
    // (64 % (g/4) == 0 and nu % (g/4) == 0, so a group's lanes run the same
    // iterations and only the last iteration drops whole groups).
    const int g4 = 1 << (glog - 2);
    const int ngroups = K >> glog;
    for (int u = tid; u < nu; u += kThreads) {
        float v[4];
        load4<FP16>(wr + 4 * u, v);
        float m = absmax4(v);
        for (int o = 1; o < g4; o <<= 1)
            m = fmaxf(m, __shfl_xor(m, o));
        const uint16_t sb = f32_to_f16_rne(m);
        if ((u & (g4 - 1)) == 0)
            scale[row * ngroups + (u >> (glog - 2))] = sb;
        pr[u] = codes4(v, f16_bits_to_f32(sb));
    }
}

template <bool FP16>
__global__ void __launch_bounds__(kThreads)
    quantize_kernel(const uint16_t *__restrict__ w, int N, int K, int glog,
                    uint8_t *__restrict__ packed, uint16_t *__restrict__ scale)
{
    // Rows are walked grid-stride, so the grid stays within the launch
    // limits at every N; the loop bound is uniform across the workgroup.
    for (int64_t row = blockIdx.x; row < N; row += gridDim.x)
        quantize_row<FP16>(w, K, glog, packed, scale, row);
}

}  // namespace

hipError_t launch_quantize(const uint16_t *w, bool fp16, int N, int K, int group, uint8_t *packed,
                           uint16_t *scale, hipStream_t stream)
{
    const int glog = group ? group_log2(group) : 0;
    const dim3 grid(N < kMaxRowBlocks ? N : kMaxRowBlocks);
    if (fp16)
        hipLaunchKernelGGL(quantize_kernel<true>, grid, dim3(kThreads), 0, stream, w, N, K, glog,
                           packed, scale);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, grid, dim3(kThreads), 0, stream, w, N, K, glog,
                           packed, scale);
    return hipGetLastError();
}

}  // namespace ternary
