// Plain kernel for the ternary linear layer: one thread per output element.
//
// Takes every valid shape (any K % 4 == 0), so it serves the shapes the fast
// kernels do not take and is a third, structurally different GPU evaluation
// for cross-checks.  It follows the pages' sign-select formulation directly:
// +x for code 01, -x for code 10, nothing for 00 and the reserved 11
// ([nxbn] m.nxbn.cn/news/169761 §4.1; code table [trdm] trdm.cn
// "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1), with the sum kept
// in fp32 partials of 128 K (of one group when groups are shorter) so no
// fp32 chain grows longer than 128 + K/32.
#include "common.h"
#include "internal.h"

namespace ternary {

namespace {

template <bool FP16>
__device__ __forceinline__ float load_act(const uint16_t *p)
{
    const uint16_t b = *p;
    if constexpr (FP16)
        return f16_bits_to_f32(b);
    else
        return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Byte j of row n's codes: row-major at n * K/4 + j; tiled (the library's
// layout: 16-row x 256-code blocks of 1 KB, [4 quarters][16 rows][16 bytes])
// at ((n/16) * ceil(K/256) + j/64) KB + ((j/16) % 4) * 256 + (n%16) * 16 + j%16.
__device__ __forceinline__ uint32_t code_byte(const uint8_t *packed, int n, int j, int K, bool tiled)
{
    if (!tiled)
        return packed[(int64_t)n * (K >> 2) + j];
    const int64_t ks = (K + 255) >> 8;
    return packed[((int64_t)(n >> 4) * ks + (j >> 6)) * 1024 + ((j >> 4) & 3) * 256 +
                  (n & 15) * 16 + (j & 15)];
}

// glog: log2 of the group size (group-scaled instances).
template <bool FP16, bool GROUPED>
__global__ void __launch_bounds__(256)
    simple_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed,
                  const uint16_t *__restrict__ scale, uint16_t *__restrict__ y, int M, int N, int K,
                  int glog, int tiled)
{
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N)
        return;
    const int ngroups = GROUPED ? K >> glog : 1;
    const int plen = GROUPED && glog < 7 ? 1 << glog : 128;  // K of one fp32 partial
    for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const uint16_t *xrow = x + (int64_t)m * K;
    float acc = 0.f;
    for (int k0 = 0; k0 < K; k0 += plen) {
        const int k1 = k0 + plen < K ? k0 + plen : K;
        float part = 0.f;
        for (int k = k0; k < k1; k += 4) {
            const uint32_t byte = code_byte(packed, n, k >> 2, K, tiled != 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t c = (byte >> (2 * i)) & 3u;
                const float xv = load_act<FP16>(xrow + k + i);
                part += c == 1u ? xv : (c == 2u ? -xv : 0.f);
            }
        }
        if constexpr (GROUPED)
            acc += f16_bits_to_f32(scale[(int64_t)n * ngroups + (k0 >> glog)]) * part;
        else
            acc += part;
    }
    if constexpr (!GROUPED)
        acc *= f16_bits_to_f32(scale[n]);
    y[(int64_t)m * N + n] = round_out<FP16>(acc);
    }
}

template <bool FP16, bool GROUPED>
hipError_t launch_simple_t(const uint16_t *x, int M, int N, int K, const uint8_t *packed,
                           const uint16_t *scale, int glog, uint16_t *y, hipStream_t stream,
                           bool tiled)
{
    const dim3 grid((N + 255) / 256, M < 65535 ? M : 65535);
    hipLaunchKernelGGL((simple_kernel<FP16, GROUPED>), grid, dim3(256), 0, stream, x, packed,
                       scale, y, M, N, K, glog, tiled ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_simple(const uint16_t *x, bool fp16, int M, int N, int K, const uint8_t *packed,
                         const uint16_t *scale, int group, uint16_t *y, hipStream_t stream,
                         bool tiled)
{
    const int glog = group ? group_log2(group) : 0;
    if (fp16)
        return group ? launch_simple_t<true, true>(x, M, N, K, packed, scale, glog, y, stream, tiled)
                     : launch_simple_t<true, false>(x, M, N, K, packed, scale, 0, y, stream, tiled);
    return group ? launch_simple_t<false, true>(x, M, N, K, packed, scale, glog, y, stream, tiled)
                 : launch_simple_t<false, false>(x, M, N, K, packed, scale, 0, y, stream, tiled);
}

}  // namespace ternary
