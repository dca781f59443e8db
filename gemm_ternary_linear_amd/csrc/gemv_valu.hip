// Decode GEMV (M = 1) on the vector ALU: sign-select accumulation in fp32 and
// a cross-lane reduction, the formulation the 7B page describes for its decode
// kernel ([nxbn] m.nxbn.cn/news/169761 §4.1: each weight adds +x, -x or
// nothing; code table [trdm] trdm.cn
// "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1).  It is a forced
// path (TERNARY_PATH_GEMV_VALU), built to be timed against the matrix-core
// decode kernels on the same shapes; the automatic choice never takes it.
//
//  * Work split.  One workgroup of 4 waves per block of 16 rows; K runs in
//    chunks of 1024 codes, chunk c going to wave c % 4.  In a chunk lane l
//    owns codes 16l .. 16l+15: one 4-byte load per lane and row reads 256
//    contiguous bytes of the row, all 16 rows' loads are issued together, and
//    the lane's 16 activations sit in fp32 registers.
//  * Arithmetic.  A 2-bit code (b1 b0) becomes the signed value 0, +1 or -1:
//    the field (sign, magnitude) = (b1 & (b0 ^ b1), b0 ^ b1), read by a
//    signed 2-bit field extract (code 11 gives 0), converted to fp32 and
//    multiplied-added with x: x * (+-1) + acc is exactly an add or a
//    subtract of x, rounded once in fp32.  Three vector instructions per code.
//  * Scales.  A lane's 16 codes lie in one group (groups of 64, 128, 256):
//    its partial takes the group's scale before the row sum; per-channel
//    scales multiply the final sum.
//  * Reduction.  The 16 row sums of a wave's 64 lanes are added by a halving
//    butterfly: each exchange step keeps half of the rows in each half of the
//    lanes (32, 16, 8, 4 lanes apart), then two plain steps (2, 1); the 4
//    waves' row sums then meet in LDS and wave 0 adds them in wave order
//    (deterministic).
#include "common.h"
#include "internal.h"

namespace ternary {

namespace {

constexpr int kValuWaves = 4;
constexpr int kValuThreads = 64 * kValuWaves;
constexpr int kChunk = 1024;  // codes per wave sweep (64 lanes x 16 codes)
constexpr int kOOBv = 0x40000000;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             (int)0x00020000);
}

// GS: 0 per channel, else log2 of the group size (6, 7 or 8).
template <bool FP16, int GS>
__global__ void __launch_bounds__(kValuThreads)
    gemv_valu_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed,
                     const uint16_t *__restrict__ scale, uint16_t *__restrict__ y, int N, int K)
{
    constexpr bool GROUPED = GS != 0;
    __shared__ float red[kValuWaves][16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int row0 = (int)blockIdx.x * 16;
    const int nrows = min(16, N - row0);
    const int rowbytes = K >> 2;
    const int ngroups = GROUPED ? K >> GS : 1;
    // resources rebased at the block's first row (64-bit pointer arithmetic)
    const __amdgpu_buffer_rsrc_t wr =
        rsrc_of(packed + (int64_t)row0 * rowbytes, (uint32_t)(nrows * rowbytes));
    const __amdgpu_buffer_rsrc_t xr = rsrc_of(x, (uint32_t)K * 2u);
    const __amdgpu_buffer_rsrc_t sr =
        rsrc_of(scale + (GROUPED ? (int64_t)row0 * ngroups : (int64_t)row0),
                GROUPED ? (uint32_t)(nrows * ngroups * 2) : (uint32_t)nrows * 2u);

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        acc[r] = 0.f;

    for (int c0 = wave * kChunk; c0 < K; c0 += kValuWaves * kChunk) {
        const int k0 = c0 + 16 * lane;  // this lane's first code of the chunk
        const bool live = k0 < K;       // K % 256 == 0: a lane's 16 codes are all in or all out
        // a wave's load covers 256 whole bytes of one row, read once:
        // non-temporal, like the tiled codes of the matrix-core kernels
        uint32_t w[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            w[r] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                wr, live && r < nrows ? r * rowbytes + (k0 >> 2) : kOOBv, 0, kStreamLoad);
        float xf[16];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                xr, live ? (k0 + 8 * i) * 2 : kOOBv, 0, 0);
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (FP16) {
                    xf[8 * i + 2 * j] = f16_bits_to_f32((uint16_t)vv[j]);
                    xf[8 * i + 2 * j + 1] = f16_bits_to_f32((uint16_t)(vv[j] >> 16));
                } else {
                    xf[8 * i + 2 * j] = __builtin_bit_cast(float, vv[j] << 16);
                    xf[8 * i + 2 * j + 1] = __builtin_bit_cast(float, vv[j] & 0xffff0000u);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // (sign, magnitude) per 2-bit field, sign kept only with a
            // magnitude: 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0
            uint32_t z = __builtin_amdgcn_bitop3_b32(w[r], w[r] >> 1, 0x55555555u, 0x78);
            z &= 0x55555555u | (z << 1);
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int v = __builtin_amdgcn_sbfe((int)z, 2 * i, 2);
                part = __builtin_fmaf((float)v, xf[i], part);
            }
            if constexpr (GROUPED) {
                const uint16_t sb = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                    sr, live && r < nrows ? (r * ngroups + (k0 >> GS)) * 2 : kOOBv, 0, 0);
                part *= f16_bits_to_f32(sb);
            }
            acc[r] += part;
        }
    }

    // Halving butterfly: after the step at distance 32 >> t, lane L holds
    // 8 >> t row sums, those of the rows whose index bit (3 - t) equals lane
    // bit (5 - t).
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int half = 8 >> t, dist = 32 >> t;
        const bool upper = (lane & dist) != 0;
#pragma unroll
        for (int r = 0; r < half; ++r) {
            const float keep = upper ? acc[r + half] : acc[r];
            const float give = upper ? acc[r] : acc[r + half];
            acc[r] = keep + __shfl_xor(give, dist);
        }
    }
    float tot = acc[0];
    tot += __shfl_xor(tot, 2);
    tot += __shfl_xor(tot, 1);
    const int row = 8 * ((lane >> 5) & 1) + 4 * ((lane >> 4) & 1) + 2 * ((lane >> 3) & 1) +
                    ((lane >> 2) & 1);
    if ((lane & 3) == 0)
        red[wave][row] = tot;
    __syncthreads();
    if (wave == 0 && lane < 16 && lane < nrows) {
        float sum = red[0][lane];
#pragma unroll
        for (int v = 1; v < kValuWaves; ++v)
            sum += red[v][lane];
        if constexpr (!GROUPED)
            sum *= f16_bits_to_f32(scale[row0 + lane]);
        y[row0 + lane] = round_out<FP16>(sum);
    }
}

template <bool FP16, int GS>
hipError_t launch_valu_t(const GemvArgs &a, hipStream_t stream)
{
    const int grid = (a.N + 15) / 16;
    hipLaunchKernelGGL((gemv_valu_kernel<FP16, GS>), dim3(grid), dim3(kValuThreads), 0, stream,
                       a.x, a.packed, a.scale, a.y, a.N, a.K);
    return hipGetLastError();
}

template <bool FP16>
hipError_t launch_valu_dtype(const GemvArgs &a, hipStream_t stream)
{
    switch (a.group) {
    case 0: return launch_valu_t<FP16, 0>(a, stream);
    case 64: return launch_valu_t<FP16, 6>(a, stream);
    case 128: return launch_valu_t<FP16, 7>(a, stream);
    default: return launch_valu_t<FP16, 8>(a, stream);
    }
}

}  // namespace

bool gemv_valu_takes(int64_t M, int64_t K, int group, bool tiled)
{
    return M == 1 && !tiled && K > 0 && K % 256 == 0 && K <= kGemvMaxK &&
           (group == 0 || group == 64 || group == 128 || group == 256);
}

hipError_t launch_gemv_valu(const GemvArgs &a, bool fp16, hipStream_t stream)
{
    if (!gemv_valu_takes(a.M, a.K, a.group, a.tiled != 0))
        return hipErrorInvalidValue;
    if (a.N == 0)
        return hipSuccess;
    return fp16 ? launch_valu_dtype<true>(a, stream) : launch_valu_dtype<false>(a, stream);
}

}  // namespace ternary
