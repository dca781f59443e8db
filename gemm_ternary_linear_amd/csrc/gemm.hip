// Prefill GEMM (M > 8) for the ternary linear layer on gfx950.
//
// At large M the layer y = x @ (unpack(q) * s)^T ([xxqk] m.xxqk.cn/news/593501
// §4.3) is a dense contraction and compute-bound ([nxbn] m.nxbn.cn/news/169761
// §4.1: prefill is dominated by compute), so it runs on the matrix cores.
// The packed tile is expanded once per workgroup into LDS as 16-bit +-2 / 0
// (never to HBM: no dense weight copy exists outside LDS), and both operands
// feed v_mfma_f32_16x16x32_{bf16,f16} with fp32 accumulation.  Scales follow
// [trdm] trdm.cn "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1/§4.2
// (group of 128 K, multiplied at the group boundary) and [nxbn] §3.2/§4.2
// (per output channel, multiplied in the epilogue).
//
// Tiling: 128 tokens x 128 channels x 64 K per workgroup step, 256 threads as
// 2x2 waves of 64x64 (4x4 MFMA tiles each).  Two LDS buffers per operand: the
// global loads of step k+1 are in flight while step k runs on the matrix cores.
// Rows are padded to 72 elements (144 bytes) so the 16 rows a fragment read
// touches fall on distinct LDS banks.
#include "common.h"
#include "internal.h"

namespace ternary {

namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // 16-bit elements per LDS row
constexpr int THREADS = 256;

template <bool FP16>
__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c)
{
    if constexpr (FP16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                       0);
}

struct TileRegs {
    uint4 xa[4];  // 4 x 16 bytes of activations
    uint2 w;      // 8 packed bytes = 32 codes
};

// Thread t loads activation rows (c*32 + t/8), 8 elements at k (t%8)*8, and
// packed row t/2, bytes (t%2)*8 .. +8 of the step.
__device__ __forceinline__ void load_tile(TileRegs &r, const uint16_t *x, const uint8_t *packed,
                                          int M, int N, int K, int m0, int n0, int k0, int tid)
{
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int m = m0 + c * 32 + (tid >> 3);
        r.xa[c] = make_uint4(0, 0, 0, 0);
        if (m < M)
            r.xa[c] = *reinterpret_cast<const uint4 *>(x + (int64_t)m * K + k0 + (tid & 7) * 8);
    }
    const int n = n0 + (tid >> 1);
    r.w = make_uint2(0, 0);
    if (n < N)
        r.w = *reinterpret_cast<const uint2 *>(packed + (int64_t)n * (K >> 2) + (k0 >> 2) +
                                               (tid & 1) * 8);
}

__device__ __forceinline__ void store_tile(const TileRegs &r, uint16_t *sA, uint16_t *sB, int tid)
{
#pragma unroll
    for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint4 *>(sA + (c * 32 + (tid >> 3)) * LDS_STRIDE + (tid & 7) * 8) = r.xa[c];
    uint32_t d[16];
    decode16(r.w.x, d);
    decode16(r.w.y, d + 8);
    uint4 *dst = reinterpret_cast<uint4 *>(sB + (tid >> 1) * LDS_STRIDE + (tid & 1) * 32);
#pragma unroll
    for (int v = 0; v < 4; ++v)
        dst[v] = make_uint4(d[4 * v], d[4 * v + 1], d[4 * v + 2], d[4 * v + 3]);
}

template <bool FP16, bool GROUPED>
__global__ void __launch_bounds__(THREADS)
    gemm_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed,
                const uint16_t *__restrict__ scale, uint16_t *__restrict__ y, int M, int N, int K)
{
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;
    const int nk = K / BK;
    const int ngroups = K >> 7;

    f32x4_t acc[4][4];
    f32x4_t part[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            part[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

    TileRegs regs;
    load_tile(regs, x, packed, M, N, K, m0, n0, 0, tid);
    store_tile(regs, sA[0], sB[0], tid);
    __syncthreads();

    // Fragment addresses: lane reads row (lane & 15), k offset 8*(lane >> 4).
    const int frow = lane & 15;
    const int fk = (lane >> 4) * 8;

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk)
            load_tile(regs, x, packed, M, N, K, m0, n0, (kt + 1) * BK, tid);

        const uint16_t *a_base = sA[buf] + (wm * 64 + frow) * LDS_STRIDE + fk;
        const uint16_t *b_base = sB[buf] + (wn * 64 + frow) * LDS_STRIDE + fk;
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            uint4 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const uint4 *>(a_base + i * 16 * LDS_STRIDE + kk);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const uint4 *>(b_base + j * 16 * LDS_STRIDE + kk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (GROUPED)
                        part[i][j] = mfma<FP16>(af[i], bf[j], part[i][j]);
                    else
                        acc[i][j] = mfma<FP16>(af[i], bf[j], acc[i][j]);
                }
        }

        if constexpr (GROUPED) {
            if (kt & 1) {  // end of a 128-wide group: fold with its scale
                const int grp = kt >> 1;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = n0 + wn * 64 + j * 16 + frow;
                    const float sc = n < N ? f16_bits_to_f32(scale[(int64_t)n * ngroups + grp]) : 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            acc[i][j][r] += sc * part[i][j][r];
                            part[i][j][r] = 0.f;
                        }
                }
            }
        }

        if (kt + 1 < nk)
            store_tile(regs, sA[buf ^ 1], sB[buf ^ 1], tid);
        __syncthreads();
    }

    // Epilogue: C tile (i, j) element r of this lane is y[m][n] with
    // m = m0 + wm*64 + i*16 + 4*(lane>>4) + r, n = n0 + wn*64 + j*16 + (lane&15).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + frow;
        if (n >= N)
            continue;
        float post = 0.5f;  // decoded weights are +-2
        if constexpr (!GROUPED)
            post *= f16_bits_to_f32(scale[n]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
                if (m < M)
                    y[(int64_t)m * N + n] = round_out<FP16>(acc[i][j][r] * post);
            }
    }
}

template <bool FP16, bool GROUPED>
hipError_t launch_gemm_t(const uint16_t *x, int M, int N, int K, const uint8_t *packed,
                         const uint16_t *scale, uint16_t *y, hipStream_t stream)
{
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_kernel<FP16, GROUPED>), grid, dim3(THREADS), 0, stream, x, packed,
                       scale, y, M, N, K);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t *x, bool fp16, int M, int N, int K, const uint8_t *packed,
                       const uint16_t *scale, bool grouped, uint16_t *y, hipStream_t stream)
{
    if (fp16)
        return grouped ? launch_gemm_t<true, true>(x, M, N, K, packed, scale, y, stream)
                       : launch_gemm_t<true, false>(x, M, N, K, packed, scale, y, stream);
    return grouped ? launch_gemm_t<false, true>(x, M, N, K, packed, scale, y, stream)
                   : launch_gemm_t<false, false>(x, M, N, K, packed, scale, y, stream);
}

}  // namespace ternary
