// Decode GEMV (1 <= M <= 8) for the ternary linear layer on gfx950.
//
// The layer ([xxqk] m.xxqk.cn/news/593501 §4.3: y = x @ (unpack(q) * s)^T) at
// small M is bound by the HBM stream of packed weights ([nxbn]
// m.nxbn.cn/news/169761 §4.1/§4.4: decode is memory-bound, the 2-bit packing
// is what cuts the bytes).  Scale granularity: one fp16 per output channel
// ([nxbn] §3.2) or per 128 consecutive K weights ([trdm] trdm.cn
// "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1), applied to the
// finished partial sum of its block ([trdm] §4.2).
//
// Mapping onto CDNA4:
//  * One workgroup owns a block of 16 output channels and the whole K range;
//    its W waves take 256-wide K slabs round-robin.
//  * Per slab a lane issues ONE 16-byte load of packed codes: lane l reads
//    channel (l & 15), bytes [16*(l>>4), +16) of the slab's 64 bytes, so a
//    wave reads 16 channels x 64 contiguous bytes per instruction.
//  * The codes are decoded in registers (decode16, branch-free byte permutes)
//    into the A operand of v_mfma_f32_16x16x32_{bf16,f16}: rows = channels,
//    k in natural order.  The B operand is the activation: column 2t+p holds
//    token t restricted to 128-group p of the slab (lanes of the other group
//    keep zeros), so one MFMA chain yields both groups' partial sums
//    separately and each is scaled by its own fp16 scale before it joins the
//    fp32 accumulator.  Only the lanes that own real B entries load x.
//  * The MFMA does the add/sub accumulate (weights are exactly +-2 or 0, the
//    products exact, the sums fp32); zero codes cost no extra work.
//  * The W waves' 16x16 fp32 tiles are reduced through LDS in a fixed order,
//    the two group columns of a token are combined with a lane shuffle, and
//    the result is rounded to the output dtype (round to nearest even).
#include "common.h"
#include "internal.h"

namespace ternary {

namespace {

template <bool FP16>
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint32_t a[4], uint4 b, f32x4_t c)
{
    const uint4 av = make_uint4(a[0], a[1], a[2], a[3]);
    if constexpr (FP16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                       0);
}

struct SlabRegs {
    uint4 w;      // 64 codes of this lane's channel
    uint4 xb[8];  // B operand pieces (8 activations each), zero on idle lanes
};

__device__ __forceinline__ void load_slab(SlabRegs &r, const uint8_t *prow, const uint16_t *xrow,
                                          int s, int k_lane, int K, bool row_ok, bool b_on)
{
    const bool in_k = k_lane < K;
    r.w = make_uint4(0, 0, 0, 0);
    if (row_ok && in_k)
        r.w = *reinterpret_cast<const uint4 *>(prow + (int64_t)s * 64);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        r.xb[i] = make_uint4(0, 0, 0, 0);
    if (b_on && in_k) {
        const uint4 *src = reinterpret_cast<const uint4 *>(xrow + (int64_t)s * 256);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r.xb[i] = src[i];
    }
}

template <bool FP16, bool GROUPED>
__global__ void __launch_bounds__(1024)
    gemv_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed,
                const uint16_t *__restrict__ scale, uint16_t *__restrict__ y, int M, int N, int K)
{
    extern __shared__ f32x4_t red[];  // [waves][64]

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int rb = blockIdx.x;
    const int g = lane >> 4;          // lane group: which 64-code quarter of the slab
    const int col = lane & 15;        // MFMA column
    const int tok = col >> 1;         // token of this column
    const int par = col & 1;          // 128-group of the slab this column collects
    const int row = rb * 16 + col;    // channel whose codes this lane loads (A row)
    const bool row_ok = row < N;
    const bool b_on = tok < M && (g >> 1) == par;
    const int nslabs = (K + 255) >> 8;
    const int ngroups = K >> 7;

    const uint8_t *prow = packed + (int64_t)row * (K >> 2) + g * 16;
    const uint16_t *xrow = x + (int64_t)(tok < M ? tok : 0) * K + g * 64;

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    SlabRegs cur, nxt;
    int s = wave;
    if (s < nslabs)
        load_slab(nxt, prow, xrow, s, s * 256 + g * 64, K, row_ok, b_on);
    for (; s < nslabs; s += nwaves) {
        cur = nxt;
        const int sn = s + nwaves;
        if (sn < nslabs)
            load_slab(nxt, prow, xrow, sn, sn * 256 + g * 64, K, row_ok, b_on);

        const uint32_t wv[4] = {cur.w.x, cur.w.y, cur.w.z, cur.w.w};
        f32x4_t part = GROUPED ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t a[8];
            decode16(wv[d], a);
            part = mfma16x16x32<FP16>(a, cur.xb[2 * d], part);
            part = mfma16x16x32<FP16>(a + 4, cur.xb[2 * d + 1], part);
        }
        if constexpr (GROUPED) {
            // C rows of this lane: channels rb*16 + 4g + r; column group par.
            const int grp = 2 * s + par;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = rb * 16 + 4 * g + r;
                float sc = 0.f;
                if (ch < N && grp < ngroups)
                    sc = f16_bits_to_f32(scale[(int64_t)ch * ngroups + grp]);
                acc[r] += sc * part[r];
            }
        } else {
            acc = part;
        }
    }

    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave != 0)
        return;
    f32x4_t sum = red[lane];
    for (int w = 1; w < nwaves; ++w) {
        const f32x4_t v = red[w * 64 + lane];
        sum[0] += v[0];
        sum[1] += v[1];
        sum[2] += v[2];
        sum[3] += v[3];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float tot = sum[r] + __shfl_xor(sum[r], 1);
        const int ch = rb * 16 + 4 * g + r;
        if (par == 0 && tok < M && ch < N) {
            float o = 0.5f * tot;  // decoded weights are +-2
            if constexpr (!GROUPED)
                o *= f16_bits_to_f32(scale[ch]);
            y[(int64_t)tok * N + ch] = round_out<FP16>(o);
        }
    }
}

template <bool FP16, bool GROUPED>
hipError_t launch_gemv_t(const uint16_t *x, int M, int N, int K, const uint8_t *packed,
                         const uint16_t *scale, uint16_t *y, hipStream_t stream)
{
    const int nslabs = (K + 255) / 256;
    int waves = nslabs / 4;
    waves = waves < 1 ? 1 : (waves > 16 ? 16 : waves);
    const int blocks = (N + 15) / 16;
    const size_t lds = (size_t)waves * 64 * sizeof(f32x4_t);
    hipLaunchKernelGGL((gemv_kernel<FP16, GROUPED>), dim3(blocks), dim3(64 * waves), lds, stream,
                       x, packed, scale, y, M, N, K);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const uint16_t *x, bool fp16, int M, int N, int K, const uint8_t *packed,
                       const uint16_t *scale, bool grouped, uint16_t *y, hipStream_t stream)
{
    if (fp16)
        return grouped ? launch_gemv_t<true, true>(x, M, N, K, packed, scale, y, stream)
                       : launch_gemv_t<true, false>(x, M, N, K, packed, scale, y, stream);
    return grouped ? launch_gemv_t<false, true>(x, M, N, K, packed, scale, y, stream)
                   : launch_gemv_t<false, false>(x, M, N, K, packed, scale, y, stream);
}

}  // namespace ternary
