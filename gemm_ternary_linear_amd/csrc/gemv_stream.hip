// Streaming decode GEMV (M <= 2) for the ternary linear layer on gfx950.
//
// The layer ([xxqk] m.xxqk.cn/news/593501 §4.3: y = x @ (unpack(q) * s)^T)
// at one or two tokens reads every packed weight byte once and does little
// arithmetic per byte, so its speed is the HBM stream ([nxbn]
// m.nxbn.cn/news/169761 §4.1/§4.4).  This kernel is built so that the stream
// starts at the first instruction and never waits on anything else:
//
//  * Every wave owns one block of 16 output channels and one K part of at
//    most kRing slabs (a slab = 256 codes = 64 bytes of each of the 16 rows),
//    and issues ALL of its slab loads before it does anything else.  The
//    number of loads is fixed per kernel instance: slots past the wave's K
//    part use a buffer offset outside the resource, which returns zeros and
//    touches no memory.  With a fixed count the compiler's vmcnt waits are
//    exact, so slab i is consumed as soon as it has landed while later slabs
//    are still in flight.
//  * Rows past N and codes past the end of the weight matrix are outside
//    the buffer resource of their block as well (zeros), so no load is
//    clamped or branched around.
//  * The activation x of the workgroup (all M tokens, whole K, slab-major in
//    LDS) is fetched through registers with buffer loads issued before the
//    slab loads; pieces past K read as zeros.  Only these x loads gate the
//    LDS writes and the one workgroup barrier; the slab loads issued before
//    that point stay in flight across it.  (Direct global->LDS copies would
//    make the compiler wait for every outstanding load before the first LDS
//    read.)
//  * Decoding and MFMA are the same as in the general decode kernel: each
//    32-bit word of codes becomes 16 bf16/fp16 weights of +-2 or 0 in
//    registers (decode16), the A operand of v_mfma_f32_16x16x32_{bf16,f16}
//    (rows = channels); B column 2t+p holds token t restricted to 128-group
//    p of the slab, so group-128 scales ([trdm] trdm.cn
//    "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1/§4.2) apply
//    to each group's fp32 partial, and per-channel scales ([nxbn] §3.2) to
//    the final sum.
//  * K parts of a channel block (KP = 1, 2 or 4 waves) are reduced through
//    LDS in a fixed order, reusing the x region after a barrier, so the LDS
//    of a workgroup is x plus its scales: the K = 18944 projection at M = 1
//    needs 38 KB and four workgroups still fit a CU.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace ternary {

namespace {

constexpr int kThreads = 256;          // 4 waves
constexpr int kRing = 20;              // slab loads per wave, all in flight together
constexpr int kXPieces = 10;           // 16-byte x pieces staged per thread (x <= 40 KB)
constexpr int kSPieces = 10;           // group scales staged per thread
constexpr int kOOB = 0x40000000;       // buffer offset past every resource: reads zero
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct StreamProblem {
    const uint16_t *x;
    const uint8_t *packed;
    const uint16_t *scale;
    uint16_t *y;
    int M, N, K;
    int kp;     // waves (K parts) per 16-channel block: 1, 2 or 4
    int spart;  // slabs per K part (<= kRing)
    int unit0;  // first workgroup of this problem
};

struct StreamBatch {
    int count;
    StreamProblem p[kGemvMaxBatch];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             (int)kRsrcWord3);
}

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

template <bool FP16, bool GROUPED>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
gemv_stream_kernel(const StreamBatch batch)
{
    // LDS: x [nslabs][M][256] (reused for the K-part reduction, >= 4 KB when
    // KP > 1) | scales: grouped [RB][ngroups][16], per channel [RB*16].
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    int pi = 0;
    for (int i = 1; i < batch.count; ++i)
        if ((int)blockIdx.x >= batch.p[i].unit0)
            pi = i;
    const StreamProblem &P = batch.p[pi];
    const int M = P.M, N = P.N, K = P.K, KP = P.kp;
    const int RB = 4 / KP;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rbi = wave % RB;   // which of the workgroup's channel blocks
    const int kp = wave / RB;    // which K part of that block
    const int blk0 = ((int)blockIdx.x - P.unit0) * RB;
    const int rb = blk0 + rbi;
    const int g = lane >> 4;     // lane group: which 64-code quarter of a slab
    const int col = lane & 15;   // A row / B column / C column of this lane
    const int tok = col >> 1;    // token of this B column
    const int par = col & 1;     // 128-group of the slab this column collects
    const bool b_lane = tok < M && (g >> 1) == par;
    const int nslabs = (K + 255) >> 8;
    const int ngroups = K >> 7;
    const int rowbytes = K >> 2;
    const int s_begin = kp * P.spart;
    const int S = min(P.spart, nslabs - s_begin);  // slabs of this wave (>= 1)
    const int xbytes = M * nslabs * 512;
    const int xregion = KP > 1 ? max(xbytes, 4096) : xbytes;

    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
    uint16_t *sc = reinterpret_cast<uint16_t *>(smem + ((xregion + 15) & ~15));

    // ---- activation pieces (issued first, so they land first) -------------
    // Piece p of the LDS image: slab s = (p/32) >> log2(M), token (p/32) & (M-1),
    // elements 8*(p%32) .. +7 of that slab.
    const int npieces = M * nslabs * 32;
    const int nxp = (npieces + kThreads - 1) / kThreads;  // pieces per thread (uniform)
    const int mshift = M == 2 ? 1 : 0;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(P.x, (uint32_t)M * (uint32_t)K * 2u);
    u32x4_t xv[kXPieces];
#pragma unroll
    for (int i = 0; i < kXPieces; ++i) {
        if (i < nxp) {
            const int p = tid + i * kThreads;
            const int q = p >> 5;
            const int e = ((q >> mshift) << 8) + ((p & 31) << 3);
            const int t = q & (M - 1);
            const int off = (p < npieces && e < K) ? (t * K + e) * 2 : kOOB;
            xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
        }
    }
    // ---- scales --------------------------------------------------------
    const __amdgpu_buffer_rsrc_t sr =
        make_rsrc(P.scale, (uint32_t)N * (uint32_t)(GROUPED ? ngroups : 1) * 2u);
    constexpr int kSc = GROUPED ? kSPieces : 1;
    // grouped: entries per thread of the workgroup's scale slice (uniform)
    const int nsp = GROUPED ? (RB * 16 * ngroups + kThreads - 1) / kThreads : 1;
    uint32_t sv[kSc];
    // grouped: entry j of the workgroup's [RB*16][ngroups] slice of the scale
    // matrix, j = tid + i*256 -> channel c, group gr (stepped without division)
    int sc_c = 0, sc_g = 0, sc_dq = 0, sc_dr = 0;
    if constexpr (GROUPED) {
        sc_c = tid / ngroups;
        sc_g = tid - sc_c * ngroups;
        sc_dq = kThreads / ngroups;
        sc_dr = kThreads - sc_dq * ngroups;
    }
    {
        int c = sc_c, gr = sc_g;
#pragma unroll
        for (int i = 0; i < kSc; ++i) {
            if (i >= nsp)
                break;
            int off = kOOB;
            if constexpr (GROUPED) {
                const int ch = blk0 * 16 + c;
                if (c < RB * 16 && ch < N)
                    off = (ch * ngroups + gr) * 2;
                gr += sc_dr;
                c += sc_dq;
                if (gr >= ngroups) {
                    gr -= ngroups;
                    ++c;
                }
            } else {
                const int ch = blk0 * 16 + tid;
                if (tid < RB * 16 && ch < N)
                    off = ch * 2;
            }
            sv[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
        }
    }

    // ---- packed slabs ----------------------------------------------------
    // Lane l reads row (l & 15) of the block, bytes [16*(l>>4), +16) of each
    // slab; the resource covers exactly the block's valid rows.
    // (readfirstlane: the clamp lowers to a vector op, and a descriptor held in
    // vector registers would put every load in a waterfall loop)
    const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(16, N - rb * 16)));
    const uint8_t *wbase = nrows > 0 ? P.packed + (int64_t)rb * 16 * rowbytes : P.packed;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)(nrows * rowbytes));
    const int woff = col * rowbytes + g * 16 + s_begin * 64;
    constexpr int kEarly = kRing - (4 * kXPieces + kSc + 3) / 4;
    u32x4_t w[kRing];
    // Every wave of the workgroup has issued its x and scale loads before any
    // slab load is issued: a CU returns vector loads in issue order, so x that
    // queued behind slab loads would wait for their HBM misses.  (Issue order
    // only: s_barrier waits for no memory operation.)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kEarly; ++i)
        w[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, i < S ? woff + i * 64 : kOOB, 0, 0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage x and scales in LDS (waits for the x and scale loads only)
#pragma unroll
    for (int i = 0; i < kXPieces; ++i) {
        const int p = tid + i * kThreads;
        if (i < nxp && p < npieces)
            *reinterpret_cast<u32x4_t *>(xs + p * 8) = xv[i];
    }
    if constexpr (GROUPED) {
        int c = sc_c, gr = sc_g;
#pragma unroll
        for (int i = 0; i < kSc; ++i) {
            if (i >= nsp)
                break;
            if (c < RB * 16)
                sc[((c >> 4) * ngroups + gr) * 16 + (c & 15)] = (uint16_t)sv[i];
            gr += sc_dr;
            c += sc_dq;
            if (gr >= ngroups) {
                gr -= ngroups;
                ++c;
            }
        }
    } else {
        if (tid < RB * 16)
            sc[tid] = (uint16_t)sv[0];
    }
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = kEarly; i < kRing; ++i)
        w[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, i < S ? woff + i * 64 : kOOB, 0, 0);
    __syncthreads();

    // ---- consume the slabs in issue order ---------------------------------
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // B operand pieces: lanes without real B entries keep zeros throughout.
    uint4 b0 = make_uint4(0, 0, 0, 0), b1 = make_uint4(0, 0, 0, 0);
    const uint16_t *xw = xs + tok * 256 + g * 64;
    const int xslab = M * 256;  // LDS elements per slab
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
        if (i < S) {
            const int s = s_begin + i;
            const uint4 *xb = reinterpret_cast<const uint4 *>(xw + s * xslab);
            const uint32_t wv[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
            f32x4_t part = GROUPED ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                if (b_lane) {
                    b0 = xb[2 * d];
                    b1 = xb[2 * d + 1];
                }
                uint32_t a[8];
                decode16(wv[d], a);
                part = mfma16x16x32<FP16>(a, b0, part);
                part = mfma16x16x32<FP16>(a + 4, b1, part);
            }
            if constexpr (GROUPED) {
                // C rows of this lane: channels rb*16 + 4g + r; column group `par`.
                const int grp = 2 * s + par;
                if (grp < ngroups) {
                    const uint2 s4 = *reinterpret_cast<const uint2 *>(
                        sc + (rbi * ngroups + grp) * 16 + 4 * g);
                    acc[0] += f16_bits_to_f32((uint16_t)s4.x) * part[0];
                    acc[1] += f16_bits_to_f32((uint16_t)(s4.x >> 16)) * part[1];
                    acc[2] += f16_bits_to_f32((uint16_t)s4.y) * part[2];
                    acc[3] += f16_bits_to_f32((uint16_t)(s4.y >> 16)) * part[3];
                }
            } else {
                acc = part;
            }
        }
    }

    // ---- K-part reduction (fixed order) and epilogue ----------------------
    f32x4_t sum = acc;
    if (KP > 1) {
        f32x4_t *red = reinterpret_cast<f32x4_t *>(smem);
        __syncthreads();  // every wave is done with x
        red[wave * 64 + lane] = acc;
        __syncthreads();
        if (kp != 0)
            return;
        for (int j = 1; j < KP; ++j) {
            const f32x4_t v = red[(rbi + j * RB) * 64 + lane];
            sum[0] += v[0];
            sum[1] += v[1];
            sum[2] += v[2];
            sum[3] += v[3];
        }
    }
    uint16_t *__restrict__ y = P.y;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float tot = sum[r] + __shfl_xor(sum[r], 1);
        const int ch = rb * 16 + 4 * g + r;
        if (par == 0 && tok < M && ch < N) {
            float o = 0.5f * tot;  // decoded weights are +-2
            if constexpr (!GROUPED)
                o *= f16_bits_to_f32(sc[rbi * 16 + 4 * g + r]);
            y[(int64_t)tok * N + ch] = round_out<FP16>(o);
        }
    }
}


// K parts per channel block for one problem: the fewest whose parts fit the
// ring and whose workgroup scale slice fits the staging registers; 0 when this
// kernel cannot take the problem.
int min_parts(int M, int K, bool grouped)
{
    const int nslabs = (K + 255) / 256;
    if (M < 1 || M > kGemvStreamMaxM || M * nslabs * 32 > kXPieces * kThreads)
        return 0;
    int kp = 1;
    while (kp <= 4 && ((nslabs + kp - 1) / kp > kRing ||
                       (grouped && (4 / kp) * 16 * (K / 128) > kSPieces * kThreads)))
        kp *= 2;
    return kp <= 4 ? kp : 0;
}

size_t lds_bytes(const StreamProblem &p, bool grouped)
{
    const int nslabs = (p.K + 255) / 256;
    const int xbytes = p.M * nslabs * 512;
    const int xregion = p.kp > 1 ? std::max(xbytes, 4096) : xbytes;
    const int scb = grouped ? (4 / p.kp) * (p.K / 128) * 16 * 2 : 64 * 2;
    return (size_t)((xregion + 15) & ~15) + (size_t)scb;
}

// A launch with fewer waves than this leaves SIMDs idle; its longest K parts
// are split further while a part keeps at least kMinPart slabs.
constexpr int kMinWaves = 2048;
constexpr int kMinPart = 4;

}  // namespace

bool gemv_stream_takes(int64_t M, int64_t K, bool grouped)
{
    return K % 128 == 0 && K <= kGemvMaxK && min_parts((int)M, (int)K, grouped) > 0;
}

hipError_t launch_gemv_stream(const GemvArgs *args, const int *order, int count, bool fp16,
                              bool grouped, hipStream_t stream)
{
    StreamBatch b;
    b.count = 0;
    int nblocks[kGemvMaxBatch], nslabs[kGemvMaxBatch];
    int waves = 0;
    for (int oi = 0; oi < count; ++oi) {
        const GemvArgs &a = args[order[oi]];
        if (a.M == 0 || a.N == 0)
            continue;
        const int kp = min_parts(a.M, a.K, grouped);
        if (kp == 0 || a.grouped != grouped)
            return hipErrorInvalidValue;
        StreamProblem &p = b.p[b.count];
        p.x = a.x;
        p.packed = a.packed;
        p.scale = a.scale;
        p.y = a.y;
        p.M = a.M;
        p.N = a.N;
        p.K = a.K;
        p.kp = kp;
        nblocks[b.count] = (a.N + 15) / 16;
        nslabs[b.count] = (a.K + 255) / 256;
        waves += nblocks[b.count] * kp;
        ++b.count;
    }
    if (b.count == 0)
        return hipSuccess;
    while (waves < kMinWaves) {
        int best = -1, best_part = 0;
        for (int i = 0; i < b.count; ++i) {
            const int part = (nslabs[i] + b.p[i].kp - 1) / b.p[i].kp;
            const int half = (nslabs[i] + 2 * b.p[i].kp - 1) / (2 * b.p[i].kp);
            if (b.p[i].kp < 4 && half >= kMinPart && part > best_part) {
                best = i;
                best_part = part;
            }
        }
        if (best < 0)
            break;
        waves += nblocks[best] * b.p[best].kp;
        b.p[best].kp *= 2;
    }
    size_t lds = 0;
    int units = 0;
    for (int i = 0; i < b.count; ++i) {
        StreamProblem &p = b.p[i];
        p.spart = (nslabs[i] + p.kp - 1) / p.kp;
        p.unit0 = units;
        units += (nblocks[i] + 4 / p.kp - 1) / (4 / p.kp);
        lds = std::max(lds, lds_bytes(p, grouped));
    }
    if (fp16) {
        if (grouped)
            hipLaunchKernelGGL((gemv_stream_kernel<true, true>), dim3(units), dim3(kThreads), lds,
                               stream, b);
        else
            hipLaunchKernelGGL((gemv_stream_kernel<true, false>), dim3(units), dim3(kThreads), lds,
                               stream, b);
    } else {
        if (grouped)
            hipLaunchKernelGGL((gemv_stream_kernel<false, true>), dim3(units), dim3(kThreads), lds,
                               stream, b);
        else
            hipLaunchKernelGGL((gemv_stream_kernel<false, false>), dim3(units), dim3(kThreads), lds,
                               stream, b);
    }
    return hipGetLastError();
}

}  // namespace ternary
