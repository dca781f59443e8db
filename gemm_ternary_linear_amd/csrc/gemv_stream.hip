// Streaming decode GEMV (M <= 8) for the ternary linear layer on gfx950.
//
// The layer ([xxqk] m.xxqk.cn/news/593501 §4.3: y = x @ (unpack(q) * s)^T)
// at a few tokens reads every packed weight byte once and does little
// arithmetic per byte, so its speed is the HBM stream ([nxbn]
// m.nxbn.cn/news/169761 §4.1/§4.4).  The kernel is shaped by how gfx950
// serves such a stream (measured on MI355X with read-only probes of the same
// access pattern):
//
//  * A workgroup of 8 waves holds RB blocks of 16 output channels, each
//    block's K range split into KP = 8 / RB parts, one per wave: parts of
//    about 4 slabs at short K (K = 4096: 2 blocks x 4 parts), 8 parts at long
//    K.  A slab is 256 codes = 64 bytes of each of the block's 16 rows, one
//    16-byte buffer load per lane.  Parts of at most one_shot() slabs (8 at
//    M = 1, 4 at M = 1 with group scales, 8 / M beyond) issue every load at
//    once, as the wave's first instructions: x by DMA straight into the
//    wave's LDS, then the codes.  Longer per-channel parts of 1 or 2 tokens
//    keep kWindow slabs in flight and issue the next slab's loads as each
//    slab is consumed; other long parts run as one-shot chunks of near-equal
//    length in turn.  Instances of 1, 2, 4 and 8 tokens exist; a problem runs
//    on the smallest one that holds its M (tokens past M read zeros).  Small
//    workgroups of short-lived waves keep the memory system supplied: the
//    dispatcher refills a CU as soon as a workgroup is done.
//  * A block's K parts meet without a workgroup barrier: each wave stores its
//    partial sums in LDS and bumps the block's LDS counter; the wave that
//    arrives last adds the parts in part order (so the result does not depend
//    on arrival order) and writes y.  The other waves leave at once.
//  * A wave's loads return in issue order, so its x (512 bytes per token and
//    slab, loaded first) arrives before the codes that need it.  The MFMA B
//    lanes read x from the wave's own LDS (no workgroup barrier).  Long parts
//    load each slab's x right before its codes into registers and stage it
//    through two LDS buffers.  Buffer loads bound every access: rows past N,
//    codes past the matrix and x past K read as zeros.
//  * Decoding and MFMA: each 32-bit word of codes becomes 16 bf16/fp16
//    weights of +-2 or 0 in registers (decode16), the A operand of
//    v_mfma_f32_16x16x32_{bf16,f16} (rows = channels); B column GC*t + p
//    holds token t restricted to group p of the slab (GC = 2 halves of 128,
//    4 groups of 64, 8 groups of 32), so group scales ([trdm] trdm.cn
//    "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1/§4.2: 128;
//    [xxqk] m.xxqk.cn/news/593501 §4.2: 64; yangyitao.com vLLM book, chapter
//    13, §13.3.3: 32, 256) apply to each group's fp32 partial, and
//    per-channel scales ([nxbn] §3.2) to the final sum.
#include "common.h"
#include "internal.h"

#include <algorithm>
#include <type_traits>

namespace ternary {

namespace {

constexpr int kWaves = 8;            // waves per workgroup
constexpr int kThreads = kWaves * 64;
// Parts of up to one_shot<M, GROUPED>() slabs issue every load at once (the x
// area of a wave in LDS bounds it, 4 KB for M tokens, and so do the registers
// of the group-scaled kernels).
template <int MT, bool GROUPED>
constexpr int one_shot()
{
    return MT == 1 ? (GROUPED ? 4 : 8) : 8 / MT;
}
constexpr int kWindow = 4;           // longer parts: slabs in flight per wave
constexpr int kSlabsPerPart = 4;     // target part length when K is short
constexpr int kOOB = 0x40000000;     // buffer offset past every resource: reads zero
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

struct StreamProblem {
    const uint16_t *x;
    const uint8_t *packed;
    const uint16_t *scale;
    uint16_t *y;
    int M, N, K;  // M <= the kernel's token count MT
    int group;    // 0 (per channel) or the group size
    int tiled;    // codes in the tiled layout (else row-major [N, K/4])
    int rb;       // 16-channel blocks per workgroup
    int kp;       // K parts (waves) per block, rb * kp <= kWaves
    int unit0;    // first workgroup of this problem
    // wave w -> (block rbi, part kpi) = 4-bit fields w of these maps (15 in
    // both: the wave holds no part); precomputed so that the kernel's start
    // needs no division
    uint64_t rbi_map, kpi_map;
};

// Kernel argument.  The first workgroup of every problem comes first, in one
// array, so that a workgroup finds its problem with one round of scalar loads.
struct StreamBatch {
    int count;
    int unit0[kGemvMaxBatch];
    StreamProblem p[kGemvMaxBatch];
};

// LDS: per wave an x area of M*L*256 elements, L = one_shot<M, GROUPED>() (a
// one-shot part's x, token t at t*L*256; a long part uses the first M*512
// elements as two slab buffers; once the part is done, its first 1 KB holds
// the wave's partial sums for the K-part reduction) and (group-scaled) the
// scales of GC column groups x 16 channels for up to L slabs; then one
// counter per block.
template <int MT, bool GROUPED>
constexpr int x_area_elems()
{
    return MT * one_shot<MT, GROUPED>() * 256;
}
static_assert(x_area_elems<1, true>() * 2 >= 64 * 16, "a wave's x area holds its partial sums");
template <int GC, int MT, bool GROUPED>
constexpr int wave_lds_elems()
{
    return x_area_elems<MT, GROUPED>() + GC * one_shot<MT, GROUPED>() * 16;
}
template <int GC, int MT, bool GROUPED>
constexpr size_t cnt_offset()
{
    return (size_t)kWaves * wave_lds_elems<GC, MT, GROUPED>() * 2;
}
template <int GC, int MT, bool GROUPED>
constexpr size_t lds_bytes()
{
    return cnt_offset<GC, MT, GROUPED>() + kWaves * 4;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             (int)kRsrcWord3);
}

// One buffer-to-LDS DMA: every lane reads 16 bytes from rsrc at voff and the
// wave writes them to LDS at lds + 16 * lane.  The builtin exists for the
// device target only; the host pass (the launch stub) sees an empty body.
__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t rsrc, void *lds, int voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds,
                                             16, voff, 0, 0, 0);
#endif
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

// Lane i of each quad of lanes takes v from lane (SEL >> 2i) & 3 of its quad
// (a DPP quad permutation).
template <int SEL>
__device__ __forceinline__ int quad_perm(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, SEL, 0xf, 0xf, false);
}
template <int SEL>
__device__ __forceinline__ float quad_perm(float v)
{
    return __builtin_bit_cast(float, quad_perm<SEL>(__builtin_bit_cast(int, v)));
}

// What one wave needs to run its K part.
struct WaveCtx {
    __amdgpu_buffer_rsrc_t xr, wr, sr;
    int M, K, ngroups;  // M: the problem's tokens (<= the kernel's MT)
    int gsh;       // GC = 2 with groups: column group (128 K) -> scale index shift
    int s_begin;   // first slab of the part
    int woff;      // this lane's byte offset of slab 0 in the block resource
    int sstride;   // bytes from one slab to the next in the block resource
    int lane, g, tok, par;
    bool b_lane;
    uint16_t *xbuf;  // this wave's x area
    uint16_t *sbuf;  // this wave's group scales [GC*one_shot<M, GROUPED>()][16]
    int srow_off;    // grouped: scale offset (bytes) of this lane's row, group 0; < 0: none
    int chs_off;     // per channel: scale offset (bytes) of channel 4g + (lane & 3), or kOOB
};

// Per-channel scale of the block's channel 4g + (lane & 3), issued after the
// part's own loads: whichever wave finishes the block applies it (each quad
// of lanes holds the scales of the four channels its C rows cover).
template <bool GROUPED>
__device__ __forceinline__ uint32_t channel_scale_load(const WaveCtx &c)
{
    if constexpr (GROUPED)
        return 0u;
    else
        return __builtin_amdgcn_raw_buffer_load_b16(c.sr, c.chs_off, 0, 0);
}

// Byte offset of this lane's piece of slab s of x (M = 1: 8 bytes, M = 2:
// 16 bytes), or kOOB past K.
template <int MT>
__device__ __forceinline__ int x_piece_off(const WaveCtx &c, int s)
{
    if constexpr (MT == 1) {
        const int e = s * 256 + 4 * c.lane;
        return e < c.K ? e * 2 : kOOB;
    }
    const int e = s * 256 + 8 * (c.lane & 31);
    return e < c.K ? ((c.lane >> 5) * c.K + e) * 2 : kOOB;
}

// This lane's x piece of one slab: 4 elements (M = 1) or 8 (M = 2).
template <int MT>
using XPiece = typename std::conditional<MT == 1, u32x2_t, u32x4_t>::type;

// Store this lane's x piece of a slab into slab buffer `buf` (0 or 1) of a
// long part, laid out [M][256].
template <int MT>
__device__ __forceinline__ void x_piece_store(const WaveCtx &c, int buf, XPiece<MT> v)
{
    uint16_t *b = c.xbuf + buf * (MT * 256);
    if constexpr (MT == 1)
        *reinterpret_cast<u32x2_t *>(b + 4 * c.lane) = v;
    else
        *reinterpret_cast<u32x4_t *>(b + (c.lane >> 5) * 256 + 8 * (c.lane & 31)) = v;
}

template <int MT>
__device__ __forceinline__ XPiece<MT> x_piece_load(const WaveCtx &c, int s)
{
    const int off = x_piece_off<MT>(c, s);
    if constexpr (MT == 1)
        return __builtin_amdgcn_raw_buffer_load_b64(c.xr, off, 0, 0);
    else
        return __builtin_amdgcn_raw_buffer_load_b128(c.xr, off, 0, 0);
}

// Scale load j of this lane for a run of slabs starting at part slab i0:
// lane l covers row l & 15 and local column group (l >> 4) + 4j of the run's
// GC*nsl column groups; its scale is that of group gr (of half slab gr when
// GC = 2).  Rows past N, groups past K and columns past the run read zero.
template <int GC>
__device__ __forceinline__ uint32_t scale_load(const WaveCtx &c, int i0, int nsl, int j)
{
    const int lg = (c.lane >> 4) + 4 * j;
    const int gr = (GC * (c.s_begin + i0) + lg) >> (GC == 2 ? c.gsh : 0);
    const int off =
        (c.srow_off >= 0 && lg < GC * nsl && gr < c.ngroups) ? c.srow_off + gr * 2 : kOOB;
    return __builtin_amdgcn_raw_buffer_load_b16(c.sr, off, 0, 0);
}

// The MFMAs of one slab whose x sits in LDS at xs (token t at xs + t *
// tstride); returns the slab's fp32 sums (C rows 4g..4g+3 of the block,
// column GC*tok + par) added to `part`.
template <bool FP16, int GC>
__device__ __forceinline__ f32x4_t slab_mfma(const WaveCtx &c, const uint16_t *xs, int tstride,
                                             u32x4_t w, f32x4_t part, uint4 &b0, uint4 &b1)
{
    const uint4 *xb = reinterpret_cast<const uint4 *>(xs + c.tok * tstride + c.g * 64);
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    // B operand pieces b0, b1 (zeroed once per part by the caller): lanes
    // without real B entries keep the zeros (GC = 8: every lane rewrites
    // both, the 32-groups change with d).
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if constexpr (GC == 8) {
            if (c.b_lane && c.par == 2 * c.g + (d >> 1)) {
                b0 = xb[2 * d];
                b1 = xb[2 * d + 1];
            } else {
                b0 = zero4;
                b1 = zero4;
            }
        } else if (c.b_lane) {
            b0 = xb[2 * d];
            b1 = xb[2 * d + 1];
        }
        uint32_t a[8];
        decode16(wv[d], a);
        part = mfma16x16x32<FP16>(a, b0, part);
        part = mfma16x16x32<FP16>(a + 4, b1, part);
    }
    return part;
}

// acc += the group partial `part` times the scales of column group col of
// this wave's scale buffer (C rows 4g..4g+3; scales past K or N are zeros).
template <int GC>
__device__ __forceinline__ void fold_scales(const WaveCtx &c, int col, f32x4_t part,
                                            f32x4_t &acc)
{
    const uint2 s4 = *reinterpret_cast<const uint2 *>(c.sbuf + col * 16 + 4 * c.g);
    acc[0] += f16_bits_to_f32((uint16_t)s4.x) * part[0];
    acc[1] += f16_bits_to_f32((uint16_t)(s4.x >> 16)) * part[1];
    acc[2] += f16_bits_to_f32((uint16_t)s4.y) * part[2];
    acc[3] += f16_bits_to_f32((uint16_t)(s4.y >> 16)) * part[3];
}

// Run a K part of exactly S <= one_shot<MT, GROUPED>() slabs, every load
// issued up front; returns this lane's fp32 accumulator.
template <int CP, bool FP16, bool GROUPED, int GC, int MT, int S>
__device__ __forceinline__ f32x4_t run_part(const WaveCtx &c, uint32_t &chs)
{
    // ---- issue every load of the part: scales, x (by DMA into this wave's
    // LDS x area, 1 KB per instruction), then the codes slab by slab --------
    constexpr int kSL = GROUPED ? (GC * S + 3) / 4 : 0;  // scale loads per lane
    uint32_t sv[kSL > 0 ? kSL : 1];
#pragma unroll
    for (int j = 0; j < kSL; ++j)
        sv[j] = scale_load<GC>(c, 0, S, j);
    // The x area is [MT][kTok]; DMA j fills its elements 512j .. 512j + 511
    // (one token, or two when a token takes 256), DMAs that would only write
    // slabs past the part are skipped, and lanes past the part, K or the
    // problem's tokens write zeros.
    constexpr int kTok = one_shot<MT, GROUPED>() * 256;  // token stride of the x area
    constexpr int kXD = (MT * kTok + 511) / 512;          // DMAs that cover the area
    int xoff[kXD];
#pragma unroll
    for (int j = 0; j < kXD; ++j) {
        const int a = 512 * j + 8 * c.lane;
        const int t = a / kTok, e = a % kTok;
        const int k = c.s_begin * 256 + e;
        xoff[j] = e < S * 256 && k < c.K && t < c.M ? (t * c.K + k) * 2 : kOOB;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kXD; ++j)
        if ((512 * j) % kTok < S * 256)  // folds: j, S and kTok are constants
            dma16_to_lds(c.xr, c.xbuf + 512 * j, xoff[j]);
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t w[S];
    // in issue order = consumption order
    load_code_run<CP>(w, c.wr, [&](int i) { return c.woff + (c.s_begin + i) * c.sstride; });
    chs = channel_scale_load<GROUPED>(c);

    // ---- scales into this wave's LDS ---------------------------------------
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
        const int lg = (c.lane >> 4) + 4 * j;
        if (lg < GC * S)
            c.sbuf[lg * 16 + (c.lane & 15)] = (uint16_t)sv[j];
    }
    __builtin_amdgcn_wave_barrier();

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    uint4 b0 = make_uint4(0, 0, 0, 0), b1 = b0;
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const uint16_t *xs = c.xbuf + i * 256;
        if constexpr (GROUPED) {
            const f32x4_t part =
                slab_mfma<FP16, GC>(c, xs, kTok, w[i], f32x4_t{0.f, 0.f, 0.f, 0.f}, b0, b1);
            fold_scales<GC>(c, GC * i + c.par, part, acc);
        } else {
            acc = slab_mfma<FP16, GC>(c, xs, kTok, w[i], acc, b0, b1);
        }
    }
    return acc;
}

// Run a per-channel K part of S > one_shot<MT, false>() slabs with kWindow
// slabs in flight: slab i's loads (its x and codes) sit in ring slot
// i % kWindow, and the loads of slab i + kWindow are issued as soon as slab i
// is consumed.  Slots past the part load as zeros without touching memory, so
// every pass issues the same loads and the compiler's waits stay exact.
template <int CP, bool FP16, int GC, int MT>
__device__ __forceinline__ f32x4_t run_rolling(const WaveCtx &c, int S, uint32_t &chs)
{
    constexpr int W = kWindow;
    XPiece<MT> xv[W];
    u32x4_t w[W];
    auto issue = [&](int slot, int i) {
        const bool in = i < S;
        xv[slot] = x_piece_load<MT>(c, in ? c.s_begin + i : (1 << 20));
        w[slot] = load_codes<CP>(c.wr, in ? c.woff + (c.s_begin + i) * c.sstride : kOOB);
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int j = 0; j < W; ++j)
        issue(j, j);
    chs = channel_scale_load<false>(c);
    x_piece_store<MT>(c, 0, xv[0]);

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    uint4 b0 = make_uint4(0, 0, 0, 0), b1 = b0;
    for (int base = 0; base < S; base += W) {
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const int i = base + j;
            if (i < S) {
                if (i + 1 < S)
                    x_piece_store<MT>(c, (i + 1) & 1, xv[(j + 1) % W]);
                __builtin_amdgcn_wave_barrier();
                acc = slab_mfma<FP16, GC>(c, c.xbuf + (i & 1) * (MT * 256), 256, w[j], acc, b0,
                                          b1);
                __builtin_amdgcn_wave_barrier();
            }
            issue(j, i + W);
        }
    }
    return acc;
}

// A part of exactly n <= one_shot<MT, GROUPED>() slabs (S counts up to n).
template <int CP, bool FP16, bool GROUPED, int GC, int MT, int S = 1>
__device__ __forceinline__ f32x4_t run_short(const WaveCtx &c, int n, uint32_t &chs)
{
    if (n == S || S == one_shot<MT, GROUPED>())
        return run_part<CP, FP16, GROUPED, GC, MT, S>(c, chs);
    if constexpr (S < one_shot<MT, GROUPED>())
        return run_short<CP, FP16, GROUPED, GC, MT, S + 1>(c, n, chs);
    else
        return f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// A part of n slabs: one-shot up to L = one_shot<MT, GROUPED>() slabs;
// beyond, per-channel parts of 1 or 2 tokens run with a window, and the rest
// (grouped parts, whose scales take registers of their own, and 4 or 8 tokens,
// whose x per slab would take too many) as ceil(n / L) one-shot chunks of
// near-equal length in turn.
template <int CP, bool FP16, bool GROUPED, int GC, int MT>
__device__ __forceinline__ f32x4_t run_part_n(const WaveCtx &c, int n, uint32_t &chs)
{
    constexpr int L = one_shot<MT, GROUPED>();
    if (n == 0) {
        chs = channel_scale_load<GROUPED>(c);
        return f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (n <= L)
        return run_short<CP, FP16, GROUPED, GC, MT>(c, n, chs);
    if constexpr (MT <= 2 && !GROUPED) {
        return run_rolling<CP, FP16, GC, MT>(c, n, chs);
    } else {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        WaveCtx cc = c;
        const int chunks = (n + L - 1) / L, len = (n + chunks - 1) / chunks;
        for (int done = 0; done < n; done += len) {
            cc.s_begin = c.s_begin + done;
            const f32x4_t part =
                run_short<CP, FP16, GROUPED, GC, MT>(cc, min(len, n - done), chs);
            acc[0] += part[0];
            acc[1] += part[1];
            acc[2] += part[2];
            acc[3] += part[3];
        }
        return acc;
    }
}

// GC: B columns per token (gemv_cols of the group size: 2 for per-channel
// scales and groups of 128 K or more, 4 for 64, 8 for 32); column GC*t + p
// holds token t restricted to group p of each slab (half p when GC = 2).
// (per-channel instances of 2 or more tokens are held to 64 VGPRs, 8 waves per
// SIMD; the 1-token per-channel instance, whose one-shot parts hold 8 slabs of
// codes, and the group-scaled ones keep the registers they need: no scratch)
template <bool FP16, bool GROUPED, int GC, int MT, int CP>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(GROUPED || MT == 1 ? 1 : 8))) gemv_stream_kernel(const StreamBatch batch)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    int pi = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxBatch; ++i)
        if (i < batch.count && (int)blockIdx.x >= batch.unit0[i])
            pi = i;
    const StreamProblem &P = batch.p[pi];
    const int M = P.M, N = P.N, K = P.K, RB = P.rb, KP = P.kp;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rbi = (int)((P.rbi_map >> (4 * wave)) & 15);  // the workgroup's channel block
    const int kpi = (int)((P.kpi_map >> (4 * wave)) & 15);  // K part of that block
    const bool active = kpi < KP;        // waves past RB*KP hold no part
    const int rb = ((int)blockIdx.x - P.unit0) * RB + rbi;
    const int nslabs = (K + 255) >> 8;
    const int glog = GROUPED ? 31 - __builtin_clz((unsigned)P.group) : 7;
    const int ngroups = K >> glog;
    const int rowbytes = K >> 2;

    // block counters: zero before any wave of the workgroup can bump one
    int *const cnt = reinterpret_cast<int *>(smem + cnt_offset<GC, MT, GROUPED>());
    if (KP > 1) {
        if (tid < kWaves)
            cnt[tid] = 0;
        __syncthreads();
    }
    if (!active)
        return;

    WaveCtx c;
    c.M = M;
    c.K = K;
    c.ngroups = ngroups;
    c.gsh = glog >= 7 ? glog - 7 : 0;
    c.lane = lane;
    c.g = lane >> 4;                // lane group: which 64-code quarter of a slab
    const int col = lane & 15;      // A row / B column / C column of this lane
    c.tok = col / GC;               // token of this B column
    c.par = col % GC;               // column group of the slab this column collects
    // Lane group g holds codes 64g .. 64g+63 of a slab, word d of them codes
    // 64g + 16d .. +15: in half g/2, in 64-group g, in 32-group 2g + d/2.
    c.b_lane = c.tok < MT && (GC == 2 ? (c.g >> 1) == c.par : (GC == 4 ? c.g == c.par : true));
    // Parts split the block's slabs evenly: part p = [p*n/KP, (p+1)*n/KP).
    c.s_begin = kpi * nslabs / KP;
    const int S = __builtin_amdgcn_readfirstlane((kpi + 1) * nslabs / KP - c.s_begin);
    // (readfirstlane: the clamp lowers to a vector op, and a descriptor in
    // vector registers would put every load in a waterfall loop)
    const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(16, N - rb * 16)));
    // Row-major codes: lane (g, col) reads bytes 16g .. 16g+15 of slab s of row
    // col (64 bytes a slab).  Tiled codes: a slab of the block is 1 KB in the
    // lane order [g][col][16 bytes], so the lane reads 16 contiguous bytes at
    // 16 * (16g + col) and the wave one kilobyte.
    const bool tiled = P.tiled != 0;
    const uint8_t *wbase = nrows == 0 ? P.packed
                           : tiled    ? P.packed + (int64_t)rb * nslabs * kTileBytes
                                      : P.packed + (int64_t)rb * 16 * rowbytes;
    c.wr = make_rsrc(wbase, nrows == 0 ? 0u : tiled ? (uint32_t)nslabs * kTileBytes
                                                    : (uint32_t)(nrows * rowbytes));
    c.woff = tiled ? (c.g * 16 + col) * 16 : col * rowbytes + c.g * 16;
    c.sstride = tiled ? kTileBytes : 64;
    c.xr = make_rsrc(P.x, (uint32_t)M * (uint32_t)K * 2u);
    // the scale resource starts at the block's first row (64-bit pointer
    // arithmetic), so its 32-bit offsets stay below 16 rows of scales
    const int spr = GROUPED ? ngroups : 1;  // scales per row
    const uint16_t *sbase = nrows > 0 ? P.scale + (int64_t)rb * 16 * spr : P.scale;
    c.sr = make_rsrc(sbase, (uint32_t)(nrows * spr * 2));
    c.srow_off = (lane & 15) < nrows ? (lane & 15) * spr * 2 : -1;
    uint16_t *wlds = reinterpret_cast<uint16_t *>(smem) + wave * wave_lds_elems<GC, MT, GROUPED>();
    c.xbuf = wlds;
    c.sbuf = wlds + x_area_elems<MT, GROUPED>();

    const int chs_r = 4 * c.g + (lane & 3);
    c.chs_off = chs_r < nrows ? chs_r * 2 : kOOB;

    uint32_t chs = 0u;
    const f32x4_t acc = run_part_n<CP, FP16, GROUPED, GC, MT>(c, S, chs);

    // ---- K-part reduction (the last wave of the block, fixed order) --------
    f32x4_t sum = acc;
    if (KP > 1) {
        // wave w's partial sums: the first 1 KB of its own x area
        constexpr int kStride = wave_lds_elems<GC, MT, GROUPED>() * 2 / 16;  // in f32x4
        f32x4_t *red = reinterpret_cast<f32x4_t *>(smem);
        red[wave * kStride + lane] = acc;
        // release the partial, learn whether every other part has arrived
        int before = 0;
        if (lane == 0)
            before = __hip_atomic_fetch_add(&cnt[rbi], 1, __ATOMIC_ACQ_REL,
                                            __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(before) != KP - 1)
            return;
        sum = red[rbi * kStride + lane];  // part 0 is wave rbi
        for (int j = 1; j < KP; ++j) {
            const f32x4_t v = red[(rbi + j * RB) * kStride + lane];
            sum[0] += v[0];
            sum[1] += v[1];
            sum[2] += v[2];
            sum[3] += v[3];
        }
    }

    // ---- epilogue: the token's GC columns, channel scale, rounding ----------
    // channel 4g + r's scale: lane r of this lane's quad
    float chsc[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (!GROUPED) {
        chsc[0] = f16_bits_to_f32((uint16_t)quad_perm<0x00>((int)chs));
        chsc[1] = f16_bits_to_f32((uint16_t)quad_perm<0x55>((int)chs));
        chsc[2] = f16_bits_to_f32((uint16_t)quad_perm<0xaa>((int)chs));
        chsc[3] = f16_bits_to_f32((uint16_t)quad_perm<0xff>((int)chs));
    }
    uint16_t o16[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        // the GC columns of a token (adjacent lanes) hold disjoint K sets:
        // within a quad, swap lanes 1 apart, then 2 apart (DPP)
        float tot = sum[r] + quad_perm<0xb1>(sum[r]);
        if constexpr (GC >= 4)
            tot += quad_perm<0x4e>(tot);
        if constexpr (GC >= 8)
            tot += __shfl_xor(tot, 4);
        float o = 0.5f * tot;  // decoded weights are +-2
        if constexpr (!GROUPED)
            o *= chsc[r];
        o16[r] = round_out<FP16>(o);
    }
    // lane (g, token t, par 0) holds channels 4g..4g+3 of token t
    if (c.par == 0 && c.tok < M) {
        const int ch0 = rb * 16 + 4 * c.g;
        uint16_t *__restrict__ yt = P.y + (int64_t)c.tok * N;
        if (ch0 + 4 <= N && ((N & 3) == 0 || M == 1)) {
            // 8-byte aligned: y is 16-byte aligned and tok*N + ch0 is a multiple of 4
            *reinterpret_cast<uint2 *>(yt + ch0) =
                make_uint2(o16[0] | (uint32_t)o16[1] << 16, o16[2] | (uint32_t)o16[3] << 16);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (ch0 + r < N)
                    yt[ch0 + r] = o16[r];
        }
    }
}

// K split of one problem: KP parts per block, a power of two up to kWaves so
// that RB = kWaves / KP blocks fill the workgroup.  KP is the largest power
// of two with parts of at least `target` slabs, doubled while a part would
// exceed the one-shot length `one` (up to kWaves parts; longer parts run with
// a window or in chunks).
void split_k(int K, int one, int target, int &kp, int &rb)
{
    const int nslabs = (K + 255) / 256;
    kp = 1;
    while (2 * kp <= kWaves && 2 * kp * target <= nslabs)
        kp *= 2;
    while (kp < kWaves && (nslabs + kp - 1) / kp > one)
        kp *= 2;
    rb = kWaves / kp;
}

}  // namespace

bool gemv_stream_takes(int64_t M, int64_t K, int group)
{
    return M >= 1 && M <= kGemvStreamMaxM && K % 128 == 0 && K <= kGemvMaxK &&
           M * gemv_cols(group) <= 16 && (group == 0 || K % group == 0);
}

namespace {
// Token count of the kernel instance that runs M tokens.
int kernel_mt(int M) { return M <= 1 ? 1 : (M == 2 ? 2 : (M <= 4 ? 4 : 8)); }

template <bool FP16, bool GROUPED, int GC, int MT, int CP>
void launch_one(dim3 grid, dim3 block, hipStream_t stream, const StreamBatch &b)
{
    constexpr size_t lds = lds_bytes<GC, MT, GROUPED>();
    hipLaunchKernelGGL((gemv_stream_kernel<FP16, GROUPED, GC, MT, CP>), grid, block, lds, stream,
                       b);
}

// MT * GC <= 16: the instances that exist.
template <bool FP16, bool GROUPED, int GC, int CP>
void launch_m(int mt, dim3 grid, dim3 block, hipStream_t stream, const StreamBatch &b)
{
    if (mt == 1)
        launch_one<FP16, GROUPED, GC, 1, CP>(grid, block, stream, b);
    else if (mt == 2)
        launch_one<FP16, GROUPED, GC, 2, CP>(grid, block, stream, b);
    else if constexpr (GC <= 4) {
        if (mt == 4)
            launch_one<FP16, GROUPED, GC, 4, CP>(grid, block, stream, b);
        else if constexpr (GC == 2)
            launch_one<FP16, GROUPED, GC, 8, CP>(grid, block, stream, b);
    }
}

template <bool FP16, int CP>
void launch_group(int group, int mt, dim3 grid, dim3 block, hipStream_t stream,
                  const StreamBatch &b)
{
    if (group == 0)
        launch_m<FP16, false, 2, CP>(mt, grid, block, stream, b);
    else if (group == 32)
        launch_m<FP16, true, 8, CP>(mt, grid, block, stream, b);
    else if (group == 64)
        launch_m<FP16, true, 4, CP>(mt, grid, block, stream, b);
    else
        launch_m<FP16, true, 2, CP>(mt, grid, block, stream, b);
}

// Code-load policy of a launch (kStreamLoad when every problem holds tiled codes).
template <bool FP16>
void launch_policy(int group, int mt, dim3 grid, dim3 block, hipStream_t stream,
                   const StreamBatch &b)
{
    bool all_tiled = true;
    for (int i = 0; i < b.count; ++i)
        all_tiled = all_tiled && b.p[i].tiled != 0;
    if (all_tiled)
        launch_group<FP16, kStreamLoad>(group, mt, grid, block, stream, b);
    else
        launch_group<FP16, 0>(group, mt, grid, block, stream, b);
}

// One-shot part length of the instance (one_shot<MT, GROUPED>() at run time).
int one_shot_of(int mt, int group) { return mt == 1 ? (group ? 4 : 8) : 8 / mt; }
static_assert(one_shot<1, false>() == 8 && one_shot<1, true>() == 4 && one_shot<2, true>() == 4 &&
                  one_shot<4, false>() == 2 && one_shot<8, true>() == 1,
              "one_shot_of mirrors one_shot");

}  // namespace

hipError_t launch_gemv_stream(const GemvArgs *args, const int *order, int count, bool fp16,
                              int group, hipStream_t stream)
{
    // One workgroup per block of 16 channels (per RB blocks at short K), in
    // the caller's problem order (longest K first: those workgroups live
    // longest and start first).  Parts of about `target` slabs.
    StreamBatch b;
    int units = 0, mt = 0;
    auto fill = [&](int target) -> hipError_t {
        b.count = 0;
        units = 0;
        mt = 0;
        for (int oi = 0; oi < count; ++oi) {
            const GemvArgs &a = args[order[oi]];
            if (a.M == 0 || a.N == 0)
                continue;
            if (a.group != group || (mt != 0 && a.M != mt) || !gemv_stream_takes(a.M, a.K, group))
                return hipErrorInvalidValue;
            mt = a.M;
            StreamProblem &p = b.p[b.count];
            p.x = a.x;
            p.packed = a.packed;
            p.scale = a.scale;
            p.y = a.y;
            p.M = a.M;
            p.N = a.N;
            p.K = a.K;
            p.group = group;
            p.tiled = a.tiled;
            split_k(a.K, one_shot_of(kernel_mt(a.M), group), target, p.kp, p.rb);
            const int nblocks = (a.N + 15) / 16;
            p.rb = std::min(p.rb, nblocks);
            p.rbi_map = 0;
            p.kpi_map = 0;
            for (int w = 0; w < kWaves; ++w) {
                const bool act = w < p.rb * p.kp;
                p.rbi_map |= (uint64_t)(act ? w % p.rb : 15) << (4 * w);
                p.kpi_map |= (uint64_t)(act ? w / p.rb : 15) << (4 * w);
            }
            p.unit0 = units;
            b.unit0[b.count] = units;
            units += (nblocks + p.rb - 1) / p.rb;
            ++b.count;
        }
        return hipSuccess;
    };
    // Parts of kSlabsPerPart slabs; a launch whose workgroups would not cover
    // the compute units once takes parts of half that, twice the workgroups
    // (such launches are latency-bound: a 512 x 4096 problem at M = 1 takes
    // 3.5 against 4.3 us).
    hipError_t e = fill(kSlabsPerPart);
    if (e == hipSuccess && b.count > 0 && units < device_cus())
        e = fill(kSlabsPerPart / 2);
    if (e != hipSuccess)
        return e;
    if (b.count == 0)
        return hipSuccess;
    const dim3 grid(units), block(kThreads);
    if (fp16)
        launch_policy<true>(group, kernel_mt(mt), grid, block, stream, b);
    else
        launch_policy<false>(group, kernel_mt(mt), grid, block, stream, b);
    return hipGetLastError();
}

}  // namespace ternary
