// Streaming decode GEMV (M <= 2) for the ternary linear layer on gfx950.
//
// The layer ([xxqk] m.xxqk.cn/news/593501 §4.3: y = x @ (unpack(q) * s)^T)
// at one or two tokens reads every packed weight byte once and does little
// arithmetic per byte, so its speed is the HBM stream ([nxbn]
// m.nxbn.cn/news/169761 §4.1/§4.4).  The kernel is shaped by how gfx950
// serves such a stream (measured on MI355X):
//
//  * HBM is fastest when the 16 rows x 1 KB of a block of output channels
//    are requested together by several waves with a few loads each; one wave
//    streaming a whole block alone, or a wave with many loads in flight, is
//    markedly slower.  So a channel block's K range is split over KP waves
//    (KP up to 16) and every wave issues all loads of its short K part
//    (S <= kMaxS slabs; a slab = 256 codes = 64 bytes of each of the 16 rows)
//    at once, as its first instructions.  Workgroups are short-lived; the
//    dispatcher keeps the CUs supplied.
//  * A wave's loads return in issue order, so each slab's activations (512
//    bytes per token) are loaded right before that slab's codes: x arrives
//    with the codes that need it.  (x fetched once per workgroup up front
//    would queue behind the flood of code requests at the L2 and DRAM and
//    hold every wave back.)  All 64 lanes load x; the wave moves it into the
//    lanes that feed the MFMA B operand through two small LDS buffers of its
//    own (no workgroup barrier).
//  * The number of loads of a wave is exactly what its part needs: the wave
//    body is instantiated per part length S (a switch on S), so the compiler's
//    vmcnt waits are exact and no placeholder load takes a slot in the memory
//    pipeline.  Buffer loads bound every access: rows past N, codes past the
//    matrix and x past K read as zeros.
//  * Decoding and MFMA: each 32-bit word of codes becomes 16 bf16/fp16
//    weights of +-2 or 0 in registers (decode16), the A operand of
//    v_mfma_f32_16x16x32_{bf16,f16} (rows = channels); B column GC*t + p
//    holds token t restricted to group p of the slab (GC = 2 halves of 128,
//    4 groups of 64, 8 groups of 32), so group scales ([trdm] trdm.cn
//    "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1/§4.2: 128;
//    [xxqk] m.xxqk.cn/news/593501 §4.2: 64; yangyitao.com vLLM book, chapter
//    13, §13.3.3: 32, 256) apply to each group's fp32 partial, and
//    per-channel scales ([nxbn] §3.2) to the final sum.
//  * A workgroup holds RB channel blocks x KP K parts (RB * KP <= 16 waves);
//    the K parts of a block are reduced through LDS in a fixed order.
#include "common.h"
#include "internal.h"

#include <algorithm>
#include <type_traits>

namespace ternary {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxS = 8;             // slabs per wave (all its loads in flight at once)
constexpr int kOOB = 0x40000000;     // buffer offset past every resource: reads zero
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

struct StreamProblem {
    const uint16_t *x;
    const uint8_t *packed;
    const uint16_t *scale;
    uint16_t *y;
    int N, K;
    int group;  // 0 (per channel) or the group size
    int rb;     // 16-channel blocks per workgroup
    int kp;     // K parts (waves) per block, rb * kp <= kWaves
    int spart;  // slabs per K part (<= kMaxS)
    int unit0;  // first workgroup of this problem
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

// LDS per wave: two x buffers of M*256 elements, then (group-scaled) the
// scales of the wave's GC*kMaxS column groups x 16 channels (GC: B columns
// per token, gemv_cols of the group size).
constexpr int kXBufElems = kGemvStreamMaxM * 256;
template <int GC>
constexpr int wave_lds_elems()
{
    return 2 * kXBufElems + GC * kMaxS * 16;
}

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

// What one wave needs to run its K part.
struct WaveCtx {
    __amdgpu_buffer_rsrc_t xr, wr, sr;
    int K, ngroups;
    int gsh;       // GC = 2 with groups: column group (128 K) -> scale index shift
    int s_begin;   // first slab of the part
    int woff;      // this lane's byte offset of slab 0 in the block resource
    int lane, g, tok, par;
    bool b_lane;
    uint16_t *xbuf;  // this wave's two x buffers
    uint16_t *sbuf;  // this wave's group scales [GC*kMaxS][16]
    int srow_off;    // grouped: scale offset (bytes) of this lane's row, group 0; < 0: none
};

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

// Store this lane's x piece of a slab into buffer `buf`, laid out [M][256].
template <int MT>
__device__ __forceinline__ void x_piece_store(const WaveCtx &c, int buf, XPiece<MT> v)
{
    uint16_t *b = c.xbuf + buf * kXBufElems;
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

// Run a K part of exactly S slabs; returns this lane's fp32 accumulator
// (C rows 4g..4g+3 of the block, column GC*tok + par).
template <bool FP16, bool GROUPED, int GC, int MT, int S>
__device__ __forceinline__ f32x4_t run_part(const WaveCtx &c)
{
    // ---- issue every load of the part: scales, then (x, codes) per slab ----
    constexpr int kSL = GROUPED ? (GC * S + 3) / 4 : 0;  // scale loads per lane
    uint32_t sv[kSL > 0 ? kSL : 1];
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
        // lane l: row l & 15, local column group (l >> 4) + 4j of the part's
        // GC*S; its scale is that of group gr (of half slab gr when GC = 2)
        const int lg = (c.lane >> 4) + 4 * j;
        const int gr = (GC * c.s_begin + lg) >> (GC == 2 ? c.gsh : 0);
        const int off = (c.srow_off >= 0 && lg < GC * S && gr < c.ngroups) ? c.srow_off + gr * 2
                                                                           : kOOB;
        sv[j] = __builtin_amdgcn_raw_buffer_load_b16(c.sr, off, 0, 0);
    }
    XPiece<MT> xv[S];
    u32x4_t w[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
        xv[i] = x_piece_load<MT>(c, c.s_begin + i);
        w[i] = __builtin_amdgcn_raw_buffer_load_b128(c.wr, c.woff + (c.s_begin + i) * 64, 0, 0);
        __builtin_amdgcn_sched_barrier(0);  // keep issue order = consumption order
    }

    // ---- scales and the first x piece into this wave's LDS -----------------
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
        const int lg = (c.lane >> 4) + 4 * j;
        if (lg < GC * S)
            c.sbuf[lg * 16 + (c.lane & 15)] = (uint16_t)sv[j];
    }
    x_piece_store<MT>(c, 0, xv[0]);

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // B operand pieces: lanes without real B entries keep zeros throughout
    // (GC = 8: every lane rewrites both, the 32-groups change with d).
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
    uint4 b0 = zero4, b1 = zero4;
#pragma unroll
    for (int i = 0; i < S; ++i) {
        // the next slab's x goes into the other buffer while this slab runs
        if (i + 1 < S)
            x_piece_store<MT>(c, (i + 1) & 1, xv[i + 1]);
        __builtin_amdgcn_wave_barrier();
        const uint4 *xb =
            reinterpret_cast<const uint4 *>(c.xbuf + (i & 1) * kXBufElems + c.tok * 256 + c.g * 64);
        const uint32_t wv[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
        f32x4_t part = GROUPED ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc;
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
        if constexpr (GROUPED) {
            // C rows of this lane: channels 4g + r of the block; column group
            // GC*i + par of the part (scales past K or N were loaded as zeros).
            const uint2 s4 =
                *reinterpret_cast<const uint2 *>(c.sbuf + (GC * i + c.par) * 16 + 4 * c.g);
            acc[0] += f16_bits_to_f32((uint16_t)s4.x) * part[0];
            acc[1] += f16_bits_to_f32((uint16_t)(s4.x >> 16)) * part[1];
            acc[2] += f16_bits_to_f32((uint16_t)s4.y) * part[2];
            acc[3] += f16_bits_to_f32((uint16_t)(s4.y >> 16)) * part[3];
        } else {
            acc = part;
        }
        // this buffer is rewritten two slabs on; LDS ops of a wave run in order
        __builtin_amdgcn_wave_barrier();
    }
    return acc;
}

// Parts of up to kMaxS slabs; the kernel for parts of at most kShortS slabs
// (every problem with K <= kShortS * 16 * 256) is a separate instance, because
// the longer parts' loads need more registers than 8 waves per SIMD allow.
constexpr int kShortS = 6;

template <bool FP16, bool GROUPED, int GC, int MT, bool LONG>
__device__ __forceinline__ f32x4_t run_part_n(const WaveCtx &c, int S)
{
    if constexpr (LONG) {
        if (S == 7)
            return run_part<FP16, GROUPED, GC, MT, 7>(c);
        if (S == 8)
            return run_part<FP16, GROUPED, GC, MT, 8>(c);
    }
    switch (S) {
    case 1: return run_part<FP16, GROUPED, GC, MT, 1>(c);
    case 2: return run_part<FP16, GROUPED, GC, MT, 2>(c);
    case 3: return run_part<FP16, GROUPED, GC, MT, 3>(c);
    case 4: return run_part<FP16, GROUPED, GC, MT, 4>(c);
    case 5: return run_part<FP16, GROUPED, GC, MT, 5>(c);
    case 6: return run_part<FP16, GROUPED, GC, MT, 6>(c);
    default: return f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
}
static_assert(kMaxS == 8 && kShortS == 6, "run_part_n covers S = 1..kMaxS");

// GC: B columns per token (gemv_cols of the group size: 2 for per-channel
// scales and groups of 128 K or more, 4 for 64, 8 for 32); column GC*t + p
// holds token t restricted to group p of each slab (half p when GC = 2).
template <bool FP16, bool GROUPED, int GC, int MT, bool LONG>

__global__ void __launch_bounds__(kThreads) gemv_stream_kernel(const StreamBatch batch)
{
    // LDS: per wave [2][M*256] x buffers + [2*kMaxS][16] group scales; the
    // K-part reduction reuses it after a barrier.
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    int pi = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxBatch; ++i)
        if (i < batch.count && (int)blockIdx.x >= batch.unit0[i])
            pi = i;
    const StreamProblem &P = batch.p[pi];
    constexpr int M = MT;
    const int N = P.N, K = P.K, RB = P.rb, KP = P.kp;

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

    WaveCtx c;
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
    c.b_lane = c.tok < M && (GC == 2 ? (c.g >> 1) == c.par : (GC == 4 ? c.g == c.par : true));
    c.s_begin = kpi * P.spart;
    const int S = active ? min(P.spart, nslabs - c.s_begin) : 0;
    // (readfirstlane: the clamp lowers to a vector op, and a descriptor in
    // vector registers would put every load in a waterfall loop)
    const int nrows = __builtin_amdgcn_readfirstlane(active ? max(0, min(16, N - rb * 16)) : 0);
    const uint8_t *wbase = nrows > 0 ? P.packed + (int64_t)rb * 16 * rowbytes : P.packed;
    c.wr = make_rsrc(wbase, (uint32_t)(nrows * rowbytes));
    c.woff = col * rowbytes + c.g * 16;
    c.xr = make_rsrc(P.x, (uint32_t)M * (uint32_t)K * 2u);
    c.sr = make_rsrc(P.scale, (uint32_t)N * (uint32_t)(GROUPED ? ngroups : 1) * 2u);
    c.srow_off = (lane & 15) < nrows ? (rb * 16 + (lane & 15)) * ngroups * 2 : -1;
    uint16_t *wlds = reinterpret_cast<uint16_t *>(smem) + wave * wave_lds_elems<GC>();
    c.xbuf = wlds;
    c.sbuf = wlds + 2 * kXBufElems;

    // per-channel scales: lane l < 16 of the wave that finishes the block
    // loads channel l (issued before the part's loads, used at the end)
    uint32_t chs = 0u;
    if constexpr (!GROUPED) {
        if (active && kpi == 0) {
            const int ch = rb * 16 + lane;
            chs = __builtin_amdgcn_raw_buffer_load_b16(c.sr, lane < 16 && ch < N ? ch * 2 : kOOB,
                                                       0, 0);
        }
    }

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (S > 0)
        acc = run_part_n<FP16, GROUPED, GC, MT, LONG>(c, S);

    // ---- K-part reduction (fixed order) and epilogue ------------------------
    f32x4_t sum = acc;
    if (KP > 1) {
        f32x4_t *red = reinterpret_cast<f32x4_t *>(smem);
        __syncthreads();  // every wave is done with its LDS buffers
        if (active)
            red[wave * 64 + lane] = acc;
        __syncthreads();
        if (!active || kpi != 0)
            return;
        for (int j = 1; j < KP; ++j) {
            const f32x4_t v = red[(rbi + j * RB) * 64 + lane];
            sum[0] += v[0];
            sum[1] += v[1];
            sum[2] += v[2];
            sum[3] += v[3];
        }
    } else if (!active) {
        return;
    }
    uint16_t *__restrict__ y = P.y;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        // the GC columns of a token (adjacent lanes) hold disjoint K sets
        float tot = sum[r] + __shfl_xor(sum[r], 1);
        if constexpr (GC >= 4)
            tot += __shfl_xor(tot, 2);
        if constexpr (GC >= 8)
            tot += __shfl_xor(tot, 4);
        const int ch = rb * 16 + 4 * c.g + r;
        float o = 0.5f * tot;  // decoded weights are +-2
        if constexpr (!GROUPED)
            o *= f16_bits_to_f32((uint16_t)__shfl((int)chs, 4 * c.g + r));
        if (c.par == 0 && c.tok < M && ch < N)
            y[(int64_t)c.tok * N + ch] = round_out<FP16>(o);
    }
}

// LDS bytes of a workgroup: the per-wave buffers, or the K-part reduction
// area if larger.
template <int GC>
constexpr size_t lds_bytes()
{
    return std::max<size_t>((size_t)kWaves * wave_lds_elems<GC>() * 2, (size_t)kWaves * 64 * 16);
}

// K split of one problem: parts of about `target` slabs, at most kMaxS, on at
// most kWaves waves per block.  Returns false when this kernel cannot take it.
bool split_k(int M, int K, int target, int &kp, int &spart)
{
    if (M < 1 || M > kGemvStreamMaxM)
        return false;
    const int nslabs = (K + 255) / 256;
    if (nslabs > kWaves * kMaxS)
        return false;
    kp = std::min(kWaves, (nslabs + target - 1) / target);
    spart = (nslabs + kp - 1) / kp;
    kp = (nslabs + spart - 1) / spart;  // no empty parts
    return spart <= kMaxS;
}

}  // namespace

bool gemv_stream_takes(int64_t M, int64_t K, int group)
{
    int kp = 0, spart = 0;
    return K % 128 == 0 && K <= kGemvMaxK && M * gemv_cols(group) <= 16 &&
           (group == 0 || K % group == 0) && split_k((int)M, (int)K, 2, kp, spart);
}

namespace {
template <bool FP16, bool GROUPED, int GC>
void launch_m(int mt, bool long_parts, dim3 grid, dim3 block, hipStream_t stream,
              const StreamBatch &b)
{
    constexpr size_t lds = lds_bytes<GC>();
    if (long_parts) {
        if (mt == 1)
            hipLaunchKernelGGL((gemv_stream_kernel<FP16, GROUPED, GC, 1, true>), grid, block, lds,
                               stream, b);
        else
            hipLaunchKernelGGL((gemv_stream_kernel<FP16, GROUPED, GC, 2, true>), grid, block, lds,
                               stream, b);
    } else if (mt == 1) {
        hipLaunchKernelGGL((gemv_stream_kernel<FP16, GROUPED, GC, 1, false>), grid, block, lds,
                           stream, b);
    } else {
        hipLaunchKernelGGL((gemv_stream_kernel<FP16, GROUPED, GC, 2, false>), grid, block, lds,
                           stream, b);
    }
}

template <bool FP16>
void launch_group(int group, int mt, bool long_parts, dim3 grid, dim3 block, hipStream_t stream,
                  const StreamBatch &b)
{
    if (group == 0)
        launch_m<FP16, false, 2>(mt, long_parts, grid, block, stream, b);
    else if (group == 32)
        launch_m<FP16, true, 8>(mt, long_parts, grid, block, stream, b);
    else if (group == 64)
        launch_m<FP16, true, 4>(mt, long_parts, grid, block, stream, b);
    else
        launch_m<FP16, true, 2>(mt, long_parts, grid, block, stream, b);
}

template <bool GROUPED, int GC>
int occupancy(int mt, bool long_parts)
{
    const void *k = long_parts
                        ? (mt == 1 ? (const void *)gemv_stream_kernel<false, GROUPED, GC, 1, true>
                                   : (const void *)gemv_stream_kernel<false, GROUPED, GC, 2, true>)
                        : (mt == 1 ? (const void *)gemv_stream_kernel<false, GROUPED, GC, 1, false>
                                   : (const void *)gemv_stream_kernel<false, GROUPED, GC, 2, false>);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kThreads, lds_bytes<GC>()) !=
            hipSuccess ||
        n < 1)
        n = 1;
    return n;
}

// Workgroups of one kernel instance that fit on a CU (cached).
int stream_slots_per_cu(int mt, bool long_parts, int group)
{
    const int gi = group == 0 ? 0 : (group == 32 ? 1 : (group == 64 ? 2 : 3));
    static int cache[2][2][4] = {};
    int &v = cache[mt - 1][long_parts][gi];
    if (v == 0)
        v = gi == 0   ? occupancy<false, 2>(mt, long_parts)
            : gi == 1 ? occupancy<true, 8>(mt, long_parts)
            : gi == 2 ? occupancy<true, 4>(mt, long_parts)
                      : occupancy<true, 2>(mt, long_parts);
    return v;
}

}  // namespace

hipError_t launch_gemv_stream(const GemvArgs *args, const int *order, int count, bool fp16,
                              int group, hipStream_t stream)
{
    // The part length (slabs per wave) of the whole batch, a function of the
    // batch only (so deterministic): 4 slabs, or 2 when 4 leaves fewer than
    // 512 workgroups (both measured best on MI355X); and when the workgroups
    // exceed the resident slots by less than a quarter of a round, the
    // shortest longer part (up to kShortS slabs) that removes that round
    // while still filling three quarters of the remaining rounds' slots,
    // since the few left-over workgroups would cost a round of their own
    // (27B up at M=1: 534 workgroups at 4 slabs, 14.5 us; 400 at 5, 12.8 us;
    // 7B gate: 592 at 2 slabs, 9.5 us, beats 296 at 4, 9.9 us).
    StreamBatch b;
    int units = 0, mt = 0, max_spart = 0;
    auto build = [&](int target) -> bool {
        b.count = 0;
        units = 0;
        mt = 0;
        max_spart = 0;
        for (int oi = 0; oi < count; ++oi) {
            const GemvArgs &a = args[order[oi]];
            if (a.M == 0 || a.N == 0)
                continue;
            StreamProblem &p = b.p[b.count];
            if (a.group != group || (mt != 0 && a.M != mt) ||
                !split_k(a.M, a.K, target, p.kp, p.spart))
                return false;
            mt = a.M;
            p.x = a.x;
            p.packed = a.packed;
            p.scale = a.scale;
            p.y = a.y;
            p.N = a.N;
            p.K = a.K;
            p.group = group;
            const int nblocks = (a.N + 15) / 16;
            p.rb = std::min(kWaves / p.kp, nblocks);
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
            max_spart = std::max(max_spart, p.spart);
            ++b.count;
        }
        return true;
    };
    int base_target = 4;
    if (!build(base_target))
        return hipErrorInvalidValue;
    if (units < 512) {
        base_target = 2;
        if (!build(base_target))
            return hipErrorInvalidValue;
    }
    if (b.count > 0 && max_spart <= kShortS) {
        const int slots = device_cus() * stream_slots_per_cu(mt, false, group);
        const int rounds = (units + slots - 1) / slots;
        if (rounds > 1 && units - (rounds - 1) * slots < slots / 4) {
            int pick = 0;
            for (int t = base_target + 1; t <= kShortS && !pick; ++t)
                if (build(t) && max_spart <= kShortS &&
                    (units + slots - 1) / slots < rounds && 4 * units >= 3 * (rounds - 1) * slots)
                    pick = t;
            if (!build(pick ? pick : base_target))
                return hipErrorInvalidValue;
        }
    }
    if (b.count == 0)
        return hipSuccess;
    bool long_parts = false;
    for (int i = 0; i < b.count; ++i)
        long_parts = long_parts || b.p[i].spart > kShortS;
    const dim3 grid(units), block(kThreads);
    if (fp16)
        launch_group<true>(group, mt, long_parts, grid, block, stream, b);
    else
        launch_group<false>(group, mt, long_parts, grid, block, stream, b);
    return hipGetLastError();
}

}  // namespace ternary
