// Decode GEMV (1 <= M <= 8) for the ternary linear layer on gfx950, for one
// projection or a batch of projections fused into one launch.
//
// The layer ([xxqk] m.xxqk.cn/news/593501 §4.3: y = x @ (unpack(q) * s)^T) at
// small M is bound by the HBM stream of packed weights ([nxbn]
// m.nxbn.cn/news/169761 §4.1/§4.4: decode is memory-bound, the 2-bit packing
// is what cuts the bytes).  Scale granularity: one fp16 per output channel
// ([nxbn] §3.2) or per group of 128 consecutive K weights ([trdm] trdm.cn
// "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1; 64 in [xxqk]
// m.xxqk.cn/news/593501 §4.2, 32 and 256 in the yangyitao.com vLLM book,
// chapter 13, §13.3.3), applied to the finished partial sum of its group
// ([trdm] §4.2).  Several projections (for
// instance the segments of a fused QKV weight, [trdm] §2.2) can share one
// launch, which pays the fixed launch and first-byte latency once.
//
// Mapping onto CDNA4:
//  * A workgroup is 4 waves and owns RB blocks of 16 output channels: each
//    wave takes one block and 1/KP of its K slabs (KP = 4/RB, chosen by K and
//    M), a slab being 256 codes (64 bytes) of every channel.
//  * Per slab a lane issues ONE 16-byte load of packed codes: lane l reads
//    channel (l & 15), bytes [16*(l>>4), +16) of the slab, so a wave reads
//    16 channels x 64 contiguous bytes per instruction.  Slabs stream in
//    groups of four, the next group's loads in flight while the current one
//    is decoded.
//  * The codes are decoded in registers (decode16, branch-free byte permutes)
//    into the A operand of v_mfma_f32_16x16x32_{bf16,f16}: rows = channels,
//    k in natural order.  The B operand is the activation: column GC*t + p
//    holds token t restricted to group p of the slab (GC = 2 halves of 128
//    for per-channel scales and groups of 128 or 256, 4 groups of 64, 8 of
//    32; lanes of the other groups keep zeros), so one MFMA chain yields every
//    group's partial sum separately and each is scaled by its own fp16 scale
//    before it joins the fp32 accumulator.  Only the lanes that own real B
//    entries read x.
//  * Each scale mode (per channel, each group size) is a separate kernel
//    instance, so a batch that mixes them takes one launch per mode.
//  * x (all M tokens) is copied into LDS with direct global->LDS loads, whole
//    K when it fits 64 KB, otherwise in K chunks (then KP = 1 and the waves
//    walk the chunks together).  Group scales of the workgroup's channels are
//    staged in LDS too.
//  * The MFMA does the add/sub accumulate (weights are exactly +-2 or 0, the
//    products exact, the sums fp32).
//  * The KP partial tiles of a channel block are reduced through LDS in a
//    fixed order, the two group columns of a token are combined with a lane
//    shuffle, and the result is rounded to the output dtype (nearest even).
#include "common.h"
#include "internal.h"

namespace ternary {

namespace {

constexpr int kThreads = 256;         // 4 waves
constexpr int kGroup = 4;             // slabs per load group
constexpr int kXLdsBytes = 64 << 10;  // activation chunk staged in LDS per workgroup

struct GemvProblem {
    const uint16_t *x;
    const uint8_t *packed;
    const uint16_t *scale;
    uint16_t *y;
    int M, N, K;
    int group;    // 0 (per channel) or the group size
    int rb;       // 16-channel blocks per workgroup: 1, 2 or 4
    int spart;    // slabs per wave (one K part)
    int kc;       // K elements staged in LDS at once (multiple of 1024)
    int unit0;    // first workgroup of this problem
};

struct GemvBatch {
    int count;
    GemvProblem p[kGemvMaxBatch];
};

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

typedef __attribute__((address_space(3))) void lds_void;

// Copy x[:, k0 : k0 + kc] into xs[t][kk] (t < M) with direct global->LDS
// loads, one 16-byte piece per lane; pieces past K are written as zeros, so
// codes read past the end of a row (clamped loads below) meet zero activations.
__device__ __forceinline__ void stage_x(const uint16_t *x, uint16_t *xs, int M, int K, int k0,
                                        int kc, int wave, int lane)
{
    const int per_tok = kc >> 3;  // 16-byte pieces per token
    for (int t = 0; t < M; ++t) {
        const uint16_t *src = x + (int64_t)t * K + k0;
        uint16_t *dst = xs + t * kc;
        for (int v = wave * 64; v < per_tok; v += kThreads) {
            const int p = v + lane;
            if (p < per_tok) {
                if (k0 + p * 8 < K)
                    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src + p * 8),
                                                     (lds_void *)(dst + v * 8), 16, 0, 0);
                else
                    *reinterpret_cast<uint4 *>(dst + p * 8) = make_uint4(0, 0, 0, 0);
            }
        }
    }
}

// GC: MFMA B columns per token (gemv_cols of the group size): 2 for
// per-channel scales and groups of 128 K or more, 4 for groups of 64, 8 for
// groups of 32.  Column GC*t + p holds token t restricted to group p of each
// slab (to half p of it when GC = 2).
template <bool FP16, bool GROUPED, int GC>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5, 8)))
gemv_kernel(const GemvBatch batch)
{
    // LDS: [4][64] fp32x4 reduction tiles | scales ([RB][K/group][16] grouped,
    // [RB*16] per channel, 128 bytes) | x [M][kc]
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    int pi = 0;
    for (int i = 1; i < batch.count; ++i)
        if ((int)blockIdx.x >= batch.p[i].unit0)
            pi = i;
    const GemvProblem &P = batch.p[pi];
    const uint16_t *__restrict__ x = P.x;
    const uint8_t *__restrict__ packed = P.packed;
    const uint16_t *__restrict__ scale = P.scale;
    const int M = P.M, N = P.N, K = P.K, RB = P.rb, kc = P.kc;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int KP = 4 / RB;
    const int rbi = wave % RB;        // which of the workgroup's channel blocks
    const int kp = wave / RB;         // which K part of that block
    const int blk0 = ((int)blockIdx.x - P.unit0) * RB;
    const int rb = blk0 + rbi;
    const int g = lane >> 4;          // lane group: which 64-code quarter of a slab
    const int col = lane & 15;        // MFMA column (B) and row (A) index of this lane
    const int tok = col / GC;         // token of this B column
    const int par = col % GC;         // group (or half) of the slab this column collects
    const int row = rb * 16 + col;    // channel whose codes this lane loads (A row)
    const bool row_ok = row < N;
    // Lane group g holds codes 64g .. 64g+63 of a slab, word d of them codes
    // 64g + 16d .. +15: in half g/2, in 64-group g, in 32-group 2g + d/2.
    const bool b_lane = tok < M && (GC == 2 ? (g >> 1) == par : (GC == 4 ? g == par : true));
    const int nslabs = (K + 255) >> 8;
    const int glog = GROUPED ? 31 - __builtin_clz((unsigned)P.group) : 7;
    const int ngroups = K >> glog;
    const int s_begin = kp * P.spart;
    const int s_end = s_begin + P.spart < nslabs ? s_begin + P.spart : nslabs;
    const int chunk_slabs = kc >> 8;

    f32x4_t *red = reinterpret_cast<f32x4_t *>(smem);
    uint16_t *sc = reinterpret_cast<uint16_t *>(smem + 4 * 1024);
    uint16_t *xs = sc + (GROUPED ? ((RB * ngroups * 16 + 7) & ~7) : 64);
    const uint4 zero4 = make_uint4(0, 0, 0, 0);

    // Packed codes: every load is in bounds.  Rows past N read row N-1 (their
    // C rows are never stored); slabs past this wave's range repeat its last
    // slab (never decoded); a slab quarter past K reads the row's last 16
    // bytes (its activations are zero in LDS).
    const int rowbytes = K >> 2;
    const uint8_t *prow = packed + (int64_t)(row_ok ? row : N - 1) * rowbytes;
    const int s_last = s_end > s_begin ? s_end - 1 : s_begin;
    auto load_group = [&](uint4 (&buf)[kGroup], int s0) {
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const int s = s0 + i < s_last ? s0 + i : s_last;
            int off = s * 64 + g * 16;
            off = off + 16 <= rowbytes ? off : rowbytes - 16;
            buf[i] = *reinterpret_cast<const uint4 *>(prow + off);
        }
    };
    uint4 wa[kGroup], wb[kGroup];
    if (s_begin < s_end)
        load_group(wa, s_begin);

    if constexpr (GROUPED) {
        // sc[(bi*ngroups + gr)*16 + r] = scale of channel (blk0 + bi)*16 + r, group gr
        for (int e = tid; e < RB * 16 * ngroups; e += kThreads) {
            const int rr = e / ngroups, gr = e - rr * ngroups;
            const int ch = blk0 * 16 + rr;
            sc[((rr >> 4) * ngroups + gr) * 16 + (rr & 15)] =
                ch < N ? scale[(int64_t)ch * ngroups + gr] : (uint16_t)0;
        }
    } else {
        // sc[r] = scale of channel blk0*16 + r (read by the epilogue)
        if (tid < RB * 16) {
            const int ch = blk0 * 16 + tid;
            sc[tid] = ch < N ? scale[ch] : (uint16_t)0;
        }
    }
    stage_x(x, xs, M, K, 0, kc, wave, lane);
    __syncthreads();
    int chunk = 0;

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // B operand pieces (two per decoded word).  Lanes without real B entries
    // keep zeros for the whole kernel; lanes with them overwrite both each time.
    uint4 b0 = make_uint4(0, 0, 0, 0), b1 = make_uint4(0, 0, 0, 0);

    // Decode + MFMA one held group of slabs starting at s0.
    auto compute_group = [&](const uint4 (&buf)[kGroup], int s0) {
        const int c = s0 / chunk_slabs;
        if (c != chunk) {
            // Only when x is chunked: then KP == 1 and every wave of the
            // workgroup reaches this point at the same iteration.
            __syncthreads();
            stage_x(x, xs, M, K, c * kc, kc, wave, lane);
            __syncthreads();
            chunk = c;
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const int s = s0 + i;
            if (s >= s_end)
                break;
            const uint4 *xb = reinterpret_cast<const uint4 *>(
                xs + tok * kc + (s - chunk * chunk_slabs) * 256 + g * 64);
            const uint32_t wv[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
            f32x4_t part = GROUPED ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                if constexpr (GC == 8) {
                    // the 32-groups change with d: every lane rewrites both
                    if (b_lane && par == 2 * g + (d >> 1)) {
                        b0 = xb[2 * d];
                        b1 = xb[2 * d + 1];
                    } else {
                        b0 = zero4;
                        b1 = zero4;
                    }
                } else if (b_lane) {
                    b0 = xb[2 * d];
                    b1 = xb[2 * d + 1];
                }
                uint32_t a[8];
                decode16(wv[d], a);
                part = mfma16x16x32<FP16>(a, b0, part);
                part = mfma16x16x32<FP16>(a + 4, b1, part);
            }
            if constexpr (GROUPED) {
                // C rows of this lane: channels rb*16 + 4g + r; column group
                // `par` (for GC = 2 a half slab: 128 K, within group
                // (2s + par) * 128 / group when groups are longer).
                const int grp = GC == 2 ? (2 * s + par) >> (glog - 7) : GC * s + par;
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
    };

    // Two register buffers in turn: the next group's loads are in flight
    // while the current group is decoded.
    for (int s0 = s_begin; s0 < s_end; s0 += 2 * kGroup) {
        if (s0 + kGroup < s_end)
            load_group(wb, s0 + kGroup);
        compute_group(wa, s0);
        if (s0 + kGroup >= s_end)
            break;
        if (s0 + 2 * kGroup < s_end)
            load_group(wa, s0 + 2 * kGroup);
        compute_group(wb, s0 + kGroup);
    }

    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (kp != 0)
        return;
    f32x4_t sum = acc;
    for (int j = 1; j < KP; ++j) {
        const f32x4_t v = red[(rbi + j * RB) * 64 + lane];
        sum[0] += v[0];
        sum[1] += v[1];
        sum[2] += v[2];
        sum[3] += v[3];
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
        const int ch = rb * 16 + 4 * g + r;
        if (par == 0 && tok < M && ch < N) {
            float o = 0.5f * tot;  // decoded weights are +-2
            if constexpr (!GROUPED)
                o *= f16_bits_to_f32(sc[rbi * 16 + 4 * g + r]);
            y[(int64_t)tok * N + ch] = round_out<FP16>(o);
        }
    }
}

// Launch shape of one problem; returns its LDS bytes.  The K split KP (waves
// per channel block) keeps a wave's slab run long enough to amortise its
// fixed costs but bounded for long K; larger M puts more channel blocks in a
// workgroup so the x it stages serves more rows.
size_t plan(GemvProblem &p)
{
    const int nslabs = (p.K + 255) / 256;
    int kp = nslabs >= 32 ? 4 : (nslabs >= 8 ? 2 : 1);
    if (p.M >= 3) {
        // From M = 3 the x a workgroup stages grows to a multiple of its
        // weights: share it over more channel blocks when there are blocks to
        // spare (2 for M <= 4, 4 beyond), but keep one block per workgroup
        // when fewer than 512 blocks would otherwise leave CUs idle
        // (measured on the 7B and 0.6B shapes at M = 8).
        const int nblocks = (p.N + 15) / 16;
        const int rb = nblocks >= 1024 ? (p.M >= 5 ? 4 : 2) : (nblocks >= 512 ? 2 : 1);
        kp = nslabs >= 8 ? 4 / rb : 1;
    }
    p.rb = 4 / kp;
    int kc = ((nslabs + 3) / 4) * 1024;  // whole K, padded to a multiple of 1024
    if ((size_t)p.M * kc * 2 > (size_t)kXLdsBytes) {
        // x does not fit: walk K in chunks, each wave on a whole channel block
        p.rb = 4;
        kc = (kXLdsBytes / (2 * p.M)) / 1024 * 1024;
    }
    p.kc = kc;
    const int KP = 4 / p.rb;
    p.spart = (nslabs + KP - 1) / KP;
    return 4 * 1024 + (p.group ? (size_t)((p.rb * (p.K / p.group) * 16 + 7) & ~7) * 2 : 128) +
           (size_t)p.M * kc * 2;
}

int units_of(const GemvProblem &p) { return ((p.N + 15) / 16 + p.rb - 1) / p.rb; }

}  // namespace

namespace {

// One launch for the problems of one group value.
template <bool FP16>
void launch_kernel(int group, int units, size_t lds, hipStream_t stream, const GemvBatch &b)
{
    if (group == 0)
        hipLaunchKernelGGL((gemv_kernel<FP16, false, 2>), dim3(units), dim3(kThreads), lds, stream, b);
    else if (group == 32)
        hipLaunchKernelGGL((gemv_kernel<FP16, true, 8>), dim3(units), dim3(kThreads), lds, stream, b);
    else if (group == 64)
        hipLaunchKernelGGL((gemv_kernel<FP16, true, 4>), dim3(units), dim3(kThreads), lds, stream, b);
    else
        hipLaunchKernelGGL((gemv_kernel<FP16, true, 2>), dim3(units), dim3(kThreads), lds, stream, b);
}

hipError_t launch_mode(const GemvArgs *args, const int *order, int count, bool fp16, int group,
                       hipStream_t stream)
{
    GemvBatch b;
    b.count = 0;
    size_t lds = 0;
    int units = 0;
    for (int oi = 0; oi < count; ++oi) {
        const GemvArgs &a = args[order[oi]];
        if (a.M == 0 || a.N == 0 || a.group != group)
            continue;
        GemvProblem &p = b.p[b.count++];
        p.x = a.x;
        p.packed = a.packed;
        p.scale = a.scale;
        p.y = a.y;
        p.M = a.M;
        p.N = a.N;
        p.K = a.K;
        p.group = group;
        const size_t l = plan(p);
        lds = l > lds ? l : lds;
        p.unit0 = units;
        units += units_of(p);
    }
    if (b.count == 0)
        return hipSuccess;
    if (fp16)
        launch_kernel<true>(group, units, lds, stream, b);
    else
        launch_kernel<false>(group, units, lds, stream, b);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_batch(const GemvArgs *args, int count, bool fp16, hipStream_t stream)
{
    if (count < 1 || count > kGemvMaxBatch)
        return hipErrorInvalidValue;
    // Longest workgroups first (most K each), so they start early and the
    // short ones fill in behind them.
    int order[kGemvMaxBatch];
    for (int i = 0; i < count; ++i)
        order[i] = i;
    for (int i = 1; i < count; ++i)
        for (int j = i; j > 0 && args[order[j]].K > args[order[j - 1]].K; --j) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    // Each group value (per channel, 32, 64, 128, 256) is a separate kernel
    // instance, and so are the problems the streaming kernel takes (M = 1,
    // M = 2) and the others: one launch per non-empty class.
    static const int kGroups[] = {0, 32, 64, 128, 256};
    for (const int group : kGroups) {
        int stream_idx[kGemvStreamMaxM][kGemvMaxBatch], other_idx[kGemvMaxBatch];
        int ns[kGemvStreamMaxM] = {}, no = 0;
        for (int oi = 0; oi < count; ++oi) {
            const GemvArgs &a = args[order[oi]];
            if (a.group != group || a.M == 0 || a.N == 0)
                continue;
            if (gemv_stream_takes(a.M, a.K, group))
                stream_idx[a.M - 1][ns[a.M - 1]++] = order[oi];
            else
                other_idx[no++] = order[oi];
        }
        for (int m = 0; m < kGemvStreamMaxM; ++m) {
            if (ns[m] == 0)
                continue;
            const hipError_t e = launch_gemv_stream(args, stream_idx[m], ns[m], fp16, group, stream);
            if (e != hipSuccess)
                return e;
        }
        if (no > 0) {
            const hipError_t e = launch_mode(args, other_idx, no, fp16, group, stream);
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_gemv(const uint16_t *x, bool fp16, int M, int N, int K, const uint8_t *packed,
                       const uint16_t *scale, int group, uint16_t *y, hipStream_t stream)
{
    const GemvArgs a = {x, packed, scale, y, M, N, K, group};
    return launch_gemv_batch(&a, 1, fp16, stream);
}

}  // namespace ternary
