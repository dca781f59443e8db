// Few-token streaming GEMM (1 <= M <= 32) for the ternary linear layer on gfx950.
//
// The layer y = x @ (unpack(q) * s)^T ([xxqk] m.xxqk.cn/news/593501 §4.3) at a
// handful of tokens still reads every packed weight byte once and does
// little arithmetic per byte ([nxbn] m.nxbn.cn/news/169761 §4.1/§4.4), but x
// is no longer small: 16 tokens of a 256-code slab are 8 KB of bf16 against
// the 1 KB of codes a 16-row block holds in that slab.  A kernel that gives
// every 16-row block its own copy of x moves several times more x than code
// bytes.  Here the eight waves of a workgroup own eight 16-row blocks (or
// 4 x 2, 2 x 4 blocks x K parts) and share one copy of each slab of x:
//
//  * Steps of one slab (256 K).  At step j every wave computes slab j of its
//    block and part: its codes (one 16-byte buffer load per lane, one
//    contiguous kilobyte per wave in the tiled layout) sit in registers, x
//    sits in LDS stage j % 4.  Loads run three slabs ahead: after the
//    step's barrier a wave DMAs its share of x slab j+3 into the stage that
//    slab j-1 used, then loads its codes of slab j+3 into the registers slab
//    j-1 used.  Its x DMA is issued before its codes of the same slab, loads
//    return in issue order, so the compiler's wait for a slab's codes also
//    covers the wave's x of that slab; the barrier then covers every wave's.
//  * x stage layout: per part, per token, 256 elements as 32 chunks of 16
//    bytes; logical chunk c of token row t sits at physical chunk c ^ swz(t)
//    so that the 16 token rows an MFMA B read touches spread over the banks.
//    Each 1-KB DMA fills two token rows, every lane fetching the logical
//    chunk of its physical slot; tokens past M and slabs past K read zeros.
//  * MFMA: v_mfma_f32_16x16x32_{bf16,f16}, rows = channels, columns =
//    tokens (a 32-token tile runs two MFMAs per decoded A operand, one per
//    16-token half; groups of 128 need two columns per token, so they stop
//    at 16 tokens).  Lane group g of the A operand holds codes 64g .. 64g+63 of the
//    slab (its 16-byte load), decoded to 16-bit +-2 / 0 (decode16); MFMA i
//    takes codes 64g + 8i .. 64g + 8i + 7 from every lane group, and the B
//    read of lane group g takes the same K positions of x (logical chunk
//    8g + i), so the eight MFMAs of a slab cover its 256 K exactly once.
//  * Scales ([trdm] trdm.cn "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战"
//    §3.1/§4.2; yangyitao.com vLLM book, chapter 13, §13.3.3: groups of 256):
//    per channel, the final sum takes 0.5 * s (codes decode to +-2); groups
//    of 256 are whole slabs, so each slab's sum takes its scale; groups of
//    128 split a slab into the K quarters {0, 1} and {2, 3}: B columns are
//    (token, group) pairs whose lanes outside the group read zeros, so each
//    column's slab sum belongs to one group and takes that group's scale.
//  * K parts of one block meet in LDS after the last step and are added in
//    part order (deterministic); y is written as 4 channels per lane.
#include "common.h"
#include "internal.h"

#include <algorithm>
#include <utility>

namespace ternary {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kS = 4;           // x stages in LDS = code slabs in registers per wave
constexpr int kAhead = kS - 1;  // slabs loaded ahead of the one computed
constexpr int kFN = 1;          // 16-channel blocks per wave
constexpr int kOOB = 0x40000000;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr int kMaxSlices = 16;  // K slices of one problem over workgroups

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u4;

struct FewProblem {
    const uint16_t *x;
    const uint8_t *packed;
    const uint16_t *scale;
    uint16_t *y;
    int M, N, K;
    int tiled;  // codes in the tiled layout (else row-major [N, K/4])
    int L;      // slabs per K piece (the last pieces may hold fewer or none)
    int ks;     // K slices over workgroups; > 1: fp32 sums to `partial`
    float *partial;  // [ks][M][N] when ks > 1
};

struct FewBatch {
    int count;
    int unit0[kGemvMaxBatch];  // first workgroup of each problem
    FewProblem p[kGemvMaxBatch];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             (int)kRsrcWord3);
}

// One buffer-to-LDS DMA: every lane reads 16 bytes at voff and the wave
// writes them to LDS at lds + 16 * lane.  Device target only (the host pass
// emits just the launch stub).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, lds_u4 *lds, int voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds,
                                             16, voff, 0, 0, 0);
#endif
}

// The same with 4 bytes per lane (LDS at lds + 4 * lane).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t *lds, int voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void *)lds, 4, voff, 0, 0, 0);
#endif
}

template <bool FP16>
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c)
{
    if constexpr (FP16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// x stage swizzle: logical chunk c of token row t sits at physical chunk
// c ^ swz(t).  The low three bits spread the 8 rows t & 7 over one
// 128-byte bank span, bit 4 moves rows 8 .. 15 half a row further: in an LDS
// read-pattern probe on MI355X this layout read 151 B/clk per CU against 120
// for c ^ t and 114 for plain contiguous 16-byte lanes.
__device__ __forceinline__ int swz(int t) { return (t & 7) | ((t & 8) << 1); }

// s_waitcnt with only the vector-memory count limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N <= 63, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// GM: 0 per-channel scales, 1 groups of 256, 2 groups of 128.  MT: tokens of
// the tile (8, 16 or 32).  KP: K parts (the workgroup's waves are RB = 8 / KP row
// groups x KP parts).  FN: 16-channel blocks per wave (each B read of x feeds
// FN MFMAs), so a workgroup holds RB * FN blocks.  CP: the cache policy of the
// code loads (kStreamLoad when every problem holds tiled codes).
template <bool FP16, int GM, int MT, int KP, int FN, int CP>
__global__ void __launch_bounds__(kThreads) few_kernel(const FewBatch batch)
{
    constexpr int RB = kWaves / KP;
    constexpr int GC = GM == 2 ? 2 : 1;               // B columns per token
    constexpr int CF = MT * GC > 16 ? 2 : 1;          // 16-column B fragments
    constexpr int TH = GC == 1 ? CF : 1;              // 16-token halves of the tile
    constexpr int XI = KP * MT / 2;                   // 1-KB x DMAs per stage
    constexpr int XW = (XI + kWaves - 1) / kWaves;    // x DMAs per wave and stage
    constexpr int ZC = KP * MT * 32;                  // chunk index of a stage's zero area
    constexpr int SU4 = ZC + 64;                      // stage: x chunks + 1 KB of zeros
    static_assert(MT == 8 || MT == 16 || MT == 32, "tile tokens");
    static_assert(MT <= 16 || GC == 1, "32-token tiles take one B column per token");
    static_assert(KP == 1 || KP == 2 || KP == 4, "parts");
    static_assert(FN == 1 || FN == 2 || FN == 4, "blocks per wave");
    static_assert(KP * MT <= 32, "stage size");
    static_assert(KP == 1 || kWaves * 64 <= SU4, "the part reduction fits in stage 0");
    // One LDS object per stage, so that the compiler knows a DMA into one
    // stage never writes the stage being read.
    static_assert(kS >= 3 && kS <= 8, "stages");
    __shared__ __attribute__((aligned(16))) u32x4_t st0[SU4], st1[SU4], st2[SU4],
        st3[kS > 3 ? SU4 : 1], st4[kS > 4 ? SU4 : 1], st5[kS > 5 ? SU4 : 1],
        st6[kS > 6 ? SU4 : 1], st7[kS > 7 ? SU4 : 1];
    lds_u4 *const ls[8] = {(lds_u4 *)st0, (lds_u4 *)st1, (lds_u4 *)st2, (lds_u4 *)st3,
                           (lds_u4 *)st4, (lds_u4 *)st5, (lds_u4 *)st6, (lds_u4 *)st7};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;   // K lane group of the MFMA operands
    const int col = lane & 15; // A row (channel in the block) / B column

    int pi = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxBatch; ++i)
        pi += (i < batch.count && (int)blockIdx.x >= batch.unit0[i]) ? 1 : 0;
    const FewProblem &P = batch.p[pi];
    const int M = P.M, N = P.N, K = P.K, L = P.L;
    const int unit = (int)blockIdx.x - batch.unit0[pi];
    const int ks = P.ks, slice = unit % ks;
    const int kp = wave / RB, rb = wave % RB;
    const int blk0 = ((unit / ks) * RB + rb) * FN;  // this wave's first block
    const int nblk = (N + 15) >> 4;
    const int nslabs = K >> 8;
    // K piece (slice, part) covers slabs [piece * L, piece * L + L)
    const int s_lo = (slice * KP + kp) * L;

    // Codes and scales of block f: resources rebased at the block's first
    // row (32-bit offsets).
    const int rowbytes = K >> 2;
    const int ngroups = GM == 0 ? 1 : (GM == 1 ? nslabs : 2 * nslabs);
    __amdgpu_buffer_rsrc_t wr[FN], sr[FN];
    int nrows[FN], woff[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
        const int blk = blk0 + f;
        nrows[f] = blk < nblk ? min(16, N - 16 * blk) : 0;
        if (P.tiled) {
            wr[f] = make_rsrc(P.packed + (int64_t)blk * nslabs * 1024, nrows[f] ? nslabs * 1024u : 0u);
            woff[f] = lane * 16;
        } else {
            wr[f] = make_rsrc(P.packed + (int64_t)blk * 16 * rowbytes, (uint32_t)(nrows[f] * rowbytes));
            woff[f] = col < nrows[f] ? col * rowbytes + g * 16 : kOOB;
        }
        sr[f] = make_rsrc(P.scale + (int64_t)blk * 16 * ngroups, (uint32_t)(nrows[f] * ngroups * 2));
    }
    const int sstride = P.tiled ? 1024 : 64;

    // x: DMA xi of this wave is stage instruction q = wave + 8 xi; its lanes
    // fill physical chunks 64 q + lane: part qp, token row t, chunk p.
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(P.x, (uint32_t)(M * K * 2));
    int xbase[XW], xpart[XW];
#pragma unroll
    for (int xi = 0; xi < XW; ++xi) {
        const int q = wave + kWaves * xi;
        const int c = 64 * q + lane;
        const int qp = c / (MT * 32), t = (c >> 5) % MT, p = c & 31;
        const int lc = p ^ swz(t);
        xpart[xi] = qp;
        xbase[xi] = q < XI && t < M ? (t * K + 8 * lc) * 2 : kOOB;
    }

    // B read offsets (bytes in a stage) per column fragment: token row t of
    // this wave's part, logical chunk 8 g + i at b ^ (16 i); lanes whose
    // column lies outside the tile or outside its group read the zero area.
    int boff[CF];
#pragma unroll
    for (int c = 0; c < CF; ++c) {
        int t, p;
        if constexpr (GC == 1) {
            t = 16 * c + col;  // fragment c: tokens 16c .. 16c + 15
            p = 0;
        } else if constexpr (MT == 16) {
            t = col;
            p = c;
        } else {
            t = col & 7;
            p = col >> 3;
        }
        const bool on = t < MT && (GC == 1 || (g >> 1) == p);
        boff[c] = on ? ((kp * MT + t) * 32 + ((8 * g) ^ (swz(t) & 24))) * 16 + 16 * (t & 7) : ZC * 16;
    }
    if (tid < 8) {  // B reads of masked lanes stay in the first 128 bytes
        const u32x4_t z = {0u, 0u, 0u, 0u};
        [&]<int... I>(std::integer_sequence<int, I...>) {
            ((ls[I][ZC + tid] = z), ...);
        }(std::make_integer_sequence<int, kS>{});
    }
    __syncthreads();

    // ---- loads of slab j (x share, then codes and scales) ---------------
    u32x4_t w[kS][FN];
    uint32_t sc[GM == 1 ? kS : 1][FN][4];  // groups of 256: per slot, C rows 4 g + r
    // Groups of 128: per wave and block, a round's (kS slabs') scales (one
    // dword: two groups) as [slab][row], DMA'd with the round's first slab
    // and read into registers (sq, C rows 4 g + r) when the round starts;
    // sq_shift: slabs by which the DMA started early (see issue()).
    static_assert(GM != 2 || kS == 4, "a round's scales are four dwords per row");
    constexpr int SQN = GM == 2 ? kWaves * FN * 64 : 1;
    __shared__ __attribute__((aligned(16))) uint32_t sqs[SQN];
    u32x4_t sq[GM == 2 ? FN : 1][4];
    int sq_shift = 0;
    auto issue = [&](auto SL, int j) __attribute__((always_inline)) {
        constexpr int s = decltype(SL)::value;
        const bool in = j < L;
#pragma unroll
        for (int xi = 0; xi < XW; ++xi) {
            const int q = wave + kWaves * xi;
            const int sl = (slice * KP + xpart[xi]) * L + j;
            const int off = in && sl < nslabs ? xbase[xi] + sl * 512 : kOOB;
            dma16(xr, ls[s] + (q < XI ? 64 * q : ZC), off);  // spare DMAs write zeros
        }
        __builtin_amdgcn_sched_barrier(0);
        const int sl = s_lo + j;
        const bool live = in && sl < nslabs;
        if constexpr (GM == 2 && s == 0) {
            // The round's slabs sl .. sl+3, before the codes of slab sl (the
            // wait for those covers it): lane l takes row l & 15's dword of
            // slab l >> 4, one 256-byte DMA per block.  The start is held at
            // most 4 slabs before the row's end (K >= 1024) so that no load
            // leaves the block; rows past N read a real row's scales.
            // (the last round's reads of the buffer are done)
            __builtin_amdgcn_s_waitcnt((15 << 0) | (3 << 14) | (7 << 4) | (0 << 8));
            const int lo = min(sl, nslabs - 4);
            sq_shift = sl - lo;
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                const int row = min(col, nrows[f] - 1);
                dma4(sr[f], sqs + (wave * FN + f) * 64, (row * ngroups + 2 * (lo + g)) * 2);
            }
        }
#pragma unroll
        for (int f = 0; f < FN; ++f)
            w[s][f] = load_codes<CP>(wr[f], live ? woff[f] + sl * sstride : kOOB);
        // Scale offsets are clamped into the block instead of selected, so
        // that no lane condition splits a load: rows past N and slabs past
        // the part read scales that are never used (a dead block's empty
        // resource reads zeros).
        if constexpr (GM == 1) {
            const int slc = min(sl, nslabs - 1);
#pragma unroll
            for (int f = 0; f < FN; ++f)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = min(4 * g + r, nrows[f] - 1);
                    sc[s][f][r] = __builtin_amdgcn_raw_buffer_load_b16(
                        sr[f], (row * ngroups + slc) * 2, 0, 0);
                }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // per channel: running sums; groups: scaled sums; per 16-token half
    f32x4_t acc[FN][TH], tot[FN][TH];
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int th = 0; th < TH; ++th)
            acc[f][th] = tot[f][th] = zero4;

    // Vector memory ops issued after this wave's last code load of slab j
    // (slot s) when step j starts: slab j's scale loads (groups of 256), then
    // the x DMAs, scale DMAs (groups of 128, a round's first slab), code and
    // scale loads of slabs j+1 .. j+kAhead-1.
    constexpr auto kAfter = [](int s) constexpr {
        int n = GM == 1 ? 4 * FN : 0;
        for (int i = 1; i < kAhead; ++i)
            n += XW + FN + (GM == 1 ? 4 * FN : (GM == 2 && (s + i) % kS == 0 ? FN : 0));
        return n;
    };
    static_assert(kAfter(0) <= 63 && kAfter(1) <= 63 && kAfter(2) <= 63 && kAfter(3) <= 63,
                  "vmcnt range");

    // One step: slab j from slot / stage s.
    auto step = [&](auto SL, int j) __attribute__((always_inline)) {
        constexpr int s = decltype(SL)::value;
        // This wave's codes of slab j have landed, and with them (issued
        // earlier, returned in order) its x DMAs of slab j; after the barrier
        // every wave's have, and every wave is done with stage s - 1.
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<kAfter(s)>();
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (GM == 2 && s == 0) {
            // the round's scales, before the next round's DMA reuses the
            // buffer: slab i is the DMA's slab i + shift (past the row's end
            // only for dead slabs, which take the last one's scales)
#pragma unroll
            for (int f = 0; f < FN; ++f)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k = min(i + sq_shift, 3);
                    sq[f][i] = *(const lds_u4 *)(sqs + (wave * FN + f) * 64 + k * 16 + 4 * g);
                }
        }
        issue(std::integral_constant<int, (s + kAhead) % kS>{}, j + kAhead);

        f32x4_t part[FN][CF];
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int c = 0; c < CF; ++c)
                part[f][c] = GM == 0 ? acc[f][c] : zero4;  // per channel: GC == 1, TH == CF
        const lds_u4 *stg = ls[s];
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {  // code word wd: MFMAs 2 wd, 2 wd + 1
            uint32_t d[FN][8];
#pragma unroll
            for (int f = 0; f < FN; ++f)
                decode16(w[s][f][wd], d[f]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int i = 2 * wd + h;
#pragma unroll
                for (int c = 0; c < CF; ++c) {
                    const u32x4_t bv = *(const lds_u4 *)((const __attribute__((address_space(3))) char *)stg +
                                                         (boff[c] ^ (16 * i)));
#pragma unroll
                    for (int f = 0; f < FN; ++f) {
                        const uint4 a = h ? make_uint4(d[f][4], d[f][5], d[f][6], d[f][7])
                                          : make_uint4(d[f][0], d[f][1], d[f][2], d[f][3]);
                        part[f][c] = mfma16<FP16>(a, __builtin_bit_cast(uint4, bv), part[f][c]);
                    }
                }
            }
        }
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            if constexpr (GM == 0) {
#pragma unroll
                for (int c = 0; c < CF; ++c)
                    acc[f][c] = part[f][c];
            } else {
                u32x4_t sv = {0u, 0u, 0u, 0u};
                if constexpr (GM == 2)
                    sv = sq[f][s];
#pragma unroll
                for (int c = 0; c < CF; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        uint32_t h;
                        if constexpr (GM == 1) {
                            h = sc[s][f][r];
                        } else {
                            const uint32_t v = sv[r];
                            if constexpr (MT == 16)
                                h = c ? v >> 16 : v;
                            else
                                h = (col >> 3) ? v >> 16 : v;
                        }
                        tot[f][GC == 1 ? c : 0][r] += f16_bits_to_f32((uint16_t)h) * part[f][c][r];
                    }
            }
        }
    };

    // Prologue: slabs 0 .. kAhead-1; then rounds of kS steps, then the rest.
    [&]<int... I>(std::integer_sequence<int, I...>) {
        (issue(std::integral_constant<int, I>{}, I), ...);
    }(std::make_integer_sequence<int, kAhead>{});
    int j = 0;
    for (; j + kS <= L; j += kS) {
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (step(std::integral_constant<int, I>{}, j + I), ...);
        }(std::make_integer_sequence<int, kS>{});
    }
    [&]<int... I>(std::integer_sequence<int, I...>) {
        ((j + I < L ? step(std::integral_constant<int, I>{}, j + I) : void()), ...);
    }(std::make_integer_sequence<int, kAhead>{});
    // No DMA may still write LDS when it is reused or the workgroup ends.
    wait_vm<0>();

#pragma unroll
    for (int ft = 0; ft < FN * TH; ++ft) {
        const int f = ft / TH, th = ft % TH;
        f32x4_t res = GM == 0 ? acc[f][th] : tot[f][th];
        if constexpr (GC == 2 && MT == 8) {
            // columns t and t + 8 hold token t's two groups
#pragma unroll
            for (int r = 0; r < 4; ++r)
                res[r] += __shfl_xor(res[r], 8);
        }
        if constexpr (KP > 1) {
            // parts meet in stage 0: [part][row group][lane] f32x4, one
            // block of each wave at a time
            __syncthreads();
            f32x4_t *red = (f32x4_t *)st0;
            red[(kp * RB + rb) * 64 + lane] = res;
            __syncthreads();
            if (kp == 0) {
#pragma unroll
                for (int q = 1; q < KP; ++q) {
                    const f32x4_t o = red[(q * RB + rb) * 64 + lane];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        res[r] += o[r];
                }
            }
        }
        // Epilogue: lane holds channels 16 blk + 4 g + r of token 16 th + col.
        const int t = 16 * th + col;
        if (kp != 0 || t >= M || t >= MT || 4 * g >= nrows[f])
            continue;
        const int n = 16 * (blk0 + f) + 4 * g;
        if (ks > 1) {
            // this slice's sums (group scales in, per-channel scale not)
            float *pr = P.partial + ((int64_t)slice * M + t) * N + n;
            if ((N & 3) == 0 && 4 * g + 3 < nrows[f]) {
                *reinterpret_cast<float4 *>(pr) = make_float4(res[0], res[1], res[2], res[3]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g + r < nrows[f])
                        pr[r] = res[r];
            }
            continue;
        }
        float post[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            post[r] = 4 * g + r >= nrows[f] ? 0.f
                      : GM == 0             ? 0.5f * f16_bits_to_f32(P.scale[n + r])
                                            : 0.5f;
        uint16_t o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            o[r] = round_out<FP16>(res[r] * post[r]);
        uint16_t *yr = P.y + (int64_t)t * N + n;
        if ((N & 3) == 0 && 4 * g + 3 < nrows[f]) {
            *reinterpret_cast<uint2 *>(yr) = make_uint2((uint32_t)o[0] | (uint32_t)o[1] << 16,
                                                        (uint32_t)o[2] | (uint32_t)o[3] << 16);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r < nrows[f])
                    yr[r] = o[r];
        }
    }
}

// Second half of a K-sliced problem: thread e of a problem takes token
// e / N4 and channels 4 (e % N4) .. + 3 (N4 = ceil(N / 4)), adds the slices'
// sums in slice order, applies 0.5 * s (per channel) or 0.5 (group scales are
// in the sums) and rounds once.
struct FewReduce {
    const float *partial;
    const uint16_t *scale;
    uint16_t *y;
    int M, N, ks;
};
struct FewReduceBatch {
    int count;
    int unit0[kGemvMaxBatch];
    FewReduce p[kGemvMaxBatch];
};
constexpr int kReduceThreads = 256;

template <bool FP16, bool PC>
__global__ void __launch_bounds__(kReduceThreads) few_reduce(const FewReduceBatch batch)
{
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxBatch; ++i)
        pi += (i < batch.count && (int)blockIdx.x >= batch.unit0[i]) ? 1 : 0;
    const FewReduce &R = batch.p[pi];
    const int N4 = (R.N + 3) >> 2;
    const int e = ((int)blockIdx.x - batch.unit0[pi]) * kReduceThreads + (int)threadIdx.x;
    if (e >= R.M * N4)
        return;
    const int t = e / N4, n = 4 * (e - t * N4);
    const int nv = min(4, R.N - n);
    const int64_t slice_stride = (int64_t)R.M * R.N;
    const float *src = R.partial + (int64_t)t * R.N + n;
    uint16_t *yr = R.y + (int64_t)t * R.N + n;
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    if (nv == 4 && (R.N & 3) == 0 && (int64_t)R.ks * slice_stride * 4 < ((int64_t)1 << 31)) {
        // 16-byte aligned, whole, 32-bit offsets: the scales and every slice's partials
        // are loaded before the first add (one memory round trip instead of
        // one per slice), then the sums are taken in slice order
        uint16_t sc[4] = {0, 0, 0, 0};
        if constexpr (PC)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sc[r] = R.scale[n + r];
        // (slices past ks take an offset past the resource: no load issued
        // to memory, no branch between the loads; they are not added)
        const __amdgpu_buffer_rsrc_t pr =
            make_rsrc(R.partial, (uint32_t)((int64_t)R.ks * slice_stride * 4));
        const int off0 = (int)(((int64_t)t * R.N + n) * 4);
        u32x4_t v[kMaxSlices];
#pragma unroll
        for (int s = 0; s < kMaxSlices; ++s)
            v[s] = __builtin_amdgcn_raw_buffer_load_b128(
                pr, s < R.ks ? off0 + (int)(s * slice_stride * 4) : kOOB, 0, 0);
        // (each element is copied to a scalar before the bit cast: this
        // compiler's __builtin_bit_cast of a vector element expression read
        // element 0 whatever the index)
#pragma unroll
        for (int s = 0; s < kMaxSlices; ++s)
            if (s < R.ks)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t u = v[s][r];
                    sum[r] += __builtin_bit_cast(float, u);
                }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            yr[r] = round_out<FP16>(sum[r] * (PC ? 0.5f * f16_bits_to_f32(sc[r]) : 0.5f));
        return;
    }
    for (int s = 0; s < R.ks; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (r < nv)
                sum[r] += src[s * slice_stride + r];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (r < nv)
            yr[r] = round_out<FP16>(sum[r] * (PC ? 0.5f * f16_bits_to_f32(R.scale[n + r]) : 0.5f));
}

template <bool FP16, int GM, int MT, int KP, int CP>
hipError_t launch_inst(unsigned grid, hipStream_t stream, const FewBatch &b)
{
    hipLaunchKernelGGL((few_kernel<FP16, GM, MT, KP, kFN, CP>), dim3(grid), dim3(kThreads), 0,
                       stream, b);
    return hipGetLastError();
}

template <bool FP16, int GM, int MT, int CP>
hipError_t launch_kp(int kp, unsigned grid, hipStream_t stream, const FewBatch &b)
{
    if (kp == 1)
        return launch_inst<FP16, GM, MT, 1, CP>(grid, stream, b);
    if constexpr (MT * 2 <= 32)
        if (kp == 2)
            return launch_inst<FP16, GM, MT, 2, CP>(grid, stream, b);
    if constexpr (MT * 4 <= 32)
        if (kp == 4)
            return launch_inst<FP16, GM, MT, 4, CP>(grid, stream, b);
    return hipErrorInvalidValue;
}

template <bool FP16, int CP>
hipError_t launch_mode(int gm, int mt, int kp, unsigned grid, hipStream_t stream,
                       const FewBatch &b)
{
    switch (gm * 3 + (mt == 32 ? 2 : mt == 16 ? 1 : 0)) {
    case 0: return launch_kp<FP16, 0, 8, CP>(kp, grid, stream, b);
    case 1: return launch_kp<FP16, 0, 16, CP>(kp, grid, stream, b);
    case 2: return launch_kp<FP16, 0, 32, CP>(kp, grid, stream, b);
    case 3: return launch_kp<FP16, 1, 8, CP>(kp, grid, stream, b);
    case 4: return launch_kp<FP16, 1, 16, CP>(kp, grid, stream, b);
    case 5: return launch_kp<FP16, 1, 32, CP>(kp, grid, stream, b);
    case 6: return launch_kp<FP16, 2, 8, CP>(kp, grid, stream, b);
    case 7: return launch_kp<FP16, 2, 16, CP>(kp, grid, stream, b);
    default: return hipErrorInvalidValue;  // groups of 128 take at most 16 tokens
    }
}

// Code-load policy of a launch (kStreamLoad when every problem holds tiled codes).
template <bool FP16>
hipError_t launch_policy(int gm, int mt, int kp, unsigned grid, hipStream_t stream,
                         const FewBatch &b)
{
    bool all_tiled = true;
    for (int i = 0; i < b.count; ++i)
        all_tiled = all_tiled && b.p[i].tiled != 0;
    return all_tiled ? launch_mode<FP16, kStreamLoad>(gm, mt, kp, grid, stream, b)
                     : launch_mode<FP16, 0>(gm, mt, kp, grid, stream, b);
}

}  // namespace

bool gemm_few_takes(int64_t M, int64_t N, int64_t K, int group, const void *scale)
{
    // 32-token tiles take one B column per token: per-channel scales and
    // groups of 256; groups of 128 (two columns per token) stop at 16, and
    // need four slabs per row (a round's scales are one 16-byte load)
    return M >= 1 && M <= (group == 128 ? 16 : kFewMaxM) && N >= 1 &&
           K >= (group == 128 ? 1024 : 256) &&
           K % 256 == 0 && K <= kGemvMaxK &&
           (group == 0 || group == 256 || (group == 128 && ((uintptr_t)scale & 3) == 0));
}

namespace {

// Slab steps a workgroup aims at: long K ranges are sliced over workgroups
// so that the workgroups of one launch run about equally long.  Measured on
// MI355X (fused 7B layer at 9 / 16 / 24 / 32 tokens, µs): 16 steps 25.4 /
// 26.6 / 34.7 / 35.9, 32 steps 22.7 / 23.5 / 28.8 / 30.0, 40 or 48 steps
// 26.0 / 26.7 / 33.0 / 34.0; fewer slices also save partial-sum traffic.
constexpr int kFewSteps = 32;

struct FewPlan {
    int kp, mt, group;
    int ks[kGemvMaxBatch], L[kGemvMaxBatch];
    size_t off[kGemvMaxBatch];  // partial sums of problem i at workspace + off[i]
    size_t ws_bytes;
};

// Tile, K parts and K slices of one launch.  Parts: the fewest (1, 2, 4)
// whose workgroups cover the compute units, within a 16-KB x stage.
// Slices: enough that a workgroup runs about kFewSteps slabs, then doubled
// (while pieces keep 4 slabs) until the workgroups cover the compute units.
hipError_t plan_few(const GemvArgs *args, const int *order, int count, FewPlan &pl)
{
    if (count < 1 || count > kGemvMaxBatch)
        return hipErrorInvalidValue;
    pl.group = -1;
    pl.mt = 0;
    int64_t blocks = 0;
    for (int oi = 0; oi < count; ++oi) {
        const GemvArgs &a = args[order[oi]];
        if (!gemm_few_takes(a.M, a.N, a.K, a.group, a.scale))
            return hipErrorInvalidValue;
        const int t = few_tile(a.M);
        if ((pl.group >= 0 && a.group != pl.group) || (pl.mt && t != pl.mt))
            return hipErrorInvalidValue;
        pl.group = a.group;
        pl.mt = t;
        blocks += (a.N + 15) / 16;
    }
    const int cus = device_cus();
    int kp = 1;
    while (kp < 4 && 2 * kp * pl.mt <= 32 && (blocks * kp + kWaves * kFN - 1) / (kWaves * kFN) < cus)
        kp *= 2;
    pl.kp = kp;
    const int rb = kWaves / kp * kFN;  // blocks per workgroup
    auto units = [&]() {
        int64_t u = 0;
        for (int oi = 0; oi < count; ++oi)
            u += (int64_t)((args[order[oi]].N + 15) / 16 + rb - 1) / rb * pl.ks[oi];
        return u;
    };
    for (int oi = 0; oi < count; ++oi) {
        const int nslabs = args[order[oi]].K / 256;
        pl.ks[oi] = std::min(kMaxSlices, std::max(1, (nslabs + kp * kFewSteps - 1) / (kp * kFewSteps)));
    }
    for (bool grew = true; grew && units() < cus;) {
        grew = false;
        for (int oi = 0; oi < count; ++oi) {
            const int nslabs = args[order[oi]].K / 256;
            if (pl.ks[oi] < kMaxSlices && nslabs >= 8 * kp * pl.ks[oi]) {
                pl.ks[oi] *= 2;
                grew = true;
            }
        }
    }
    pl.ws_bytes = 0;
    for (int oi = 0; oi < count; ++oi) {
        const GemvArgs &a = args[order[oi]];
        const int nslabs = a.K / 256;
        pl.L[oi] = (nslabs + kp * pl.ks[oi] - 1) / (kp * pl.ks[oi]);
        pl.ks[oi] = (nslabs + kp * pl.L[oi] - 1) / (kp * pl.L[oi]);  // no empty slices
        pl.off[oi] = pl.ws_bytes;
        if (pl.ks[oi] > 1)
            pl.ws_bytes += ((size_t)pl.ks[oi] * a.M * a.N * 4 + 255) & ~(size_t)255;
    }
    return hipSuccess;
}

}  // namespace

size_t gemm_few_scratch_need(const GemvArgs *args, const int *order, int count)
{
    FewPlan pl;
    return plan_few(args, order, count, pl) == hipSuccess ? pl.ws_bytes : 0;
}

hipError_t launch_gemm_few(const GemvArgs *args, const int *order, int count, bool fp16,
                           hipStream_t stream, const FixedScratch *fixed)
{
    FewPlan pl;
    hipError_t e = plan_few(args, order, count, pl);
    if (e != hipSuccess)
        return e;
    char *ws = nullptr;
    if (pl.ws_bytes) {
        if (fixed) {
            if (pl.ws_bytes > fixed->bytes)
                return hipErrorInvalidValue;
            ws = static_cast<char *>(fixed->ptr);
        } else {
            void *w = nullptr;
            e = stream_workspace(stream, pl.ws_bytes, &w);
            if (e != hipSuccess)
                return e;
            ws = static_cast<char *>(w);
        }
    }
    FewBatch b = {};
    FewReduceBatch rb = {};
    int units = 0, runits = 0;
    const int rbk = kWaves / pl.kp * kFN;  // blocks per workgroup
    for (int oi = 0; oi < count; ++oi) {
        const GemvArgs &a = args[order[oi]];
        FewProblem &p = b.p[b.count];
        p.x = a.x;
        p.packed = a.packed;
        p.scale = a.scale;
        p.y = a.y;
        p.M = a.M;
        p.N = a.N;
        p.K = a.K;
        p.tiled = a.tiled;
        p.L = pl.L[oi];
        p.ks = pl.ks[oi];
        p.partial = p.ks > 1 ? reinterpret_cast<float *>(ws + pl.off[oi]) : nullptr;
        b.unit0[b.count] = units;
        units += ((a.N + 15) / 16 + rbk - 1) / rbk * p.ks;
        ++b.count;
        if (p.ks > 1) {
            FewReduce &r = rb.p[rb.count];
            r.partial = p.partial;
            r.scale = a.scale;
            r.y = a.y;
            r.M = a.M;
            r.N = a.N;
            r.ks = p.ks;
            rb.unit0[rb.count] = runits;
            runits += (a.M * ((a.N + 3) / 4) + kReduceThreads - 1) / kReduceThreads;
            ++rb.count;
        }
    }
    if (units == 0)
        return hipSuccess;
    const int gm = pl.group == 0 ? 0 : (pl.group == 256 ? 1 : 2);
    e = fp16 ? launch_policy<true>(gm, pl.mt, pl.kp, (unsigned)units, stream, b)
             : launch_policy<false>(gm, pl.mt, pl.kp, (unsigned)units, stream, b);
    if (e != hipSuccess || runits == 0)
        return e;
    const bool pc = pl.group == 0;
    if (fp16) {
        if (pc)
            hipLaunchKernelGGL((few_reduce<true, true>), dim3(runits), dim3(kReduceThreads), 0, stream, rb);
        else
            hipLaunchKernelGGL((few_reduce<true, false>), dim3(runits), dim3(kReduceThreads), 0, stream, rb);
    } else {
        if (pc)
            hipLaunchKernelGGL((few_reduce<false, true>), dim3(runits), dim3(kReduceThreads), 0, stream, rb);
        else
            hipLaunchKernelGGL((few_reduce<false, false>), dim3(runits), dim3(kReduceThreads), 0, stream, rb);
    }
    return hipGetLastError();
}

}  // namespace ternary
