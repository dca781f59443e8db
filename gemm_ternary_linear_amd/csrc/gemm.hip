// Prefill GEMM (M > 8) for the ternary linear layer on gfx950.
//
// At large M the layer y = x @ (unpack(q) * s)^T ([xxqk] m.xxqk.cn/news/593501
// §4.3) is a dense contraction and compute-bound ([nxbn] m.nxbn.cn/news/169761
// §4.1: prefill is dominated by compute), so it runs on the matrix cores.
// The packed tile is expanded once per workgroup into LDS as 16-bit +-2 / 0
// (never to HBM: no dense weight copy exists outside LDS), and both operands
// feed v_mfma_f32_16x16x32_{bf16,f16} with fp32 accumulation.  Scales follow
// [trdm] trdm.cn "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1/§4.2
// (group of 128 K, multiplied at the group boundary; groups of 64 in [xxqk]
// §4.2, of 32 and 256 in the yangyitao.com vLLM book, chapter 13, §13.3.3)
// and [nxbn] §3.2/§4.2 (per output channel, multiplied in the epilogue).
//
// Tiling: 128 tokens x 128 channels x 64 K per workgroup step, 256 threads as
// 2x2 waves of 64x64 (4x4 MFMA tiles each).  Two LDS buffers per operand: the
// global loads of step k+1 are in flight while step k runs on the matrix cores.
// Rows are padded to 72 elements (144 bytes) so the 16 rows a fragment read
// touches fall on distinct LDS banks.
#include <algorithm>
#include <cstdint>
#include <type_traits>

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

// glog: log2 of the group size (group-scaled instances, groups of 32 K or
// more: every 32-K MFMA step lies inside one group).
template <bool FP16, bool GROUPED>
__global__ void __launch_bounds__(THREADS)
    gemm_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed,
                const uint16_t *__restrict__ scale, uint16_t *__restrict__ y, int M, int N, int K,
                int glog)
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
    const int ngroups = K >> glog;

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
            if constexpr (GROUPED) {
                const int kend = kt * BK + kk + 32;  // K covered so far
                if ((kend & ((1 << glog) - 1)) == 0) {
                    // end of a group: fold its sums with the group's scales
                    const int grp = (kend >> glog) - 1;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int n = n0 + wn * 64 + j * 16 + frow;
                        const float sc =
                            n < N ? f16_bits_to_f32(scale[(int64_t)n * ngroups + grp]) : 0.f;
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


// ---------------------------------------------------------------------------
// Pipelined kernel for per-channel scales.  x and the packed weights reach LDS
// by buffer-to-LDS DMA (no register staging), NS stages deep, so the loads of
// K step kt+NS-1 are in flight while step kt runs on the matrix cores.  Each
// wave reads its packed codes (one dword = 16 codes per lane and fragment)
// from LDS and expands them in registers straight into MFMA A operands: the
// decoded weights never pass through LDS.
//
// K order inside one 64-wide step: lane group g (lanes 16g..16g+15) of an
// MFMA operand holds k = 16g + 8*kk + (0..7) for the two 32-deep MFMAs kk of
// the step, which is exactly what the packed dword g of a row decodes to;
// the x fragment reads use the same order, so the contraction is unchanged.
//
// x stage layout: token row r of the stage is 128 bytes = 8 chunks of 8
// elements; logical chunk c sits in physical chunk c ^ f(r) with
// f(r) = (r & 7) ^ ((r >> 3) & 1), which spreads the 16 rows a fragment read
// touches over all LDS banks.  The DMA gathers each chunk from the global
// address that belongs to its physical slot.
namespace dma {

constexpr int TK = 64;
constexpr int kOOB = 0x40000000;  // buffer offset past every record: reads as 0

template <int TN_, int TM_, int WGN_, int WGM_, int NS_, int OCC_>
struct Cfg {
    static constexpr int TN = TN_, TM = TM_, WGN = WGN_, WGM = WGM_, NS = NS_, OCC = OCC_;
    static constexpr int THREADS = WGN * WGM * 64;
    static constexpr int FN = TN / WGN / 16;  // 16-channel fragments per wave
    static constexpr int FM = TM / WGM / 16;  // 16-token fragments per wave
    static constexpr int XI = TM * 8 / THREADS;  // 16-byte x DMAs per thread and stage
    static constexpr int WI = TN * 4 / THREADS;  // 4-byte packed DMAs per thread and stage
    static constexpr int VPS = XI + WI;          // vector memory ops per thread and stage
    static constexpr int XSTAGE = TM * 8;        // 16-byte chunks per x stage
    static constexpr int WSTAGE = TN * 4;        // dwords per packed stage
    static_assert(TM * 8 % THREADS == 0 && TN * 4 % THREADS == 0, "stage split");
    static_assert(FN >= 1 && FM >= 1 && NS >= 2 && NS <= 8, "tile");
    static_assert((NS - 2) * VPS <= 63, "vmcnt range");
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u4;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ __forceinline__ int xswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// One buffer-to-LDS DMA: every lane reads BYTES from rsrc at voff + soff and
// the wave writes them to LDS at lds + lane * BYTES.  The builtin exists for
// the device target only; the host pass (which emits just the launch stub)
// sees an empty body.
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t rsrc, void *lds, int voff, int soff)
{
    static_assert(BYTES == 4 || BYTES == 16, "DMA size");
#if defined(__HIP_DEVICE_COMPILE__)
    auto *l = (__attribute__((address_space(3))) void *)lds;
    if constexpr (BYTES == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, l, 16, voff, soff, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, l, 4, voff, soff, 0, 0);
#endif
}

// s_waitcnt with only the vector-memory count limited (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their
// maxima).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N <= 63, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most N of this wave's DMAs are outstanding, then meet the
// other waves at a barrier; afterwards every wave's older DMAs have landed.
// The scheduling fences keep the wait from being hoisted into the compute
// before it, and the memory clobber keeps LDS accesses on their side.
template <int N>
__device__ __forceinline__ void wait_and_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<N>();
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// One problem of a launch: y = x * (q (.) s)^T, K range split into ksplit
// slices whose fp32 partial tiles go to `partial` when ksplit > 1.
struct BigProblem {
    const uint16_t *x;
    const uint8_t *packed;
    const uint16_t *scale;
    uint16_t *y;
    float4 *partial;
    int M, N, K, ksplit;
    int tiled;  // codes in the tiled layout (else row-major [N, K/4])
};

// The problems of one launch; workgroups wg0[i] .. wg0[i+1]-1 belong to
// problem i (wg0 ascending, wg0[0] == 0).
struct BigBatch {
    int count;
    int wg0[kGemvMaxBatch];
    BigProblem p[kGemvMaxBatch];
};

// GS: 0 for per-channel scales, else the group size (64, 128 or 256 K: one,
// two or four K steps).  ZS: skip zero blocks ([trdm] trdm.cn
// "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §6: ternary weights often
// come with block sparsity, and a kernel can skip all-zero blocks): a wave
// whose channels (16 FN) x 64 K of a step are all code 00 or 11 skips the
// step's decode and MFMAs (their products are zeros; the sums are the same
// bits).
template <bool FP16, int GS, class C, bool ZS = false>
__global__ void __launch_bounds__(C::THREADS, C::OCC) gemm_dma_kernel(const BigBatch batch)
{
    constexpr int NS = C::NS, FN = C::FN, FM = C::FM, THREADS = C::THREADS;
    constexpr bool GROUPED = GS != 0;
    constexpr int SPG = GROUPED ? GS / TK : 1;  // K steps per group
    constexpr int GSH = SPG == 1 ? 0 : (SPG == 2 ? 1 : 2);
    // Group scales: a channel's dword holds the scales of a pair of groups
    // (2 SPG K steps).  The workgroup gathers it once per LS steps (the
    // pair's steps, at most one round of NS) into one of NB buffers of the
    // round's parity, the buffer of the step's position in the round; the
    // stages in between issue, in its place, a DMA that reads past the
    // resource (no memory access) into a buffer that is never read, so every
    // stage still issues the same number of DMAs.  Rounds alternate between
    // the two parities, so a gather into the next round's buffer never
    // overwrites scales that the current round still reads.
    static_assert(!GROUPED || (C::TN == THREADS && NS % 4 == 0 && (GS == 64 || GS == 128 ||
                                                                   GS == 256)),
                  "one scale dword per thread; groups of 1, 2 or 4 steps");
    constexpr int VPS = C::VPS + (GROUPED ? 1 : 0);  // vector memory ops per thread and stage
    constexpr int LS = !GROUPED ? NS : (2 * SPG < NS ? 2 * SPG : NS);  // steps per scale gather
    constexpr int NB = NS / LS;  // scale buffers per round parity
    static_assert(NS % LS == 0 && NB <= 4, "scale gathers per round");
    // One LDS object per stage: the compiler then knows that a DMA into one
    // stage does not write the stage being read and waits for nothing there.
    constexpr int XS = C::XSTAGE, WS = C::WSTAGE, SS = GROUPED ? C::TN : 1;
#define TERNARY_STAGES(T, name, n)                                                               \
    __shared__ __attribute__((aligned(16))) T name##0[n], name##1[n], name##2[NS > 2 ? n : 1],  \
        name##3[NS > 3 ? n : 1], name##4[NS > 4 ? n : 1], name##5[NS > 5 ? n : 1],            \
        name##6[NS > 6 ? n : 1], name##7[NS > 7 ? n : 1]
    TERNARY_STAGES(uint4, sx, XS);
    TERNARY_STAGES(uint32_t, sw, WS);
#undef TERNARY_STAGES
    __shared__ __attribute__((aligned(16))) uint32_t sc00[SS], sc01[NB > 1 ? SS : 1],
        sc02[NB > 2 ? SS : 1], sc03[NB > 3 ? SS : 1], sc10[SS], sc11[NB > 1 ? SS : 1],
        sc12[NB > 2 ? SS : 1], sc13[NB > 3 ? SS : 1], scx[SS];
    lds_u4 *const lx[8] = {(lds_u4 *)sx0, (lds_u4 *)sx1, (lds_u4 *)sx2, (lds_u4 *)sx3,
                           (lds_u4 *)sx4, (lds_u4 *)sx5, (lds_u4 *)sx6, (lds_u4 *)sx7};
    lds_u32 *const lw[8] = {(lds_u32 *)sw0, (lds_u32 *)sw1, (lds_u32 *)sw2, (lds_u32 *)sw3,
                            (lds_u32 *)sw4, (lds_u32 *)sw5, (lds_u32 *)sw6, (lds_u32 *)sw7};
    lds_u32 *const lsc[2][4] = {
        {(lds_u32 *)sc00, (lds_u32 *)sc01, (lds_u32 *)sc02, (lds_u32 *)sc03},
        {(lds_u32 *)sc10, (lds_u32 *)sc11, (lds_u32 *)sc12, (lds_u32 *)sc13}};
    lds_u32 *const lscx = (lds_u32 *)scx;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave % C::WGN;
    const int wm = wave / C::WGN;

    // This workgroup's problem: one round of scalar loads and compares.
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxBatch; ++i)
        pi += (i < batch.count && (int)blockIdx.x >= batch.wg0[i]) ? 1 : 0;
    const BigProblem &P = batch.p[pi];
    const uint16_t *__restrict__ x = P.x;
    const uint8_t *__restrict__ packed = P.packed;
    const uint16_t *__restrict__ scale = P.scale;
    uint16_t *__restrict__ y = P.y;
    float4 *__restrict__ partial = P.partial;
    const int M = P.M, N = P.N, K = P.K, ksplit = P.ksplit;

    // Tile order: workgroup b runs on XCD b % 8.  Without a K split, when the
    // token tiles split evenly over the 8 XCDs, XCD k owns token tiles k,
    // k+8, ... (their x stays in its L2) and walks the channel tiles, running
    // all its token tiles of one channel tile back to back so that each
    // weight tile is read once per XCD.  With a K split of `ksplit` slices,
    // the slices of one tile go to one XCD when the tiles split evenly over
    // the XCDs.
    const int ntn = (N + C::TN - 1) / C::TN, ntm = (M + C::TM - 1) / C::TM;
    int tn, tm, tile = 0, slice = 0;
    const int bid = (int)blockIdx.x - batch.wg0[pi];
    if (ksplit == 1) {
        if (ntm % 8 == 0) {
            const int xcd = bid & 7, slot = bid >> 3, own = ntm >> 3;
            tm = xcd + 8 * (slot % own);
            tn = slot / own;
        } else {
            tm = bid / ntn;
            tn = bid % ntn;
        }
    } else {
        if ((ntn * ntm) % 8 == 0) {
            const int xcd = bid & 7, slot = bid >> 3;
            tile = xcd + 8 * (slot / ksplit);
            slice = slot % ksplit;
        } else {
            tile = bid / ksplit;
            slice = bid % ksplit;
        }
        tm = tile / ntn;
        tn = tile % ntn;
    }
    const int n0 = tn * C::TN;
    const int m0 = tm * C::TM;
    // This slice's K steps: rounds [r0, r1) of NS steps (slices differ by at
    // most one round).
    const int rounds = K / (TK * NS);
    const int r0 = (int)((int64_t)slice * rounds / ksplit);
    const int r1 = (int)((int64_t)(slice + 1) * rounds / ksplit);
    const int nk = (r1 - r0) * NS;
    const int kbase = r0 * NS;

    // DMA sources.  x DMA i of this thread fills physical chunk p = i*THREADS
    // + tid of the stage (lanes of a wave write consecutive chunks).
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x), (short)0, (int)((uint32_t)M * (uint32_t)K * 2u), 0x00020000);
    // Codes: a K step is 16 bytes of each row.  Row-major, row n's 16 bytes of
    // step kc sit at n * K/4 + 16 kc; tiled (K % 256 == 0 here), the 16 rows
    // of a block have their 16 bytes of step kc together, 256 contiguous
    // bytes at block * (K/256) KB + 256 kc (row n % 16 at 16 (n % 16)).
    const bool tiled = P.tiled != 0;
    const int nblk = (N + 15) >> 4;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(packed), (short)0,
        tiled ? (int)((uint32_t)nblk * 16u * (uint32_t)(K >> 2))
              : (int)((uint32_t)N * (uint32_t)(K >> 2)),
        0x00020000);
    const int wstep = tiled ? 256 : TK / 4;  // bytes between K steps of one row
    int xoff[C::XI], woff[C::WI];
#pragma unroll
    for (int i = 0; i < C::XI; ++i) {
        const int p = i * THREADS + tid;
        const int r = p >> 3, c = (p & 7) ^ xswz(p >> 3);
        xoff[i] = m0 + r < M ? ((m0 + r) * K + 8 * c) * 2 : kOOB;
    }
#pragma unroll
    for (int i = 0; i < C::WI; ++i) {
        const int d = i * THREADS + tid;
        const int row = d >> 2, n = n0 + row;
        woff[i] = n >= N ? kOOB
                  : tiled ? (n >> 4) * (K >> 8) * 1024 + (n & 15) * 16 + 4 * (d & 3)
                          : n * (K >> 2) + 4 * (d & 3);
    }
    // Scales: thread t loads channel n0 + t's pair of groups.
    const int ngroups = K / (GROUPED ? GS : 1);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(scale), (short)0,
        GROUPED ? (int)((uint32_t)N * (uint32_t)ngroups * 2u) : 0, 0x00020000);
    const int soff = GROUPED && n0 + tid < N ? (n0 + tid) * ngroups * 2 : kOOB;
    // Wave-uniform LDS destinations of this wave's DMAs (kept in SGPRs).
    const int wave_chunk = __builtin_amdgcn_readfirstlane(wave) * 64;

    // Every step issues the same number of DMAs, so that one vmcnt value
    // is right everywhere: steps past the end reload the last K step into a
    // stage that is never read again.  P: the parity of step kt's round.
    auto issue = [&](auto S, auto P, int kt) {
        constexpr int s = decltype(S)::value, p = decltype(P)::value;
        const int kc = kbase + (kt < nk ? kt : nk - 1);
#pragma unroll
        for (int i = 0; i < C::XI; ++i)
            dma_to_lds<16>(xr, (void *)(lx[s] + i * THREADS + wave_chunk), xoff[i], kc * (TK * 2));
#pragma unroll
        for (int i = 0; i < C::WI; ++i)
            dma_to_lds<4>(wr, (void *)(lw[s] + i * THREADS + wave_chunk), woff[i], kc * wstep);
        if constexpr (GROUPED) {
            if constexpr (s % LS == 0)  // the dword holding group kc / SPG
                dma_to_lds<4>(sr, (void *)(lsc[p][s / LS] + wave_chunk), soff,
                              ((kc >> GSH) >> 1) * 4);
            else
                dma_to_lds<4>(sr, (void *)(lscx + wave_chunk), kOOB, 0);
        }
    };

    f32x4_t acc[FN][FM];
    f32x4_t part[GROUPED ? FN : 1][GROUPED ? FM : 1];  // the current group's sums
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

    // Per-lane LDS read offsets.  x: token row (lane & 15) of each fragment,
    // logical chunk 2g + kk; packed: dword g of channel row (lane & 15).
    const int g = lane >> 4;
    const int fr = lane & 15;
    const int xrow0 = wm * FM * 16 + fr;
    const int xa0 = xrow0 * 8 + ((2 * g) ^ xswz(fr));  // kk = 0; kk = 1 flips bit 0
    const int xa1 = xa0 ^ 1;
    const int wa = (wn * FN * 16 + fr) * 4 + g;

    auto compute = [&](auto S, auto P, int kt) {
        constexpr int s = decltype(S)::value, p = decltype(P)::value;
        uint32_t wv[FN];
#pragma unroll
        for (int f = 0; f < FN; ++f)
            wv[f] = lw[s][wa + f * 64];
        bool skip = false;
        if constexpr (ZS) {
            // one decision per wave and step: codes 00 and 11 both decode to zero
            uint32_t nz = 0;
#pragma unroll
            for (int f = 0; f < FN; ++f)
                nz |= (wv[f] ^ (wv[f] >> 1)) & 0x55555555u;
            skip = __builtin_amdgcn_ballot_w64(nz != 0) == 0;
            if constexpr (GROUPED)
                if (skip && s % SPG == 0)
#pragma unroll
                    for (int f = 0; f < FN; ++f)
#pragma unroll
                        for (int j = 0; j < FM; ++j)
                            part[f][j] = zero4;
        }
#pragma unroll
        for (int kk = 0; kk < (skip ? 0 : 2); ++kk) {
            uint4 xf[FM];
#pragma unroll
            for (int j = 0; j < FM; ++j)
                xf[j] = __builtin_bit_cast(uint4, lx[s][(kk ? xa1 : xa0) + j * 128]);
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                uint32_t d[8];
                decode16(wv[f], d);
                const uint4 a = kk ? make_uint4(d[4], d[5], d[6], d[7])
                                   : make_uint4(d[0], d[1], d[2], d[3]);
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    if constexpr (GROUPED)  // steps kt = s mod NS (slices are whole rounds)
                        part[f][j] =
                            mfma<FP16>(a, xf[j], (s % SPG == 0 && kk == 0) ? zero4 : part[f][j]);
                    else
                        acc[f][j] = mfma<FP16>(a, xf[j], acc[f][j]);
                }
            }
        }
        if constexpr (GROUPED) {
            if constexpr (s % SPG == SPG - 1) {
                // End of a group: fold its sums with the group's scales (low
                // half of the pair's dwords for an even group, high half for
                // an odd one; known from s alone when NS spans two groups).
                int odd;
                if constexpr (NS % (2 * SPG) == 0)
                    odd = (s >> GSH) & 1;
                else
                    odd = ((kbase + kt) >> GSH) & 1;
#pragma unroll
                for (int f = 0; f < FN; ++f) {
                    const u32x4_t w = *reinterpret_cast<const lds_u4 *>(
                        lsc[p][s / LS] + wn * FN * 16 + f * 16 + 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float sc = f16_bits_to_f32((uint16_t)(odd ? w[r] >> 16 : w[r]));
#pragma unroll
                        for (int j = 0; j < FM; ++j)
                            acc[f][j][r] += sc * part[f][j][r];
                    }
                }
            }
        }
    };

    // One K step: wait for this wave's DMA of stage kt, barrier (all waves'
    // DMA of stage kt landed, all waves done with stage kt-1), start the DMA
    // of step kt+NS-1 into the stage kt-1 used (the next round's, of the
    // other parity, unless kt opens its round), then compute stage kt.
    auto step = [&](auto S, auto P, int kt) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value, p = decltype(P)::value;
        wait_and_barrier<(NS - 2) * VPS>();
        issue(std::integral_constant<int, (s + NS - 1) % NS>{},
              std::integral_constant<int, s == 0 ? p : 1 - p>{}, kt + NS - 1);
        compute(S, P, kt);
    };
    auto round = [&](auto P, int kt) __attribute__((always_inline)) {
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (step(std::integral_constant<int, I>{}, P, kt + I), ...);
        }(std::make_integer_sequence<int, NS>{});
    };
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;

    // Prologue: stages 0 .. NS-2 of round 0.
    [&]<int... I>(std::integer_sequence<int, I...>) {
        (issue(std::integral_constant<int, I>{}, Even{}, I), ...);
    }(std::make_integer_sequence<int, NS - 1>{});

    // K is a whole number of NS-step rounds (the host checks), so every
    // stage index below is a constant; group-scaled kernels run rounds in
    // pairs so that the parity is one too.
    if constexpr (GROUPED) {
        int kt = 0;
        for (; kt + 2 * NS <= nk; kt += 2 * NS) {
            round(Even{}, kt);
            round(Odd{}, kt + NS);
        }
        if (kt < nk)
            round(Even{}, kt);
    } else {
        for (int kt = 0; kt < nk; kt += NS)
            round(Even{}, kt);
    }
    // No DMA may still be writing LDS when the workgroup ends.
    wait_vm<0>();

    if (ksplit > 1) {
        // Split K: store this slice's fp32 partial tile, fragment by fragment
        // (lane-contiguous float4s); gemm_split_reduce adds the slices.
        float4 *mine = partial + ((int64_t)tile * ksplit + slice) * (C::TN * C::TM / 4);
        const int lo = wave * FN * FM * 64 + lane;
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int j = 0; j < FM; ++j)
                mine[lo + (f * FM + j) * 64] = __builtin_bit_cast(float4, acc[f][j]);
        return;
    }

    // Epilogue: C tile (f, j) element r of this lane is channel
    // n0 + (wn*FN + f)*16 + 4*g + r of token m0 + (wm*FM + j)*16 + fr.
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
        const int n = n0 + (wn * FN + f) * 16 + 4 * g;
        float post[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)  // weights are +-2; group scales are already in
            post[r] = n + r >= N ? 0.f : GROUPED ? 0.5f : 0.5f * f16_bits_to_f32(scale[n + r]);
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int m = m0 + (wm * FM + j) * 16 + fr;
            if (m >= M)
                continue;
            uint16_t *yr = y + (int64_t)m * N;
            if (vec && n + 3 < N) {
                const uint32_t lo = (uint32_t)round_out<FP16>(acc[f][j][0] * post[0]) |
                                    (uint32_t)round_out<FP16>(acc[f][j][1] * post[1]) << 16;
                const uint32_t hi = (uint32_t)round_out<FP16>(acc[f][j][2] * post[2]) |
                                    (uint32_t)round_out<FP16>(acc[f][j][3] * post[3]) << 16;
                *reinterpret_cast<uint2 *>(yr + n) = make_uint2(lo, hi);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N)
                        yr[n + r] = round_out<FP16>(acc[f][j][r] * post[r]);
            }
        }
    }
}

// Second half of a split-K product: thread t of the grid takes float4 t of
// the partial tiles (the layout gemm_dma_kernel stores), adds the `ksplit`
// slices in slice order, applies the per-channel scale (group scales are
// already in the partials) and writes four outputs of one token.
template <bool FP16, bool GROUPED, class C>
__global__ void __launch_bounds__(256)
    gemm_split_reduce(const float4 *__restrict__ partial, const uint16_t *__restrict__ scale,
                      uint16_t *__restrict__ y, int M, int N, int ksplit)
{
    constexpr int FN = C::FN, FM = C::FM, TILE4 = C::TN * C::TM / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int ntn = (N + C::TN - 1) / C::TN, ntm = (M + C::TM - 1) / C::TM;
    if (idx >= (int64_t)ntn * ntm * TILE4)
        return;
    const int tile = (int)(idx / TILE4), e = (int)(idx % TILE4);
    const int lane = e & 63, t = e >> 6;
    const int j = t % FM, f = (t / FM) % FN, wave = t / (FM * FN);
    const int n = (tile % ntn) * C::TN + ((wave % C::WGN) * FN + f) * 16 + 4 * (lane >> 4);
    const int m = (tile / ntn) * C::TM + ((wave / C::WGN) * FM + j) * 16 + (lane & 15);
    if (m >= M || n >= N)
        return;
    // Slices in batches of kBatch loads issued together (one memory round
    // trip per batch, not per slice); slices past ksplit take an offset past
    // the resource (no memory access) and are not added.  The partial tiles
    // of one launch hold at most 2 GiB, so byte offsets fit in 32 bits.
    constexpr int kBatch = 8;
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float4 *>(partial), (short)0,
        (int)((int64_t)ntn * ntm * ksplit * TILE4 * 16), 0x00020000);
    const int64_t first = (int64_t)tile * ksplit * TILE4 + e;  // float4 index of slice 0
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < ksplit; q0 += kBatch) {
        u32x4_t w[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            w[b] = __builtin_amdgcn_raw_buffer_load_b128(
                pr, q0 + b < ksplit ? (int)((first + (int64_t)(q0 + b) * TILE4) * 16) : kOOB, 0,
                0);
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            if (q0 + b < ksplit)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // (element copied to a scalar before the bit cast: this
                    // compiler's bit cast of a vector element expression read
                    // element 0 whatever the index)
                    const uint32_t u = w[b][r];
                    const float x = __builtin_bit_cast(float, u);
                    a[r] = q0 + b == 0 ? x : a[r] + x;  // slice 0 as is, then in order
                }
    }
    uint16_t *yr = y + (int64_t)m * N;
    if ((N & 3) == 0 && n + 3 < N) {
        uint32_t o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            o[r] = round_out<FP16>(a[r] * (GROUPED ? 0.5f : 0.5f * f16_bits_to_f32(scale[n + r])));
        *reinterpret_cast<uint2 *>(yr + n) = make_uint2(o[0] | o[1] << 16, o[2] | o[3] << 16);
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (n + r < N)
                yr[n + r] = round_out<FP16>(a[r] * (GROUPED ? 0.5f : 0.5f * f16_bits_to_f32(scale[n + r])));
    }
}

}  // namespace dma

template <bool FP16, bool GROUPED>
hipError_t launch_gemm_t(const uint16_t *x, int M, int N, int K, const uint8_t *packed,
                         const uint16_t *scale, int glog, uint16_t *y, hipStream_t stream)
{
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_kernel<FP16, GROUPED>), grid, dim3(THREADS), 0, stream, x, packed,
                       scale, y, M, N, K, glog);
    return hipGetLastError();
}

}  // namespace

// Tile shape, wave grid, stage count and waves per SIMD of the pipelined
// kernel: per-channel problems run two workgroups per CU; group-scaled ones
// keep a second set of accumulators (the current group's sums) and run one.
typedef dma::Cfg<256, 128, 4, 1, 4, 2> BigCfg;  // per-channel, M > 64
// Few tokens: the MFMAs are not the limit, the weight stream is, so the
// tiles take fewer tokens and (M <= 32) the pipeline runs 8 stages deep to
// keep more weight bytes in flight per CU, in two-wave workgroups of 128
// channels: twice the tiles of 256 channels, which spreads shapes of few
// channel tiles over more CUs (a 25600 x 5120 problem at M = 16: 33 against
// 40 us); up to 16 tokens the tile takes 16 (30 us).  Group-scaled problems,
// which keep a second set of accumulators, use these at every M so that they
// still run two workgroups per CU.
typedef dma::Cfg<256, 64, 4, 1, 4, 2> MidCfg;   // 32 < M <= 64 (or K % 512 != 0)
typedef dma::Cfg<128, 32, 2, 1, 8, 2> SmallCfg; // 16 < M <= 32, K % 512 == 0
typedef dma::Cfg<128, 16, 2, 1, 8, 2> TinyCfg;  // M <= 16, K % 512 == 0

// Which configuration a problem runs with: 0 tiny, 1 small, 2 mid, 3 large.
int big_cfg_of(int M, int K, int group)
{
    static_assert(TinyCfg::NS == SmallCfg::NS, "one K condition for both");
    const bool grouped = group != 0;
    if (M <= 32 && K % (dma::TK * SmallCfg::NS) == 0)
        return M <= 16 ? 0 : 1;
    return M <= 64 || grouped ? 2 : 3;
}

// The pipelined kernel takes problems whose K is a whole number of 4-step
// rounds (256), whose buffer offsets stay below the out-of-range marker, and
// (group scales) groups of 64, 128 or 256 K whose scale array is 4-byte
// aligned with an even number of groups per row: it loads a channel's scales
// of two consecutive groups as one dword.
bool gemm_big_takes(int M, int N, int K, int group, const void *scale, bool tiled)
{
    if (M < 1 || N < 1 || K % (dma::TK * BigCfg::NS) != 0 || (int64_t)M * K * 2 >= dma::kOOB ||
        (tiled ? tiled_bytes(N, K) : (int64_t)N * (K / 4)) >= dma::kOOB)
        return false;
    if (group == 0)
        return true;
    return (group == 64 || group == 128 || group == 256) && (K / group) % 2 == 0 &&
           ((uintptr_t)scale & 3) == 0 && (int64_t)N * (K / group) * 2 < dma::kOOB;
}

// Compute units of the current device (cached per device).
int device_cus()
{
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// K slices of the pipelined kernel (whole rounds of NS steps each, at most
// one round apart): enough that tiles x slices cover the compute units once,
// keeping at least two rounds per slice, within a 2 GiB workspace.  When the
// tiles alone fill at most a quarter of the units and twice the slices would
// still hold three rounds each, they cover the units twice (more workgroups
// in flight).  Measured on MI355X: the 5120 x 25600 projection (group 128,
// 40 or 20 tiles, 3.8 rounds per doubled slice) at M = 16 / 32 / 64 takes
// 35 / 40 / 51 against 43 / 48 / 53 us; the 4096 x 18944 one (per channel,
// 2.3 rounds per doubled slice) slowed from 19 / 22 / 23 to 21 / 24 / 31 us
// and the 25600 x 5120 one at M = 64 (100 tiles) from 43 to 44.5 us, on the
// extra partial-tile traffic.
int big_ksplit(int tiles, int K, int ns, int tile_elems)
{
    const int rounds = K / (dma::TK * ns), cus = device_cus();
    if ((int64_t)tiles >= cus)
        return 1;
    int ks = (cus + tiles - 1) / tiles;
    const int ks2 = (2 * cus + tiles - 1) / tiles;
    if (4 * tiles <= cus && rounds >= 3 * ks2)
        ks = ks2;
    ks = std::min(ks, rounds / 2);
    while (ks > 1 && (int64_t)tiles * ks * tile_elems * 4 > (int64_t(1) << 31))
        --ks;
    return std::max(ks, 1);
}

// The plan of one grouped launch: problem order (longest K first, so that the
// longest tiles start first), tiles and K slices per problem, and the bytes
// of fp32 partial tiles the split problems need.  When all the tiles together
// do not cover the compute units, each problem's K range is split as
// big_ksplit() says.
template <class C>
size_t plan_big_mode(const GemvArgs *args, const int *idx, int count, int *order, int *tiles,
                     int *ks, size_t cap = SIZE_MAX)
{
    int64_t total = 0;
    for (int i = 0; i < count; ++i) {
        order[i] = i;
        const GemvArgs &a = args[idx[i]];
        tiles[i] = ((a.N + C::TN - 1) / C::TN) * ((a.M + C::TM - 1) / C::TM);
        total += tiles[i];
    }
    for (int i = 1; i < count; ++i)  // stable insertion sort, K descending
        for (int j = i; j > 0 && args[idx[order[j]]].K > args[idx[order[j - 1]]].K; --j) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    // Tiles that cover the compute units but differ in length (a long-K
    // problem among short ones): a problem whose tiles run at least twice a
    // workgroup slot's fair share of the launch (the sum of tiles x K over
    // the compute units x workgroups per unit) is split into slices of about
    // that share, whole rounds of NS steps, at least two per slice.  Measured
    // on MI355X: the 7B-shaped layer at M = 32, whose 32 down tiles (K =
    // 18944) ran 4.6 times as long as the other 368, from 102 us unsplit.
    int64_t work = 0;
    for (int i = 0; i < count; ++i)
        work += (int64_t)tiles[i] * args[idx[i]].K;
    const int64_t share = std::max<int64_t>(1, work / ((int64_t)device_cus() * C::OCC));
    // The balanced slices are a speed-up, not a need: when their partial
    // tiles would not fit in `cap` (the fixed scratch of the allocation-free
    // call), the launch runs without them.
    bool balance = true;
    size_t ws_bytes;
again:
    ws_bytes = 0;
    for (int i = 0; i < count; ++i) {
        const int K = args[idx[i]].K;
        if (total < device_cus()) {
            ks[i] = big_ksplit(tiles[i], K, C::NS, C::TN * C::TM);
        } else if (balance && count > 1 && K >= 2 * share) {
            const int rounds = K / (dma::TK * C::NS);
            ks[i] = (int)std::min<int64_t>((K + share - 1) / share, rounds / 2);
            while (ks[i] > 1 && (int64_t)tiles[i] * ks[i] * C::TN * C::TM * 4 > (int64_t(1) << 31))
                --ks[i];
            ks[i] = std::max(ks[i], 1);
        } else {
            ks[i] = 1;
        }
        if (ks[i] > 1)
            ws_bytes += (size_t)tiles[i] * ks[i] * C::TN * C::TM * 4;
    }
    if (balance && total >= device_cus() && ws_bytes > cap) {
        balance = false;
        goto again;
    }
    return ws_bytes;
}

// Launches the problems args[idx[0..count)) (all gemm_big_takes(), one scale
// mode) as one grouped launch of the pipelined kernel, plus one reduce launch
// per problem whose K range is split.  The fp32 partials of split problems go
// to `fixed` when given (the caller checked its size), else to the stream's
// workspace.
template <bool FP16, int GS, class C, bool ZS>
hipError_t launch_big_mode(const GemvArgs *args, const int *idx, int count, hipStream_t stream,
                           const FixedScratch *fixed)
{
    int order[kGemvMaxBatch], tiles[kGemvMaxBatch], ks[kGemvMaxBatch];
    const size_t ws_bytes =
        plan_big_mode<C>(args, idx, count, order, tiles, ks, fixed ? fixed->bytes : SIZE_MAX);
    char *ws = nullptr;
    if (ws_bytes) {
        if (fixed) {
            if (ws_bytes > fixed->bytes)
                return hipErrorInvalidValue;
            ws = static_cast<char *>(fixed->ptr);
        } else {
            void *w = nullptr;
            const hipError_t e = stream_workspace(stream, ws_bytes, &w);
            if (e != hipSuccess)
                return e;
            ws = static_cast<char *>(w);
        }
    }
    dma::BigBatch b = {};
    b.count = count;
    int wg = 0;
    size_t off = 0;
    for (int r = 0; r < count; ++r) {
        const int i = order[r];
        const GemvArgs &a = args[idx[i]];
        dma::BigProblem &p = b.p[r];
        p.x = a.x;
        p.packed = a.packed;
        p.scale = a.scale;
        p.y = a.y;
        p.partial = nullptr;
        if (ks[i] > 1) {
            p.partial = reinterpret_cast<float4 *>(ws + off);
            off += (size_t)tiles[i] * ks[i] * C::TN * C::TM * 4;
        }
        p.M = a.M;
        p.N = a.N;
        p.K = a.K;
        p.ksplit = ks[i];
        p.tiled = a.tiled;
        b.wg0[r] = wg;
        wg += tiles[i] * ks[i];
    }
    hipLaunchKernelGGL((dma::gemm_dma_kernel<FP16, GS, C, ZS>), dim3(wg), dim3(C::THREADS), 0,
                       stream, b);
    hipError_t e = hipGetLastError();
    for (int r = 0; r < count && e == hipSuccess; ++r) {
        const dma::BigProblem &p = b.p[r];
        if (p.ksplit == 1)
            continue;
        const int i = order[r];
        const int64_t n4 = (int64_t)tiles[i] * (C::TN * C::TM / 4);
        hipLaunchKernelGGL((dma::gemm_split_reduce<FP16, GS != 0, C>),
                           dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, p.partial,
                           p.scale, p.y, p.M, p.N, p.ksplit);
        e = hipGetLastError();
    }
    return e;
}

template <bool FP16, int GS, bool ZS>
hipError_t launch_big_group(const GemvArgs *args, const int (*idx)[kGemvMaxBatch], const int *n,
                            hipStream_t stream, const FixedScratch *fixed)
{
    hipError_t e = hipSuccess;
    if (n[0] && e == hipSuccess)
        e = launch_big_mode<FP16, GS, TinyCfg, ZS>(args, idx[0], n[0], stream, fixed);
    if (n[1] && e == hipSuccess)
        e = launch_big_mode<FP16, GS, SmallCfg, ZS>(args, idx[1], n[1], stream, fixed);
    if (n[2] && e == hipSuccess)
        e = launch_big_mode<FP16, GS, MidCfg, ZS>(args, idx[2], n[2], stream, fixed);
    if constexpr (GS == 0)  // group-scaled problems never take the large configuration
        if (n[3] && e == hipSuccess)
            e = launch_big_mode<FP16, GS, BigCfg, ZS>(args, idx[3], n[3], stream, fixed);
    return e;
}

// The batch's problems by (scale mode, configuration): one grouped launch each.
struct BigClasses {
    int idx[4][4][kGemvMaxBatch];
    int n[4][4] = {};
    BigClasses(const GemvArgs *args, int count)
    {
        static_assert(kGemvMaxBatch <= 8, "batch table");
        for (int i = 0; i < count; ++i) {
            const int g = args[i].group;
            const int mode = g == 0 ? 0 : (g == 64 ? 1 : (g == 128 ? 2 : 3));
            const int c = big_cfg_of(args[i].M, args[i].K, g);
            idx[mode][c][n[mode][c]++] = i;
        }
    }
};

template <bool FP16, bool ZS>
hipError_t launch_gemm_big_batch(const GemvArgs *args, int count, hipStream_t stream,
                                 const FixedScratch *fixed)
{
    const BigClasses cl(args, count);
    hipError_t e = launch_big_group<FP16, 0, ZS>(args, cl.idx[0], cl.n[0], stream, fixed);
    if (e == hipSuccess)
        e = launch_big_group<FP16, 64, ZS>(args, cl.idx[1], cl.n[1], stream, fixed);
    if (e == hipSuccess)
        e = launch_big_group<FP16, 128, ZS>(args, cl.idx[2], cl.n[2], stream, fixed);
    if (e == hipSuccess)
        e = launch_big_group<FP16, 256, ZS>(args, cl.idx[3], cl.n[3], stream, fixed);
    return e;
}

size_t gemm_batch_scratch_need(const GemvArgs *args, int count, size_t cap)
{
    // the launches of one call run in stream order and reuse the buffer from
    // its start: the need is the largest single launch's (planned as the
    // launch will be planned with a fixed scratch of `cap` bytes)
    const BigClasses cl(args, count);
    int order[kGemvMaxBatch], tiles[kGemvMaxBatch], ks[kGemvMaxBatch];
    size_t need = 0;
    for (int mode = 0; mode < 4; ++mode) {
        const int *n = cl.n[mode];
        if (n[0])
            need = std::max(need, plan_big_mode<TinyCfg>(args, cl.idx[mode][0], n[0], order, tiles, ks, cap));
        if (n[1])
            need = std::max(need, plan_big_mode<SmallCfg>(args, cl.idx[mode][1], n[1], order, tiles, ks, cap));
        if (n[2])
            need = std::max(need, plan_big_mode<MidCfg>(args, cl.idx[mode][2], n[2], order, tiles, ks, cap));
        if (n[3] && mode == 0)
            need = std::max(need, plan_big_mode<BigCfg>(args, cl.idx[mode][3], n[3], order, tiles, ks, cap));
    }
    return need;
}

hipError_t launch_gemm_batch(const GemvArgs *args, int count, bool fp16, hipStream_t stream,
                             const FixedScratch *fixed, bool zero_skip)
{
    if (zero_skip)
        return fp16 ? launch_gemm_big_batch<true, true>(args, count, stream, fixed)
                    : launch_gemm_big_batch<false, true>(args, count, stream, fixed);
    return fp16 ? launch_gemm_big_batch<true, false>(args, count, stream, fixed)
                : launch_gemm_big_batch<false, false>(args, count, stream, fixed);
}

hipError_t launch_gemm(const uint16_t *x, bool fp16, int M, int N, int K, const uint8_t *packed,
                       const uint16_t *scale, int group, uint16_t *y, hipStream_t stream,
                       bool tiled, bool zero_skip)
{
    if (gemm_big_takes(M, N, K, group, scale, tiled)) {
        const GemvArgs a = {x, packed, scale, y, M, N, K, group, tiled ? 1 : 0};
        return launch_gemm_batch(&a, 1, fp16, stream, nullptr, zero_skip);
    }
    if (tiled || zero_skip)  // the 128 x 128 kernel: row-major codes, no zero skipping
        return hipErrorInvalidValue;
    const int glog = group ? group_log2(group) : 0;
    if (fp16)
        return group ? launch_gemm_t<true, true>(x, M, N, K, packed, scale, glog, y, stream)
                     : launch_gemm_t<true, false>(x, M, N, K, packed, scale, 0, y, stream);
    return group ? launch_gemm_t<false, true>(x, M, N, K, packed, scale, glog, y, stream)
                 : launch_gemm_t<false, false>(x, M, N, K, packed, scale, 0, y, stream);
}

}  // namespace ternary
