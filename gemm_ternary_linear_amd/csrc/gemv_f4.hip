// Decode GEMV (M <= 8) on gfx950's scaled fp4 x fp8 matrix instruction.
//
// The layer ([xxqk] m.xxqk.cn/news/593501 §4.3: y = x @ (unpack(q) * s)^T) at
// a few tokens reads every packed byte once and does little arithmetic per
// byte ([nxbn] m.nxbn.cn/news/169761 §4.1/§4.4), so the kernel is built to
// spend as few vector instructions per code as possible and to issue its
// weight reads the way HBM serves them best (short parts, every load issued
// at once).
//
//  * Codes -> fp4.  A 2-bit code (b1 b0) becomes (sign, magnitude) =
//    (b1, b0 ^ b1), placed at the top of a 4-bit e2m1 field with two zero bits
//    below: 00 -> +0, 01 -> +2, 10 -> -2, 11 -> -0 (read as 0, [trdm]
//    trdm.cn "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1).  Sixteen codes
//    (one 32-bit word) cost five vector instructions and give two fp4 words:
//    the odd codes and the even codes.  These are the A operand of
//    v_mfma_scale_f32_16x16x128_f8f6f4 (A: fp4, 16 channels x 128 K), whose
//    K order inside a 32-code block is therefore odd codes then even codes.
//  * x -> exact fp8 pieces.  The matrix instruction multiplies fp4 by fp8, so
//    each activation is written as the sum of e4m3 pieces: x = X1*S1 + X2*S2
//    for bf16 (8 significant bits = 4 + 4), plus X3*S3 for fp16 (11 bits),
//    with S1 a power of two per 32 elements chosen from their largest
//    magnitude (so |x / S1| < 256 <= 448) and S2 = S1 / 16, S3 = S1 / 256.
//    X1 = RNE(x / S1), X2 = RNE((x - X1 S1) / S2), ...: every piece is exact
//    for elements within 2^13 of their block's largest (the e4m3 normal
//    range), and below that the error is under 2^-9 S1 per element, far
//    inside 1e-3 * sum |x| s.  The pieces are separate B columns, the S's
//    the instruction's per-32-element B scales, and fp4 x e4m3 products are
//    exact, so the result is the fp32 sum of the exact products.
//  * Work split.  A workgroup of 8 waves holds RB blocks of 16 channels x KP
//    K parts (RB * KP = 8).  It converts its problem's whole x into LDS once
//    (all 512 lanes, 8 elements each), while every wave's first code loads
//    are already in flight; then each wave runs its part in one-shot chunks
//    of 4 slabs (8 for instances with several MFMA passes; a slab is 256
//    codes = 64 bytes of each of the block's 16 rows, one 16-byte buffer load
//    per lane).  K parts meet in LDS: the last wave of a block adds them in
//    part order (deterministic) and writes y.
//  * Code layouts.  Row-major codes ([trdm] §3.1) give each load instruction
//    16 rows x 64 bytes; the library's tiled layout stores every slab of a
//    block as one kilobyte in the A operand's lane order, so the same load
//    reads one contiguous kilobyte (measured 14.2 against 15.3 us for the 7B
//    decode layer at M = 1).  Only the address arithmetic differs.
//  * Scales.  Per-channel scales ([nxbn] §3.2) multiply the final sum.  Group
//    scales ([trdm] §3.1/§4.2: 128; [xxqk] §4.2: 64; yangyitao.com vLLM book,
//    chapter 13, §13.3.3: 32, 256) multiply each group's fp32 partial: a
//    token's B columns are split by group (GC = 1, 2 or 4 columns), so every
//    column of a slab's product holds one group, which takes its scale in
//    fp32 before the sum over slabs.
#include "common.h"
#include "internal.h"

#include <algorithm>
#include <atomic>
#include <mutex>

namespace ternary {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kOOB = 0x40000000;
constexpr int kPad = 64;      // bytes between two pieces in LDS (B reads of
                              // neighbouring columns fall on other banks)
// x loads per lane issued before the codes: all of a single token's x up to
// K = 24576, fewer with more tokens (registers)
template <int MT>
constexpr int pre_loads() { return MT == 1 ? 6 : 2; }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x2_t __attribute__((__vector_size__(4)));

// Kernel geometry of one instance.
template <bool FP16, int GMODE, int MT>
struct Geo {
    // GMODE: 0 per channel, 1 groups of 256, 2 of 128, 3 of 64, 4 of 32
    static constexpr int NP = FP16 ? 3 : 2;                       // pieces of x
    static constexpr int GC = GMODE <= 1 ? 1 : (GMODE == 2 ? 2 : 4);  // columns per piece
    static constexpr int CPT = NP * GC <= 2 ? 2 : (NP * GC <= 4 ? 4 : (NP * GC <= 8 ? 8 : 16));
    static constexpr int TP = 16 / CPT;                           // tokens per MFMA pass
    static constexpr int NPASS = (MT + TP - 1) / TP;
    // slabs per one-shot chunk of code loads: 4 with one MFMA pass (measured
    // faster than 8 on the 7B decode layer), 8 with more (4 costs registers)
    static constexpr int SP = NPASS == 1 ? 4 : 8;
    static constexpr int GPS = GMODE == 0 ? 0 : (GMODE == 1 ? 1 : (GMODE == 2 ? 2 : (GMODE == 3 ? 4 : 8)));  // groups per slab
    static constexpr int GLOG = GMODE == 1 ? 8 : (GMODE == 2 ? 7 : (GMODE == 3 ? 6 : 5));
};

// LDS layout, from a problem's padded K (Kp = slabs * 256):
//   pieces  [MT][NP][Kp + kPad] bytes   e4m3, per slab two 128-byte MFMA chunks
//                                       (K block kb of MFMA j at s*256 + j*128
//                                       + 32 kb, in the fp4 operand's order)
//   scales  [MT][NP][Kp / 32] bytes     E8M0 of 32-element block 8 s + 2 kb + j
//   gscale  [kWaves][SP * GPS][16]      fp16 group scales of a wave's chunk
//   red     [kWaves][NPASS][64] f32x4   K-part partial sums
//   cnt     [kWaves] int
struct Lds {
    int piece_stride, sc_base, sc_stride, gs_base, red_base, cnt_base, bytes;
};
template <bool FP16, int GMODE, int MT>
__host__ __device__ inline Lds lds_layout(int K)
{
    using G = Geo<FP16, GMODE, MT>;
    Lds L;
    const int Kp = (K + 255) & ~255;
    L.piece_stride = Kp + kPad;
    L.sc_base = MT * G::NP * L.piece_stride;
    L.sc_stride = Kp >> 5;
    L.gs_base = (L.sc_base + MT * G::NP * L.sc_stride + 15) & ~15;
    L.red_base = L.gs_base + (G::GPS ? kWaves * G::SP * G::GPS * 16 * 2 : 0);
    L.cnt_base = L.red_base + kWaves * G::NPASS * 64 * 16;
    L.bytes = L.cnt_base + kWaves * 4;
    return L;
}

struct F4Problem {
    const uint16_t *x;
    const uint8_t *packed;
    const uint16_t *scale;
    uint16_t *y;
    int M, N, K;
    int rb, kp;   // 16-channel blocks per workgroup, K parts per block (rb * kp = kWaves)
    int unit0;    // first workgroup of the problem
    int tiled;    // codes in the tiled layout (else row-major [N, K/4])
};
struct F4Batch {
    int count;
    int unit0[kGemvMaxBatch];
    F4Problem p[kGemvMaxBatch];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             (int)0x00020000);
}

// Lane i of each quad of lanes takes v from lane (SEL >> 2i) & 3 of its quad.
template <int SEL>
__device__ __forceinline__ uint32_t quad_perm(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, SEL, 0xf, 0xf, false);
}
__device__ __forceinline__ float xor_lanes(float v, int m)
{
    if (m == 1)
        return __builtin_bit_cast(float, quad_perm<0xb1>(__builtin_bit_cast(uint32_t, v)));
    if (m == 2)
        return __builtin_bit_cast(float, quad_perm<0x4e>(__builtin_bit_cast(uint32_t, v)));
    return __shfl_xor(v, m);
}

// 16 codes (one word) -> the fp4 words of its odd and of its even codes.
__device__ __forceinline__ void codes_to_fp4(uint32_t w, uint32_t &odd, uint32_t &even)
{
    // field (b1 b0) -> (sign, magnitude) = (b1, b0 ^ b1): truth table 0x78 of
    // (w, w >> 1, mask): mask ? w ^ (w >> 1) : w
    const uint32_t z = __builtin_amdgcn_bitop3_b32(w, w >> 1, 0x55555555u, 0x78);
    odd = z & 0xccccccccu;          // field 2n+1 at the top of nibble n
    even = (z << 2) & 0xccccccccu;  // field 2n at the top of nibble n
}

// Convert 8 activations (task `t`: elements 8*(t%4) .. +7 of 32-block b of
// token `tok`) into their pieces in LDS.  The four lanes of a quad hold one
// block; all four take part in the block maximum.
template <bool FP16, int MT>
__device__ __forceinline__ void convert8(u32x4_t v, int tok, int b, int mq, bool store,
                                         unsigned char *lds, const Lds &L)
{
    constexpr int NP = FP16 ? 3 : 2;
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
    float xf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (FP16) {
            xf[2 * i] = f16_bits_to_f32((uint16_t)vv[i]);
            xf[2 * i + 1] = f16_bits_to_f32((uint16_t)(vv[i] >> 16));
        } else {
            xf[2 * i] = __builtin_bit_cast(float, vv[i] << 16);
            xf[2 * i + 1] = __builtin_bit_cast(float, vv[i] & 0xffff0000u);
        }
    }
    float m = fmaxf(fmaxf(fmaxf(fabsf(xf[0]), fabsf(xf[1])), fmaxf(fabsf(xf[2]), fabsf(xf[3]))),
                    fmaxf(fmaxf(fabsf(xf[4]), fabsf(xf[5])), fmaxf(fabsf(xf[6]), fabsf(xf[7]))));
    uint32_t mb = __builtin_bit_cast(uint32_t, m);
    mb = max(mb, quad_perm<0xb1>(mb));
    mb = max(mb, quad_perm<0x4e>(mb));
    // S1 = 2^(e1 - 127) with e1 = (exponent of the block max) - 7, so |x / S1| < 256
    const int ef = (int)(mb >> 23);
    int e[3];
    e[0] = max(ef - 7, 1);
    e[1] = max(e[0] - 4, 1);
    e[2] = max(e[0] - 8, 1);
    uint32_t pw[3][2];
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        r[i] = xf[i];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const float sc = __builtin_bit_cast(float, (uint32_t)e[p] << 23);
        s16x2_t q0 = {0, 0}, q1 = {0, 0};
        q0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q0, r[0], r[1], sc, false);
        q0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q0, r[2], r[3], sc, true);
        q1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q1, r[4], r[5], sc, false);
        q1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q1, r[6], r[7], sc, true);
        pw[p][0] = __builtin_bit_cast(uint32_t, q0);
        pw[p][1] = __builtin_bit_cast(uint32_t, q1);
        if (p + 1 < NP) {
            // the remainder, exact in fp32
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(pw[p][h], sc, false);
                const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(pw[p][h], sc, true);
                r[4 * h] -= lo.x;
                r[4 * h + 1] -= lo.y;
                r[4 * h + 2] -= hi.x;
                r[4 * h + 3] -= hi.y;
            }
        }
    }
    if (!store)
        return;
    // element c of the block: odd c -> byte (c-1)/2, even c -> byte 8 + c/2,
    // within its 16-element half; this lane holds c = 8 mq .. 8 mq + 7
    const int s = b >> 3, q = b & 7;
    const int off = s * 256 + (q & 1) * 128 + 32 * (q >> 1) + 16 * (mq >> 1) + 4 * (mq & 1);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        unsigned char *dst = lds + (tok * NP + p) * L.piece_stride + off;
        *reinterpret_cast<uint32_t *>(dst) = __builtin_amdgcn_perm(pw[p][1], pw[p][0], 0x07050301u);
        *reinterpret_cast<uint32_t *>(dst + 8) =
            __builtin_amdgcn_perm(pw[p][1], pw[p][0], 0x06040200u);
        if (mq == 0)
            lds[L.sc_base + (tok * NP + p) * L.sc_stride + b] = (unsigned char)e[p];
    }
}

// GMODE as in Geo; MT: the instance's token count (M <= MT); CP: the cache
// policy of the code loads (kStreamLoad when every problem holds tiled codes).
template <bool FP16, int GMODE, int MT, int CP>
__global__ void __launch_bounds__(kThreads) gemv_f4_kernel(const F4Batch batch)
{
    using G = Geo<FP16, GMODE, MT>;
    constexpr int NP = G::NP, GC = G::GC, CPT = G::CPT, TP = G::TP, NPASS = G::NPASS;
    constexpr bool GROUPED = GMODE != 0;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    int pi = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxBatch; ++i)
        if (i < batch.count && (int)blockIdx.x >= batch.unit0[i])
            pi = i;
    const F4Problem &P = batch.p[pi];
    const int M = P.M, N = P.N, K = P.K, RB = P.rb, KP = P.kp;
    const Lds L = lds_layout<FP16, GMODE, MT>(K);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rbi = wave % RB, kpi = wave / RB;
    const int rb = ((int)blockIdx.x - P.unit0) * RB + rbi;
    const int nslabs = (K + 255) >> 8, rowbytes = K >> 2;
    const int g = lane >> 4, col = lane & 15;

    // ---- x loads for the conversion come first (they return before the codes)
    const int tasks_per_tok = (nslabs * 256) >> 3;
    const int ntask = M * tasks_per_tok;
    const int npass_x = (ntask + kThreads - 1) / kThreads;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(P.x, (uint32_t)M * (uint32_t)K * 2u);
    auto x_off = [&](int t) -> int {
        const int tok = t / tasks_per_tok, e = (t - tok * tasks_per_tok) * 8;
        return (t < ntask && e < K) ? (tok * K + e) * 2 : kOOB;
    };
    constexpr int kPreLoads = pre_loads<MT>();
    u32x4_t xv[kPreLoads];
#pragma unroll
    for (int p = 0; p < kPreLoads; ++p) {
        xv[p] = u32x4_t{0, 0, 0, 0};
        if (p < npass_x)
            xv[p] = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off(p * kThreads + tid), 0, 0);
    }

    // ---- this wave's part: slabs [s_begin, s_begin + S); waves past RB * KP
    // hold none (they only help convert x)
    const bool active = wave < RB * KP;
    const int s_begin = active ? kpi * nslabs / KP : 0;
    const int S = __builtin_amdgcn_readfirstlane(active ? (kpi + 1) * nslabs / KP - s_begin : 0);
    const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(16, N - rb * 16)));
    // Row-major codes: lane (g, col) reads bytes 16g .. 16g+15 of slab s of
    // row col, 64 bytes a slab.  Tiled codes: slab s of the block is 1 KB,
    // [4 quarters g][16 rows][16 bytes], so the lane reads bytes 16 * lane of
    // it: one contiguous kilobyte per wave instruction.
    const bool tiled = P.tiled != 0;
    const uint8_t *wbase = nrows == 0 ? P.packed
                           : tiled    ? P.packed + (int64_t)rb * nslabs * kTileBytes
                                      : P.packed + (int64_t)rb * 16 * rowbytes;
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(wbase, nrows == 0 ? 0u : tiled ? (uint32_t)nslabs * kTileBytes
                                                 : (uint32_t)(nrows * rowbytes));
    const int woff = tiled ? lane * 16 : col * rowbytes + g * 16;
    const int sstride = tiled ? kTileBytes : 64;
    // row-major codes at or past K within a row read as whatever follows
    // (tiled ones as the zero padding); their x pieces are zero
    constexpr int kSP = G::SP;
    u32x4_t w[kSP];
    __builtin_amdgcn_sched_barrier(0);
    load_code_run<CP>(w, wr,
                      [&](int j) { return j < S ? woff + (s_begin + j) * sstride : kOOB; });
    // channel scale of row 4g + (lane & 3): each quad of lanes holds the four
    // rows its C fragment covers (shared by DPP in the epilogue)
    const int ch0 = rb * 16 + 4 * g;
    uint32_t chs = 0;
    if constexpr (!GROUPED) {
        const __amdgpu_buffer_rsrc_t sr =
            make_rsrc(nrows > 0 ? P.scale + (int64_t)rb * 16 : P.scale, (uint32_t)nrows * 2u);
        const int r = 4 * g + (lane & 3);
        chs = __builtin_amdgcn_raw_buffer_load_b16(sr, r < nrows ? r * 2 : kOOB, 0, 0);
    }
    int *const cnt = reinterpret_cast<int *>(smem + L.cnt_base);
    if (KP > 1 && tid < kWaves)
        cnt[tid] = 0;

    // ---- convert x into LDS: task t = 8 elements of token t / tasks_per_tok
#pragma unroll
    for (int p = 0; p < kPreLoads; ++p) {
        if (p < npass_x) {
            const int t = p * kThreads + tid;
            const int tok = t / tasks_per_tok, tk = t - tok * tasks_per_tok;
            convert8<FP16, MT>(xv[p], tok, tk >> 2, tk & 3, t < ntask, smem, L);
        }
    }
    for (int p = kPreLoads; p < npass_x; ++p) {
        const int t = p * kThreads + tid;
        const int tok = t / tasks_per_tok, tk = t - tok * tasks_per_tok;
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off(t), 0, 0);
        convert8<FP16, MT>(v, tok, tk >> 2, tk & 3, t < ntask, smem, L);
    }
    __syncthreads();
    if (!active)
        return;

    // ---- this lane's B column in every pass
    const int slot = col % CPT;
    const int cpiece = slot / GC, chalf = slot % GC;
    // group index of K block kb within a slab's column split (GC columns)
    auto hk = [](int kb) { return GC == 1 ? 0 : (GC == 2 ? kb >> 1 : kb); };
    const bool keep_lo = hk(g >> 1) == chalf, keep_hi = hk(2 + (g >> 1)) == chalf;
    int bbase[NPASS], sbase[NPASS];
    bool bvalid[NPASS];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const int tok = ps * TP + col / CPT;
        bvalid[ps] = cpiece < NP && tok < M;
        const int pc = (bvalid[ps] ? tok * NP + cpiece : 0);
        bbase[ps] = pc * L.piece_stride + 16 * g;
        sbase[ps] = L.sc_base + pc * L.sc_stride + 2 * g;
    }
    // group scales: this wave's staging area and this lane's row offset
    uint16_t *const gsb = reinterpret_cast<uint16_t *>(smem + L.gs_base) + wave * (kSP * G::GPS * 16);
    const int ngroups = GROUPED ? (K >> G::GLOG) : 1;
    // groups of 128 or smaller come two to a 4-byte load when every such
    // load is aligned and holds two groups of one row (a wave-uniform choice)
    const bool pair_loads = GROUPED && (ngroups & 1) == 0 && ((uintptr_t)P.scale & 3) == 0;
    // group scales: the resource starts at the block's first row (64-bit
    // pointer arithmetic), so offsets stay below 16 rows of scales
    const __amdgpu_buffer_rsrc_t gsr =
        make_rsrc(GROUPED && nrows > 0 ? P.scale + (int64_t)rb * 16 * ngroups : P.scale,
                  GROUPED ? (uint32_t)(nrows * ngroups * 2) : 0u);

    f32x4_t acc[NPASS];
    // B operands of every pass.  With one pass they are kept across slabs:
    // lanes whose column holds no piece, and the half of a grouped column's K
    // blocks that is not its group's, stay zero, and only the rest is reloaded
    // from LDS every slab.  With more passes, keeping them would take more
    // than 128 registers (half the occupancy) in some instances, so they are
    // cleared and reloaded every slab.
    constexpr bool KEEPB = NPASS == 1;
    i32x8_t bo[NPASS][2];
    uint32_t bsw[NPASS];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        acc[ps] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        bo[ps][0] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        bo[ps][1] = bo[ps][0];
        bsw[ps] = 0;
    }

    for (int c0 = 0; c0 < S; c0 += kSP) {
        if (c0 > 0) {
            __builtin_amdgcn_sched_barrier(0);
            load_code_run<CP>(w, wr, [&](int j) {
                return c0 + j < S ? woff + (s_begin + c0 + j) * sstride : kOOB;
            });
        }
        if constexpr (GROUPED) {
            // stage the chunk's group scales: [local group][16 rows]
            constexpr int NG = kSP * G::GPS;
            const int g_first = ((s_begin + c0) * 256) >> G::GLOG;
            if (G::GPS >= 2 && pair_loads) {
                // two groups per 4-byte load: lane l takes row l & 15's pair
                // (l >> 4) + 4 i, so a row's 16 lanes-worth of groups come in
                // half the requests (g_first is even: a chunk is whole slabs)
#pragma unroll
                for (int i = 0; i < NG / 8; ++i) {
                    const int pr = (lane >> 4) + 4 * i, row = lane & 15;
                    const int gi = g_first + 2 * pr;
                    const int off = row < nrows && gi < ngroups ? (row * ngroups + gi) * 2 : kOOB;
                    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(gsr, off, 0, 0);
                    gsb[2 * pr * 16 + row] = (uint16_t)v;
                    gsb[(2 * pr + 1) * 16 + row] = (uint16_t)(v >> 16);
                }
            } else {
#pragma unroll
                for (int i = 0; i < NG / 4; ++i) {
                    const int lg = (lane >> 4) + 4 * i, row = lane & 15;
                    const int gi = g_first + lg;
                    const int off = row < nrows && gi < ngroups ? (row * ngroups + gi) * 2 : kOOB;
                    gsb[lg * 16 + row] =
                        (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(gsr, off, 0, 0);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int jj = 0; jj < kSP; ++jj) {
            const int i = c0 + jj;
            if (i >= S)
                break;
            const int s = s_begin + i;
            uint32_t a[2][4];
            codes_to_fp4(w[jj].x, a[0][0], a[0][1]);
            codes_to_fp4(w[jj].y, a[0][2], a[0][3]);
            codes_to_fp4(w[jj].z, a[1][0], a[1][1]);
            codes_to_fp4(w[jj].w, a[1][2], a[1][3]);
            const i32x8_t A0 = {(int)a[0][0], (int)a[0][1], (int)a[0][2], (int)a[0][3], 0, 0, 0, 0};
            const i32x8_t A1 = {(int)a[1][0], (int)a[1][1], (int)a[1][2], (int)a[1][3], 0, 0, 0, 0};
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps) {
                if constexpr (!KEEPB) {
                    bo[ps][0] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
                    bo[ps][1] = bo[ps][0];
                    bsw[ps] = 0;
                }
                if (bvalid[ps]) {
                    const unsigned char *src = smem + bbase[ps] + s * 256;
                    if (keep_lo) {
                        const u32x4_t p0 = *reinterpret_cast<const u32x4_t *>(src);
                        const u32x4_t p2 = *reinterpret_cast<const u32x4_t *>(src + 128);
                        bo[ps][0][0] = (int)p0.x; bo[ps][0][1] = (int)p0.y;
                        bo[ps][0][2] = (int)p0.z; bo[ps][0][3] = (int)p0.w;
                        bo[ps][1][0] = (int)p2.x; bo[ps][1][1] = (int)p2.y;
                        bo[ps][1][2] = (int)p2.z; bo[ps][1][3] = (int)p2.w;
                    }
                    if (keep_hi) {
                        const u32x4_t p1 = *reinterpret_cast<const u32x4_t *>(src + 64);
                        const u32x4_t p3 = *reinterpret_cast<const u32x4_t *>(src + 192);
                        bo[ps][0][4] = (int)p1.x; bo[ps][0][5] = (int)p1.y;
                        bo[ps][0][6] = (int)p1.z; bo[ps][0][7] = (int)p1.w;
                        bo[ps][1][4] = (int)p3.x; bo[ps][1][5] = (int)p3.y;
                        bo[ps][1][6] = (int)p3.z; bo[ps][1][7] = (int)p3.w;
                    }
                    bsw[ps] = *reinterpret_cast<const uint16_t *>(smem + sbase[ps] + 8 * s);
                }
                if constexpr (!GROUPED) {
                    acc[ps] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A0, bo[ps][0], acc[ps], 4, 0, 0, 127, 0, (int)bsw[ps]);
                    acc[ps] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A1, bo[ps][1], acc[ps], 4, 0, 0, 127, 1, (int)bsw[ps]);
                } else {
                    // this lane's column holds one group of the slab (per
                    // MFMA for groups of 32): fold its partial with the scale
                    // of rows 4g .. 4g+3
                    const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
                    f32x4_t d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A0, bo[ps][0], z4, 4, 0, 0, 127, 0, (int)bsw[ps]);
                    f32x4_t d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A1, bo[ps][1], GMODE == 4 ? z4 : d0, 4, 0, 0, 127, 1, (int)bsw[ps]);
                    auto fold = [&](int lgrp, f32x4_t d) {
                        const uint2 s4 = *reinterpret_cast<const uint2 *>(gsb + lgrp * 16 + 4 * g);
                        acc[ps][0] += f16_bits_to_f32((uint16_t)s4.x) * d[0];
                        acc[ps][1] += f16_bits_to_f32((uint16_t)(s4.x >> 16)) * d[1];
                        acc[ps][2] += f16_bits_to_f32((uint16_t)s4.y) * d[2];
                        acc[ps][3] += f16_bits_to_f32((uint16_t)(s4.y >> 16)) * d[3];
                    };
                    if constexpr (GMODE == 4) {
                        fold(G::GPS * jj + 2 * chalf, d0);
                        fold(G::GPS * jj + 2 * chalf + 1, d1);
                    } else {
                        fold(G::GPS * jj + chalf, d1);
                    }
                }
            }
        }
    }

    // ---- K-part reduction: the last wave of a block adds the parts in order
    f32x4_t sum[NPASS];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps)
        sum[ps] = acc[ps];
    if (KP > 1) {
        f32x4_t *red = reinterpret_cast<f32x4_t *>(smem + L.red_base);
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps)
            red[(wave * NPASS + ps) * 64 + lane] = acc[ps];
        int before = 0;
        if (lane == 0)
            before = __hip_atomic_fetch_add(&cnt[rbi], 1, __ATOMIC_ACQ_REL,
                                            __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(before) != KP - 1)
            return;
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
            sum[ps] = red[(rbi * NPASS + ps) * 64 + lane];
            for (int j = 1; j < KP; ++j) {
                const f32x4_t v = red[((rbi + j * RB) * NPASS + ps) * 64 + lane];
                sum[ps][0] += v[0];
                sum[ps][1] += v[1];
                sum[ps][2] += v[2];
                sum[ps][3] += v[3];
            }
        }
    }

    // ---- epilogue: a token's CPT columns, scales, rounding, store
    float chsc[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (!GROUPED) {
        chsc[0] = f16_bits_to_f32((uint16_t)quad_perm<0x00>(chs));
        chsc[1] = f16_bits_to_f32((uint16_t)quad_perm<0x55>(chs));
        chsc[2] = f16_bits_to_f32((uint16_t)quad_perm<0xaa>(chs));
        chsc[3] = f16_bits_to_f32((uint16_t)quad_perm<0xff>(chs));
    }
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        uint16_t o16[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float tot = sum[ps][r];
#pragma unroll
            for (int m = 1; m < CPT; m <<= 1)
                tot += xor_lanes(tot, m);
            o16[r] = round_out<FP16>(0.5f * chsc[r] * tot);  // decoded weights are +-2
        }
        const int tok = ps * TP + col / CPT;
        if (slot == 0 && tok < M && ch0 < N) {
            uint16_t *__restrict__ yt = P.y + (int64_t)tok * N;
            if (ch0 + 4 <= N && ((N & 3) == 0 || M == 1)) {
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
}

int gmode_of(int group)
{
    return group == 0 ? 0 : (group == 256 ? 1 : (group == 128 ? 2 : (group == 64 ? 3 : 4)));
}
int kernel_mt(int M) { return M <= 1 ? 1 : (M == 2 ? 2 : (M <= 4 ? 4 : 8)); }

template <bool FP16, int GMODE, int MT>
int lds_need(int K) { return lds_layout<FP16, GMODE, MT>(K).bytes; }

template <bool FP16, int GMODE>
int lds_need_mt(int mt, int K)
{
    switch (mt) {
    case 1: return lds_need<FP16, GMODE, 1>(K);
    case 2: return lds_need<FP16, GMODE, 2>(K);
    case 4: return lds_need<FP16, GMODE, 4>(K);
    default: return lds_need<FP16, GMODE, 8>(K);
    }
}
int lds_need_of(bool fp16, int group, int M, int K)
{
    const int mt = kernel_mt(M);
    switch (gmode_of(group)) {
    case 0: return fp16 ? lds_need_mt<true, 0>(mt, K) : lds_need_mt<false, 0>(mt, K);
    case 1: return fp16 ? lds_need_mt<true, 1>(mt, K) : lds_need_mt<false, 1>(mt, K);
    case 2: return fp16 ? lds_need_mt<true, 2>(mt, K) : lds_need_mt<false, 2>(mt, K);
    case 3: return fp16 ? lds_need_mt<true, 3>(mt, K) : lds_need_mt<false, 3>(mt, K);
    default: return fp16 ? lds_need_mt<true, 4>(mt, K) : lds_need_mt<false, 4>(mt, K);
    }
}

// The kernel instance of (fp16, group mode, token tile, code-load policy),
// with its dynamic-LDS limit raised to kGemvF4MaxLds when `lds` exceeds the
// default 64 KB (once per instance).
template <bool FP16, int GMODE, int MT, int CP>
hipError_t instance(int lds, const void **fn)
{
    auto *k = gemv_f4_kernel<FP16, GMODE, MT, CP>;
    static std::atomic<bool> raised{false};
    if (lds > 64 * 1024 && !raised.load(std::memory_order_acquire)) {
        const hipError_t e = hipFuncSetAttribute(
            (const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, kGemvF4MaxLds);
        if (e != hipSuccess)
            return e;
        raised.store(true, std::memory_order_release);
    }
    *fn = (const void *)k;
    return hipSuccess;
}

hipError_t instance_of(bool fp16, int gm, int mt, int cp, int lds, const void **fn)
{
    auto by_mt = [&]<bool FP16, int GMODE, int CP>() -> hipError_t {
        switch (mt) {
        case 1: return instance<FP16, GMODE, 1, CP>(lds, fn);
        case 2: return instance<FP16, GMODE, 2, CP>(lds, fn);
        case 4: return instance<FP16, GMODE, 4, CP>(lds, fn);
        default: return instance<FP16, GMODE, 8, CP>(lds, fn);
        }
    };
    auto by_gm = [&]<bool FP16, int CP>() -> hipError_t {
        switch (gm) {
        case 0: return by_mt.template operator()<FP16, 0, CP>();
        case 1: return by_mt.template operator()<FP16, 1, CP>();
        case 2: return by_mt.template operator()<FP16, 2, CP>();
        case 3: return by_mt.template operator()<FP16, 3, CP>();
        default: return by_mt.template operator()<FP16, 4, CP>();
        }
    };
    if (cp == kStreamLoad)
        return fp16 ? by_gm.template operator()<true, kStreamLoad>()
                    : by_gm.template operator()<false, kStreamLoad>();
    return fp16 ? by_gm.template operator()<true, 0>() : by_gm.template operator()<false, 0>();
}

// Workgroups of kernel `fn` with `lds` bytes of dynamic LDS that one compute
// unit holds at once (the occupancy calculator; cached per kernel and size).
int resident_per_cu(const void *fn, int lds)
{
    struct Entry {
        const void *fn;
        int lds, n;
    };
    static Entry cache[64];
    static int used = 0;
    static std::mutex mu;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].fn == fn && cache[i].lds == lds)
            return cache[i].n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, (size_t)lds) != hipSuccess ||
        n < 1)
        n = 1;
    if (used < 64)
        cache[used++] = {fn, lds, n};
    return n;
}

// K parts per block: the smallest power of two (up to kWaves) whose parts hold
// at most `target` slabs.
int parts_for(int nslabs, int target)
{
    int kp = 1;
    while (kp < kWaves && (nslabs + kp - 1) / kp > target)
        kp *= 2;
    return kp;
}

// MFMA passes of an instance (tokens per pass = 16 / columns per token).
int passes_of(bool fp16, int group, int M)
{
    const int np = fp16 ? 3 : 2, gc = group == 0 || group == 256 ? 1 : (group == 128 ? 2 : 4);
    const int c = np * gc <= 2 ? 2 : (np * gc <= 4 ? 4 : (np * gc <= 8 ? 8 : 16));
    const int tp = 16 / c;
    return (kernel_mt((int)M) + tp - 1) / tp;
}

}  // namespace

bool gemv_f4_takes(int64_t M, int64_t K, int group, bool fp16)
{
    return M >= 1 && M <= kGemvF4MaxM && K % 128 == 0 && K <= kGemvMaxK &&
           passes_of(fp16, group, (int)M) <= 4 &&
           (group == 0 || group == 32 || group == 64 || group == 128 || group == 256) &&
           (group == 0 || K % group == 0) &&
           lds_need_of(fp16, group, (int)M, (int)K) <= kGemvF4MaxLds;
}

hipError_t launch_gemv_f4(const GemvArgs *args, const int *order, int count, bool fp16, int group,
                          hipStream_t stream)
{
    F4Batch b;
    int units = 0, mt = 0, lds = 0;
    // Parts of at most 12 slabs (32 beyond K = 8192, whose x costs more to
    // convert per workgroup); a launch that would not cover the compute units
    // once takes parts of half that, twice the workgroups.
    auto fill = [&](int shrink) -> hipError_t {
        b.count = 0;
        units = 0;
        mt = 0;
        lds = 0;
        for (int oi = 0; oi < count; ++oi) {
            const GemvArgs &a = args[order[oi]];
            if (a.M == 0 || a.N == 0)
                continue;
            if (a.group != group || (mt != 0 && a.M != mt) || !gemv_f4_takes(a.M, a.K, group, fp16))
                return hipErrorInvalidValue;
            mt = a.M;
            F4Problem &p = b.p[b.count];
            p.x = a.x;
            p.packed = a.packed;
            p.scale = a.scale;
            p.y = a.y;
            p.M = a.M;
            p.N = a.N;
            p.K = a.K;
            p.tiled = a.tiled;
            const int nslabs = (a.K + 255) / 256;
            // (measured, fused launches at one token: 12 / 32 against the
            // earlier 8 / 20 took the 27B-shaped group-128 pair from 20.9 to
            // 17.1 us and the 7B layer from 12.97 to 12.90 us)
            const int target = std::max(1, (a.K > 8192 ? 32 : 12) >> shrink);
            p.kp = parts_for(nslabs, target);
            const int nblocks = (a.N + 15) / 16;
            p.rb = kWaves / p.kp;
            if (p.rb > nblocks) {
                // fewer blocks than the workgroup holds: more K parts per block
                p.rb = nblocks;
                p.kp = 1;
                while (2 * p.kp * p.rb <= kWaves && 2 * p.kp <= nslabs)
                    p.kp *= 2;
            }
            p.unit0 = units;
            b.unit0[b.count] = units;
            units += (nblocks + p.rb - 1) / p.rb;
            lds = std::max(lds, lds_need_of(fp16, group, a.M, a.K));
            ++b.count;
        }
        return hipSuccess;
    };
    hipError_t e = fill(0);
    if (e == hipSuccess && b.count > 0 && units < device_cus())
        e = fill(1);
    if (e != hipSuccess)
        return e;
    if (b.count == 0)
        return hipSuccess;
    bool all_tiled = true;
    for (int i = 0; i < b.count; ++i)
        all_tiled = all_tiled && b.p[i].tiled != 0;
    const void *fn = nullptr;
    e = instance_of(fp16, gmode_of(group), kernel_mt(mt), all_tiled ? kStreamLoad : 0, lds, &fn);
    if (e != hipSuccess)
        return e;
    if (b.count == 1 && (b.p[0].N + 15) / 16 >= kWaves) {
        // One problem: its workgroups are all alike.  A wave loads its part in
        // chunks of SP slabs, one memory round trip each, so a part of 5
        // slabs costs two round trips for 5 KB where one of 4 costs one.
        // Take the most K parts per block whose parts are whole chunks (or at
        // least two), whose workgroups fit in one round of what the device
        // holds at once and cover half the compute units; failing that, the
        // most parts that fit in one round.  Measured on MI355X at one token:
        // the 25600 x 5120 projection (20 slabs) with 2 parts (400
        // workgroups) 10.5 us, against 11.9 with 4 (800, 5-slab parts) and
        // 13.3 with 8; the 18944 x 4096 one with 4 parts (592) 6.8 us,
        // against 6.9 with 2 and 8.2 with 8.
        F4Problem &p = b.p[0];
        const int nblocks = (p.N + 15) / 16, nslabs = (p.K + 255) / 256;
        const int slots = resident_per_cu(fn, lds) * device_cus();
        const int sp = passes_of(fp16, group, mt) == 1 ? 4 : 8;
        int best = 0, fit = 0;
        for (int kp = kWaves; kp >= 1; kp /= 2) {
            const int n = (nblocks + kWaves / kp - 1) / (kWaves / kp);
            const int per = (nslabs + kp - 1) / kp;
            if (kp > nslabs || n > slots)
                continue;
            if (fit == 0)
                fit = kp;
            if ((per % sp == 0 || per >= 2 * sp) && 2 * n >= device_cus()) {
                best = kp;
                break;
            }
        }
        if (best == 0)
            best = fit;
        if (best != 0) {
            p.kp = best;
            p.rb = kWaves / best;
            units = (nblocks + p.rb - 1) / p.rb;
        }
    }
    void *kargs[] = {&b};
    return hipLaunchKernel(fn, dim3(units), dim3(kThreads), kargs, (size_t)lds, stream);
}

}  // namespace ternary
