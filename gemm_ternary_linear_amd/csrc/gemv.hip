// Decode GEMV routing (1 <= M <= 8) for the ternary linear layer on gfx950:
// one projection, or a batch of projections fused into as few launches as
// the kernel instances allow ([trdm] trdm.cn
// "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §2.2: the segments of a
// fused QKV weight share one launch, which pays the fixed launch and
// first-byte latency once).  Two decode kernels exist: gemv_f4.hip (codes as
// fp4, activations as exact fp8 pieces, on the scaled fp4 x fp8 matrix
// instruction) and gemv_stream.hip (codes as 16-bit +-2 / 0 on the bf16/fp16
// matrix instruction).  Both read row-major and tiled codes.
//
// The automatic choice takes the fp4 kernel for one token and the 16-bit one
// for 2 to 8 tokens wherever it takes the shape (the fp4 kernel otherwise):
// every fp4 workgroup converts the whole activation block into fp8 pieces,
// work that grows with the tokens, while the 16-bit kernel feeds x to the
// matrix cores as it is.  Measured on MI355X (tiled codes, fused launches of
// the 7B layer): 2 / 4 / 8 tokens 18.1 / 21.5 / 27.2 us on the 16-bit kernel
// against 20.7 / 23.4 / 33.8 us with the fp4 one; the 27B group-128 pair at
// 4 tokens 23.0 against 36.6 us.  At one token the fp4 kernel wins in fused
// launches (7B layer 13.0 against 16.1 us) and on lone projections with
// K <= 8192 (tiled codes, weights rotating over 1 GiB: 7B gate 6.7 against
// 7.5 us, 27B up 10.5 against 12.7, 7B q 3.8 against 4.1, 1024 x 1024 3.8
// against 3.9), while a lone projection of fewer than 8192 channels with
// longer K runs faster on the 16-bit kernel, whose workgroups stage only their
// own part of x instead of converting all of it (27B down 15.0 against 16.1
// us, 7B down 7.9 against 8.8).
#include "internal.h"

namespace ternary {

bool gemv_kernel_takes(GemvKernel k, int64_t M, int64_t K, int group, bool fp16, bool tiled)
{
    switch (k) {
    case GemvKernel::F4: return gemv_f4_takes(M, K, group, fp16);
    case GemvKernel::B16: return gemv_stream_takes(M, K, group);
    default: return gemv_f4_takes(M, K, group, fp16) || gemv_stream_takes(M, K, group);
    }
}

hipError_t launch_gemv_batch(const GemvArgs *args, int count, bool fp16, hipStream_t stream,
                             GemvKernel kernel)
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
    // Each group value (per channel, 32, 64, 128, 256), each M and each kernel
    // is a separate instance: one launch per non-empty class.  A lone
    // one-token problem of fewer than 8192 channels and K > 8192 prefers the
    // 16-bit kernel.
    int n_m1 = 0;
    for (int i = 0; i < count; ++i)
        n_m1 += args[i].M == 1 && args[i].N > 0 ? 1 : 0;
    static const int kGroups[] = {0, 32, 64, 128, 256};
    for (const int group : kGroups) {
        int f4[kGemvMaxM][kGemvMaxBatch], b16[kGemvMaxM][kGemvMaxBatch];
        int nf[kGemvMaxM] = {}, nb[kGemvMaxM] = {};
        for (int oi = 0; oi < count; ++oi) {
            const GemvArgs &a = args[order[oi]];
            if (a.group != group || a.M == 0 || a.N == 0)
                continue;
            const bool f4_first = a.M == 1 && !(n_m1 == 1 && a.N < 8192 && a.K > 8192);
            const bool use_f4 =
                kernel != GemvKernel::B16 && gemv_f4_takes(a.M, a.K, group, fp16) &&
                (kernel == GemvKernel::F4 || f4_first || !gemv_stream_takes(a.M, a.K, group));
            if (use_f4)
                f4[a.M - 1][nf[a.M - 1]++] = order[oi];
            else if (kernel != GemvKernel::F4 && gemv_stream_takes(a.M, a.K, group))
                b16[a.M - 1][nb[a.M - 1]++] = order[oi];
            else
                return hipErrorInvalidValue;
        }
        for (int m = 0; m < kGemvMaxM; ++m) {
            if (nf[m]) {
                const hipError_t e = launch_gemv_f4(args, f4[m], nf[m], fp16, group, stream);
                if (e != hipSuccess)
                    return e;
            }
            if (nb[m]) {
                const hipError_t e = launch_gemv_stream(args, b16[m], nb[m], fp16, group, stream);
                if (e != hipSuccess)
                    return e;
            }
        }
    }
    return hipSuccess;
}

hipError_t launch_gemv(const uint16_t *x, bool fp16, int M, int N, int K, const uint8_t *packed,
                       const uint16_t *scale, int group, uint16_t *y, hipStream_t stream,
                       GemvKernel kernel, bool tiled)
{
    const GemvArgs a = {x, packed, scale, y, M, N, K, group, tiled ? 1 : 0};
    return launch_gemv_batch(&a, 1, fp16, stream, kernel);
}

}  // namespace ternary
