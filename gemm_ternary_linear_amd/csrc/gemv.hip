// Decode GEMV routing (1 <= M <= 8) for the ternary linear layer on gfx950:
// one projection, or a batch of projections fused into as few launches as
// the kernel instances allow ([trdm] trdm.cn
// "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §2.2: the segments of a
// fused QKV weight share one launch, which pays the fixed launch and
// first-byte latency once).  The kernel itself is gemv_stream.hip.
#include "internal.h"

namespace ternary {

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
    // Each group value (per channel, 32, 64, 128, 256) and each M is a
    // separate kernel instance: one launch per non-empty class.
    static const int kGroups[] = {0, 32, 64, 128, 256};
    for (const int group : kGroups) {
        int idx[kGemvStreamMaxM][kGemvMaxBatch];
        int n[kGemvStreamMaxM] = {};
        for (int oi = 0; oi < count; ++oi) {
            const GemvArgs &a = args[order[oi]];
            if (a.group != group || a.M == 0 || a.N == 0)
                continue;
            if (!gemv_stream_takes(a.M, a.K, group))
                return hipErrorInvalidValue;
            idx[a.M - 1][n[a.M - 1]++] = order[oi];
        }
        for (int m = 0; m < kGemvStreamMaxM; ++m) {
            if (n[m] == 0)
                continue;
            const hipError_t e = launch_gemv_stream(args, idx[m], n[m], fp16, group, stream);
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
