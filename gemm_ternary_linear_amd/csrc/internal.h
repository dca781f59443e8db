// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ternary {

// Largest M the decode GEMV takes (two MFMA B columns per token, 16 columns).
constexpr int kGemvMaxM = 8;
// Most projections one fused decode launch takes.
constexpr int kGemvMaxBatch = 8;

// Scale granularity of a problem: 0 = one scale per output channel, else the
// group size along K (32, 64, 128 or 256; scales [N, K/group]).
inline bool group_valid(int64_t group)
{
    return group == 0 || group == 32 || group == 64 || group == 128 || group == 256;
}
inline int group_log2(int group) { return 31 - __builtin_clz((unsigned)group); }

// The decode GEMVs hand each token GEMV_COLS MFMA B columns, one per group of
// a 256-code slab (two halves for per-channel scales and groups of 128 or
// more), so a token takes 2, 4 or 8 of the 16 columns.
constexpr int gemv_cols(int group) { return group == 32 ? 8 : (group == 64 ? 4 : 2); }

// One decode GEMV problem (shapes already validated).
struct GemvArgs {
    const uint16_t *x;
    const uint8_t *packed;
    const uint16_t *scale;
    uint16_t *y;
    int M, N, K;
    int group;  // 0 (per channel) or the group size
    int tiled;  // codes in the tiled layout (else row-major [N, K/4])
};

// The tiled layout of an [N, K] code matrix (include/ternary.h): blocks of 16
// rows x 256 codes, 1 KB each, blocks of one row band consecutive.
constexpr int kTileRows = 16, kTileK = 256, kTileBytes = 1024;
inline int64_t tiled_slabs(int64_t K) { return (K + kTileK - 1) / kTileK; }
inline int64_t tiled_bytes(int64_t N, int64_t K)
{
    return (N + kTileRows - 1) / kTileRows * tiled_slabs(K) * kTileBytes;
}
// Row-major <-> tiled, one thread per 16 tiled bytes (pack.hip).
hipError_t launch_tile(const uint8_t *packed, int64_t N, int64_t K, uint8_t *tiled,
                       hipStream_t stream);
hipError_t launch_untile(const uint8_t *tiled, int64_t N, int64_t K, uint8_t *packed,
                         hipStream_t stream);

hipError_t launch_pack(const int8_t *q, int64_t nbytes, uint8_t *packed, int32_t *invalid_count,
                       hipStream_t stream);
hipError_t launch_unpack(const uint8_t *packed, int64_t nbytes, int8_t *q, hipStream_t stream);
// Codes and scales of 16-bit weights w [N, K] (`group` as in GemvArgs).
hipError_t launch_quantize(const uint16_t *w, bool fp16, int N, int K, int group, uint8_t *packed,
                           uint16_t *scale, hipStream_t stream);

// All linear launchers: x/y are 2-byte elements (bf16 or fp16 by `fp16`),
// `group` as in GemvArgs, shapes already validated by the caller.
// Which decode kernel runs a GEMV problem: AUTO takes the fp4 x fp8 one for
// M == 1 (the 16-bit one for a launch's lone one-token problem of fewer than
// 8192 channels and K > 8192) and the 16-bit one for larger M, each where it takes the
// shape, else the other; F4 and B16 force one (parity tests, tuning).
// Both read row-major and tiled codes.
enum class GemvKernel { AUTO, F4, B16 };
bool gemv_kernel_takes(GemvKernel k, int64_t M, int64_t K, int group, bool fp16,
                       bool tiled = false);
hipError_t launch_gemv(const uint16_t *x, bool fp16, int M, int N, int K, const uint8_t *packed,
                       const uint16_t *scale, int group, uint16_t *y, hipStream_t stream,
                       GemvKernel kernel = GemvKernel::AUTO, bool tiled = false);
// Up to kGemvMaxBatch decode problems (all taken by `kernel`), one launch per
// (kernel, scale mode, M) class.
hipError_t launch_gemv_batch(const GemvArgs *args, int count, bool fp16, hipStream_t stream,
                             GemvKernel kernel = GemvKernel::AUTO);
// Largest M the streaming decode kernel takes (M * gemv_cols(group) <= 16).
constexpr int kGemvStreamMaxM = 8;
// Whether the 16-bit streaming decode kernel (gemv_stream.hip) takes a shape.
bool gemv_stream_takes(int64_t M, int64_t K, int group);
// The problems args[order[0..count)] (all gemv_stream_takes(), one group
// value, one M) in one launch of the streaming decode kernel.
hipError_t launch_gemv_stream(const GemvArgs *args, const int *order, int count, bool fp16,
                              int group, hipStream_t stream);
// Decode GEMV on the scaled fp4 x fp8 matrix instruction (gemv_f4.hip):
// largest M, and the most dynamic LDS a workgroup may take (the activations of
// a problem live in LDS as fp8 pieces, 2 or 3 bytes per element and token).
constexpr int kGemvF4MaxM = 8;
constexpr int kGemvF4MaxLds = 80 * 1024;
// Whether the fp4 x fp8 decode kernel takes a shape (M <= 8, K % 128 == 0,
// the activation pieces fit in LDS).
bool gemv_f4_takes(int64_t M, int64_t K, int group, bool fp16);
// The problems args[order[0..count)] (all gemv_f4_takes(), one group value,
// one M) in one launch of the fp4 x fp8 decode kernel.
hipError_t launch_gemv_f4(const GemvArgs *args, const int *order, int count, bool fp16,
                          int group, hipStream_t stream);
// Decode GEMV on the vector ALU (gemv_valu.hip; a forced path only): M == 1,
// K % 256 == 0, per-channel scales or groups of 64, 128 or 256, row-major
// codes.
bool gemv_valu_takes(int64_t M, int64_t K, int group, bool tiled);
hipError_t launch_gemv_valu(const GemvArgs &a, bool fp16, hipStream_t stream);
// Few-token streaming GEMM (gemm_few.hip): 1 <= M <= kFewMaxM (16 for groups
// of 128), K % 256 == 0, K <= kGemvMaxK, per-channel scales or groups of 128
// (4-byte aligned scale array, K >= 1024) or 256; row-major and tiled codes.  One launch
// for up to kGemvMaxBatch problems that share the scale mode and the token
// tile (few_tile(M): 8, 16 or 32 tokens).
constexpr int kFewMaxM = 32;
inline int few_tile(int64_t M) { return M <= 8 ? 8 : (M <= 16 ? 16 : 32); }
bool gemm_few_takes(int64_t M, int64_t N, int64_t K, int group, const void *scale);
struct FixedScratch;
// K ranges long against the launch's other problems, or launches with few
// channel blocks, are sliced over workgroups: their fp32 sums go to `fixed`
// when given (it must hold gemm_few_scratch_need() bytes), else to the
// stream's workspace, and a second kernel adds the slices in order.
hipError_t launch_gemm_few(const GemvArgs *args, const int *order, int count, bool fp16,
                           hipStream_t stream, const struct FixedScratch *fixed = nullptr);
size_t gemm_few_scratch_need(const GemvArgs *args, const int *order, int count);
// Compute units of the current device (cached per device).
int device_cus();
// Tiled codes need the pipelined kernel (gemm_big_takes with tiled), and so
// does zero_skip (the pipelined kernel skipping a wave's all-zero steps).
hipError_t launch_gemm(const uint16_t *x, bool fp16, int M, int N, int K, const uint8_t *packed,
                       const uint16_t *scale, int group, uint16_t *y, hipStream_t stream,
                       bool tiled = false, bool zero_skip = false);
// Whether the pipelined (grouped) prefill kernel takes a problem (it reads
// row-major and tiled codes; the 128 x 128 kernel only row-major ones).
bool gemm_big_takes(int M, int N, int K, int group, const void *scale, bool tiled = false);
// A caller-provided scratch buffer for split-K partial tiles (device memory
// of `bytes` bytes), used instead of the per-stream workspace.
struct FixedScratch {
    void *ptr;
    size_t bytes;
};
// Up to kGemvMaxBatch prefill problems (all gemm_big_takes()) in one grouped
// launch per scale mode (plus one reduce launch per problem whose K range is
// split).  Split-K partials go to `fixed` if given (it must hold
// gemm_batch_scratch_need() bytes), else to the stream's workspace.
hipError_t launch_gemm_batch(const GemvArgs *args, int count, bool fp16, hipStream_t stream,
                             const FixedScratch *fixed = nullptr, bool zero_skip = false);
// Scratch bytes launch_gemm_batch needs for these problems (0: no K split)
// when its fixed scratch holds `cap` bytes (work-balanced K slices that would
// not fit are left out).
size_t gemm_batch_scratch_need(const GemvArgs *args, int count, size_t cap);

// Library-owned scratch of at least `bytes` for work on `stream` of the
// current device.  While `stream` is being captured nothing is allocated: a
// stream without a workspace that large returns kErrCaptureWorkspace.  A
// workspace replaced by a larger one stays allocated until
// release_workspaces() (a graph captured earlier may still use it).
hipError_t stream_workspace(hipStream_t stream, size_t bytes, void **out);
// The error stream_workspace() returns under capture when the stream's
// workspace is too small (reported as TERNARY_ERR_WORKSPACE).
constexpr hipError_t kErrCaptureWorkspace = hipErrorStreamCaptureUnsupported;
// Frees every workspace, retired ones included, after waiting for the
// devices that hold them.
hipError_t release_workspaces();

// The allocation-free variant's scratch (noalloc.hip): the device address of
// this device's copy of the library's static scratch array (looked up once per
// device), and its size.
hipError_t noalloc_scratch(void **out);
size_t noalloc_scratch_bytes();

hipError_t launch_simple(const uint16_t *x, bool fp16, int M, int N, int K, const uint8_t *packed,
                         const uint16_t *scale, int group, uint16_t *y, hipStream_t stream,
                         bool tiled = false);

// Shape requirements of the fast kernels.  The decode kernels take K up to
// 65536 (a multiple of 128).
constexpr int64_t kGemvMaxK = 65536;
inline bool gemm_takes(int64_t M, int64_t K, int group)
{
    return M >= 1 && K % 128 == 0 && (group == 0 || K % group == 0);
}
// The automatic GEMV/GEMM choice, the same for both activation dtypes: the
// decode GEMV wherever one of its kernels takes the shape (fp16 activations
// need the most LDS in the fp4 x fp8 kernel).  Measured on MI355X, the decode
// kernels beat the GEMM at every M <= 8 they take (7B down 4096 x 18944 at
// M = 8: GEMV 12.8 us, pipelined GEMM with split K 23.7 us).
inline bool gemv_preferred(int64_t M, int64_t K, int group)
{
    return gemv_kernel_takes(GemvKernel::AUTO, M, K, group, true);
}

}  // namespace ternary
