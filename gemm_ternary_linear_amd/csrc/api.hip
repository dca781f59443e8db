// C ABI of the ternary linear layer (declared in include/ternary.h).
//
// Host-side argument validation, then an asynchronous launch on the caller's
// stream.  Validation never dereferences a pointer and never calls HIP, so an
// invalid call returns its status without touching the device.
#include <stdint.h>

#include "../../include/ternary.h"
#include "internal.h"

#include <algorithm>

namespace {

constexpr int kAbiVersion = 7;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges; empty ranges never overlap).
bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    if (na <= 0 || nb <= 0)
        return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return TERNARY_OK;
    return e == ternary::kErrCaptureWorkspace ? TERNARY_ERR_WORKSPACE : TERNARY_ERR_HIP;
}

// Largest M, N or K accepted: kernels index channels, tokens and K with
// 32-bit ints (element offsets are 64-bit) and grids stay far inside the
// launch limits.
constexpr int64_t kMaxDim = (int64_t)1 << 24;

// The library's group value of a group_size (-1 -> 0), or -1 if unsupported.
int group_of(int64_t group_size)
{
    if (group_size == -1)
        return 0;
    return group_size > 0 && ternary::group_valid(group_size) ? (int)group_size : -1;
}

// Scale elements of one problem.
int64_t scale_elems(int64_t N, int64_t K, int64_t group_size)
{
    return group_size == -1 ? N : N * (K / group_size);
}

int check_shape(int64_t M, int64_t N, int64_t K, int64_t group_size)
{
    if (group_of(group_size) < 0)
        return TERNARY_ERR_GROUP;
    if (M < 0 || N < 0 || K <= 0 || K % 4 != 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return TERNARY_ERR_SHAPE;
    if (group_size > 0 && K % group_size != 0)
        return TERNARY_ERR_SHAPE;
    return TERNARY_OK;
}

// Bytes of a problem's codes in its layout.
int64_t code_bytes(int64_t N, int64_t K, bool tiled)
{
    return tiled ? ternary::tiled_bytes(N, K) : N * (K / 4);
}

int check_linear(const void *x, int dtype, int64_t M, int64_t N, int64_t K, const uint8_t *packed,
                 const uint16_t *scale, int64_t group_size, const void *y, bool tiled = false)
{
    if (dtype != TERNARY_BF16 && dtype != TERNARY_FP16)
        return TERNARY_ERR_DTYPE;
    const int sh = check_shape(M, N, K, group_size);
    if (sh != TERNARY_OK)
        return sh;
    if (M == 0 || N == 0)
        return TERNARY_OK;
    if (!x || !packed || !scale || !y)
        return TERNARY_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(packed, 16) || !aligned(scale, 2))
        return TERNARY_ERR_ALIGN;
    const int64_t ybytes = 2 * M * N;
    const int64_t sbytes = 2 * scale_elems(N, K, group_size);
    if (overlap(y, ybytes, x, 2 * M * K) || overlap(y, ybytes, packed, code_bytes(N, K, tiled)) ||
        overlap(y, ybytes, scale, sbytes))
        return TERNARY_ERR_ALIAS;
    return TERNARY_OK;
}

// Whether the automatic choice gives a problem to the few-token GEMM: the
// token counts just past the decode GEMV (9 .. 32, groups of 128 up to 16),
// where it runs every measured shape faster than the GEMM.
bool few_preferred(int64_t M, int64_t N, int64_t K, int group, const void *scale)
{
    return M > ternary::kGemvMaxM && ternary::gemm_few_takes(M, N, K, group, scale);
}

int select_path(int64_t M, int64_t N, int64_t K, int group, const void *scale)
{
    if (ternary::gemv_preferred(M, K, group))
        return TERNARY_PATH_GEMV;
    if (few_preferred(M, N, K, group, scale))
        return TERNARY_PATH_FEW;
    if (ternary::gemm_takes(M, K, group))
        return TERNARY_PATH_GEMM;
    return TERNARY_PATH_SIMPLE;
}

// The automatic choice for tiled codes: the decode GEMV as for row-major
// codes, else the pipelined GEMM (the 128 x 128 kernel reads row-major codes
// only), else the plain kernel.
int select_path_tiled(int64_t M, int64_t N, int64_t K, int group, const void *scale)
{
    if (ternary::gemv_preferred(M, K, group))
        return TERNARY_PATH_GEMV;
    if (few_preferred(M, N, K, group, scale))
        return TERNARY_PATH_FEW;
    if (ternary::gemm_big_takes((int)M, (int)N, (int)K, group, scale, true))
        return TERNARY_PATH_GEMM;
    return TERNARY_PATH_SIMPLE;
}

// One linear problem after validation: path choice (AUTO or forced) and launch.
int linear_one(const void *x, int dtype, int64_t M, int64_t N, int64_t K, const uint8_t *packed,
               const uint16_t *scale, int64_t group_size, void *y, int path, bool tiled,
               hipStream_t stream)
{
    const int group = group_of(group_size);
    const bool fp16 = dtype == TERNARY_FP16;
    if (path == TERNARY_PATH_AUTO)
        path = tiled ? select_path_tiled(M, N, K, group, scale) : select_path(M, N, K, group, scale);
    ternary::GemvKernel gk = ternary::GemvKernel::AUTO;
    switch (path) {
    case TERNARY_PATH_GEMV_F4:
    case TERNARY_PATH_GEMV_B16:
    case TERNARY_PATH_GEMV:
        gk = path == TERNARY_PATH_GEMV_F4 ? ternary::GemvKernel::F4
             : path == TERNARY_PATH_GEMV_B16 ? ternary::GemvKernel::B16
                                             : ternary::GemvKernel::AUTO;
        if (!(M == 0 || N == 0 || ternary::gemv_kernel_takes(gk, M, K, group, fp16, tiled)))
            return TERNARY_ERR_PATH;
        path = TERNARY_PATH_GEMV;
        break;
    case TERNARY_PATH_GEMM:
        if (!(M == 0 || N == 0 ||
              (tiled ? ternary::gemm_big_takes((int)M, (int)N, (int)K, group, scale, true)
                     : ternary::gemm_takes(M, K, group))))
            return TERNARY_ERR_PATH;
        break;
    case TERNARY_PATH_SIMPLE: break;
    case TERNARY_PATH_GEMV_VALU:
        if (!(M == 0 || N == 0 || ternary::gemv_valu_takes(M, K, group, tiled)))
            return TERNARY_ERR_PATH;
        break;
    case TERNARY_PATH_FEW:
        if (!(M == 0 || N == 0 || ternary::gemm_few_takes(M, N, K, group, scale)))
            return TERNARY_ERR_PATH;
        break;
    case TERNARY_PATH_GEMM_ZSKIP:
        if (!(M == 0 || N == 0 ||
              ternary::gemm_big_takes((int)M, (int)N, (int)K, group, scale, tiled)))
            return TERNARY_ERR_PATH;
        break;
    default: return TERNARY_ERR_PATH;
    }
    if (M == 0 || N == 0)
        return TERNARY_OK;
    const uint16_t *xv = static_cast<const uint16_t *>(x);
    uint16_t *yv = static_cast<uint16_t *>(y);
    hipError_t e;
    switch (path) {
    case TERNARY_PATH_GEMV:
        e = ternary::launch_gemv(xv, fp16, (int)M, (int)N, (int)K, packed, scale, group, yv, stream,
                                 gk, tiled);
        break;
    case TERNARY_PATH_GEMM:
        e = ternary::launch_gemm(xv, fp16, (int)M, (int)N, (int)K, packed, scale, group, yv, stream,
                                 tiled);
        break;
    case TERNARY_PATH_GEMV_VALU: {
        const ternary::GemvArgs a = {xv, packed, scale, yv, (int)M, (int)N, (int)K, group,
                                     tiled ? 1 : 0};
        e = ternary::launch_gemv_valu(a, fp16, stream);
        break;
    }
    case TERNARY_PATH_FEW: {
        const ternary::GemvArgs a = {xv, packed, scale, yv, (int)M, (int)N, (int)K, group,
                                     tiled ? 1 : 0};
        const int order = 0;
        e = ternary::launch_gemm_few(&a, &order, 1, fp16, stream);
        break;
    }
    case TERNARY_PATH_GEMM_ZSKIP:
        e = ternary::launch_gemm(xv, fp16, (int)M, (int)N, (int)K, packed, scale, group, yv, stream,
                                 tiled, true);
        break;
    default:
        e = ternary::launch_simple(xv, fp16, (int)M, (int)N, (int)K, packed, scale, group, yv,
                                   stream, tiled);
        break;
    }
    return hip_status(e);
}

// Shape checks of ternary_tile / ternary_untile (and the size they imply).
int check_tile_shape(int64_t N, int64_t K)
{
    if (N < 0 || K < 0 || K % 4 != 0 || N > kMaxDim || K > kMaxDim)
        return TERNARY_ERR_SHAPE;
    // one thread per 16 bytes, grids below 2^32 workgroups
    if (ternary::tiled_bytes(N, K) > ((int64_t)1 << 40))
        return TERNARY_ERR_SHAPE;
    return TERNARY_OK;
}

}  // namespace

namespace ternary {

int linear_batch(const ternary_problem *problems, int count, int dtype, hipStream_t stream,
                 bool noalloc)
{
    if (count < 1 || count > TERNARY_MAX_BATCH)
        return TERNARY_ERR_SHAPE;
    if (!problems)
        return TERNARY_ERR_NULL;
    for (int i = 0; i < count; ++i) {
        const ternary_problem &p = problems[i];
        if (p.layout != TERNARY_LAYOUT_ROWS && p.layout != TERNARY_LAYOUT_TILED)
            return TERNARY_ERR_SHAPE;
        const int st = check_linear(p.x, dtype, p.M, p.N, p.K, p.packed, p.scale, p.group_size, p.y,
                                    p.layout == TERNARY_LAYOUT_TILED);
        if (st != TERNARY_OK)
            return st;
    }
    // No output may overlap another problem's inputs or output.
    for (int i = 0; i < count; ++i) {
        const ternary_problem &a = problems[i];
        const int64_t ya = 2 * a.M * a.N;
        for (int j = 0; j < count; ++j) {
            if (i == j)
                continue;
            const ternary_problem &b = problems[j];
            const int64_t sb = 2 * scale_elems(b.N, b.K, b.group_size);
            if (overlap(a.y, ya, b.x, 2 * b.M * b.K) ||
                overlap(a.y, ya, b.packed, code_bytes(b.N, b.K, b.layout == TERNARY_LAYOUT_TILED)) ||
                overlap(a.y, ya, b.scale, sb) ||
                overlap(a.y, ya, b.y, 2 * b.M * b.N))
                return TERNARY_ERR_ALIAS;
        }
    }
    // Plan every launch before the first one: decode problems fused, the
    // pipelined GEMM's problems grouped, the rest one call each.
    const bool fp16 = dtype == TERNARY_FP16;
    GemvArgs fused[TERNARY_MAX_BATCH], grouped_gemm[TERNARY_MAX_BATCH], few[TERNARY_MAX_BATCH];
    int others[TERNARY_MAX_BATCH];
    int nf = 0, ng = 0, no = 0, nw = 0;
    for (int i = 0; i < count; ++i) {
        const ternary_problem &p = problems[i];
        if (p.M == 0 || p.N == 0)
            continue;
        const bool tiled = p.layout == TERNARY_LAYOUT_TILED;
        const GemvArgs a = {static_cast<const uint16_t *>(p.x), p.packed, p.scale,
                            static_cast<uint16_t *>(p.y), (int)p.M, (int)p.N, (int)p.K,
                            group_of(p.group_size), tiled ? 1 : 0};
        if (gemv_kernel_takes(GemvKernel::AUTO, p.M, p.K, a.group, fp16, tiled))
            fused[nf++] = a;
        else if (few_preferred(p.M, p.N, p.K, a.group, a.scale))
            few[nw++] = a;
        else if (gemm_takes(p.M, p.K, a.group) &&
                 gemm_big_takes(a.M, a.N, a.K, a.group, a.scale, tiled))
            grouped_gemm[ng++] = a;
        else
            others[no++] = i;
    }
    // Few-token problems: one launch per scale mode and token tile, longest K
    // first.
    int few_order[TERNARY_MAX_BATCH], few_first[TERNARY_MAX_BATCH + 1], nfl = 0;
    {
        int n = 0;
        for (const int group : {0, 128, 256})
        for (const int tile : {8, 16, 32}) {
            const int first = n;
            for (int i = 0; i < nw; ++i)
                if (few[i].group == group && few_tile(few[i].M) == tile)
                    few_order[n++] = i;
            for (int i = first + 1; i < n; ++i)  // stable insertion sort, K descending
                for (int j = i; j > first && few[few_order[j]].K > few[few_order[j - 1]].K; --j)
                    std::swap(few_order[j], few_order[j - 1]);
            if (n > first)
                few_first[nfl++] = first;
        }
        few_first[nfl] = n;
    }
    FixedScratch fs = {nullptr, 0};
    if (noalloc) {
        // split-K partials go to the library's static scratch (one launch
        // after another on the stream): check its size before anything is
        // enqueued
        size_t need = ng ? gemm_batch_scratch_need(grouped_gemm, ng, noalloc_scratch_bytes()) : 0;
        for (int l = 0; l < nfl; ++l)
            need = std::max(need, gemm_few_scratch_need(few, few_order + few_first[l],
                                                        few_first[l + 1] - few_first[l]));
        if (need > noalloc_scratch_bytes())
            return TERNARY_ERR_SCRATCH;
        const int st = hip_status(noalloc_scratch(&fs.ptr));
        if (st != TERNARY_OK)
            return st;
        fs.bytes = noalloc_scratch_bytes();
    }
    for (int oi = 0; oi < no; ++oi) {
        // (the 128 x 128 GEMM and the plain kernel use no scratch)
        const ternary_problem &p = problems[others[oi]];
        const int st = linear_one(p.x, dtype, p.M, p.N, p.K, p.packed, p.scale, p.group_size, p.y,
                                  TERNARY_PATH_AUTO, p.layout == TERNARY_LAYOUT_TILED, stream);
        if (st != TERNARY_OK)
            return st;
    }
    if (ng) {
        const int st = hip_status(launch_gemm_batch(grouped_gemm, ng, fp16, stream,
                                                    noalloc ? &fs : nullptr));
        if (st != TERNARY_OK)
            return st;
    }
    for (int l = 0; l < nfl; ++l) {
        const int st = hip_status(launch_gemm_few(few, few_order + few_first[l],
                                                  few_first[l + 1] - few_first[l], fp16, stream,
                                                  noalloc ? &fs : nullptr));
        if (st != TERNARY_OK)
            return st;
    }
    if (nf)
        return hip_status(launch_gemv_batch(fused, nf, fp16, stream));
    return TERNARY_OK;
}

}  // namespace ternary

extern "C" {

int ternary_abi_version(void) { return kAbiVersion; }

int ternary_shutdown(void)
{
    return ternary::release_workspaces() == hipSuccess ? TERNARY_OK : TERNARY_ERR_HIP;
}

int ternary_gemv_max_m(void) { return ternary::kGemvMaxM; }

const char *ternary_status_string(int status)
{
    switch (status) {
    case TERNARY_OK: return "ok";
    case TERNARY_ERR_NULL: return "null pointer argument";
    case TERNARY_ERR_SHAPE: return "invalid shape (negative size, K % 4 != 0, or K not a multiple of the group size)";
    case TERNARY_ERR_GROUP: return "group_size must be -1 (per channel), 32, 64, 128 or 256";
    case TERNARY_ERR_DTYPE: return "activation dtype must be TERNARY_BF16 or TERNARY_FP16";
    case TERNARY_ERR_ALIGN: return "pointer not aligned (data 16 bytes, scale 2 bytes)";
    case TERNARY_ERR_ALIAS: return "output overlaps an input";
    case TERNARY_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case TERNARY_ERR_PATH: return "forced kernel path cannot take this shape";
    case TERNARY_ERR_WORKSPACE:
        return "the stream is being captured and its split-K workspace is too small: run the same "
               "call once outside capture first";
    case TERNARY_ERR_SCRATCH:
        return "the call needs more split-K scratch than the library's static buffer holds";
    default: return "unknown status";
    }
}

int ternary_pack(const int8_t *q, int64_t N, int64_t K, uint8_t *packed, int32_t *invalid_count,
                 hipStream_t stream)
{
    if (N < 0 || K < 0 || K % 4 != 0)
        return TERNARY_ERR_SHAPE;
    if (N == 0 || K == 0)
        return TERNARY_OK;
    if (N > INT64_MAX / K)
        return TERNARY_ERR_SHAPE;
    if (!q || !packed)
        return TERNARY_ERR_NULL;
    if (!aligned(q, 16) || !aligned(packed, 16) || !aligned(invalid_count, 4))
        return TERNARY_ERR_ALIGN;
    const int64_t nbytes = N * (K / 4);
    if (overlap(packed, nbytes, q, N * K) || overlap(invalid_count, 4, q, N * K) ||
        overlap(invalid_count, 4, packed, nbytes))
        return TERNARY_ERR_ALIAS;
    return hip_status(ternary::launch_pack(q, nbytes, packed, invalid_count, stream));
}

int ternary_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *q, hipStream_t stream)
{
    if (N < 0 || K < 0 || K % 4 != 0)
        return TERNARY_ERR_SHAPE;
    if (N == 0 || K == 0)
        return TERNARY_OK;
    if (N > INT64_MAX / K)
        return TERNARY_ERR_SHAPE;
    if (!q || !packed)
        return TERNARY_ERR_NULL;
    if (!aligned(q, 16) || !aligned(packed, 16))
        return TERNARY_ERR_ALIGN;
    const int64_t nbytes = N * (K / 4);
    if (overlap(packed, nbytes, q, N * K))
        return TERNARY_ERR_ALIAS;
    return hip_status(ternary::launch_unpack(packed, nbytes, q, stream));
}

int ternary_quantize(const void *w, int dtype, int64_t N, int64_t K, int64_t group_size,
                     uint8_t *packed, uint16_t *scale, hipStream_t stream)
{
    if (dtype != TERNARY_BF16 && dtype != TERNARY_FP16)
        return TERNARY_ERR_DTYPE;
    const int sh = check_shape(0, N, K, group_size);
    if (sh != TERNARY_OK)
        return sh;
    if (N == 0)
        return TERNARY_OK;
    if (!w || !packed || !scale)
        return TERNARY_ERR_NULL;
    if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scale, 2))
        return TERNARY_ERR_ALIGN;
    const int64_t wbytes = 2 * N * K, pbytes = N * (K / 4),
                  sbytes = 2 * scale_elems(N, K, group_size);
    if (overlap(packed, pbytes, w, wbytes) || overlap(scale, sbytes, w, wbytes) ||
        overlap(scale, sbytes, packed, pbytes))
        return TERNARY_ERR_ALIAS;
    return hip_status(ternary::launch_quantize(static_cast<const uint16_t *>(w),
                                               dtype == TERNARY_FP16, (int)N, (int)K,
                                               group_of(group_size), packed, scale, stream));
}

int ternary_select_path(int64_t M, int64_t N, int64_t K, int64_t group_size)
{
    const int sh = check_shape(M, N, K, group_size);
    if (sh != TERNARY_OK)
        return sh;
    // (the few-token GEMM's group-128 scale alignment is assumed met)
    return select_path(M, N, K, group_of(group_size), reinterpret_cast<const void *>(16));
}

int ternary_linear_ex(const void *x, int dtype, int64_t M, int64_t N, int64_t K,
                      const uint8_t *packed, const uint16_t *scale, int64_t group_size, void *y,
                      int path, hipStream_t stream)
{
    const int st = check_linear(x, dtype, M, N, K, packed, scale, group_size, y);
    if (st != TERNARY_OK)
        return st;
    return linear_one(x, dtype, M, N, K, packed, scale, group_size, y, path, false, stream);
}

int ternary_linear_tiled(const void *x, int dtype, int64_t M, int64_t N, int64_t K,
                         const uint8_t *tiled, const uint16_t *scale, int64_t group_size, void *y,
                         int path, hipStream_t stream)
{
    const int st = check_linear(x, dtype, M, N, K, tiled, scale, group_size, y, true);
    if (st != TERNARY_OK)
        return st;
    return linear_one(x, dtype, M, N, K, tiled, scale, group_size, y, path, true, stream);
}

int64_t ternary_tiled_bytes(int64_t N, int64_t K)
{
    const int st = check_tile_shape(N, K);
    return st != TERNARY_OK ? st : ternary::tiled_bytes(N, K);
}

int ternary_tile(const uint8_t *packed, int64_t N, int64_t K, uint8_t *tiled, hipStream_t stream)
{
    const int st = check_tile_shape(N, K);
    if (st != TERNARY_OK)
        return st;
    if (N == 0 || K == 0)
        return TERNARY_OK;
    if (!packed || !tiled)
        return TERNARY_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(tiled, 16))
        return TERNARY_ERR_ALIGN;
    if (overlap(tiled, ternary::tiled_bytes(N, K), packed, N * (K / 4)))
        return TERNARY_ERR_ALIAS;
    return hip_status(ternary::launch_tile(packed, N, K, tiled, stream));
}

int ternary_untile(const uint8_t *tiled, int64_t N, int64_t K, uint8_t *packed, hipStream_t stream)
{
    const int st = check_tile_shape(N, K);
    if (st != TERNARY_OK)
        return st;
    if (N == 0 || K == 0)
        return TERNARY_OK;
    if (!packed || !tiled)
        return TERNARY_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(tiled, 16))
        return TERNARY_ERR_ALIGN;
    if (overlap(tiled, ternary::tiled_bytes(N, K), packed, N * (K / 4)))
        return TERNARY_ERR_ALIAS;
    return hip_status(ternary::launch_untile(tiled, N, K, packed, stream));
}

int ternary_linear_batch(const ternary_problem *problems, int count, int dtype,
                         hipStream_t stream)
{
    return ternary::linear_batch(problems, count, dtype, stream, false);
}

int ternary_linear(const void *x, int dtype, int64_t M, int64_t N, int64_t K,
                   const uint8_t *packed, const uint16_t *scale, int64_t group_size, void *y,
                   hipStream_t stream)
{
    return ternary_linear_ex(x, dtype, M, N, K, packed, scale, group_size, y, TERNARY_PATH_AUTO,
                             stream);
}

}  // extern "C"
