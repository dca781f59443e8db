/*
 * ternary.h - C ABI of the MI355X (gfx950) ternary-weight linear layer.
 *
 *     y[m,n] = sum_k x[m,k] * q[n,k] * s(n,k)          (y = x * (q (.) s)^T)
 *
 * Sources (page titles and sections):
 *   [trdm] trdm.cn, "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战":
 *          §3.1 packing rule; §4.2 operand shapes; §4.4 2-D contiguous input.
 *   [nxbn] m.nxbn.cn/news/169761 (a 7B ternary checkpoint into vLLM):
 *          §2.2 code table and bit order; §3.2 per-channel scale broadcast
 *          over rows; §5.2 the layer's forward takes (x, weight, scale).
 *   [xxqk] m.xxqk.cn/news/593501 (Bonsai 2 27B into vLLM): §4.3 the layer is
 *          dequantise-then-matmul; §4.2/§5.2 checkpoints grouped by 64.
 *   [ch13] yangyitao.com vLLM book, "第13章 量化：精度与速度的工程平衡":
 *          §13.1.3 symmetric linear quantization; §13.1.4 its s/2 error
 *          bound; §13.3 scale granularity (per channel, per group; §13.3.3 group
 *          sizes 128, 32, 256); §13.8.2 group_size = -1 means one group per
 *          row.
 *
 * Format (fixed by [trdm §3.1] and [nxbn §2.2]):
 *   - each weight is a 2-bit code: 00 -> 0, 01 -> +1, 10 -> -1, 11 -> reserved,
 *     read as 0 by every function here and never written by ternary_pack;
 *   - four codes per byte, little-endian: weight 4j+i of a row lives in bits
 *     [2i+1:2i] of byte j of that row;
 *   - packed weights are [N, K/4] bytes, row-major (one row per output channel,
 *     K contiguous);
 *   - scales are IEEE binary16 bit patterns: [N] when group_size == -1 (one per
 *     output channel, [nxbn §3.2]) or [N, K/g] row-major when group_size == g
 *     (g consecutive K weights of a row share one: g = 128 in [trdm §3.1], 64
 *     in [xxqk §4.2], 32 and 256 in [ch13 §13.3.3]).
 *
 * Tiled layout (this library's, not the pages'; TERNARY_LAYOUT_TILED): the same
 * bytes as the row-major packing, permuted so that the matrix-core kernels read
 * one contiguous kilobyte per wave instruction.  Rows are padded to a multiple
 * of 16 and K to a multiple of 256 with code 00; with Ks = ceil(K / 256), byte
 * j of row n of the row-major packing (j < K/4) sits at
 *     ((n / 16) * Ks + j / 64) * 1024 + ((j % 64) / 16) * 256 + (n % 16) * 16 + j % 16
 * i.e. block (n/16, j/64) of 16 rows x 64 bytes is 1 KB, stored as four
 * [16 rows][16 bytes] quarters in K order.  ternary_tiled_bytes() gives the
 * size, ternary_tile()/ternary_untile() convert; every linear entry point that
 * takes a layout reads either.
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers, owned by the caller.  The library
 *     keeps no reference after a call returns and never allocates or frees
 *     caller memory.
 *   - The library owns one device workspace per (device, stream) for GEMM
 *     shapes whose K range it splits over several workgroups (fp32 partial
 *     tiles, added in a fixed order by a second kernel): shapes with few
 *     output tiles, few-token shapes with long K, and batches in which one
 *     problem's K is much longer than the others'.  The first call on a
 *     stream that needs a larger one allocates it (hipMalloc); the one it
 *     replaces stays allocated (a graph captured earlier may use it) until
 *     ternary_shutdown(), which frees them all.  Under stream capture nothing
 *     is allocated: a call that would need a larger workspace returns
 *     TERNARY_ERR_WORKSPACE, so warm a stream up (one call per shape) before
 *     capturing on it.  ternary_linear_batch_noalloc allocates nothing.
 *   - Work is enqueued asynchronously on `stream` (NULL = the default stream).
 *     Arguments are validated on the host before anything is launched; on any
 *     error a negative ternary_status is returned and nothing is enqueued.
 *     Faults during execution surface at the next synchronisation of the
 *     stream, as for any HIP kernel.
 *   - Every call is deterministic: the same inputs give the same bits.
 *   - No function throws; C++ exceptions never cross this boundary.
 */
#ifndef TERNARY_LINEAR_H
#define TERNARY_LINEAR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TERNARY_OK = 0,
    TERNARY_ERR_NULL = -1,   /* a required pointer is NULL                       */
    TERNARY_ERR_SHAPE = -2,  /* negative size, K % 4 != 0, K % group != 0, ...   */
    TERNARY_ERR_GROUP = -3,  /* group_size is not -1, 32, 64, 128 or 256         */
    TERNARY_ERR_DTYPE = -4,  /* activation dtype is not TERNARY_BF16/TERNARY_FP16*/
    TERNARY_ERR_ALIGN = -5,  /* a pointer is not aligned as documented           */
    TERNARY_ERR_ALIAS = -6,  /* the output overlaps an input                     */
    TERNARY_ERR_HIP = -7,    /* a HIP runtime call or kernel launch failed       */
    TERNARY_ERR_PATH = -8,   /* a forced kernel path cannot take this shape      */
    TERNARY_ERR_WORKSPACE = -9, /* stream under capture, its split-K workspace too
                                   small: run the same call once outside capture */
    TERNARY_ERR_SCRATCH = -10   /* ternary_linear_batch_noalloc: the call needs more
                                   split-K scratch than TERNARY_NOALLOC_SCRATCH_BYTES */
} ternary_status;

/* Weight layout of a linear call (see "Tiled layout" above). */
typedef enum { TERNARY_LAYOUT_ROWS = 0, TERNARY_LAYOUT_TILED = 1 } ternary_layout;

/* Activation / output element type (2 bytes per element). */
typedef enum { TERNARY_BF16 = 0, TERNARY_FP16 = 1 } ternary_dtype;

/* Kernel path for ternary_linear_ex.  AUTO picks by M (see ternary_linear). */
typedef enum {
    TERNARY_PATH_AUTO = 0,
    TERNARY_PATH_GEMV = 1,     /* decode GEMV, requires 1 <= M <= ternary_gemv_max_m();
                                  at M == 1 the fp4 x fp8 kernel (a single call of
                                  fewer than 8192 channels and K > 8192: the
                                  16-bit one), at
                                  larger M the 16-bit one, each where it takes the
                                  shape, else the other                                */
    TERNARY_PATH_GEMM = 2,     /* prefill kernel (bf16/fp16 MFMA)                       */
    TERNARY_PATH_SIMPLE = 3,   /* plain one-output-per-thread kernel, any valid shape   */
    TERNARY_PATH_GEMV_F4 = 4,  /* decode GEMV on the scaled fp4 x fp8 matrix
                                  instruction (codes as fp4, x as exact fp8 pieces)     */
    TERNARY_PATH_GEMV_B16 = 5, /* decode GEMV on the bf16/fp16 matrix instruction
                                  (codes as 16-bit +-2 / 0)                            */
    TERNARY_PATH_GEMV_VALU = 6, /* decode GEMV on the vector ALU: each code adds +x, -x
                                  or nothing in fp32 ([nxbn §4.1]), lanes reduced by
                                  cross-lane exchange; M == 1, K % 256 == 0, per
                                  channel or groups of 64/128/256, row-major codes
                                  only.  Never chosen by AUTO (measured slower); kept
                                  for comparison                                        */
    TERNARY_PATH_FEW = 7,      /* few-token streaming GEMM: 1 <= M <= 32 (16 for groups
                                  of 128), K % 256 == 0, K <= 65536 (groups of 128:
                                  K >= 1024), per channel or groups of 128 / 256; x
                                  shared in LDS by the eight 16-channel blocks of a
                                  workgroup, codes streamed into registers             */
    TERNARY_PATH_GEMM_ZSKIP = 8 /* the pipelined GEMM skipping all-zero code blocks
                                  ([trdm §6]; a wave's channels x 64 K): the shapes
                                  TERNARY_PATH_GEMM takes on the pipelined kernel
                                  (K % 256 == 0, ...); the same bits as that path.
                                  Pays only on block-sparse codes; never chosen by
                                  AUTO                                                 */
} ternary_path;

/*
 * ternary_pack - encode ternary values as 2-bit codes ([trdm §3.1]).
 *   q             int8 [N, K], row-major, values in {-1, 0, +1}; 16-byte aligned.
 *   N, K          N >= 0, K >= 0, K % 4 == 0.
 *   packed        uint8 [N, K/4] output, 16-byte aligned, must not overlap q.
 *   invalid_count optional int32 (device).  Each value outside {-1, 0, +1} is
 *                 written as code 00 and counted; the count is ADDED to
 *                 *invalid_count (the caller zeroes it).  NULL skips counting.
 * N == 0 or K == 0 is a successful no-op.
 */
int ternary_pack(const int8_t *q, int64_t N, int64_t K, uint8_t *packed,
                 int32_t *invalid_count, hipStream_t stream);

/*
 * ternary_unpack - decode 2-bit codes to int8 {-1, 0, +1} ([trdm §3.1],
 * [nxbn §2.2]); code 11 decodes to 0.  Bit-exact inverse of ternary_pack for
 * bytes that hold no code 11.
 *   packed  uint8 [N, K/4], 16-byte aligned.
 *   q       int8 [N, K] output, 16-byte aligned, must not overlap packed.
 */
int ternary_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *q, hipStream_t stream);

/*
 * ternary_tiled_bytes - size in bytes of the tiled layout of an [N, K] code
 * matrix: ceil(N/16) * 16 * ceil(K/256) * 64.  Returns TERNARY_ERR_SHAPE for
 * N < 0, K < 0, K % 4 != 0, N or K above 2^24, or more than 2^40 bytes (the
 * limits of ternary_tile / ternary_untile as well).
 */
int64_t ternary_tiled_bytes(int64_t N, int64_t K);

/*
 * ternary_tile - row-major packed codes -> tiled layout (a byte permutation;
 * padding bytes are written as 0).
 *   packed  uint8 [N, K/4], 16-byte aligned.
 *   tiled   uint8 [ternary_tiled_bytes(N, K)] output, 16-byte aligned, must not
 *           overlap packed.
 * N == 0 or K == 0 is a successful no-op.  ternary_untile is the inverse
 * (same arguments, tiled -> packed; padding bytes are not read).
 */
int ternary_tile(const uint8_t *packed, int64_t N, int64_t K, uint8_t *tiled,
                 hipStream_t stream);
int ternary_untile(const uint8_t *tiled, int64_t N, int64_t K, uint8_t *packed,
                   hipStream_t stream);

/*
 * ternary_quantize - codes and scales of 16-bit weights (the step before the
 * layer: its packed and scale inputs).
 *   w           [N, K] weights, dtype `dtype` (TERNARY_BF16 or TERNARY_FP16),
 *               row-major, 16-byte aligned.
 *   N, K        N >= 0, K > 0, K % 4 == 0, K % group_size == 0 when grouped;
 *               N == 0 is a successful no-op.
 *   group_size  -1 (one scale per row) or 32, 64, 128, 256.
 *   packed      uint8 [N, K/4] output, 16-byte aligned.
 *   scale       fp16 [N] or [N, K/group_size] output, 2-byte aligned.
 * No output may overlap w or the other output.  Rule: the symmetric linear
 * quantizer of [ch13 §13.1.3] with the code range {-1, 0, +1}: per group,
 * s = max |w| rounded to fp16 (nearest even), and q = round(w / s) with ties
 * to even, i.e. q = sign(w) where |w| > s/2 and 0 elsewhere; a group with
 * s == 0 gets q = 0.  Then |w - q*s| <= s/2 for every weight ([ch13 §13.1.4]).
 * w must be finite with every group's max |w| below 65520 (s finite in
 * fp16); results are unspecified otherwise.  Deterministic, bit-exact.
 */
int ternary_quantize(const void *w, int dtype, int64_t N, int64_t K, int64_t group_size,
                     uint8_t *packed, uint16_t *scale, hipStream_t stream);

/*
 * ternary_linear - y = x * (q (.) s)^T ([xxqk §4.3]; operand shapes [trdm §4.2]).
 *   x           [M, K] activations, dtype `dtype`, row-major contiguous
 *               ([trdm §4.4]: callers flatten leading dims to M), 16-byte aligned.
 *   dtype       TERNARY_BF16 or TERNARY_FP16; y has the same dtype.
 *   M, N, K     M >= 0, N >= 0, K > 0, K % 4 == 0; K % group_size == 0 when
 *               grouped.  M == 0 or N == 0 is a successful no-op.
 *   packed      uint8 [N, K/4] codes as above, 16-byte aligned.
 *   scale       fp16 bit patterns, [N] (group_size == -1) or [N, K/group_size]
 *               (grouped), 2-byte aligned.
 *   group_size  -1 (per output channel, [ch13 §13.8.2] convention) or the
 *               group size: 32, 64, 128 or 256.
 *   y           [M, N] output, 16-byte aligned, must not overlap any input.
 * Products are formed exactly and accumulated in fp32; the scale multiplies
 * each group's (or the row's) fp32 partial sum; y is rounded from fp32 to the
 * output dtype, round-to-nearest-even.  x and s must be finite (results for
 * non-finite inputs are unspecified) and |x| < 2^126.
 * Path choice: M <= ternary_gemv_max_m() runs the decode GEMV (the fp4 x fp8
 * kernel at M == 1 except for N < 8192 with K > 8192, the 16-bit one otherwise, each where
 * it takes the shape); 9 <= M <= 32 the few-token GEMM (TERNARY_PATH_FEW) where it takes
 * the shape (groups of 128: M <= 16); larger M and the rest the MFMA GEMM; shapes no fast kernel
 * takes (K % 128 != 0) run the plain kernel.  The GEMV gives each token 2
 * MFMA columns (per channel, groups of 128 or 256), 4 (groups of 64) or 8
 * (groups of 32) of 16, so it takes M <= 4 for groups of 64 and 32 (M <= 2
 * where the fp4 kernel's LDS cannot hold x), and K <= 65536.  Results of different paths agree within the bound
 * |y - y_ref| <= 1e-3 * sum_k |x_k| * s(n,k) + 1e-6, not bitwise.
 */
int ternary_linear(const void *x, int dtype, int64_t M, int64_t N, int64_t K,
                   const uint8_t *packed, const uint16_t *scale, int64_t group_size,
                   void *y, hipStream_t stream);

/* ternary_linear with an explicit kernel path (ternary_path); AUTO is the
 * default choice above.  A forced path that cannot take the shape returns
 * TERNARY_ERR_PATH without launching. */
int ternary_linear_ex(const void *x, int dtype, int64_t M, int64_t N, int64_t K,
                      const uint8_t *packed, const uint16_t *scale, int64_t group_size,
                      void *y, int path, hipStream_t stream);

/*
 * ternary_linear_tiled - ternary_linear_ex with the codes in the tiled layout:
 *   tiled  uint8 [ternary_tiled_bytes(N, K)], 16-byte aligned; every other
 *          argument as for ternary_linear_ex.
 * The same products, sums and rounding as the row-major call.  Paths: both
 * decode GEMVs, the pipelined GEMM and the plain kernel read the tiled
 * layout; the GEMM shapes only the 128 x 128 kernel takes (K % 256 != 0, group
 * size 32, an odd number of groups per row, scales not 4-byte aligned) run the
 * plain kernel under TERNARY_PATH_AUTO and return TERNARY_ERR_PATH when
 * TERNARY_PATH_GEMM is forced.  A forced path runs the same kernel, with the
 * same launch shape, on tiled as on row-major codes: the results are the
 * same bits.
 */
int ternary_linear_tiled(const void *x, int dtype, int64_t M, int64_t N, int64_t K,
                         const uint8_t *tiled, const uint16_t *scale, int64_t group_size,
                         void *y, int path, hipStream_t stream);

/* Most problems one ternary_linear_batch call takes. */
#define TERNARY_MAX_BATCH 8

/* One projection of a batched call: the arguments of ternary_linear. */
typedef struct {
    const void *x;          /* [M, K] activations, 16-byte aligned                  */
    const uint8_t *packed;  /* [N, K/4] codes, 16-byte aligned                      */
    const uint16_t *scale;  /* fp16 [N] or [N, K/group_size], 2-byte aligned        */
    void *y;                /* [M, N] output, 16-byte aligned                       */
    int64_t M, N, K;        /* as for ternary_linear                                */
    int64_t group_size;     /* -1, 32, 64, 128 or 256                               */
    int64_t layout;         /* TERNARY_LAYOUT_ROWS ([N, K/4] as above) or
                               TERNARY_LAYOUT_TILED (packed holds
                               ternary_tiled_bytes(N, K) bytes)                    */
} ternary_problem;

/*
 * ternary_linear_batch - several independent ternary_linear problems in as
 * few launches as possible, for the projections of one layer: the segments of
 * a fused QKV (or gate+up) weight, each with its own packed rows and scales
 * ([trdm §2.2]), or any set of projections that are ready together.
 *   problems  host array of `count` problems (1 <= count <= TERNARY_MAX_BATCH),
 *             read during the call only.
 *   dtype     activation/output dtype shared by all problems.
 * Every problem is validated as by ternary_linear (or ternary_linear_tiled);
 * an unknown layout returns TERNARY_ERR_SHAPE; in addition no output may
 * overlap any input or any other output of the batch (TERNARY_ERR_ALIAS).  On
 * any error nothing is launched.  Problems the automatic path sends to the
 * decode GEMV (see ternary_linear) run together in one launch per scale
 * mode (per channel, or each group size) and token count M; problems the
 * automatic path sends to the few-token GEMM run together in one launch per
 * scale mode (plus one launch adding the K slices of sliced problems);
 * the GEMM problems the pipelined kernel takes (K % 256 == 0; group sizes 64,
 * 128 or 256 with an even number of groups per row and 4-byte-aligned scales)
 * run together in one grouped GEMM launch per scale mode and tile shape
 * (longest K first); the others run as separate launches on the same stream.  Results are
 * deterministic (the same batch gives the same bits) and each satisfies the
 * bound of ternary_linear; they may differ from a single ternary_linear call on
 * the same problem in the last bits, because a batch may split a problem's K
 * range into a different number of partial sums.
 */
int ternary_linear_batch(const ternary_problem *problems, int count, int dtype,
                         hipStream_t stream);

/* The path ternary_linear_ex(..., TERNARY_PATH_AUTO, ...) takes for a shape
 * (a ternary_path value), or a negative status for invalid shapes.  A
 * group-128 scale array is assumed 4-byte aligned (else the few-token GEMM's
 * shapes take the GEMM). */
int ternary_select_path(int64_t M, int64_t N, int64_t K, int64_t group_size);

/* Largest M the decode GEMV accepts. */
int ternary_gemv_max_m(void);

/* Human-readable name of a ternary_status value (static storage). */
const char *ternary_status_string(int status);

/* Library ABI version (increments when a signature or a convention changes). */
int ternary_abi_version(void);

/*
 * ternary_shutdown - free the library's workspaces, those replaced by larger
 * ones included.  Waits for every device that holds one, then frees them;
 * later calls allocate again as needed.  A HIP graph captured before with a
 * split-K GEMM launch in it must not be replayed afterwards.  Returns
 * TERNARY_ERR_HIP if a synchronisation or free failed (the remaining
 * workspaces are still released).
 */
int ternary_shutdown(void);

/* Bytes of the static scratch array of ternary_linear_batch_noalloc. */
#define TERNARY_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * ternary_linear_batch_noalloc - ternary_linear_batch for callers that cannot
 * allocate device memory: code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, validation, results (the
 * same bits) and launches as ternary_linear_batch, but the fp32 partial tiles
 * of a split-K GEMM and the K-slice sums of the few-token GEMM (one launch
 * after another, so they share it) go to a static device array of the library
 * (TERNARY_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends) instead
 * of the per-stream workspace: the call never allocates or frees.  A batch
 * whose split-K partials need more returns TERNARY_ERR_SCRATCH and enqueues
 * nothing.  Every call on one GPU shares that GPU's array: calls that overlap
 * on a GPU (other streams, other host threads) race, and a graph captured with
 * it must not be replayed while another such call runs on the GPU.
 */
int ternary_linear_batch_noalloc(const ternary_problem *problems, int count, int dtype,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TERNARY_LINEAR_H */
