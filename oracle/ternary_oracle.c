/*
 * Plain CPU oracle for the ternary-weight linear layer y = x * (q (.) s)^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Everything here is written straight from the definitions on the pages:
 *   [trdm]  trdm.cn, "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战"
 *           (ternary model into vLLM, from reverse-engineered loading to
 *           kernel optimisation): §3.1 states the packing rule (2 bits per
 *           weight, 00->0, 01->+1, 10->-1, 11 reserved and read as 0, four
 *           weights per byte little-endian with the first weight in the lowest
 *           two bits, 128 consecutive K weights sharing one fp16 scale);
 *           §4.2 gives the operand shapes x[M,K], w[N,K/4], scale[N,K/128].
 *   [nxbn]  m.nxbn.cn/news/169761 (a 7B ternary checkpoint into vLLM):
 *           §2.2 gives the same code table and decodes a byte field by field
 *           from the low bits; §3.2 dequantises as unpack(q) * scale.view(-1,1)
 *           with one fp16 scale per output channel; §4.2 applies the scale to
 *           the finished accumulator.
 *   [xxqk]  m.xxqk.cn/news/593501 (Bonsai 2 27B into vLLM): §4.3 defines the
 *           layer as dequantise-then-matmul, y = x @ (unpack(q) * s)^T; §4.2
 *           and §5.2 meet checkpoints whose groups are 64 weights (and the
 *           garbage that reading them as 128 gives).
 *   [ch13]  yangyitao.com vLLM book, chapter 13 (quantization): §13.3.3
 *           per-group scales, group_size 128 the usual default, 32 and 256
 *           the finer and coarser alternatives.
 *
 * The oracle evaluates exactly that definition in fp64: each product of a
 * bf16/fp16 activation, a ternary value and an fp16 scale is exact in fp64,
 * and the K-term sum is taken in ascending k.
 *
 * Readings where the pages are silent or garbled (also listed in the design doc):
 *   - code 11 decodes to 0 (reserved on [trdm], unused on [nxbn]);
 *   - pack writes 00 for any value outside {-1,0,1} and counts it;
 *   - scale layout is [N] for per-channel, [N, K/g] row-major for groups of
 *     g consecutive K weights (any g dividing K; the GPU library takes 32,
 *     64, 128 and 256);
 *   - the tolerance bound uses B = sum_k |x_k| * |s(n,k)|.
 * Parity for every function below is pinned by tests that do not re-use it
 * (see tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_VERSION 1

int ternary_oracle_version(void) { return ORACLE_VERSION; }

/* ---- number formats, from their definitions -------------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent field 0 is zero/subnormal (fraction * 2^-24); 31 is Inf/NaN. */
double ternary_oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * Exponent field 0 is zero/subnormal (fraction * 2^-133); 255 is Inf/NaN. */
double ternary_oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);
    return sign ? -v : v;
}

/* ---- the 2-bit code --------------------------------------------------------- */

/* Table form of the code map [trdm §3.1]: 00->0, 01->+1, 10->-1, 11->0. */
static const int8_t CODE_TABLE[4] = {0, 1, -1, 0};

int ternary_oracle_code_table(int c) { return CODE_TABLE[c & 3]; }

/* Comparison form [nxbn §2.2]: (c == 1) - (c == 2). */
int ternary_oracle_code_eq(int c) { return (c == 1) - (c == 2); }

/* Bit form: low bit counts +1, high bit counts -1; 11 cancels to 0. */
int ternary_oracle_code_bits(int c) { return (c & 1) - ((c >> 1) & 1); }

/* Field i (0..3) of a byte: weights are stored least-significant pair first
 * [trdm §3.1; nxbn §2.2]. */
static int field_of(uint8_t byte, int i) { return (byte >> (2 * i)) & 3; }

/* q(n,k) from packed [N, K/4]. */
static int q_at(const uint8_t *packed, int64_t K, int64_t n, int64_t k)
{
    uint8_t byte = packed[n * (K / 4) + k / 4];
    return CODE_TABLE[field_of(byte, (int)(k % 4))];
}

/* unpack: packed [N, K/4] bytes -> int8 [N, K] in {-1,0,1}. */
void ternary_oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *q)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            q[n * K + k] = (int8_t)q_at(packed, K, n, k);
}

/* pack: int8 [N, K] in {-1,0,1} -> bytes [N, K/4].  Returns how many inputs
 * were outside {-1,0,1}; those are written as code 00. */
int64_t ternary_oracle_pack(const int8_t *q, int64_t N, int64_t K, uint8_t *packed)
{
    int64_t invalid = 0;
    memset(packed, 0, (size_t)(N * (K / 4)));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int v = q[n * K + k];
            int code;
            if (v == 1)
                code = 1;
            else if (v == -1)
                code = 2;
            else {
                code = 0;
                if (v != 0)
                    ++invalid;
            }
            packed[n * (K / 4) + k / 4] |= (uint8_t)(code << (2 * (k % 4)));
        }
    }
    return invalid;
}

/* ---- the linear layer ------------------------------------------------------- */

static double x_at(const uint16_t *x, int x_fp16, int64_t K, int64_t m, int64_t k)
{
    uint16_t bits = x[m * K + k];
    return x_fp16 ? ternary_oracle_f16_to_f64(bits) : ternary_oracle_bf16_to_f64(bits);
}

/* s(n,k): one scale per output channel (group_size == -1, [nxbn §3.2]) or one
 * per group_size consecutive K weights of a row ([trdm §3.1] with 128,
 * [xxqk §4.2] with 64, [ch13 §13.3.3]; layout [N, K/group_size]). */
static double s_at(const uint16_t *scale, int64_t K, int64_t group_size, int64_t n, int64_t k)
{
    if (group_size < 0)
        return ternary_oracle_f16_to_f64(scale[n]);
    return ternary_oracle_f16_to_f64(scale[n * (K / group_size) + k / group_size]);
}

/* Dequantised row n of W = q (.) s, in fp64 [xxqk §4.3]. */
static void dequant_row(const uint8_t *packed, const uint16_t *scale, int64_t K,
                        int64_t group_size, int64_t n, double *w, double *abs_s)
{
    for (int64_t k = 0; k < K; ++k) {
        double s = s_at(scale, K, group_size, n, k);
        w[k] = (double)q_at(packed, K, n, k) * s;
        abs_s[k] = fabs(s);
    }
}

/* y[m,n] = sum_k x[m,k] * W[n,k] and bound[m,n] = sum_k |x[m,k]| * |s(n,k)|,
 * k ascending, all in fp64.  x is bf16 (x_fp16 == 0) or fp16 bit patterns.
 * Returns the number of threads that ran (for reporting), or -1 on bad args.
 * Threads split the output channels n; each (m, n) sum runs in one thread. */
int ternary_oracle_linear(const uint16_t *x, int x_fp16, int64_t M, int64_t N, int64_t K,
                          const uint8_t *packed, const uint16_t *scale, int64_t group_size,
                          double *y, double *bound, int nthreads)
{
    if (K <= 0 || K % 4 != 0 || (group_size > 0 && K % group_size != 0))
        return -1;
    int used = 1;
    if (nthreads <= 0)
        nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
        double *a = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            dequant_row(packed, scale, K, group_size, n, w, a);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0, b = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double xv = x_at(x, x_fp16, K, m, k);
                    acc += xv * w[k];
                    b += fabs(xv) * a[k];
                }
                y[m * N + n] = acc;
                if (bound)
                    bound[m * N + n] = b;
            }
        }
        free(w);
        free(a);
    }
    return used;
}

/* The same definition evaluated only at the listed (m, n) outputs, for
 * checking full-size launches on a sample.  Returns threads used or -1. */
int ternary_oracle_linear_at(const uint16_t *x, int x_fp16, int64_t M, int64_t N, int64_t K,
                             const uint8_t *packed, const uint16_t *scale, int64_t group_size,
                             const int64_t *ms, const int64_t *ns, int64_t count,
                             double *y, double *bound, int nthreads)
{
    if (K <= 0 || K % 4 != 0 || (group_size > 0 && K % group_size != 0))
        return -1;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return -1;
    int used = 1;
    if (nthreads <= 0)
        nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
        double *a = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < count; ++i) {
            int64_t m = ms[i], n = ns[i];
            dequant_row(packed, scale, K, group_size, n, w, a);
            double acc = 0.0, b = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = x_at(x, x_fp16, K, m, k);
                acc += xv * w[k];
                b += fabs(xv) * a[k];
            }
            y[i] = acc;
            if (bound)
                bound[i] = b;
        }
        free(w);
        free(a);
    }
    return used;
}

/* Count of reserved (11) fields in a packed buffer [nxbn §2.2 census]. */
int64_t ternary_oracle_count_reserved(const uint8_t *packed, int64_t nbytes)
{
    int64_t c = 0;
    for (int64_t i = 0; i < nbytes; ++i)
        for (int f = 0; f < 4; ++f)
            c += field_of(packed[i], f) == 3;
    return c;
}
