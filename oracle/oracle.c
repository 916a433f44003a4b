/*
 * Plain CPU oracle for the weight-only-quantized decode GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * reference that the GPU path is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links, calls or falls back to it, and the two share
 * no code (this file includes nothing from the product tree).
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (no fast-math), so
 * every float operation below is one IEEE binary32 operation in program order.
 *
 * Sources (pages are cited by title and section; no listing line numbers):
 *   [Q2]  "gemv_q2_vec.rs" (spark_model layers/ops), module doc and the
 *         fn docs of q2_0_gemv_vec / q2_0_gemv_vec_batchm: a block_q2_0 holds
 *         128 ternary 2-bit codes plus an inline fp16 scale d; w = (code-1)*d;
 *         A and C are BF16.
 *   [Q2T] same page, `mod tests`, helper `gemv_row`: the per-row reference
 *         is an fp32 accumulator starting at 0, summed in ascending k, with
 *         w = ((code & 3) - 1) * d and d round-tripped through fp16, and the
 *         result stored as BF16 (round to nearest even).
 *   [W8]  "w8a16_gemm_m16.rs" (metrale_model_layers layers/ops), module doc
 *         and the doc of w8a16_gemm_m16: FP8 E4M3 weights [N,K], FP32 scales
 *         [N/128, K/128]; per output, each 128-K block's fp32 sum times the
 *         block's scale is added to an fp32 total (one scaling per block, no
 *         BF16 in between); BF16 input and output.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - block_q2_0 byte layout: fp16 d little-endian in bytes 0-1, then 32
 *     bytes of codes; code k of the block sits in bits 2*(k mod 4) of byte
 *     2 + k/4 (equivalently bits 2*(k mod 16) of little-endian word k/16).
 *   - FP8 variant: OCP E4M3FN (bias 7, max 448, NaN = S.1111.111, no inf).
 *   - FP8 fold: inner = sequential fp32 sum over the 128-K block, then
 *     outer = outer + s * inner, multiply then add, unfused.
 *   - Scale row for weight row n is n/128 (ceil(N/128) rows of scales).
 *
 * Parity pins live in the tests: brute-force float32 emulation, closed
 * forms, the exact-integer regime, an f64 error bound, codec tables checked
 * against numpy/torch, and worked examples.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------ codecs */

/* IEEE binary16 -> binary32, exact for every pattern (subnormals included). */
float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t e = (uint32_t)(h >> 10) & 0x1fu;
    uint32_t m = (uint32_t)h & 0x3ffu;
    float mag;
    if (e == 0) {
        mag = ldexpf((float)m, -24);              /* 0 or subnormal m * 2^-24 */
    } else if (e == 31) {
        mag = m ? NAN : INFINITY;
    } else {
        mag = ldexpf((float)(1024u + m), (int)e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

/* bfloat16 -> binary32: the 16 bits are the top half of the binary32. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even.  NaN stays a quiet
 * NaN with the same sign; values that round past the largest finite bfloat16
 * become infinity, as IEEE rounding prescribes. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;                               /* carries into the exponent correctly */
    return (uint16_t)upper;
}

/* OCP OFP8 E4M3FN -> binary32 (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent field 0 is subnormal m * 2^-9; S.1111.111 is NaN;
 * there is no infinity). */
float oracle_e4m3fn_to_f32(uint8_t q)
{
    uint32_t sign = (q >> 7) & 1u;
    uint32_t e = (q >> 3) & 0xfu;
    uint32_t m = q & 0x7u;
    float mag;
    if (e == 0xfu && m == 0x7u)
        mag = NAN;
    else if (e == 0)
        mag = ldexpf((float)m, -9);
    else
        mag = ldexpf((float)(8u + m), (int)e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -mag : mag;
}

/* ------------------------------------------------------- q2_0 unpacker */

/* Unpack a [N][K/128] array of 34-byte block_q2_0 into codes [N][K] and
 * fp16 scale bits [N][K/128].  Written byte-wise from the layout reading
 * above (the product packer is written word-wise), so a round trip through
 * both checks one formulation against the other.  Returns 0, or -1 when K is
 * not a multiple of 128. */
int oracle_q2_0_unpack(const uint8_t *packed, uint32_t N, uint32_t K,
                       uint8_t *codes, uint16_t *d_f16)
{
    if (K % 128u != 0)
        return -1;
    size_t nb = K / 128u;
    for (size_t n = 0; n < N; ++n) {
        for (size_t b = 0; b < nb; ++b) {
            const uint8_t *blk = packed + (n * nb + b) * 34u;
            d_f16[n * nb + b] = (uint16_t)(blk[0] | ((uint16_t)blk[1] << 8));
            for (size_t j = 0; j < 128; ++j) {
                uint8_t byte = blk[2 + j / 4];
                codes[n * (size_t)K + b * 128 + j] = (uint8_t)((byte >> (2 * (j % 4))) & 3u);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------ threading */

typedef struct {
    int kind; /* 0 = q2_0, 1 = w8a16 */
    const uint16_t *A;
    const uint8_t *Wb;    /* q2_0 codes or e4m3fn bytes, [N][K] */
    const uint16_t *d;    /* q2_0 fp16 scale bits [N][K/128] */
    const float *S;       /* w8a16 scales [ceil(N/128)][K/128] */
    uint16_t *C;
    uint32_t M, N, K;
    uint32_t n0, n1;
} job_t;

/* One output of the Q2_0 GEMV, as [Q2T] defines it. */
static uint16_t q2_0_one(const uint16_t *a_row, const uint8_t *c_row,
                         const uint16_t *d_row, uint32_t K)
{
    float acc = 0.0f;
    for (uint32_t k = 0; k < K; ++k) {
        float d = oracle_f16_to_f32(d_row[k / 128u]);
        float w = (float)((int)(c_row[k] & 3u) - 1) * d;
        acc = acc + oracle_bf16_to_f32(a_row[k]) * w;
    }
    return oracle_f32_to_bf16(acc);
}

/* One output of the W8A16 GEMM, as [W8] defines it. */
static uint16_t w8a16_one(const uint16_t *a_row, const uint8_t *w_row,
                          const float *s_row, uint32_t K)
{
    float outer = 0.0f;
    for (uint32_t b = 0; b < K / 128u; ++b) {
        float inner = 0.0f;
        for (uint32_t k = b * 128u; k < b * 128u + 128u; ++k)
            inner = inner + oracle_bf16_to_f32(a_row[k]) * oracle_e4m3fn_to_f32(w_row[k]);
        float scaled = s_row[b] * inner;
        outer = outer + scaled;
    }
    return oracle_f32_to_bf16(outer);
}

static void *run_job(void *p)
{
    const job_t *j = (const job_t *)p;
    size_t K = j->K, nb = j->K / 128u;
    for (uint32_t n = j->n0; n < j->n1; ++n) {
        for (uint32_t m = 0; m < j->M; ++m) {
            const uint16_t *a_row = j->A + (size_t)m * K;
            uint16_t out;
            if (j->kind == 0)
                out = q2_0_one(a_row, j->Wb + (size_t)n * K, j->d + (size_t)n * nb, j->K);
            else
                out = w8a16_one(a_row, j->Wb + (size_t)n * K, j->S + (size_t)(n / 128u) * nb, j->K);
            j->C[(size_t)m * j->N + n] = out;
        }
    }
    return NULL;
}

/* Split the output columns n over threads; every output's own k order is
 * fixed, so the result does not depend on the thread count. */
static int run_all(job_t base, int nthreads)
{
    if (nthreads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = c > 0 ? (int)c : 1;
    }
    if ((uint32_t)nthreads > base.N)
        nthreads = base.N ? (int)base.N : 1;
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    if (!tid || !jobs) {
        free(tid);
        free(jobs);
        return -2;
    }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].n0 = (uint32_t)((uint64_t)base.N * t / nthreads);
        jobs[t].n1 = (uint32_t)((uint64_t)base.N * (t + 1) / nthreads);
    }
    /* threads 1.. run concurrently; the calling thread takes range 0; a
     * thread that cannot be created has its range run inline instead */
    char *joined = (char *)calloc((size_t)nthreads, 1);
    for (int t = 1; t < nthreads; ++t) {
        if (joined && pthread_create(&tid[t], NULL, run_job, &jobs[t]) == 0)
            joined[t] = 1;
        else
            run_job(&jobs[t]);
    }
    run_job(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (joined && joined[t])
            pthread_join(tid[t], NULL);
    free(joined);
    free(tid);
    free(jobs);
    return 0;
}

/* ----------------------------------------------------------- entry points */

/* C[m][n] = bf16( sum_k a[m][k] * (code[n][k]-1) * d[n][k/128] ), fp32
 * sequential in ascending k.  A: bf16 bits [M][K]; codes: [N][K] (values 0..3,
 * code 3 decodes to +2d); d_f16: fp16 bits [N][K/128]; C: bf16 bits [M][N].
 * nthreads <= 0 uses every online core.  Returns 0, or -1 if K % 128 != 0. */
int oracle_q2_0_gemv(const uint16_t *A, const uint8_t *codes, const uint16_t *d_f16,
                     uint16_t *C, uint32_t M, uint32_t N, uint32_t K, int nthreads)
{
    if (K % 128u != 0)
        return -1;
    if (M == 0 || N == 0)
        return 0;
    job_t j = {0, A, codes, d_f16, NULL, C, M, N, K, 0, 0};
    return run_all(j, nthreads);
}

/* C[m][n] = bf16( sum_b S[n/128][b] * sum_{k in block b} a[m][k] * w[n][k] ).
 * A: bf16 bits [M][K]; W: E4M3FN bytes [N][K]; S: fp32 [ceil(N/128)][K/128];
 * C: bf16 bits [M][N].  Returns 0, or -1 if K % 128 != 0. */
int oracle_w8a16_gemm(const uint16_t *A, const uint8_t *W, const float *S,
                      uint16_t *C, uint32_t M, uint32_t N, uint32_t K, int nthreads)
{
    if (K % 128u != 0)
        return -1;
    if (M == 0 || N == 0)
        return 0;
    job_t j = {1, A, W, NULL, S, C, M, N, K, 0, 0};
    return run_all(j, nthreads);
}

/* Threads the oracle would use for nthreads <= 0 (reported by the CPU
 * baseline). */
int oracle_default_threads(void)
{
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    return c > 0 ? (int)c : 1;
}
