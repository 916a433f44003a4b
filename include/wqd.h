/*
 * wqd.h - C ABI of the weight-only-quantized decode GEMV library (libwqd.so)
 * for AMD Instinct MI355X (gfx950).
 *
 *   C[M,N] = A[M,K] (BF16) . dequant(B)^T,  fp32 accumulation, BF16 store.
 *
 * Two weight formats:
 *   - Q2_0 ternary (page "gemv_q2_vec.rs", module doc and the docs of
 *     q2_0_gemv_vec / q2_0_gemv_vec_batchm): 128-weight blocks, each an
 *     inline fp16 scale d followed by 2-bit codes, w = (code - 1) * d.
 *   - W8A16 (page "w8a16_gemm_m16.rs", module doc and the doc of
 *     w8a16_gemm_m16): FP8 E4M3 weights [N,K] with FP32 block scales
 *     [ceil(N/128), K/128], each scale folded once per 128-K block onto an
 *     fp32 outer accumulator.
 *
 * Conventions for every GPU entry point:
 *   - A, B/W, S and C are DEVICE pointers owned by the caller; the library
 *     never frees or keeps them, and allocates nothing per call.
 *   - Work is enqueued on `stream` (0 = the default stream) and the call
 *     returns without synchronising.  Results are visible once the stream
 *     has reached that point.
 *   - Arguments are validated before any HIP call, so every argument error is
 *     reported identically with or without a GPU.  Nothing is launched when a
 *     call fails.
 *   - C must not overlap A, B, W or S.
 *   - Return value: WQD_OK (0) or one of the WQD_E* codes below; the text of
 *     the last failure on the calling thread is returned by wqd_last_error().
 *   - No C++ exception crosses this interface.
 */
#ifndef WQD_H
#define WQD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes */
#define WQD_OK            0
#define WQD_EINVAL        1  /* a size or count outside the documented range */
#define WQD_ENULL         2  /* a required pointer is NULL */
#define WQD_EALIGN        3  /* a pointer lacks the documented alignment */
#define WQD_EUNSUPPORTED  4  /* valid input this library does not implement */
#define WQD_ENODEV        5  /* no usable HIP device */
#define WQD_EHIP          6  /* a HIP runtime error; its text is in wqd_last_error() */

/* ---------------------------------------------------------------- layout */
#define WQD_Q2_0_GROUP         128  /* weights per block_q2_0 */
#define WQD_Q2_0_BLOCK_BYTES   34   /* fp16 d (2 B) + 128 x 2-bit codes (32 B) */
#define WQD_Q2_0_BATCHM_MAX_M  8    /* rows per batched launch */
#define WQD_Q2_0_MAX_K         (1u << 24)  /* largest K the Q2_0 entry points take */
#define WQD_W8A16_MAX_M        16   /* rows per W8A16 call (the MFMA M tile) */
#define WQD_W8A16_BLOCK        128  /* K and N extent of one FP8 scale */

/*
 * block_q2_0 (34 bytes, no padding, 2-byte aligned in an array):
 *   bytes 0-1 : d, IEEE binary16, little-endian
 *   bytes 2-33: 128 codes in {0,1,2} (3 decodes to +2d); code k of the block
 *               sits in bits 2*(k mod 16) of little-endian 32-bit word k/16,
 *               i.e. bits 2*(k mod 4) of byte 2 + k/4.
 * A Q2_0 weight matrix is block_q2_0[N][K/128], row-major (weight row n holds
 * the K/128 blocks of output column n in ascending k).
 * The pages give the inline fp16 scale and 16 codes per 32-bit word
 * (gemv_q2_vec.rs, module doc and q2_0_gemv_vec doc); the byte order and field
 * order are this library's fixed reading of them.
 */

/*
 * q2_0_gemv - M = 1 Q2_0 GEMV: C[1,N] = A[1,K] . dequant(B)^T.
 * Defined by page "gemv_q2_vec.rs", doc of q2_0_gemv_vec (A BF16 [1,K], B raw
 * block_q2_0, C BF16 [1,N], dequant (code-1)*d inside the dot product).
 *
 *   A      device, BF16 [K], 16-byte aligned
 *   B      device, block_q2_0 [N][K/128], 4-byte aligned
 *   C      device, BF16 [N], 2-byte aligned
 *   N      >= 1 output columns
 *   K      >= 128, a multiple of 128 (else WQD_EINVAL), at most
 *          WQD_Q2_0_MAX_K (else WQD_EUNSUPPORTED)
 *   group  must be 128 (the block size; other values give WQD_EINVAL)
 *
 * Each output is an fp32 sum over k stored as BF16 (round to nearest even);
 * it matches the CPU reference within 2 BF16 ulp or 1e-2 of the output row's
 * RMS, and is bit-identical to row 0 of q2_0_gemv_batchm with the same inputs.
 */
int q2_0_gemv(const void *A, const void *B, void *C,
              uint32_t N, uint32_t K, uint32_t group, hipStream_t stream);

/*
 * q2_0_gemv_batchm - batched Q2_0 GEMV for M concurrent decode rows:
 * C[M,N] = A[M,K] . dequant(B)^T.
 * Defined by page "gemv_q2_vec.rs", doc of q2_0_gemv_vec_batchm: each weight
 * word is read once per launch and used for all rows; every output row is
 * bit-identical to running q2_0_gemv on that row alone.  M above 8 is served
 * by ceil(M/8) launches of at most 8 rows, A and C advanced by whole rows
 * (the page's Q2_BATCHM_MAX_M chunking).
 *
 *   A  device, BF16 [M][K] row-major, 16-byte aligned
 *   B, C, N, K, group as for q2_0_gemv; C is BF16 [M][N] row-major
 *   M  number of rows; M = 0 returns WQD_OK and launches nothing
 */
int q2_0_gemv_batchm(const void *A, const void *B, void *C,
                     uint32_t N, uint32_t K, uint32_t group, uint32_t M,
                     hipStream_t stream);

/*
 * w8a16_gemm_m16 - W8A16 decode GEMM with a 16-row M tile:
 * C[m,n] = bf16( sum_b S[n/128][b] * sum_{k in block b} A[m,k] * W[n,k] ).
 * Defined by page "w8a16_gemm_m16.rs", module doc (scale folded once per
 * 128-K block onto an fp32 outer accumulator, matrix-core reduction order)
 * and the doc of w8a16_gemm_m16 (1 <= m <= 16, K a multiple of 128; callers
 * with 17..32 rows make two calls on contiguous row halves).
 *
 *   A  device, BF16 [M][K] row-major, 16-byte aligned
 *   W  device, FP8 E4M3FN [N][K] row-major, 16-byte aligned
 *   S  device, fp32 [ceil(N/128)][K/128] row-major, 4-byte aligned
 *   C  device, BF16 [M][N] row-major, 2-byte aligned; only rows < M written
 *   M  1..16 (else WQD_EINVAL);  N >= 1;  K >= 128, a multiple of 128
 *
 * Matches the CPU reference within 2 BF16 ulp or 1e-2 of the row RMS; each
 * output row depends only on its own A row, so it is bit-identical for any M.
 */
int w8a16_gemm_m16(const void *A, const void *W, const float *S, void *C,
                   uint32_t M, uint32_t N, uint32_t K, hipStream_t stream);

/*
 * w8a16_gemm_m16_n64 - the same GEMM with each workgroup owning 64
 * consecutive weight rows (four 16-row tiles) instead of spreading tiles over
 * the matrix: a quarter as many workgroups as there are 16-row tiles.
 * Defined by page "w8a16_gemm_m16.rs", docs of W8A16_GEMM_M16_N_TILE_WIDE and
 * w8a16_gemm_m16_n64 (same arguments and guards as w8a16_gemm_m16, wider N
 * tile, fewer workgroups).  Arguments, checks and error codes are those of
 * w8a16_gemm_m16; the output is bit-identical to it (same sums, same order).
 */
int w8a16_gemm_m16_n64(const void *A, const void *W, const float *S, void *C,
                       uint32_t M, uint32_t N, uint32_t K, hipStream_t stream);

/*
 * w8a16_gemm_m16_strided - w8a16_gemm_m16 with row pitches for A and C, so
 * the rows may be slices of wider row-major buffers.
 * Defined by page "w8a16_gemm_m16.rs", doc of w8a16_gemm_m16_strided (pitches
 * in elements, each covering its row, the activation pitch a multiple of 8 so
 * every row starts on a 16-byte boundary).
 *
 *   A             device, BF16, row m at A + m * a_row_stride, 16-byte aligned
 *   C             device, BF16, row m at C + m * c_row_stride, 2-byte aligned;
 *                 only elements [0, N) of rows < M are written, the padding
 *                 between rows is never touched
 *   a_row_stride  >= K and a multiple of 8 (else WQD_EINVAL)
 *   c_row_stride  >= N (else WQD_EINVAL)
 *   W, S, M, N, K as for w8a16_gemm_m16; (M-1)*pitch + row must stay below
 *   2^32 elements for both A and C (else WQD_EINVAL)
 *
 * With a_row_stride = K and c_row_stride = N it is w8a16_gemm_m16, bit for
 * bit; in general each output row is bit-identical to w8a16_gemm_m16 on the
 * same row stored contiguously.
 */
int w8a16_gemm_m16_strided(const void *A, const void *W, const float *S, void *C,
                           uint32_t M, uint32_t N, uint32_t K,
                           uint32_t a_row_stride, uint32_t c_row_stride,
                           hipStream_t stream);

/*
 * w8a16_gemv_batch16 - W8A16 decode GEMV on the vector ALUs for 1..16 rows:
 * the same operation as w8a16_gemm_m16 (FP8 E4M3FN weights, 128x128 fp32
 * block scales folded once per 128-K block onto an fp32 outer accumulator),
 * computed without matrix instructions.
 * Defined by page "w8a16_gemm_m16.rs", module doc (the scalar GEMV
 * w8a16_gemv_batch16 beside the matrix-core kernel, one multiply-add per
 * weight byte and activation row, not bit-identical to the matrix-core
 * kernel) and the scale-fold rule stated there.
 *
 *   A, W, S, C, M, N, K as for w8a16_gemm_m16 (M 1..16, K a multiple of 128)
 *   K must also be at most 81920 (one activation row is staged on chip):
 *     larger K gives WQD_EUNSUPPORTED
 *
 * Rows are served by launches of at most 8 rows (fewer when 8 rows of K do not
 * fit on chip), A and C advanced by whole rows.  Matches the CPU reference
 * within 2 BF16 ulp or 1e-2 of the row RMS; each output row is bit-identical
 * for every M (its arithmetic does not depend on the other rows), but not to
 * w8a16_gemm_m16, whose matrix instructions add in their own order.
 */
int w8a16_gemv_batch16(const void *A, const void *W, const float *S, void *C,
                       uint32_t M, uint32_t N, uint32_t K, hipStream_t stream);

/*
 * w8a16_gemv_batch16_strided - w8a16_gemv_batch16 with A and C row pitches,
 * with the argument order and pitch rules of w8a16_gemm_m16_strided (page
 * "w8a16_gemm_m16.rs", doc of w8a16_gemm_m16_strided, which names the
 * strided scalar GEMV as having the same argument order).  Each output row is
 * bit-identical to w8a16_gemv_batch16 on the same row stored contiguously.
 */
int w8a16_gemv_batch16_strided(const void *A, const void *W, const float *S, void *C,
                               uint32_t M, uint32_t N, uint32_t K,
                               uint32_t a_row_stride, uint32_t c_row_stride,
                               hipStream_t stream);

/* ----------------------------------------------------------- host helpers */

/* Bytes of a packed Q2_0 matrix: N * (K/128) * 34, or 0 if K % 128 != 0. */
size_t q2_0_packed_bytes(uint32_t N, uint32_t K);

/*
 * q2_0_pack - host packer into the block_q2_0 layout above.
 *   codes  host, uint8 [N][K], each 0, 1 or 2 (3 is rejected: WQD_EINVAL)
 *   d_f16  host, IEEE binary16 bit patterns [N][K/128]
 *   out    host, q2_0_packed_bytes(N, K) bytes
 * K must be a positive multiple of 128.  Pure host code; no HIP call.
 */
int q2_0_pack(const uint8_t *codes, const uint16_t *d_f16,
              uint32_t N, uint32_t K, void *out);

/*
 * q2_0_batchm_chunks - the launch plan q2_0_gemv_batchm uses for M rows, per
 * page "gemv_q2_vec.rs" (batchm_row_chunks / batchm_launch_chunks): writes up
 * to `cap` triples (A byte offset, C byte offset, rows) into out3[3*i..3*i+2]
 * with rows in 1..8, contiguous from row 0, summing to M (BF16 = 2 bytes per
 * element).  Returns the number of launches, ceil(M/8) (0 when M = 0), even if
 * it exceeds `cap`.  Pure host code; no HIP call.
 */
uint32_t q2_0_batchm_chunks(uint32_t M, uint32_t K, uint32_t N,
                            uint64_t *out3, uint32_t cap);

/*
 * Q2_0 row tiers.  The matrix-core kernel is compiled for launches of at most
 * 1, 2, 4, 6 and 8 rows (WQD_Q2_0_TIER_WIDTHS, narrowest first); a launch of m
 * rows runs on the narrowest compiled width that covers m.  Every width gives
 * the same bits for a row (its arithmetic does not depend on the width), a
 * narrower one only skips work for rows that are not there.  Widths 1 and 8
 * are the base tiers (the page's single-row GEMV and its 8-row batched
 * launch); 2, 4 and 6 are exact-row tiers, which the presence of the
 * environment variable WQD_NO_EXACT_M_TIERS (any value, "0" included; read
 * once per process) removes from the decision without unloading anything.
 * Follows page "w4a16_gemv_tiers.rs": "Why this module exists" (a wider tier
 * pays for rows that are not there), "Kill switch" and select_tier
 * (narrowest present tier that covers m, none for m = 0).
 *
 * q2_0_select_tier - the pure decision: index into WQD_Q2_0_TIER_WIDTHS of the
 *   narrowest width >= m whose bit is set in present_mask and that is allowed
 *   (exact_m != 0 allows the exact-row tiers), or -1 when m = 0 or nothing
 *   covers m.  Pure host code; no HIP call, no environment access.
 * q2_0_tier_width - the width q2_0_gemv / q2_0_gemv_batchm launch m rows on
 *   in this process (every width compiled, the switch as read), or 0 when the
 *   matrix-core family cannot serve m (m = 0 or m > 8).  No HIP call.
 * q2_0_exact_m_tiers_enabled - 1 unless WQD_NO_EXACT_M_TIERS is present.
 */
#define WQD_Q2_0_TIER_COUNT 5
#define WQD_Q2_0_TIER_WIDTHS {1u, 2u, 4u, 6u, 8u}
int q2_0_select_tier(uint32_t m, uint32_t present_mask, int exact_m);
uint32_t q2_0_tier_width(uint32_t m);
int q2_0_exact_m_tiers_enabled(void);

/* Text of the last failing call on this thread ("" if none). */
const char *wqd_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* WQD_H */
