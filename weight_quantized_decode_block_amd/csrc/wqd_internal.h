// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wqd {

// Rows [r0, r1) of workgroup b when N rows are split evenly over G
// workgroups: the first N % G get one row more.  Wave-uniform 32-bit
// arithmetic (a 64-bit division here cost about 100 instructions per wave
// before the first load).
__device__ __forceinline__ void even_rows(uint32_t N, uint32_t b, uint32_t G, uint32_t &r0, uint32_t &r1) {
  const uint32_t q = N / G, rem = N - q * G;
  r0 = b * q + (b < rem ? b : rem);
  r1 = r0 + q + (b < rem ? 1u : 0u);
}

// Output stores: a BF16 result is written as a relaxed atomic store at agent
// scope, which the compiler emits as an ordinary global store with the sc1
// cache-policy bit (the store goes through the XCD's L2 instead of leaving a
// dirty line there).  Measured on MI355X against the plain store (Q2_0,
// graph-replayed, interleaved A/B): N = K = 5120 M = 1 4.29 -> 4.22 us, M = 2
// 4.54 -> 4.45, N = K = 4096 3.52 -> 3.40, N = K = 8192 6.73 -> 6.65,
// N = 5120 K = 17408 8.95 -> 8.87; M = 8 6.41 -> 6.45.  The same bit on a
// buffer store, or a non-temporal store, was slower at most shapes.
__device__ __forceinline__ void store_out(uint16_t *p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Enqueue one batched Q2_0 launch for 1..8 rows (A [m][K], C [m][N]) on the
// vector-ALU kernel.  Shapes are validated by the caller.
hipError_t launch_q2_0_valu(const void *A, const void *B, void *C, uint32_t N,
                            uint32_t K, uint32_t m, hipStream_t stream);

// Same operation on the matrix-core kernels, 1..8 rows per launch, for K a
// multiple of 256 from 1024 up and weights under 2^31 bytes
// (q2_0_pairs_supports).  `width` (1, 2, 4, 6 or 8, at least m) picks the
// compiled row tier; every tier gives a row the same bits.
bool q2_0_pairs_supports(uint32_t N, uint32_t K);
hipError_t launch_q2_0_pairs(const void *A, const void *B, void *C, uint32_t N,
                             uint32_t K, uint32_t m, uint32_t width, hipStream_t stream);

// Enqueue the W8A16 M16 GEMM for 1..16 rows; A and C row pitches lda / ldc
// in elements; band = 0 (the weight rows split evenly over the workgroups) or
// b > 0 (each workgroup owns 16 * b consecutive weight rows).  Every choice
// gives the same bits.  Shapes validated by the caller.
hipError_t launch_w8a16_m16(const void *A, const void *W, const float *S,
                            void *C, uint32_t M, uint32_t N, uint32_t K,
                            uint32_t lda, uint32_t ldc, uint32_t band,
                            hipStream_t stream);

// Enqueue the vector-ALU W8A16 GEMV for 1..w8a16_gemv_rows_per_launch(K)
// rows (at most 8); A and C row pitches lda / ldc in elements.  Shapes
// validated by the caller.
hipError_t launch_w8a16_gemv(const void *A, const void *W, const float *S,
                             void *C, uint32_t M, uint32_t N, uint32_t K,
                             uint32_t lda, uint32_t ldc, hipStream_t stream);

// Activation rows one vector-ALU GEMV launch can stage in LDS (0 when one
// row of K does not fit).
uint32_t w8a16_gemv_rows_per_launch(uint32_t K);

}  // namespace wqd
