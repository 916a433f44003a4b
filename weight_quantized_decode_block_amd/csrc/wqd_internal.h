// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wqd {

// Enqueue one batched Q2_0 launch for 1..8 rows (A [m][K], C [m][N]).
// `total_bytes` is the size of B (N * K/128 * 34).  Shapes are validated by
// the caller.
hipError_t launch_q2_0(const void *A, const void *B, void *C, uint32_t N,
                       uint32_t K, uint32_t m, hipStream_t stream);

// Enqueue the W8A16 M16 GEMM for 1..16 rows.  Shapes validated by the caller.
hipError_t launch_w8a16_m16(const void *A, const void *W, const float *S,
                            void *C, uint32_t M, uint32_t N, uint32_t K,
                            hipStream_t stream);

}  // namespace wqd
