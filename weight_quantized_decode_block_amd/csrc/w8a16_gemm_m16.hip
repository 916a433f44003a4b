// W8A16 decode GEMM with a 16-row M tile for gfx950 (MI355X).
//
//   C[m,n] = bf16( sum_b S[n/128][b] * sum_{k in block b} A[m,k] * W[n,k] ),  m < M <= 16
//
// Operation: page "w8a16_gemm_m16.rs", module doc (FP8 E4M3 weights [N,K],
// FP32 block scales [N/128, K/128] folded once per 128-K block onto an fp32
// outer accumulator, never per element and never into BF16; the M tile is the
// matrix instruction's 16 rows) and the doc of w8a16_gemm_m16 (BF16 A [m,k],
// BF16 C [m,n], rows >= m untouched).  The pages' Hopper design (mma.sync
// m16n8k16, 32 columns and 128 threads per CTA, A staged with cp.async) is
// not used; this kernel is laid out for gfx950 as follows.
//
// Work layout
//   * A workgroup of 4 waves owns 16 weight rows (one 16x16 output tile); the
//     K blocks are split into 4 contiguous ranges, one per wave.
//   * Per 128-K block, lane l (i = l%16, g = l/16) loads 32 bytes of weight
//     row n0+i at k = 32g..32g+31 (two 16-byte loads) and 64 bytes of
//     activation row i at the same k, converts the FP8 bytes to BF16 with the
//     hardware conversion (exact for every finite E4M3FN value), and issues
//     four v_mfma_f32_16x16x32_bf16 whose k-slot 8g+e is k = 32g + 8j + e of
//     the block for the j-th instruction, identically for both operands.
//     The dequantised weights live in registers, where the matrix unit reads
//     its operands; they never pass through LDS.
//   * The four instructions start from zero, so they produce the block's
//     inner sum; the block's scale is then folded once:
//     outer = outer + s * inner (multiply, then add).
//   * The four waves' fp32 tiles are added in LDS in fixed wave order and the
//     rows m < M are stored as BF16, round to nearest even.
//
// Each output row depends only on its own activation row (rows >= M are
// zero operands), so a row's bits do not depend on M.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wqd_internal.h"

namespace wqd {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kNTile = 16;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI));
}

struct Stage {
  u32x4_t w0, w1;          // 32 FP8 weights
  u32x4_t a0, a1, a2, a3;  // 32 BF16 activations
};

__device__ __forceinline__ void load_stage(const uint8_t *__restrict__ wrow, const uint16_t *__restrict__ arow,
                                           bool w_ok, bool a_ok, uint32_t kofs, Stage &s) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  if (w_ok) {
    const u32x4_t *p = reinterpret_cast<const u32x4_t *>(wrow + kofs);
    s.w0 = p[0];
    s.w1 = p[1];
  } else {
    s.w0 = z;
    s.w1 = z;
  }
  if (a_ok) {
    const u32x4_t *p = reinterpret_cast<const u32x4_t *>(arow + kofs);
    s.a0 = p[0];
    s.a1 = p[1];
    s.a2 = p[2];
    s.a3 = p[3];
  } else {
    s.a0 = z;
    s.a1 = z;
    s.a2 = z;
    s.a3 = z;
  }
}

__device__ __forceinline__ bf16x8_t weights8(uint32_t lo4, uint32_t hi4) {
  u32x4_t v;
  v.x = fp8x2_to_bf16x2<false>(lo4);
  v.y = fp8x2_to_bf16x2<true>(lo4);
  v.z = fp8x2_to_bf16x2<false>(hi4);
  v.w = fp8x2_to_bf16x2<true>(hi4);
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x4_t block_inner(const Stage &s) {
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, s.a0), weights8(s.w0.x, s.w0.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, s.a1), weights8(s.w0.z, s.w0.w), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, s.a2), weights8(s.w1.x, s.w1.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, s.a3), weights8(s.w1.z, s.w1.w), acc, 0, 0, 0);
  return acc;
}

__global__ __launch_bounds__(kThreads) void w8a16_gemm_m16_kernel(const uint16_t *__restrict__ A,
                                                                  const uint8_t *__restrict__ W,
                                                                  const float *__restrict__ S,
                                                                  uint16_t *__restrict__ C, uint32_t M,
                                                                  uint32_t N, uint32_t K) {
  __shared__ float part[kWaves][16][kNTile];

  const uint32_t nb = K >> 7;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t i = lane & 15u;
  const uint32_t g = lane >> 4;
  const uint32_t n0 = blockIdx.x * kNTile;
  const uint32_t n = n0 + i;
  const bool w_ok = n < N;
  const bool a_ok = i < M;
  const uint8_t *wrow = W + (size_t)(w_ok ? n : 0) * K + 32u * g;
  const uint16_t *arow = A + (size_t)(a_ok ? i : 0) * K + 32u * g;
  const float *srow = S + (size_t)(n0 >> 7) * nb;

  const uint32_t b0 = (uint32_t)(((uint64_t)nb * wave) / kWaves);
  const uint32_t b1 = (uint32_t)(((uint64_t)nb * (wave + 1)) / kWaves);

  f32x4_t outer = {0.0f, 0.0f, 0.0f, 0.0f};
  if (b0 < b1) {
    Stage cur;
    load_stage(wrow, arow, w_ok, a_ok, b0 * 128u, cur);
    for (uint32_t b = b0; b < b1; ++b) {
      Stage nxt;
      if (b + 1 < b1) load_stage(wrow, arow, w_ok, a_ok, (b + 1) * 128u, nxt);
      const f32x4_t inner = block_inner(cur);
      const float s = srow[b];
#pragma unroll
      for (int r = 0; r < 4; ++r) outer[r] = __fadd_rn(outer[r], __fmul_rn(s, inner[r]));
      cur = nxt;
    }
  }

  // D layout: this lane holds rows m = 4g + r of column i.
#pragma unroll
  for (int r = 0; r < 4; ++r) part[wave][4 * g + r][i] = outer[r];
  __syncthreads();
  const uint32_t t = threadIdx.x;
  const uint32_t m = t >> 4;
  const uint32_t col = t & 15u;
  if (m < M && n0 + col < N) {
    float v = part[0][m][col];
    v = v + part[1][m][col];
    v = v + part[2][m][col];
    v = v + part[3][m][col];
    C[(size_t)m * N + n0 + col] = f32_to_bf16_rne(v);
  }
}

}  // namespace

hipError_t launch_w8a16_m16(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                            uint32_t K, hipStream_t stream) {
  const dim3 grid((N + kNTile - 1) / kNTile);
  hipLaunchKernelGGL(w8a16_gemm_m16_kernel, grid, dim3(kThreads), 0, stream,
                     static_cast<const uint16_t *>(A), static_cast<const uint8_t *>(W), S,
                     static_cast<uint16_t *>(C), M, N, K);
  return hipGetLastError();
}

}  // namespace wqd
