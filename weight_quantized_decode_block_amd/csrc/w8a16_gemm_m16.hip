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
//   * A workgroup of 8 waves owns a tile of 16 weight rows and walks K in
//     phases of up to 8 blocks (1024 k).  Each phase's bytes - 16 weight-row
//     segments of 1 KB and the M activation-row segments of 2 KB - are fetched
//     with 16-byte loads in which consecutive lanes read consecutive addresses,
//     kept kDepth phases ahead in registers and written to one of two LDS
//     buffers; one barrier per phase separates writing a buffer from reading it.
//   * In a phase, wave w handles block w.  Lane l (i = l%16, g = l/16) reads the
//     32 FP8 weights k = 32g..32g+31 of row i and the 32 activations of row
//     m = i at the same k, converts the weights to BF16 with the hardware
//     conversion (exact for every finite E4M3FN value) and issues four
//     v_mfma_f32_16x16x32_bf16, the j-th on k = 32g + 8j .. 32g + 8j + 7 of
//     both operands.  Starting from zero, they give the block's inner sum;
//     the block's scale is folded once: outer = outer + s * inner.
//   * The 8 waves' partial tiles are added in LDS in fixed wave order and rows
//     m < M are stored as BF16, round to nearest even.
//
// Each output row depends only on its own activation row (rows >= M are zero
// operands) and the fixed block / wave order, so a row's bits do not depend
// on M.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wqd_internal.h"

namespace wqd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kPhaseBlocks = 8;                      // 1024 k per phase
constexpr int kDepth = 3;                            // phases of loads in flight
constexpr int kWPitch = kPhaseBlocks * 128 + 16;     // LDS pitch of a weight row segment
constexpr int kWBytes = 16 * kWPitch;
constexpr int kAPitch = kPhaseBlocks * 256 + 16;     // LDS pitch of an activation row segment

__host__ __device__ constexpr int slots_for(int m) { return 2 + (m * (kPhaseBlocks * 16) + kThreads - 1) / kThreads; }
__host__ __device__ constexpr int buffer_bytes(int m) { return kWBytes + m * kAPitch; }

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

__device__ __forceinline__ bf16x8_t weights8(uint32_t lo4, uint32_t hi4) {
  u32x4_t v;
  v.x = fp8x2_to_bf16x2<false>(lo4);
  v.y = fp8x2_to_bf16x2<true>(lo4);
  v.z = fp8x2_to_bf16x2<false>(hi4);
  v.w = fp8x2_to_bf16x2<true>(hi4);
  return __builtin_bit_cast(bf16x8_t, v);
}

// Chunk slot s of a phase for this thread: slots 0-1 carry weight chunks (row
// tid/32, column tid%32 + 32s of the row's 64), the rest carry activation
// chunks (row c/128, column c%128 with c = (s-2)*512 + tid).  Loads and LDS
// writes are branch-free so the compiler can count outstanding loads exactly:
// a slot with no chunk in this phase loads the tile's first weight chunk
// (always in bounds) and writes it to a dummy LDS slot.
struct ChunkMap {
  const uint8_t *W;
  const uint8_t *A;  // activations as bytes
  uint32_t N, K, M, n0;
};

__device__ __forceinline__ bool chunk_at(const ChunkMap &cm, uint32_t tid, int s, uint32_t p, uint32_t pbn,
                                         const uint8_t *&src, uint32_t &lds_off) {
  bool ok;
  const uint8_t *a;
  uint32_t off;
  if (s < 2) {  // s is a compile-time constant after unrolling
    const uint32_t r = tid >> 5, col = (tid & 31u) + 32u * s;
    ok = (col < pbn * 8u) && (cm.n0 + r < cm.N);
    a = cm.W + (size_t)(cm.n0 + r) * cm.K + (size_t)p * (kPhaseBlocks * 128) + 16u * col;
    off = r * kWPitch + 16u * col;
  } else {
    const uint32_t c = (uint32_t)(s - 2) * kThreads + tid;
    const uint32_t m = c >> 7, col = c & 127u;
    ok = (m < cm.M) && (col < pbn * 16u);
    a = cm.A + (size_t)m * cm.K * 2u + (size_t)p * (kPhaseBlocks * 256) + 16u * col;
    off = kWBytes + m * kAPitch + 16u * col;
  }
  src = ok ? a : cm.W + (size_t)cm.n0 * cm.K;
  lds_off = off;
  return ok;
}

template <int SLOTS>
__device__ __forceinline__ void issue_phase(const ChunkMap &cm, uint32_t tid, uint32_t p, uint32_t pbn,
                                            u32x4_t (&r)[SLOTS]) {
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const uint8_t *src;
    uint32_t off;
    chunk_at(cm, tid, s, p, pbn, src, off);
    r[s] = *reinterpret_cast<const u32x4_t *>(src);
  }
}

template <int SLOTS>
__device__ __forceinline__ void write_phase(const ChunkMap &cm, uint32_t tid, uint32_t p, uint32_t pbn,
                                            const u32x4_t (&r)[SLOTS], uint8_t *buf, uint8_t *dummy) {
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const uint8_t *src;
    uint32_t off;
    const bool ok = chunk_at(cm, tid, s, p, pbn, src, off);
    *reinterpret_cast<u32x4_t *>(ok ? buf + off : dummy) = r[s];
  }
}

__device__ __forceinline__ void mac_block(const uint8_t *buf, uint32_t lb, uint32_t i, uint32_t g, bool a_ok,
                                          float s, f32x4_t &outer) {
  const u32x4_t *pw = reinterpret_cast<const u32x4_t *>(buf + i * kWPitch + lb * 128u + 32u * g);
  const u32x4_t w0 = pw[0], w1 = pw[1];
  bf16x8_t a[4];
  if (a_ok) {
    const u32x4_t *pa = reinterpret_cast<const u32x4_t *>(buf + kWBytes + i * kAPitch + lb * 256u + 64u * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = __builtin_bit_cast(bf16x8_t, pa[j]);
  } else {
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = __builtin_bit_cast(bf16x8_t, z);
  }
  f32x4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], weights8(w0.x, w0.y), x, 0, 0, 0);
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], weights8(w0.z, w0.w), x, 0, 0, 0);
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], weights8(w1.x, w1.y), x, 0, 0, 0);
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], weights8(w1.z, w1.w), x, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) outer[r] = __fadd_rn(outer[r], __fmul_rn(s, x[r]));
}

template <int SLOTS>
__global__ __launch_bounds__(kThreads) void w8a16_gemm_m16_kernel(const uint16_t *__restrict__ A,
                                                                  const uint8_t *__restrict__ W,
                                                                  const float *__restrict__ S,
                                                                  uint16_t *__restrict__ C, uint32_t M,
                                                                  uint32_t N, uint32_t K) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t i = lane & 15u, g = lane >> 4;
  const uint32_t nb = K >> 7;
  const uint32_t nphase = (nb + kPhaseBlocks - 1) / kPhaseBlocks;
  const uint32_t buf_bytes = (uint32_t)buffer_bytes(M);  // two buffers, then a 16-byte dummy slot
  const ChunkMap cm{W, reinterpret_cast<const uint8_t *>(A), N, K, M, blockIdx.x * 16u};
  const float *srow = S + (size_t)(cm.n0 >> 7) * nb;
  const bool a_ok = i < M;

  f32x4_t outer = {0.0f, 0.0f, 0.0f, 0.0f};
  uint8_t *dummy = lds + 2u * buf_bytes;
  // Blocks in phase q; 0 past the end, which turns every slot into a safe
  // load that is written to the dummy slot.
  auto blocks_in = [&](uint32_t q) { return q < nphase ? min((uint32_t)kPhaseBlocks, nb - q * kPhaseBlocks) : 0u; };
  // One phase: store its chunks, request the phase kDepth ahead into the same
  // registers, then compute on it.  Loads are issued in a fixed order with no
  // branches around them, so each store waits only for its own phase's loads.
  auto step = [&](uint32_t p, u32x4_t(&r)[SLOTS]) {
    uint8_t *buf = lds + (p & 1u) * buf_bytes;
    const uint32_t pbn = blocks_in(p);
    write_phase<SLOTS>(cm, tid, p, pbn, r, buf, dummy);
    issue_phase<SLOTS>(cm, tid, p + kDepth, blocks_in(p + kDepth), r);
    __syncthreads();
    if (wave < pbn) mac_block(buf, wave, i, g, a_ok, srow[p * kPhaseBlocks + wave], outer);
  };

  u32x4_t ring[kDepth][SLOTS];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue_phase<SLOTS>(cm, tid, d, blocks_in(d), ring[d]);
  uint32_t p0 = 0;
  for (; p0 + kDepth <= nphase; p0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) step(p0 + d, ring[d]);
  }
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (p0 + d < nphase) step(p0 + d, ring[d]);

  // Accumulator layout: this lane holds rows m = 4g + r of weight row n0 + i.
  __syncthreads();
  float *part = reinterpret_cast<float *>(lds);  // [wave][m][n]
#pragma unroll
  for (int r = 0; r < 4; ++r) part[(wave * 16u + 4u * g + r) * 16u + i] = outer[r];
  __syncthreads();
  if (tid < 256u) {
    const uint32_t m = tid >> 4, col = tid & 15u;
    const uint32_t n = cm.n0 + col;
    if (m < M && n < N) {
      float v = part[m * 16u + col];
      for (uint32_t w = 1; w < kWaves; ++w) v = v + part[(w * 16u + m) * 16u + col];
      C[(size_t)m * N + n] = f32_to_bf16_rne(v);
    }
  }
}

template <int SLOTS>
hipError_t launch_slots(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                        uint32_t K, hipStream_t stream) {
  const size_t lds = 2 * (size_t)buffer_bytes((int)M) + 16;  // two buffers and the dummy slot
  static bool attr_set = false;  // one-time opt-in above the default LDS limit
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&w8a16_gemm_m16_kernel<SLOTS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(w8a16_gemm_m16_kernel<SLOTS>, dim3((N + 15) / 16), dim3(kThreads), lds, stream,
                     static_cast<const uint16_t *>(A), static_cast<const uint8_t *>(W), S,
                     static_cast<uint16_t *>(C), M, N, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w8a16_m16(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                            uint32_t K, hipStream_t stream) {
  if (M <= 4) return launch_slots<slots_for(4)>(A, W, S, C, M, N, K, stream);
  if (M <= 8) return launch_slots<slots_for(8)>(A, W, S, C, M, N, K, stream);
  return launch_slots<slots_for(16)>(A, W, S, C, M, N, K, stream);
}

}  // namespace wqd
