// Q2_0 ternary decode GEMV / batched GEMV for gfx950 (MI355X).
//
//   C[m,n] = bf16( sum_k A[m,k] * (code[n,k] - 1) * d[n, k/128] ),  m < MC <= 8
//
// Operation: page "gemv_q2_vec.rs", docs of q2_0_gemv_vec (M=1: A staged in
// shared memory, 16 codes per 32-bit word, dequant (code-1)*d inside the dot
// product) and q2_0_gemv_vec_batchm (each weight word read once and applied to
// all rows; every row bit-identical to the M=1 kernel).  The pages' thread map
// (one 32-lane warp per row, 8 rows per CTA) is not used; this kernel is laid
// out for 64-lane waves as described below.
//
// Work layout
//   * A workgroup is kWaves waves and owns kRowsPerWave*kWaves weight rows.
//     Lane l of a wave works on row l/8 and on the blocks b = (l%8) + 8i of
//     that row, so the 8 lanes of a row read 8 consecutive 34-byte blocks and
//     all rows of the wave read the same activation slice (LDS broadcast).
//   * Each lane loads a whole block with three dword-aligned loads (9 dwords
//     starting at the block's offset rounded down to 4 bytes), then extracts
//     the 8 code words with one v_perm each.  Every load stays inside the
//     buffer: an odd-offset block starts 2 bytes after a dword boundary whose
//     first half belongs to the previous block, and the final block of the
//     buffer reads its last dword as 16 bits when it ends mid-dword.
//   * Decode: for a code word w, (w >> 2s) & 0x03030303 puts codes s, s+4,
//     s+8, s+12 into the four bytes; read as FP8 E4M3 those bytes are 0,
//     2^-9, 2*2^-9, 3*2^-9, so the hardware FP8->BF16 conversion with scale
//     2^9 turns each byte pair into an exact BF16 pair (c_i, c_j).  Two
//     conversions per masked word, eight per 16 codes.
//   * MAC: v_dot2c_f32_bf16 against a permuted copy of the activations
//     (A' dword e of a word pairs the two activations whose codes the e-th
//     conversion produced), so no per-element shuffle happens in the loop.
//     The chain computes sum a*c over the block starting from -sum a, which
//     equals sum a*(c-1); the block's scale d is then applied once:
//     acc += d * chain.  Products a*c are exact (c in {0,1,2,3}).
//   * Activations: each workgroup stages A' and the per-block sums of A for
//     a tile of 128-K blocks in LDS (blocks padded to 68 dwords so the eight
//     block slots of a wave fall in distinct banks).
//   * The 8 lane partials of a row are added by a fixed xor-butterfly and the
//     row is stored as BF16, round to nearest even.
//
// Bit-identity across row counts: a row's arithmetic (its block sums of A,
// its dot2 chains, its fma order and the butterfly) does not depend on MC or
// on the other rows, so batched rows equal the M=1 launch bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wqd_internal.h"

namespace wqd {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct __attribute__((aligned(4))) u32x4a4 { uint32_t x, y, z, w; };
struct __attribute__((aligned(16))) u32x4 { uint32_t x, y, z, w; };

constexpr int kBlockBytes = 34;
constexpr int kRowsPerWave = 8;
constexpr int kWaves = 2;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWG = kRowsPerWave * kWaves;
constexpr int kApStride = 68;                  // dwords of A' per block (64 + 4 pad)
constexpr int kLdsBytesPerRowBlock = kApStride * 4 + 4;  // A' + one block sum
constexpr int kLdsBudget = 64 * 1024;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ float dot2(uint32_t a, bf16x2_t t, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), t, c, false);
}

// One 34-byte block as 9 dwords plus the selectors that undo its 0/2-byte
// misalignment.
struct Block {
  uint32_t w[8];
  uint32_t lo, hi;  // the two halves of the ninth dword (w[8] = lo | hi << 16)
  uint32_t sel;     // v_perm selector yielding code word q from (w[q+1], w[q])
  uint32_t dsh;     // shift of the fp16 scale inside w[0]
};

__device__ __forceinline__ void load_block(const uint8_t *__restrict__ B, uint64_t off,
                                           uint64_t total, Block &k) {
  const uint64_t o4 = off & ~uint64_t(3);
  const uint32_t *p = reinterpret_cast<const uint32_t *>(B + o4);
  const u32x4a4 v0 = *reinterpret_cast<const u32x4a4 *>(p);
  const u32x4a4 v1 = *reinterpret_cast<const u32x4a4 *>(p + 4);
  k.w[0] = v0.x; k.w[1] = v0.y; k.w[2] = v0.z; k.w[3] = v0.w;
  k.w[4] = v1.x; k.w[5] = v1.y; k.w[6] = v1.z; k.w[7] = v1.w;
  // The ninth dword as two halves, with no branch and combined only where it
  // is used (combining here would wait for these loads).  Only an odd block
  // (starting 2 bytes into a dword) uses the upper half; the buffer's last
  // block can end 2 bytes into this dword only when it is even, and then its
  // upper half is read from an in-range address and never used.
  const uint16_t *h = reinterpret_cast<const uint16_t *>(B);
  k.lo = h[(o4 + 32) >> 1];
  k.hi = h[(min(o4 + 34, total - 2)) >> 1];
  const bool odd = (off & 2) != 0;
  k.sel = odd ? 0x07060504u : 0x05040302u;
  k.dsh = odd ? 16u : 0u;
}

// Stage A' and the block sums of A for blocks [kb0, kb0+tcount) of rows 0..MC-1.
// Work item = one 16-element word of one row; the 8 words of a block sit in 8
// consecutive lanes so their partial sums combine with a fixed butterfly.
template <int MC>
__device__ __forceinline__ void stage_tile(const uint16_t *__restrict__ A, uint32_t K, uint32_t kb0,
                                           uint32_t tcount, uint32_t tb, uint32_t *ap, float *asum) {
  const uint32_t per_row = tcount * 8;
  const uint32_t items = MC * per_row;
  for (uint32_t base = 0; base < items; base += kThreads) {
    const uint32_t it = base + threadIdx.x;
    const bool valid = it < items;
    float ps = 0.0f;
    uint32_t m = 0, bl = 0, q = 0;
    if (valid) {
      m = it / per_row;
      const uint32_t rem = it - m * per_row;
      bl = rem >> 3;
      q = rem & 7;
      const uint16_t *src = A + (size_t)m * K + (size_t)(kb0 + bl) * 128 + q * 16;
      const u32x4 r0 = *reinterpret_cast<const u32x4 *>(src);
      const u32x4 r1 = *reinterpret_cast<const u32x4 *>(src + 8);
      // r[i] holds (a_{2i}, a_{2i+1}); A' pairs follow the conversion order
      // (0,4) (8,12) (1,5) (9,13) (2,6) (10,14) (3,7) (11,15).
      u32x4 o0, o1;
      o0.x = __builtin_amdgcn_perm(r0.z, r0.x, 0x05040100u);  // a0, a4
      o0.y = __builtin_amdgcn_perm(r1.z, r1.x, 0x05040100u);  // a8, a12
      o0.z = __builtin_amdgcn_perm(r0.z, r0.x, 0x07060302u);  // a1, a5
      o0.w = __builtin_amdgcn_perm(r1.z, r1.x, 0x07060302u);  // a9, a13
      o1.x = __builtin_amdgcn_perm(r0.w, r0.y, 0x05040100u);  // a2, a6
      o1.y = __builtin_amdgcn_perm(r1.w, r1.y, 0x05040100u);  // a10, a14
      o1.z = __builtin_amdgcn_perm(r0.w, r0.y, 0x07060302u);  // a3, a7
      o1.w = __builtin_amdgcn_perm(r1.w, r1.y, 0x07060302u);  // a11, a15
      uint32_t *dst = ap + ((size_t)m * tb + bl) * kApStride + q * 8;
      *reinterpret_cast<u32x4 *>(dst) = o0;
      *reinterpret_cast<u32x4 *>(dst + 4) = o1;
      const uint32_t r[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ps = ps + bf16_lo(r[i]);
        ps = ps + bf16_hi(r[i]);
      }
    }
    ps = ps + __shfl_xor(ps, 1);
    ps = ps + __shfl_xor(ps, 2);
    ps = ps + __shfl_xor(ps, 4);
    if (valid && q == 0) asum[(size_t)m * tb + bl] = ps;
  }
}

template <int MC>
__device__ __forceinline__ void mac_block(const Block &k, const uint32_t *ap, const float *asum,
                                          uint32_t tb, uint32_t bl, float (&acc)[MC]) {
  const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)((k.w[0] >> k.dsh) & 0xffffu));
  float s[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) s[m] = -asum[(size_t)m * tb + bl];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t w = __builtin_amdgcn_perm(q == 7 ? (k.lo | (k.hi << 16)) : k.w[q + 1], k.w[q], k.sel);
    const uint32_t x0 = w & 0x03030303u;
    const uint32_t x1 = (w >> 2) & 0x03030303u;
    const uint32_t x2 = (w >> 4) & 0x03030303u;
    const uint32_t x3 = (w >> 6) & 0x03030303u;
    const bf16x2_t t0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 512.0f, false);
    const bf16x2_t t1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 512.0f, true);
    const bf16x2_t t2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 512.0f, false);
    const bf16x2_t t3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 512.0f, true);
    const bf16x2_t t4 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x2, 512.0f, false);
    const bf16x2_t t5 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x2, 512.0f, true);
    const bf16x2_t t6 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x3, 512.0f, false);
    const bf16x2_t t7 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x3, 512.0f, true);
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const uint32_t *a = ap + ((size_t)m * tb + bl) * kApStride + q * 8;
      const u32x4 a0 = *reinterpret_cast<const u32x4 *>(a);
      const u32x4 a1 = *reinterpret_cast<const u32x4 *>(a + 4);
      float c = s[m];
      c = dot2(a0.x, t0, c);
      c = dot2(a0.y, t1, c);
      c = dot2(a0.z, t2, c);
      c = dot2(a0.w, t3, c);
      c = dot2(a1.x, t4, c);
      c = dot2(a1.y, t5, c);
      c = dot2(a1.z, t6, c);
      c = dot2(a1.w, t7, c);
      s[m] = c;
    }
  }
#pragma unroll
  for (int m = 0; m < MC; ++m) acc[m] = __builtin_fmaf(s[m], d, acc[m]);
}

template <int MC>
__global__ __launch_bounds__(kThreads) void q2_0_gemv_kernel(const uint16_t *__restrict__ A,
                                                             const uint8_t *__restrict__ B,
                                                             uint16_t *__restrict__ C, uint32_t N,
                                                             uint32_t K, uint32_t tb) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint32_t *ap = lds;
  float *asum = reinterpret_cast<float *>(lds + (size_t)MC * tb * kApStride);

  const uint32_t nb = K >> 7;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t j = lane & 7u;
  const uint32_t n = blockIdx.x * kRowsPerWG + wave * kRowsPerWave + (lane >> 3);
  const bool row_ok = n < N;
  const uint64_t total = (uint64_t)N * nb * kBlockBytes;
  const uint64_t row_off = (uint64_t)(row_ok ? n : 0) * nb * kBlockBytes;

  float acc[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) acc[m] = 0.0f;

  // Lane j's blocks of a tile are j, j + 8, ...: two of them in flight, each
  // refilled in place after its MAC.  A lane whose block lies past the
  // tile's last re-reads that last block (never used), so no request sits
  // behind a per-lane branch; requests past the tile's last round of 8
  // blocks are skipped (a condition the same for every lane).  Measured on
  // MI355X against one block ahead with the requests behind per-lane branches
  // (a register copy per block that waited for its request): N = 5120,
  // K = 5248 M = 1 10.1 -> 9.4 us, M = 8 34.2 -> 33.2, and with the kernel
  // forced, N = K = 5120 M = 1 9.1 -> 8.1, K = 17408 26.2 -> 23.1; small K
  // unchanged (N = 32768 K = 512 4.44 against 4.49).
  for (uint32_t kb0 = 0; kb0 < nb; kb0 += tb) {
    const uint32_t tcount = min(tb, nb - kb0);
    const uint32_t nk = (tcount + 7u) / 8u;  // rounds of 8 blocks (uniform)
    auto fetch = [&](uint32_t bl, Block &k) __attribute__((always_inline)) {
      load_block(B, row_off + (uint64_t)(kb0 + min(bl, tcount - 1u)) * kBlockBytes, total, k);
    };
    Block ring[2];
    fetch(j, ring[0]);
    if (nk > 1u) fetch(j + 8u, ring[1]);
    __syncthreads();  // all readers of the previous tile are done
    stage_tile<MC>(A, K, kb0, tcount, tb, ap, asum);
    __syncthreads();
    for (uint32_t k = 0; k < nk; k += 2u) {
      const uint32_t bl0 = j + 8u * k, bl1 = bl0 + 8u;
      if (row_ok && bl0 < tcount) mac_block<MC>(ring[0], ap, asum, tb, bl0, acc);
      if (k + 2u < nk) fetch(bl0 + 16u, ring[0]);
      if (k + 1u < nk) {
        if (row_ok && bl1 < tcount) mac_block<MC>(ring[1], ap, asum, tb, bl1, acc);
        if (k + 3u < nk) fetch(bl1 + 16u, ring[1]);
      }
    }
  }

#pragma unroll
  for (int m = 0; m < MC; ++m) {
    float v = acc[m];
    v = v + __shfl_xor(v, 1);
    v = v + __shfl_xor(v, 2);
    v = v + __shfl_xor(v, 4);
    acc[m] = v;
  }
  if (row_ok && j == 0) {
#pragma unroll
    for (int m = 0; m < MC; ++m) C[(size_t)m * N + n] = f32_to_bf16_rne(acc[m]);
  }
}

template <int MC>
hipError_t launch_mc(const void *A, const void *B, void *C, uint32_t N, uint32_t K, hipStream_t stream) {
  const uint32_t nb = K >> 7;
  const uint32_t cap = (uint32_t)(kLdsBudget / (MC * kLdsBytesPerRowBlock)) / 8 * 8;
  const uint32_t need = (nb + 7) / 8 * 8;
  const uint32_t tb = need < cap ? need : cap;
  const size_t lds = (size_t)MC * tb * kLdsBytesPerRowBlock;
  const dim3 grid((N + kRowsPerWG - 1) / kRowsPerWG);
  hipLaunchKernelGGL(q2_0_gemv_kernel<MC>, grid, dim3(kThreads), lds, stream,
                     static_cast<const uint16_t *>(A), static_cast<const uint8_t *>(B),
                     static_cast<uint16_t *>(C), N, K, tb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q2_0_valu(const void *A, const void *B, void *C, uint32_t N, uint32_t K, uint32_t m,
                       hipStream_t stream) {
  switch (m) {
    case 1: return launch_mc<1>(A, B, C, N, K, stream);
    case 2: return launch_mc<2>(A, B, C, N, K, stream);
    case 3: return launch_mc<3>(A, B, C, N, K, stream);
    case 4: return launch_mc<4>(A, B, C, N, K, stream);
    case 5: return launch_mc<5>(A, B, C, N, K, stream);
    case 6: return launch_mc<6>(A, B, C, N, K, stream);
    case 7: return launch_mc<7>(A, B, C, N, K, stream);
    case 8: return launch_mc<8>(A, B, C, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wqd
