// Vector-ALU W8A16 decode GEMV for gfx950 (MI355X), up to 8 activation rows
// per launch.
//
//   C[m,n] = bf16( sum_b S[n/128][b] * inner(m, n, b) ),
//   inner(m, n, b) = fp32 sum of A[m,k] * W[n,k] over the 128 k of block b
//
// Operation: page "w8a16_gemm_m16.rs", module doc.  Beside its matrix-core
// kernel the page keeps a scalar GEMV (w8a16_gemv_batch16): one multiply-add
// per weight and activation row on the general-purpose ALUs, with bits that
// need not equal the matrix-core kernel's.  Scales as there: a block's 128
// products are summed in fp32, that sum is multiplied by the block's scale
// and the product added to the output's fp32 total; BF16 appears only at the
// store.  This is that scalar path, laid out for gfx950; it keeps its own
// fixed order (below), the same for every M.
//
// Work layout
//   * One workgroup of 8 waves per CU owns an even share [r0, r1) of the N
//     weight rows; wave w takes rows r0 + w, r0 + w + 8, ... in groups of
//     RPW rows (as many as the wave holds, up to 3).
//   * A weight row is read in chunks of 1024 k: lane l loads the 16 FP8
//     weights k0 = 1024c + 16l .. k0 + 15 with one 16-byte load, so every load
//     instruction covers 1 KB of consecutive bytes; lanes 8j .. 8j + 7 hold
//     block b = 8c + j.  Lanes past the end of the row load through an offset
//     beyond the buffer, which the hardware range check turns into zeros.
//   * Within a group the wave goes chunk-major (chunk c of each of the
//     group's rows, then chunk c + 1), with two groups' row-chunks of loads
//     in flight; they are issued once the activations are in LDS (issuing
//     them earlier delays the activations behind them).  The activations are staged once per workgroup in LDS, laid out
//     so that the two 16-byte reads of a lane's 16 activations are each
//     contiguous across the wave, and read into registers at the first row of
//     every chunk.
//   * Per row-chunk and activation row m: the 16 weights become 8 BF16 pairs
//     (hardware conversion, exact for every finite E4M3FN value) and
//     p = dot2(a, w, p) runs over the pairs in ascending k from zero
//     (v_dot2_f32_bf16: two products and the running fp32 sum per step).  The
//     8 lanes of a block then add their p in a butterfly (neighbour, pair,
//     other half of the 8), in which both partners compute the same sum, so
//     all 8 lanes hold the block's inner sum; its scale is folded once:
//     o_j = o_j + s_b * inner_b with j = b mod 8.
//   * After the row's last chunk the result is ((o_0 + o_1) + o_2) ... + o_7
//     over the 8 lane groups, stored as BF16 (round to nearest even).
//
// Every output's arithmetic is the same sequence whatever M is, so a row's
// bits do not depend on M.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "wqd_internal.h"

namespace wqd {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kWaves = 8;
constexpr uint32_t kThreads = 64 * kWaves;
constexpr uint32_t kChunkBytes = 2048;  // LDS bytes of one activation row's 1024-k chunk
constexpr uint32_t kPastEnd = 0x80000000u;
constexpr uint32_t kMaxRowsPerLaunch = 8;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <bool HI>
__device__ __forceinline__ bf16x2_t fp8x2_to_bf16x2(uint32_t v) {
  return __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI));
}

// x + (x of the lane selected by the DPP control); both lanes of a pair add
// the same two values, so they get the same bits.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i within 8

// f(integral_constant<D>) for D = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void unroll(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    unroll<B + 1, E>(f);
  }
}

struct ChunkRegs {
  u32x4_t w;  // 16 FP8 weights of one row-chunk
  float s;    // the scale of this lane's block
};

// RPW: rows per wave group; DEPTH: row-chunks of loads in flight per wave (a
// multiple of RPW, so a ring position always serves the same row slot)
template <int MMAX, int RPW, int DEPTH>
__global__ __launch_bounds__(kThreads) void w8a16_gemv_kernel(const uint16_t *__restrict__ A,
                                                              const uint8_t *__restrict__ W,
                                                              const float *__restrict__ S,
                                                              uint16_t *__restrict__ C, uint32_t M, uint32_t N,
                                                              uint32_t K, uint32_t lda, uint32_t ldc) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t nb = K >> 7;
  const uint32_t nchunk = (K + 1023u) >> 10;
  const uint32_t a_pitch = nchunk * kChunkBytes;

  // Activations into LDS: 16-byte piece p of chunk c of row m holds
  // A[m][1024c + 8p .. +7] at m * a_pitch + 2048c + 1024(p & 1) + 16(p >> 1),
  // zeros past K.  The first round of loads is requested before any other
  // set-up (the waves of a CU issue their scalar set-up one at a time).
  const uint32_t total = M * nchunk * 128u;
  auto piece = [&](uint32_t x, u32x4_t &v, uint32_t &dst) __attribute__((always_inline)) {
    uint32_t m = 0;  // x / (nchunk * 128) with MMAX - 1 compares (no division)
#pragma unroll
    for (int j = 1; j < MMAX; ++j) m += x >= (uint32_t)j * nchunk * 128u ? 1u : 0u;
    const uint32_t rest = x - m * (nchunk * 128u);
    const uint32_t c = rest >> 7, p = rest & 127u;
    const uint32_t k = 1024u * c + 8u * p;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    v = k < K ? *reinterpret_cast<const u32x4_t *>(A + (size_t)m * lda + k) : zero;
    dst = m * a_pitch + kChunkBytes * c + 1024u * (p & 1u) + 16u * (p >> 1);
  };
  constexpr int UA = 4;
  u32x4_t av[UA];
  uint32_t adst[UA];
  auto a_load = [&](uint32_t base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const uint32_t x = base + (uint32_t)u * kThreads + tid;
      if (x < total) piece(x, av[u], adst[u]);
    }
  };
  auto a_store = [&](uint32_t base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const uint32_t x = base + (uint32_t)u * kThreads + tid;
      if (x < total) *reinterpret_cast<u32x4_t *>(lds + adst[u]) = av[u];
    }
  };
  a_load(0u);

  uint32_t r0, r1;
  even_rows(N, blockIdx.x, gridDim.x, r0, r1);
  // rows of this wave: r0 + wave + 8t for t < nrows, in groups of RPW
  const uint32_t nrows = r1 - r0 > wave ? (r1 - r0 - wave + kWaves - 1u) / kWaves : 0u;
  const uint32_t ngroups = (nrows + RPW - 1u) / RPW;
  const uint32_t nq = ngroups * nchunk * RPW;  // row-chunks, padded to whole groups
  const uint32_t k_lane = 16u * lane;           // + 1024c: this lane's first k of a chunk

  // Work cursor: row slot t of group grp, chunk c.
  struct Cursor {
    uint32_t q, t, c, grp;
  };
  auto advance = [&](Cursor &cu) __attribute__((always_inline)) {
    ++cu.q;
    if (++cu.t == (uint32_t)RPW) {
      cu.t = 0;
      if (++cu.c == nchunk) {
        cu.c = 0;
        ++cu.grp;
      }
    }
  };
  Cursor ld = {0u, 0u, 0u, 0u};
  auto issue_next = [&]() __attribute__((always_inline)) {
    const uint32_t ti = ld.grp * RPW + ld.t;  // row index within the wave
    const bool live = ld.q < nq && ti < nrows;
    const uint32_t n = live ? r0 + wave + kWaves * ti : r0;
    const uint32_t k0 = 1024u * ld.c + k_lane;
    const bool in_row = live && k0 < K;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(W + (size_t)n * K), (short)0, (int)K, 0x00020000);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(S + (size_t)(n >> 7) * nb), (short)0, (int)(nb * 4u), 0x00020000);
    ChunkRegs r;
    r.w = __builtin_amdgcn_raw_buffer_load_b128(wr, in_row ? k0 : kPastEnd, 0, 0);
    r.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, in_row ? (k0 >> 7) * 4u : kPastEnd, 0, 0));
    advance(ld);
    return r;
  };

  static_assert(DEPTH % RPW == 0, "a ring position must always serve the same row slot");
  ChunkRegs ring[DEPTH];
  {
    a_store(0u);
    for (uint32_t base = UA * kThreads; base < total; base += UA * kThreads) {
      a_load(base);
      a_store(base);
    }
    __syncthreads();
    unroll<0, DEPTH>([&](auto d) __attribute__((always_inline)) { ring[decltype(d)::value] = issue_next(); });
  }

  float o[RPW][MMAX];    // o_j of this lane's group j for row slot t, activation row m
  uint32_t a[MMAX][8];    // this lane's 16 activations of the current chunk, as BF16 pairs
#pragma unroll
  for (int t = 0; t < RPW; ++t)
#pragma unroll
    for (int m = 0; m < MMAX; ++m) o[t][m] = 0.0f;

  Cursor cc = {0u, 0u, 0u, 0u};
  // T: the row slot of this ring position (the ring is a whole number of groups' slots)
  auto step = [&](ChunkRegs &r, auto T) __attribute__((always_inline)) {
    constexpr int t = decltype(T)::value;
    const uint32_t c = cc.c, grp = cc.grp;
    if (t == 0) {
      const uint8_t *src = lds + 2048u * c + 16u * lane;
#pragma unroll
      for (int m = 0; m < MMAX; ++m) {
        const uint32_t mm = (uint32_t)m < M ? (uint32_t)m : 0u;
        const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(src + mm * a_pitch);
        const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(src + mm * a_pitch + 1024u);
        a[m][0] = lo.x; a[m][1] = lo.y; a[m][2] = lo.z; a[m][3] = lo.w;
        a[m][4] = hi.x; a[m][5] = hi.y; a[m][6] = hi.z; a[m][7] = hi.w;
      }
    }
    bf16x2_t wb[8];
    wb[0] = fp8x2_to_bf16x2<false>(r.w.x);
    wb[1] = fp8x2_to_bf16x2<true>(r.w.x);
    wb[2] = fp8x2_to_bf16x2<false>(r.w.y);
    wb[3] = fp8x2_to_bf16x2<true>(r.w.y);
    wb[4] = fp8x2_to_bf16x2<false>(r.w.z);
    wb[5] = fp8x2_to_bf16x2<true>(r.w.z);
    wb[6] = fp8x2_to_bf16x2<false>(r.w.w);
    wb[7] = fp8x2_to_bf16x2<true>(r.w.w);
#pragma unroll
    for (int m = 0; m < MMAX; ++m) {
      float p = 0.0f;
#pragma unroll
      for (int h = 0; h < 8; ++h) p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[m][h]), wb[h], p, false);
      p = add_dpp<kDppXor1>(p);
      p = add_dpp<kDppXor2>(p);
      p = add_dpp<kDppHalfMirror>(p);
      o[t][m] = __fadd_rn(o[t][m], __fmul_rn(r.s, p));
    }
    // the ring entry is refilled only once its scale has been used: a copy
    // kept across the request made the compiler move the new scale into the
    // ring's register at the loop's end, waiting for that load there
    // (measured on MI355X: N = K = 5120 M = 1 7.01 -> 6.86 us, M = 2 8.00 ->
    // 7.69, N = 17408 M = 1 18.4 -> 17.9, K = 17408 M = 1 18.6 -> 17.9)
    r = issue_next();
    advance(cc);
    if (t == RPW - 1 && c + 1u == nchunk) {  // the group's rows are complete
#pragma unroll
      for (int tt = 0; tt < RPW; ++tt) {
        const uint32_t ti = grp * RPW + tt;
        const uint32_t n = r0 + wave + kWaves * ti;
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
          float v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, o[tt][m]), 0));
#pragma unroll
          for (int j = 1; j < 8; ++j)
            v = v + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, o[tt][m]), 8 * j));
          if (lane == 0u && ti < nrows && (uint32_t)m < M) C[(size_t)m * ldc + n] = f32_to_bf16_rne(v);
          o[tt][m] = 0.0f;
        }
      }
    }
  };

  while (cc.q + DEPTH <= nq)
    unroll<0, DEPTH>([&](auto d) __attribute__((always_inline)) {
      constexpr int D = decltype(d)::value;
      step(ring[D], std::integral_constant<int, D % RPW>{});
    });
  // the rest is a whole number of groups (nq is a multiple of RPW)
  unroll<0, DEPTH>([&](auto d) __attribute__((always_inline)) {
    constexpr int D = decltype(d)::value;
    if (cc.q < nq) step(ring[D], std::integral_constant<int, D % RPW>{});
  });
}

// Workgroups: one per CU, at least 8 rows (one per wave) each.
uint32_t gemv_grid(uint32_t N, int cus) {
  const uint32_t by_rows = (N + kWaves - 1u) / kWaves;
  return by_rows < (uint32_t)cus ? by_rows : (uint32_t)cus;
}

template <int MMAX, int RPW>
hipError_t launch_cfg(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N, uint32_t K,
                      uint32_t lda, uint32_t ldc, size_t lds, uint32_t grid, hipStream_t stream) {
  constexpr auto kern = w8a16_gemv_kernel<MMAX, RPW, 2 * RPW>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, stream, static_cast<const uint16_t *>(A),
                     static_cast<const uint8_t *>(W), S, static_cast<uint16_t *>(C), M, N, K, lda, ldc);
  return hipGetLastError();
}

// Row groups as wide as a wave's share of rows, up to 3 (wider groups would
// mostly pad: a wave holds N / (8 * CUs) rows, 2.5 for N = 5120 on 256 CUs),
// with two groups' row-chunks in flight.
template <int MMAX>
hipError_t launch_mmax(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N, uint32_t K,
                       uint32_t lda, uint32_t ldc, size_t lds, hipStream_t stream) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus = n > 0 ? n : 1;
  }
  const uint32_t grid = gemv_grid(N, cus);
  const uint32_t rows_per_wave = ((N + grid - 1u) / grid + kWaves - 1u) / kWaves;
  if (rows_per_wave <= 1u) return launch_cfg<MMAX, 1>(A, W, S, C, M, N, K, lda, ldc, lds, grid, stream);
  if (rows_per_wave <= 2u) return launch_cfg<MMAX, 2>(A, W, S, C, M, N, K, lda, ldc, lds, grid, stream);
  return launch_cfg<MMAX, 3>(A, W, S, C, M, N, K, lda, ldc, lds, grid, stream);
}

}  // namespace

uint32_t w8a16_gemv_rows_per_launch(uint32_t K) {
  const uint32_t per_row = ((K + 1023u) >> 10) * kChunkBytes;
  const uint32_t fit = (160u * 1024u) / per_row;
  return fit < kMaxRowsPerLaunch ? fit : kMaxRowsPerLaunch;
}

hipError_t launch_w8a16_gemv(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                             uint32_t K, uint32_t lda, uint32_t ldc, hipStream_t stream) {
  const size_t lds = (size_t)M * ((K + 1023u) >> 10) * kChunkBytes;
  if (M <= 1) return launch_mmax<1>(A, W, S, C, M, N, K, lda, ldc, lds, stream);
  if (M <= 2) return launch_mmax<2>(A, W, S, C, M, N, K, lda, ldc, lds, stream);
  if (M <= 4) return launch_mmax<4>(A, W, S, C, M, N, K, lda, ldc, lds, stream);
  return launch_mmax<8>(A, W, S, C, M, N, K, lda, ldc, lds, stream);
}

}  // namespace wqd
