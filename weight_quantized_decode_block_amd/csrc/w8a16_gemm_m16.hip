// W8A16 decode GEMM with a 16-row M tile for gfx950 (MI355X).
//
//   C[m,n] = bf16( sum_b S[n/128][b] * sum_{k in block b} A[m,k] * W[n,k] ),  m < M <= 16
//
// Operation: page "w8a16_gemm_m16.rs", module doc (FP8 E4M3 weights [N,K]
// with FP32 scales [N/128, K/128]: each 128-K block's fp32 sum is multiplied
// by its scale once and added to the output's fp32 total, with no scaling of
// single products and no BF16 intermediate; the M tile is the matrix
// instruction's 16 rows) and the doc of w8a16_gemm_m16 (BF16 A [m,k],
// BF16 C [m,n], rows >= m untouched).  The pages' Hopper design (mma.sync
// m16n8k16, 32 columns and 128 threads per CTA, A staged with cp.async) is
// not used.
//
// Four kernels give the same bits (the same blocks per wave, chains and
// reduction order) and are chosen by shape (launch_w8a16_m16 at the end):
// the units kernel (up to 8 rows, activations resident in LDS), the
// segmented kernel (large activations, and 9..16 rows; a 16-wave form of it
// for 9..16 rows over three to five tiles), the registers kernel
// (9..16 rows over more than five tiles per workgroup, K <= 5120), and the
// per-phase kernel described next, for what the others cannot address
// (weights of 2 GB and more, very wide activation row pitches).
//
// Per-phase work layout
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

#include <type_traits>

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

// f(integral_constant<D>) for D = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void unroll(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    unroll<B + 1, E>(f);
  }
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
  uint32_t N, K, M, n0, lda;  // lda: A row pitch in elements
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
    a = cm.A + (size_t)m * cm.lda * 2u + (size_t)p * (kPhaseBlocks * 256) + 16u * col;
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
                                                                  uint32_t N, uint32_t K, uint32_t lda,
                                                                  uint32_t ldc, uint32_t band) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t i = lane & 15u, g = lane >> 4;
  const uint32_t nb = K >> 7;
  const uint32_t nphase = (nb + kPhaseBlocks - 1) / kPhaseBlocks;
  const uint32_t buf_bytes = (uint32_t)buffer_bytes(M);  // two buffers, then a 16-byte dummy slot
  // tiles of this workgroup: `band` consecutive 16-row tiles from blockIdx.x * band
  const uint32_t ntiles = (N + 15u) >> 4;
  const uint32_t t_end = min(blockIdx.x * band + band, ntiles);
  for (uint32_t t = blockIdx.x * band; t < t_end; ++t) {
    const ChunkMap cm{W, reinterpret_cast<const uint8_t *>(A), N, K, M, 16u * t, lda};
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
        C[(size_t)m * ldc + n] = f32_to_bf16_rne(v);
      }
    }
    __syncthreads();  // the partials sit in buffer 0, which the next tile's first phase overwrites
  }
}

template <int SLOTS>
hipError_t launch_slots(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                        uint32_t K, uint32_t lda, uint32_t ldc, uint32_t band, hipStream_t stream) {
  const size_t lds = 2 * (size_t)buffer_bytes((int)M) + 16;  // two buffers and the dummy slot
  static bool attr_set = false;  // one-time opt-in above the default LDS limit
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&w8a16_gemm_m16_kernel<SLOTS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const uint32_t ntiles = (N + 15u) / 16u;
  if (band == 0u) band = 1u;  // one tile per workgroup
  hipLaunchKernelGGL(w8a16_gemm_m16_kernel<SLOTS>, dim3((ntiles + band - 1u) / band), dim3(kThreads), lds, stream,
                     static_cast<const uint16_t *>(A), static_cast<const uint8_t *>(W), S,
                     static_cast<uint16_t *>(C), M, N, K, lda, ldc, band);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Resident-activation kernel (the usual decode case, when all M rows of A fit
// in LDS): same arithmetic, block order and reduction order as the kernel
// above, so both give the same bits.  Weight bytes go straight from memory to
// the lanes that use them, and each wave works on its own blocks without
// waiting for the others until the end of a tile.
//   * A workgroup of 8 waves owns a contiguous range of weight rows and walks
//     it in tiles of 16 rows (the last one may be partial); wave w owns
//     blocks w, w + 8, ... of every tile.  The ranges are either an even
//     split of the N rows over the grid (one workgroup per CU, so every CU
//     streams the same number of bytes: with 16-row tiles dealt out whole,
//     5120 rows are 320 tiles and a quarter of the CUs would stream twice as
//     much as the rest), or bands of 16 * band rows.
//   * Per block, lane (i, g) loads the 32 weights k = 32g..32g+31 of row
//     n0 + i (two 16-byte buffer loads; a lane whose row lies outside the
//     range gives an offset past the end of the buffer, which the hardware
//     range check turns into zeros without a memory access) and the block's
//     scale for that row (4 bytes), DEPTH blocks ahead of the compute.
//   * Activations are copied into LDS once per workgroup; lane (i, g) reads
//     its 64 bytes of row i (rows i >= M read row 0 and feed outputs that are
//     never stored).
//   * At the end of a tile the 8 waves' accumulators are added in LDS in wave
//     order and rows m < M are stored.
// ---------------------------------------------------------------------------
// Buffer offset of a lane with no row: beyond every weight buffer the kernel
// accepts (N * K < 2^31), and still below 2^32 after adding a block offset.
constexpr uint32_t kPastEnd = 0x80000000u;

struct UnitRegs {
  u32x4_t w0, w1;  // this lane's 32 FP8 weights of the block
  float s;         // the block's scale
};

// Scale floats the units kernel can hold in LDS: the scale rows covering a
// workgroup's weight rows.
constexpr uint32_t kUnitScales = 512;

template <int MMAX>
struct UnitLayout {
  static constexpr int kPart = 0;  // [tile parity][wave][m][16] floats
  static constexpr int kS = kPart + 2 * kWaves * MMAX * 16 * 4;  // [scale row - g0][block] floats
  static constexpr int kA = kS + (int)kUnitScales * 4;
};

template <int MMAX>
constexpr size_t unit_lds_bytes(uint32_t M, uint32_t K) {
  return (size_t)UnitLayout<MMAX>::kA + (size_t)M * (2u * K + 16u);
}

template <int MMAX, int DEPTH, int UA, bool SL>
__global__ __launch_bounds__(kThreads) void w8a16_units_kernel(const uint16_t *__restrict__ A,
                                                               const uint8_t *__restrict__ W,
                                                               const float *__restrict__ S,
                                                               uint16_t *__restrict__ C, uint32_t M, uint32_t N,
                                                               uint32_t K, uint32_t lda, uint32_t ldc,
                                                               uint32_t band) {
  using L = UnitLayout<MMAX>;
  constexpr int NF = MMAX < 4 ? MMAX : 4;  // accumulator rows that can hold outputs
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t i = lane & 15u, g = lane >> 4;
  const uint32_t nb = K >> 7;
  const uint32_t a_pitch = 2u * K + 16u;

  // A into LDS while the first DEPTH blocks are in flight; its first round is
  // requested before any other set-up.  Chunk c: row m = c / cpr, counted
  // with MMAX - 1 compares (no division); idle slots re-read chunk 0 and
  // write into the partials.
  const uint32_t cpr = K >> 3;
  const uint32_t total = M * cpr;
  u32x4_t av[UA];
  uint32_t adst[UA];
  auto a_load = [&](uint32_t base) {
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const uint32_t c = base + (uint32_t)u * kThreads + tid;
      const bool in = c < total;
      const uint32_t cc = in ? c : 0u;
      uint32_t m = 0;
#pragma unroll
      for (int x = 1; x < MMAX; ++x) m += cc >= (uint32_t)x * cpr ? 1u : 0u;
      const uint32_t col = cc - m * cpr;
      av[u] = *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const uint8_t *>(A) + (size_t)m * lda * 2u +
                                                 16u * col);
      adst[u] = in ? L::kA + m * a_pitch + 16u * col : (uint32_t)L::kPart;
    }
  };
  a_load(0u);

  // rows [r0, r1) of this workgroup: an even split over the grid (band = 0) or
  // 16 * band rows from blockIdx.x * 16 * band
  uint32_t r0, r1;
  if (band == 0u) {
    even_rows(N, blockIdx.x, gridDim.x, r0, r1);
  } else {
    r0 = blockIdx.x * 16u * band;
    r1 = min(r0 + 16u * band, N);
  }
  const uint32_t my_tiles = (r1 - r0 + 15u) >> 4;
  // SL: the scale rows of rows [r0, r1), at most kUnitScales floats (the
  // launcher checks), requested now and kept in LDS for the whole launch, so
  // the weight requests carry no 4-byte scale requests beside them
  const uint32_t g0 = r0 >> 7;
  const uint32_t nsc = SL ? (((r1 - 1u) >> 7) - g0 + 1u) * nb : 0u;
  float sv = 0.0f;
  if constexpr (SL) {
    if (tid < nsc) sv = S[g0 * nb + tid];
  }
  // blocks of a tile owned by this wave: wave, wave + 8, ...; a wave that
  // owns none (K < 1024) runs one empty unit per tile to meet the barrier
  const uint32_t upw = nb > wave ? (nb - wave + kWaves - 1) / kWaves : 1u;
  const uint32_t nq = my_tiles * upw;

  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(W), (short)0, (int)(N * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(S), (short)0, (int)(((N + 127u) >> 7) * nb * 4u), 0x00020000);

  struct Cursor {
    uint32_t q, u, j, n0;  // unit, block index within the tile's share, tile index, tile's first row
  };
  auto advance = [&](Cursor &c) {
    ++c.q;
    if (++c.u == upw) {
      c.u = 0;
      ++c.j;
      c.n0 += 16u;
    }
  };
  Cursor ld = {0u, 0u, 0u, r0};
  const uint32_t w_lane = 32u * g;
  auto issue_next = [&]() {
    const bool live = ld.q < nq;
    const uint32_t b = min(wave + kWaves * ld.u, nb - 1u);
    const uint32_t n0 = live ? ld.n0 : r0;
    const uint32_t row = n0 + i;
    // past the wave's last unit the loads fall outside the buffer (the range
    // check returns zeros without a memory access; re-reading the first
    // tile's weights, long evicted from L2 at large N, cost 10-15 % more HBM
    // traffic and the wait for it: N = 17408, K = 5120, M = 1 19.1 -> 18.2 us)
    const uint32_t voff = (live && row < r1) ? row * K + w_lane : kPastEnd;
    const uint32_t soff = 128u * b;
    UnitRegs r;
    r.w0 = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff, soff, 0);
    r.w1 = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff + 16u, soff, 0);
    if constexpr (SL) {
      r.s = 0.0f;
    } else {
      // the scale of this lane's own row: a tile need not sit inside one 128-row scale group
      const uint32_t srow = (row < r1 ? row : r1 - 1u) >> 7;
      r.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srsrc, live ? srow * nb * 4u : kPastEnd, 4u * b, 0));
    }
    advance(ld);
    return r;
  };

  const uint32_t a_lane = (i < M ? i : 0u) * a_pitch + 64u * g;  // + L::kA + 256 per block
  float *part = reinterpret_cast<float *>(lds + L::kPart);

  UnitRegs ring[DEPTH];
  {
    auto a_store = [&]() {
#pragma unroll
      for (int u = 0; u < UA; ++u) *reinterpret_cast<u32x4_t *>(lds + adst[u]) = av[u];
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) ring[d] = issue_next();
    a_store();
    if constexpr (SL) {
      if (tid < nsc) reinterpret_cast<float *>(lds + L::kS)[tid] = sv;
    }
    for (uint32_t base = UA * kThreads; base < total; base += UA * kThreads) {
      a_load(base);
      a_store();
    }
    __syncthreads();
  }

  f32x4_t outer = {0.0f, 0.0f, 0.0f, 0.0f};
  auto unit = [&](const UnitRegs &r, uint32_t b, uint32_t n0) {
    float sc = r.s;
    if constexpr (SL) {  // this lane's row's scale, from LDS
      const uint32_t row = n0 + i;
      const uint32_t srow = (row < r1 ? row : r1 - 1u) >> 7;
      sc = reinterpret_cast<const float *>(lds + L::kS)[(srow - g0) * nb + b];
    }
    const uint8_t *act = lds + L::kA + a_lane + 256u * b;
    bf16x8_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const bf16x8_t *>(act + 16 * j);
    f32x4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
    x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], weights8(r.w0.x, r.w0.y), x, 0, 0, 0);
    x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], weights8(r.w0.z, r.w0.w), x, 0, 0, 0);
    x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], weights8(r.w1.x, r.w1.y), x, 0, 0, 0);
    x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], weights8(r.w1.z, r.w1.w), x, 0, 0, 0);
#pragma unroll
    for (int rr = 0; rr < NF; ++rr) outer[rr] = __fadd_rn(outer[rr], __fmul_rn(sc, x[rr]));
  };

  Cursor cc = {0u, 0u, 0u, r0};
  auto step = [&](UnitRegs &r) {
    const uint32_t j = cc.j, u = cc.u, n0 = cc.n0;
    const uint32_t b = wave + kWaves * u;
    if (b < nb) unit(r, b, n0);
    r = issue_next();
    advance(cc);
    if (u + 1u == upw) {  // tile done: add the 8 waves' partial tiles in wave order
      const uint32_t par = j & 1u;
#pragma unroll
      for (int rr = 0; rr < NF; ++rr) {
        const uint32_t m = 4u * g + rr;
        if (m < M) part[((par * kWaves + wave) * MMAX + m) * 16u + i] = outer[rr];
      }
      outer = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
      __syncthreads();
      if (tid < M * 16u) {
        const uint32_t m = tid >> 4, col = tid & 15u;
        const uint32_t n = n0 + col;
        if (n < r1) {
          const float *pp = part + (par * kWaves * MMAX + m) * 16u + col;
          float v = pp[0];
          for (uint32_t w = 1; w < kWaves; ++w) v = v + pp[w * MMAX * 16u];
          C[(size_t)m * ldc + n] = f32_to_bf16_rne(v);
        }
      }
      // this parity's partials are next written after the following tile's barrier
    }
  };

  while (cc.q + DEPTH <= nq) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) step(ring[d]);
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (cc.q < nq) step(ring[d]);
}

// Launches KERN with one workgroup per 64-row band (band > 0), or with
// kUnitWgsPerCu workgroups per CU (fewer if registers or LDS do not allow it,
// and never fewer than 16 rows per workgroup) splitting the rows evenly.
constexpr int kUnitWgsPerCu = 1;  // two measured slower on MI355X (N = K = 5120, M = 1: 7.98 -> 10.5 us)

template <auto KERN>
hipError_t launch_units(size_t lds, uint32_t ntiles, uint32_t band, hipStream_t stream, const uint16_t *a,
                        const uint8_t *w, const float *s, uint16_t *c, uint32_t M, uint32_t N, uint32_t K,
                        uint32_t lda, uint32_t ldc) {
  struct Res {
    hipError_t err = hipSuccess;
    int wg_per_cu = 1, cus = 1;
  };
  static const Res res = [] {
    Res r;
    int dev = 0, per_cu = 0;
    if ((r.err = hipFuncSetAttribute(reinterpret_cast<const void *>(KERN),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024)) != hipSuccess)
      return r;
    if ((r.err = hipGetDevice(&dev)) != hipSuccess) return r;
    if ((r.err = hipDeviceGetAttribute(&r.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return r;
    if ((r.err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERN, kThreads, 0)) != hipSuccess) return r;
    r.wg_per_cu = per_cu > 0 ? per_cu : 1;
    if (r.cus < 1) r.cus = 1;
    return r;
  }();
  if (res.err != hipSuccess) return res.err;
  const int by_lds = (int)((160u * 1024u) / lds);
  int per_cu = by_lds < res.wg_per_cu ? (by_lds > 0 ? by_lds : 1) : res.wg_per_cu;
  if (per_cu > kUnitWgsPerCu) per_cu = kUnitWgsPerCu;
  const uint32_t resident = (uint32_t)(per_cu * res.cus);
  const uint32_t grid = band > 0u ? (ntiles + band - 1u) / band : (ntiles < resident ? ntiles : resident);
  hipLaunchKernelGGL(KERN, dim3(grid), dim3(kThreads), lds, stream, a, w, s, c, M, N, K, lda, ldc, band);
  return hipGetLastError();
}

// Whether the scale rows of every workgroup's rows fit in the kUnitScales
// floats of LDS: a range of R rows touches at most (R + 126) / 128 + 1 scale
// rows, and a workgroup holds at most ceil(N / CUs) rows (one workgroup per
// CU, fewer workgroups when there are fewer tiles) or 16 * band.
inline hipError_t unit_scales_fit(uint32_t N, uint32_t K, uint32_t band, bool &fit) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus = n > 0 ? n : 1;
  }
  const uint32_t ntiles = (N + 15u) / 16u;
  const uint32_t wgs = band > 0u ? (ntiles + band - 1u) / band : (ntiles < (uint32_t)cus ? ntiles : (uint32_t)cus);
  const uint32_t rows_max = band > 0u ? 16u * band : (N + wgs - 1u) / wgs;
  fit = (uint64_t)((rows_max + 126u) / 128u + 1u) * (K >> 7) <= kUnitScales;
  return hipSuccess;
}

// Staging chunks per thread: exactly the number that covers A in one round
// (1 .. 10; larger A is staged in rounds of 10).  Idle chunk slots re-read
// chunk 0 before the staging barrier; measured on MI355X against the coarser
// choice of 2, 3, 4, 5 or 10: N = K = 5120 M = 5 8.77 -> 8.46 us, M = 6
// 8.81 -> 8.57, M = 7 8.87 -> 8.78, N = 17408 K = 5120 M = 5 19.45 -> 19.14
// (and that choice against 10 everywhere: N = K = 5120 M = 4 8.71 -> 8.42,
// N = 5120 K = 17408 M = 1 20.5 -> 20.1).
template <int MMAX, bool SL, int UA = 1>
hipError_t launch_units_sl(uint32_t per_thread, size_t lds, uint32_t ntiles, uint32_t band, hipStream_t stream,
                           const uint16_t *a, const uint8_t *w, const float *S, uint16_t *c, uint32_t M, uint32_t N,
                           uint32_t K, uint32_t lda, uint32_t ldc) {
  if constexpr (UA < 10) {
    if (per_thread > (uint32_t)UA)
      return launch_units_sl<MMAX, SL, UA + 1>(per_thread, lds, ntiles, band, stream, a, w, S, c, M, N, K, lda, ldc);
  }
  return launch_units<w8a16_units_kernel<MMAX, 4, UA, SL>>(lds, ntiles, band, stream, a, w, S, c, M, N, K, lda, ldc);
}

template <int MMAX>
hipError_t launch_units_mmax(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                             uint32_t K, uint32_t lda, uint32_t ldc, uint32_t band, hipStream_t stream) {
  const size_t lds = unit_lds_bytes<MMAX>(M, K);
  const uint32_t ntiles = (N + 15u) / 16u;
  const auto *a = static_cast<const uint16_t *>(A);
  const auto *w = static_cast<const uint8_t *>(W);
  auto *c = static_cast<uint16_t *>(C);
  const uint32_t per_thread = (M * (K >> 3) + kThreads - 1) / kThreads;
  bool sl = false;
  const hipError_t e = unit_scales_fit(N, K, band, sl);
  if (e != hipSuccess) return e;
  if (sl) return launch_units_sl<MMAX, true>(per_thread, lds, ntiles, band, stream, a, w, S, c, M, N, K, lda, ldc);
  return launch_units_sl<MMAX, false>(per_thread, lds, ntiles, band, stream, a, w, S, c, M, N, K, lda, ldc);
}

// ---------------------------------------------------------------------------
// Register-resident-activation kernel (K up to 1024 * NBW): the same tiles,
// block ownership, arithmetic and reduction order as the two kernels above,
// so the same bits, but without staging the activations in LDS.
//   * Wave w owns blocks w, w + 8, ... of every tile, and every tile needs the
//     same activations for those blocks: lane (i, g) holds its 64 bytes of
//     activation row i (row 0 for i >= M) for each of the wave's blocks in
//     registers for the whole kernel (16 registers per block), read once from
//     memory at the start.  Nothing limits M below 16 and no barrier
//     precedes the first block.
//   * The weights of the next tile's blocks are requested as the current
//     tile's blocks are consumed (ring slot u serves the wave's u-th block of
//     every tile); past the last tile the requests use an offset beyond the
//     buffer, which fetches nothing.
// ---------------------------------------------------------------------------
template <int NBW>
__global__ __launch_bounds__(kThreads) void w8a16_regs_kernel(const uint16_t *__restrict__ A,
                                                              const uint8_t *__restrict__ W,
                                                              const float *__restrict__ S,
                                                              uint16_t *__restrict__ C, uint32_t M, uint32_t N,
                                                              uint32_t K, uint32_t lda, uint32_t ldc,
                                                              uint32_t band) {
  constexpr int MMAX = 16;
  using L = UnitLayout<MMAX>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t i = lane & 15u, g = lane >> 4;
  const uint32_t nb = K >> 7;
  // the activations of the wave's blocks, requested before any other set-up
  bf16x8_t a[NBW][4];
  {
    const uint16_t *arow = A + (size_t)(i < M ? i : 0u) * lda + 32u * g;
    unroll<0, NBW>([&](auto uu) __attribute__((always_inline)) {
      constexpr int u = decltype(uu)::value;
      const uint32_t b = min(wave + kWaves * (uint32_t)u, nb - 1u);
#pragma unroll
      for (int j = 0; j < 4; ++j) a[u][j] = *reinterpret_cast<const bf16x8_t *>(arow + 128u * b + 8u * j);
    });
  }
  uint32_t r0, r1;  // rows of this workgroup, as in the kernel above
  if (band == 0u) {
    even_rows(N, blockIdx.x, gridDim.x, r0, r1);
  } else {
    r0 = blockIdx.x * 16u * band;
    r1 = min(r0 + 16u * band, N);
  }
  const uint32_t ntile = (r1 - r0 + 15u) >> 4;
  const uint32_t upw = nb > wave ? (nb - wave + kWaves - 1u) / kWaves : 0u;  // <= NBW

  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(W), (short)0, (int)(N * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(S), (short)0, (int)(((N + 127u) >> 7) * nb * 4u), 0x00020000);
  // block u of this wave in tile t (t = ntile, or u past the wave's blocks: nothing)
  auto issue = [&](uint32_t t, uint32_t u) __attribute__((always_inline)) {
    const uint32_t b = min(wave + kWaves * u, nb - 1u);
    const uint32_t row = r0 + 16u * t + i;
    const bool ok = t < ntile && row < r1 && u < upw;
    const uint32_t voff = ok ? row * K + 32u * g : kPastEnd;
    const uint32_t srow = (ok ? row : r0) >> 7;
    UnitRegs r;
    r.w0 = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff, 128u * b, 0);
    r.w1 = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff + 16u, 128u * b, 0);
    r.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srsrc, ok ? srow * nb * 4u : kPastEnd,
                                                                         4u * b, 0));
    return r;
  };

  UnitRegs ring[NBW];
  {
    unroll<0, NBW>([&](auto uu) __attribute__((always_inline)) {
      constexpr int u = decltype(uu)::value;
      ring[u] = issue(0u, (uint32_t)u);
    });
  }

  float *part = reinterpret_cast<float *>(lds + L::kPart);
  for (uint32_t t = 0; t < ntile; ++t) {
    f32x4_t outer = {0.0f, 0.0f, 0.0f, 0.0f};
    // compute from the ring registers in place, then request the next
    // tile's block into them (no request behind a branch, no register copy
    // that would wait for a load in flight; measured on MI355X against a copy
    // taken before the request, N = K = 5120 M = 16 11.77 -> 11.42 us, M = 9
    // 10.30 -> 9.61, N = 17408 M = 16 24.4 -> 22.7)
    unroll<0, NBW>([&](auto uu) __attribute__((always_inline)) {
      constexpr int u = decltype(uu)::value;
      if ((uint32_t)u < upw) {
        const UnitRegs &r = ring[u];
        f32x4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][0], weights8(r.w0.x, r.w0.y), x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][1], weights8(r.w0.z, r.w0.w), x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][2], weights8(r.w1.x, r.w1.y), x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][3], weights8(r.w1.z, r.w1.w), x, 0, 0, 0);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) outer[rr] = __fadd_rn(outer[rr], __fmul_rn(r.s, x[rr]));
      }
      ring[u] = issue(t + 1u, (uint32_t)u);
    });
    // the 8 waves' partial tiles, added in wave order (tile parity alternates
    // the buffer, so one barrier per tile suffices)
    const uint32_t par = t & 1u;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const uint32_t m = 4u * g + rr;
      if (m < M) part[((par * kWaves + wave) * MMAX + m) * 16u + i] = outer[rr];
    }
    __syncthreads();
    if (tid < M * 16u) {
      const uint32_t m = tid >> 4, col = tid & 15u;
      const uint32_t n = r0 + 16u * t + col;
      if (n < r1) {
        const float *pp = part + (par * kWaves * MMAX + m) * 16u + col;
        float v = pp[0];
        for (uint32_t w = 1; w < kWaves; ++w) v = v + pp[w * MMAX * 16u];
        C[(size_t)m * ldc + n] = f32_to_bf16_rne(v);
      }
    }
  }
}

template <int NBW>
hipError_t launch_regs(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N, uint32_t K,
                       uint32_t lda, uint32_t ldc, uint32_t band, hipStream_t stream) {
  // Scales per block from memory.  Staging them in LDS first, as the kernel
  // above does, measured mixed here (N = K = 5120 M = 16 11.77 -> 11.60 us,
  // N = 17408 M = 16 24.31 -> 24.88: the staging barrier holds the first tile).
  return launch_units<w8a16_regs_kernel<NBW>>((size_t)UnitLayout<16>::kA, (N + 15u) / 16u, band, stream,
                                              static_cast<const uint16_t *>(A), static_cast<const uint8_t *>(W), S,
                                              static_cast<uint16_t *>(C), M, N, K, lda, ldc);
}

// ---------------------------------------------------------------------------
// Segmented kernel (activations too large for LDS): the same tiles, block
// ownership, arithmetic and reduction order as the kernels above, so the same
// bits.
//   * One workgroup per CU owns rows [r0, r1) (an even split of N, or 16 * band
//     rows) as T <= TMAX tiles of 16 rows.  K is walked in segments of SB
//     blocks; the activation rows of a segment are staged in LDS once per
//     workgroup (two buffers: the next segment's loads are in flight while the
//     current one is used, one barrier per segment) and serve all T tiles.
//   * Wave w owns blocks w, w + 8, ... (SB is a multiple of 8, so a wave meets
//     its blocks in ascending order).  A unit is one such block for all T
//     tiles: the lane's 64 activation bytes are read from LDS once and feed T
//     chains of four MFMA, one per tile, and each tile keeps its own outer
//     accumulator (outer_t = outer_t + s * inner).
//   * Weights go straight from memory to the lanes as in the units kernel,
//     DEPTH units ahead, across segment boundaries.  Every segment but the
//     last runs as straight-line code that computes from the ring registers
//     in place, and every tile is computed (one past the workgroup's rows sees
//     zero weights): measured on MI355X against requests and tiles guarded by
//     branches (which made the compiler wait for every load in flight inside
//     each unit), N = 5120 K = 17408 M = 8 24.9 -> 23.1 us, M = 16 29.9 ->
//     25.6, N = K = 17408 M = 8 59.4 -> 56.6.
//   * After the last segment the 8 waves' partial tiles are added in LDS in
//     wave order and rows m < M are stored.
// ---------------------------------------------------------------------------
template <int MMAX, int TMAX>
struct SegRegs {
  u32x4_t w0[TMAX], w1[TMAX];  // this lane's 32 FP8 weights of the block, per tile
  float s[TMAX];               // the block's scale for this lane's row, per tile
};

template <int MMAX, int NG = 1>
struct SegShape {
  static constexpr int kSB = MMAX <= 8 ? 32 : 16;             // blocks per segment
  static constexpr int kPitch = kSB * 256 + 16;               // LDS pitch of an activation row segment
  static constexpr int kBuf = MMAX * kPitch;                  // one segment buffer
  static constexpr int kThr = kThreads * NG;                  // threads: NG groups of 8 waves
  static constexpr int kChunks = MMAX * kSB * 16 / kThr;      // 16-byte chunks per thread per segment
  static_assert(kSB % kWaves == 0, "a wave must meet its blocks in ascending order");
  static_assert(MMAX * kSB * 16 % kThr == 0, "whole staging rounds");
};

template <int MMAX, int TMAX, int DEPTH>
__global__ __launch_bounds__(kThreads) void w8a16_segs_kernel(const uint16_t *__restrict__ A,
                                                              const uint8_t *__restrict__ W,
                                                              const float *__restrict__ S,
                                                              uint16_t *__restrict__ C, uint32_t M, uint32_t N,
                                                              uint32_t K, uint32_t lda, uint32_t ldc,
                                                              uint32_t band) {
  using G = SegShape<MMAX>;
  constexpr int NF = MMAX < 4 ? MMAX : 4;
  constexpr uint32_t kSB = G::kSB, kUps = kSB / kWaves;  // units per wave per full segment
  static_assert(kUps % DEPTH == 0, "a segment's units fill whole rounds of the ring");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t i = lane & 15u, g = lane >> 4;
  const uint32_t nb = K >> 7;

  // staging: chunk c = u * 512 + tid of a segment is activation row
  // c / (16 SB), 16-byte column c % (16 SB); segment sg adds sg * 256 SB bytes
  // (a scalar offset).  Rows >= M fetch nothing (their zeros land in buffer
  // rows no lane reads); columns past K in the last segment fetch the row's
  // padding, the next row's start or nothing, and no lane reads them either.
  // The first segment's loads go out before any other set-up.
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(A), (short)0, (int)(((M - 1u) * lda + K) * 2u), 0x00020000);
  u32x4_t av[G::kChunks];
  uint32_t a_src[G::kChunks], a_dst[G::kChunks];
#pragma unroll
  for (int u = 0; u < G::kChunks; ++u) {
    const uint32_t c = (uint32_t)u * kThreads + tid;
    const uint32_t m = c / (kSB * 16u), col = c % (kSB * 16u);
    a_src[u] = m < M ? m * lda * 2u + 16u * col : kPastEnd;
    a_dst[u] = m * (uint32_t)G::kPitch + 16u * col;
  }
  auto stage_load = [&](uint32_t sg) {
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u)
      av[u] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, a_src[u], sg * kSB * 256u, 0);
  };
  stage_load(0u);

  uint32_t r0, r1;
  if (band == 0u) {
    even_rows(N, blockIdx.x, gridDim.x, r0, r1);
  } else {
    r0 = blockIdx.x * 16u * band;
    r1 = min(r0 + 16u * band, N);
  }
  const uint32_t T = (r1 - r0 + 15u) >> 4;  // <= TMAX (checked by the launcher)
  const uint32_t nseg = (nb + kSB - 1u) / kSB;
  const uint32_t nq = nb > wave ? (nb - wave + kWaves - 1) / kWaves : 0u;  // the wave's blocks

  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(W), (short)0, (int)(N * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(S), (short)0, (int)(((N + 127u) >> 7) * nb * 4u), 0x00020000);

  // unit q of this wave is block wave + 8q for every tile
  uint32_t lq = 0;  // next unit to request
  const uint32_t w_lane = 32u * g;
  auto issue_next = [&]() {
    const bool live = lq < nq;
    const uint32_t b = live ? wave + kWaves * lq : 0u;
    SegRegs<MMAX, TMAX> r;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const uint32_t row = r0 + 16u * (uint32_t)t + i;
      const bool in = live && (uint32_t)t < T && row < r1;
      const uint32_t voff = in ? row * K + w_lane : kPastEnd;
      r.w0[t] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff, 128u * b, 0);
      r.w1[t] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff + 16u, 128u * b, 0);
      const uint32_t srow = (row < r1 ? row : r1 - 1u) >> 7;
      r.s[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             srsrc, in ? srow * nb * 4u : kPastEnd, 4u * b, 0));
    }
    ++lq;
    return r;
  };

  auto stage_store = [&](uint32_t sg) {
    uint8_t *buf = lds + (sg & 1u) * G::kBuf;
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u) *reinterpret_cast<u32x4_t *>(buf + a_dst[u]) = av[u];
  };

  SegRegs<MMAX, TMAX> ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) ring[d] = issue_next();
  stage_store(0u);
  __syncthreads();
  const uint32_t nlast = nseg - 1u;
  stage_load(min(1u, nlast));  // (a single segment re-reads itself, stored nowhere)

  f32x4_t outer[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) outer[t] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t a_lane = (i < M ? i : 0u) * G::kPitch + 64u * g;  // rows >= M read row 0, never stored
  auto unit = [&](const SegRegs<MMAX, TMAX> &r, uint32_t b, uint32_t sg) {
    const uint8_t *act = lds + (sg & 1u) * G::kBuf + a_lane + 256u * (b - sg * kSB);
    bf16x8_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const bf16x8_t *>(act + 16 * j);
    // every tile is computed (one past the workgroup's rows sees zero weights
    // and scales and is never stored), so the tile chains interleave
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      f32x4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
      x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], weights8(r.w0[t].x, r.w0[t].y), x, 0, 0, 0);
      x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], weights8(r.w0[t].z, r.w0[t].w), x, 0, 0, 0);
      x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], weights8(r.w1[t].x, r.w1[t].y), x, 0, 0, 0);
      x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], weights8(r.w1[t].z, r.w1[t].w), x, 0, 0, 0);
#pragma unroll
      for (int rr = 0; rr < NF; ++rr) outer[t][rr] = __fadd_rn(outer[t][rr], __fmul_rn(r.s[t], x[rr]));
    }
  };

  // Every segment but the last is full (each wave owns kUps of its blocks
  // there) and runs as straight-line code: compute from the ring registers in
  // place and request the unit DEPTH ahead into them (past the wave's last
  // block: a request that fetches nothing).  The last segment requests what
  // it still needs.
  uint32_t q = 0;  // next unit to compute
  for (uint32_t sg = 0; sg < nlast; ++sg) {
#pragma unroll
    for (int u = 0; u < (int)kUps; ++u) {
      unit(ring[u % DEPTH], wave + kWaves * q, sg);
      ring[u % DEPTH] = issue_next();
      ++q;
    }
    stage_store(sg + 1u);  // that buffer was last read in segment sg - 1, before the previous barrier
    __syncthreads();
    stage_load(min(sg + 2u, nlast));  // (the last segment re-read at the end, stored nowhere)
  }
#pragma unroll
  for (int u = 0; u < (int)kUps; ++u) {
    if (q < nq) {
      unit(ring[u % DEPTH], wave + kWaves * q, nlast);
      if (q + DEPTH < nq) ring[u % DEPTH] = issue_next();
    }
    ++q;
  }

  // the 8 waves' partial tiles, added in wave order
  __syncthreads();  // every wave is done with the segment buffers
  float *part = reinterpret_cast<float *>(lds);  // [tile][wave][m][16]
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if ((uint32_t)t < T) {
#pragma unroll
      for (int rr = 0; rr < NF; ++rr) {
        const uint32_t m = 4u * g + rr;
        if (m < M) part[(((uint32_t)t * kWaves + wave) * MMAX + m) * 16u + i] = outer[t][rr];
      }
    }
  }
  __syncthreads();
  if (tid < M * 16u) {
    const uint32_t m = tid >> 4, col = tid & 15u;
    for (uint32_t t = 0; t < T; ++t) {
      const uint32_t n = r0 + 16u * t + col;
      if (n < r1) {
        const float *pp = part + (t * kWaves * MMAX + m) * 16u + col;
        float v = pp[0];
        for (uint32_t w = 1; w < kWaves; ++w) v = v + pp[w * MMAX * 16u];
        C[(size_t)m * ldc + n] = f32_to_bf16_rne(v);
      }
    }
  }
}

// Two-group form of the segmented kernel: 16 waves, where waves w and w + 8
// own the same blocks (w, w + 8, ...) and split the workgroup's tiles, group
// 0 taking tiles 0, 2, 4, ... and group 1 tiles 1, 3, ...  Every chain, fold
// and reduction step is that of the 8-wave form, so the bits are the same;
// what changes is four waves per SIMD instead of two (each with half the
// registers) to hide the latency of the convert-MFMA-fold chains.  Measured
// on MI355X (graph-replayed, cold weights) against the 8-wave form, it pays
// only for 9 to 16 rows over three or more tiles: N = 17408 K = 5120 M = 16
// (five tiles) 21.9 -> 21.3 us, N = 10240 K = 17408 M = 12 (three) 37.6 ->
// 37.0.  Over two tiles (a 1 : 1 split) and for up to 8 rows it was slower:
// N = K = 5120 M = 16 10.1 -> 10.5, N = 5120 K = 17408 M = 16 25.6 -> 26.7,
// M = 8 23.1 -> 23.3, N = 10240 K = 17408 M = 8 36.2 -> 36.4 (the weights'
// 16-row loads keep the address unit busier here than in the Q2_0 kernel).
// A kernel of its own, like the Q2_0 one, so that the 8-wave form's machine
// code stays as measured.
template <int MMAX, int TMAX, int DEPTH>
__global__ __launch_bounds__(2 * kThreads) void w8a16_segs_groups_kernel(
    const uint16_t *__restrict__ A, const uint8_t *__restrict__ W, const float *__restrict__ S,
    uint16_t *__restrict__ C, uint32_t M, uint32_t N, uint32_t K, uint32_t lda, uint32_t ldc, uint32_t band) {
  constexpr int NG = 2;
  using G = SegShape<MMAX, NG>;
  constexpr int NF = MMAX < 4 ? MMAX : 4;
  constexpr uint32_t kSB = G::kSB, kUps = kSB / kWaves;
  constexpr uint32_t kThr = G::kThr;
  static_assert(kUps % DEPTH == 0, "a segment's units fill whole rounds of the ring");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t wave = wave_all & (uint32_t)(kWaves - 1);  // owns blocks wave, wave + 8, ...
  const uint32_t grp = wave_all / (uint32_t)kWaves;         // owns tiles grp, grp + 2, ...
  const uint32_t i = lane & 15u, g = lane >> 4;
  const uint32_t nb = K >> 7;

  // staging as in the 8-wave form over twice the threads; each chunk's
  // offsets are recomputed when used (registers are the scarce resource here)
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(A), (short)0, (int)(((M - 1u) * lda + K) * 2u), 0x00020000);
  u32x4_t av[G::kChunks];
  auto a_src = [&](int u) {
    const uint32_t c = (uint32_t)u * kThr + tid;
    const uint32_t m = c / (kSB * 16u), col = c % (kSB * 16u);
    return m < M ? m * lda * 2u + 16u * col : kPastEnd;
  };
  auto a_dst = [&](int u) {
    const uint32_t c = (uint32_t)u * kThr + tid;
    const uint32_t m = c / (kSB * 16u), col = c % (kSB * 16u);
    return m * (uint32_t)G::kPitch + 16u * col;
  };
  auto stage_load = [&](uint32_t sg) {
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u)
      av[u] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, a_src(u), sg * kSB * 256u, 0);
  };
  auto stage_store = [&](uint32_t sg) {
    uint8_t *buf = lds + (sg & 1u) * G::kBuf;
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u) *reinterpret_cast<u32x4_t *>(buf + a_dst(u)) = av[u];
  };
  stage_load(0u);

  uint32_t r0, r1;
  if (band == 0u) {
    even_rows(N, blockIdx.x, gridDim.x, r0, r1);
  } else {
    r0 = blockIdx.x * 16u * band;
    r1 = min(r0 + 16u * band, N);
  }
  const uint32_t T = (r1 - r0 + 15u) >> 4;  // <= TMAX (checked by the launcher)
  const uint32_t nseg = (nb + kSB - 1u) / kSB;
  const uint32_t nq = nb > wave ? (nb - wave + kWaves - 1) / kWaves : 0u;  // the wave's blocks
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(W), (short)0, (int)(N * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(S), (short)0, (int)(((N + 127u) >> 7) * nb * 4u), 0x00020000);
  const uint32_t w_lane = 32u * g;
  const uint32_t a_lane = (i < M ? i : 0u) * G::kPitch + 64u * g;  // rows >= M read row 0, never stored
  float *part = reinterpret_cast<float *>(lds);                      // [tile][wave][m][16], at the end

  // The group's TG tiles: its own requests, registers and chains; both
  // groups meet the same barriers.
  auto run = [&](auto TGc) {
    constexpr int TG = decltype(TGc)::value;
    uint32_t lq = 0;  // next unit to request: block wave + 8 lq of the group's tiles
    auto issue_next = [&]() {
      const bool live = lq < nq;
      const uint32_t b = live ? wave + kWaves * lq : 0u;
      SegRegs<MMAX, TG> r;
#pragma unroll
      for (int k = 0; k < TG; ++k) {
        const uint32_t t = grp + (uint32_t)NG * (uint32_t)k;
        const uint32_t row = r0 + 16u * t + i;
        const bool in = live && t < T && row < r1;
        const uint32_t voff = in ? row * K + w_lane : kPastEnd;
        r.w0[k] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff, 128u * b, 0);
        r.w1[k] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff + 16u, 128u * b, 0);
        const uint32_t srow = (row < r1 ? row : r1 - 1u) >> 7;
        r.s[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               srsrc, in ? srow * nb * 4u : kPastEnd, 4u * b, 0));
      }
      ++lq;
      return r;
    };

    SegRegs<MMAX, TG> ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) ring[d] = issue_next();
    stage_store(0u);
    __syncthreads();
    const uint32_t nlast = nseg - 1u;
    stage_load(min(1u, nlast));

    f32x4_t outer[TG];
#pragma unroll
    for (int k = 0; k < TG; ++k) outer[k] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
    auto unit = [&](const SegRegs<MMAX, TG> &r, uint32_t b, uint32_t sg) {
      const uint8_t *act = lds + (sg & 1u) * G::kBuf + a_lane + 256u * (b - sg * kSB);
      bf16x8_t a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const bf16x8_t *>(act + 16 * j);
#pragma unroll
      for (int k = 0; k < TG; ++k) {
        f32x4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], weights8(r.w0[k].x, r.w0[k].y), x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], weights8(r.w0[k].z, r.w0[k].w), x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], weights8(r.w1[k].x, r.w1[k].y), x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], weights8(r.w1[k].z, r.w1[k].w), x, 0, 0, 0);
#pragma unroll
        for (int rr = 0; rr < NF; ++rr) outer[k][rr] = __fadd_rn(outer[k][rr], __fmul_rn(r.s[k], x[rr]));
      }
    };

    // full segments straight-line, the last one peeled (as in the 8-wave form)
    uint32_t q = 0;
    for (uint32_t sg = 0; sg < nlast; ++sg) {
#pragma unroll
      for (int u = 0; u < (int)kUps; ++u) {
        unit(ring[u % DEPTH], wave + kWaves * q, sg);
        ring[u % DEPTH] = issue_next();
        ++q;
      }
      stage_store(sg + 1u);
      __syncthreads();
      stage_load(min(sg + 2u, nlast));
    }
#pragma unroll
    for (int u = 0; u < (int)kUps; ++u) {
      if (q < nq) {
        unit(ring[u % DEPTH], wave + kWaves * q, nlast);
        if (q + DEPTH < nq) ring[u % DEPTH] = issue_next();
      }
      ++q;
    }

    __syncthreads();  // every wave is done with the segment buffers
#pragma unroll
    for (int k = 0; k < TG; ++k) {
      const uint32_t t = grp + (uint32_t)NG * (uint32_t)k;
      if (t < T) {
#pragma unroll
        for (int rr = 0; rr < NF; ++rr) {
          const uint32_t m = 4u * g + rr;
          if (m < M) part[((t * kWaves + wave) * MMAX + m) * 16u + i] = outer[k][rr];
        }
      }
    }
  };
  if (grp == 0u)
    run(std::integral_constant<int, (TMAX + 1) / 2>{});
  else
    run(std::integral_constant<int, TMAX / 2>{});

  // the 8 waves' partial tiles, added in wave order
  __syncthreads();
  if (tid < M * 16u) {
    const uint32_t m = tid >> 4, col = tid & 15u;
    for (uint32_t t = 0; t < T; ++t) {
      const uint32_t n = r0 + 16u * t + col;
      if (n < r1) {
        const float *pp = part + (t * kWaves * MMAX + m) * 16u + col;
        float v = pp[0];
        for (uint32_t w = 1; w < kWaves; ++w) v = v + pp[w * MMAX * 16u];
        C[(size_t)m * ldc + n] = f32_to_bf16_rne(v);
      }
    }
  }
}

template <auto KERN, uint32_t THREADS, size_t LDS>
hipError_t launch_segs_k(uint32_t grid, hipStream_t stream, const void *A, const void *W, const float *S, void *C,
                         uint32_t M, uint32_t N, uint32_t K, uint32_t lda, uint32_t ldc, uint32_t band) {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void *>(KERN), hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(KERN, dim3(grid), dim3(THREADS), LDS, stream, static_cast<const uint16_t *>(A),
                     static_cast<const uint8_t *>(W), S, static_cast<uint16_t *>(C), M, N, K, lda, ldc, band);
  return hipGetLastError();
}

template <int MMAX, int TMAX>
hipError_t launch_segs_t(uint32_t grid, hipStream_t stream, const void *A, const void *W, const float *S, void *C,
                         uint32_t M, uint32_t N, uint32_t K, uint32_t lda, uint32_t ldc, uint32_t band) {
  constexpr size_t lds = 2u * SegShape<MMAX>::kBuf;
  static_assert(lds <= 160u * 1024u, "two segment buffers must fit in LDS");
  static_assert((size_t)TMAX * kWaves * MMAX * 16u * 4u <= lds, "the partial tiles reuse the segment buffers");
  if constexpr (MMAX == 16 && TMAX >= 3) {  // the two-group form, two units in flight up to two tiles a group
    return launch_segs_k<w8a16_segs_groups_kernel<MMAX, TMAX, (TMAX + 1) / 2 <= 2 ? 2 : 1>, 2u * kThreads, lds>(
        grid, stream, A, W, S, C, M, N, K, lda, ldc, band);
  } else {
    // two units in flight, one at five tiles (where two would not fit in registers)
    return launch_segs_k<w8a16_segs_kernel<MMAX, TMAX, TMAX >= 5 ? 1 : 2>, kThreads, lds>(grid, stream, A, W, S, C, M,
                                                                                          N, K, lda, ldc, band);
  }
}

// Tiles per workgroup of the segmented kernel's grid: one workgroup per CU
// (an even row split) or one per band of 16 * band rows.
struct SegGrid {
  uint32_t grid, tiles;
};
inline hipError_t seg_grid(uint32_t N, uint32_t band, SegGrid &sg) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus = n > 0 ? n : 1;
  }
  const uint32_t ntiles = (N + 15u) / 16u;
  if (band > 0u) {
    sg.grid = (ntiles + band - 1u) / band;
    sg.tiles = band;
  } else {
    sg.grid = ntiles < (uint32_t)cus ? ntiles : (uint32_t)cus;
    sg.tiles = ((N + sg.grid - 1u) / sg.grid + 15u) / 16u;
  }
  return hipSuccess;
}

template <int MMAX>
hipError_t launch_segs(const SegGrid &sg, hipStream_t stream, const void *A, const void *W, const float *S, void *C,
                       uint32_t M, uint32_t N, uint32_t K, uint32_t lda, uint32_t ldc, uint32_t band) {
  if (sg.tiles <= 2u) return launch_segs_t<MMAX, 2>(sg.grid, stream, A, W, S, C, M, N, K, lda, ldc, band);
  if (sg.tiles <= 3u) return launch_segs_t<MMAX, 3>(sg.grid, stream, A, W, S, C, M, N, K, lda, ldc, band);
  return launch_segs_t<MMAX, 5>(sg.grid, stream, A, W, S, C, M, N, K, lda, ldc, band);
}

// More than five 16-row tiles per workgroup: launches of the segmented kernel
// over consecutive row ranges of whole 128-row scale groups, as few as keep
// each within five tiles (rows are independent, so the bits do not change).
// Measured on MI355X against the per-phase kernel it replaces there: N =
// 20736 K = 10240 M = 8 58.1 -> 46.9 us, N = 20744 K = 6144 M = 12 50.4 ->
// 31.8, N = 21000 K = 17408 M = 5 86.3 -> 72.1.
template <int MMAX>
hipError_t launch_segs_ranges(hipStream_t stream, const void *A, const void *W, const float *S, void *C, uint32_t M,
                              uint32_t N, uint32_t K, uint32_t lda, uint32_t ldc) {
  uint32_t len = 0;
  for (uint32_t parts = 2;; ++parts) {
    len = (((N + parts - 1u) / parts) + 127u) & ~127u;
    SegGrid g;
    const hipError_t e = seg_grid(len, 0u, g);
    if (e != hipSuccess) return e;
    if (g.tiles <= 5u) break;
  }
  const size_t nb = K >> 7;
  for (uint32_t r = 0; r < N; r += len) {
    const uint32_t n = min(len, N - r);
    SegGrid g;
    hipError_t e = seg_grid(n, 0u, g);
    if (e != hipSuccess) return e;
    e = launch_segs<MMAX>(g, stream, A, static_cast<const uint8_t *>(W) + (size_t)r * K, S + (size_t)(r >> 7) * nb,
                          static_cast<uint16_t *>(C) + r, M, n, K, lda, ldc, 0u);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_w8a16_m16(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                            uint32_t K, uint32_t lda, uint32_t ldc, uint32_t band, hipStream_t stream) {
  // every kernel gives the same bits; the choice is by speed and by what fits
  const bool bounded = (uint64_t)N * K < (1ull << 31);
  const uint32_t nbw = ((K >> 7) + kWaves - 1u) / kWaves;  // blocks per wave and tile
  // Up to 8 rows whose activations fit in LDS: the units kernel (the
  // segmented kernel is slower there: N = K = 5120 M = 1 9.0 against 7.7 us,
  // M = 8 9.1 against 8.9, N = 17408 K = 5120 M = 8 20.7 against 19.6),
  // except for large activations over two or three tiles per workgroup,
  // which the segmented kernel stages in pieces behind the first units:
  // 96 KB or more at five to eight rows (N = 5120 K = 6144 M = 8 11.1 -> 10.0
  // us, K = 8192 M = 6 13.4 -> 12.5, N = K = 8192 M = 8 18.2 -> 17.4), more
  // than 100 KB at fewer (N = 5120 K = 17408 M = 4 22.5 -> 21.6, M = 3 22.3 ->
  // 21.5; at 96 KB, K = 12288 M = 4, 17.0 against 17.2, and at one tile per
  // workgroup, N = 4096, 12.9 against 14.9, the units kernel stays faster),
  // and from 84 KB at six to eight rows (N = 5120 K = 7168 M = 6 12.14 ->
  // 10.99, K = 6144 M = 7 11.16 -> 10.00; at five rows below 96 KB the units
  // kernel stays: K = 8192 11.57 against 12.40, K = 6144 9.19 against 9.99).
  const bool seg_ok = bounded && (uint64_t)(M - 1u) * lda + K < (1ull << 30);  // (its activation range fits an int)
  const uint64_t a_bytes = (uint64_t)M * K * 2u;
  if (seg_ok && M <= 8 &&
      ((M >= 6 && a_bytes >= 84u * 1024u) || (M >= 5 && a_bytes >= 96u * 1024u) || a_bytes > 100u * 1024u)) {
    SegGrid sg;
    const hipError_t e = seg_grid(N, band, sg);
    if (e != hipSuccess) return e;
    if (sg.tiles >= 2u && sg.tiles <= 3u) return launch_segs<8>(sg, stream, A, W, S, C, M, N, K, lda, ldc, band);
  }
  if (bounded && M <= 8 && unit_lds_bytes<8>(M, K) <= 160u * 1024u) {
    if (M <= 1) return launch_units_mmax<1>(A, W, S, C, M, N, K, lda, ldc, band, stream);
    if (M <= 2) return launch_units_mmax<2>(A, W, S, C, M, N, K, lda, ldc, band, stream);
    if (M <= 4) return launch_units_mmax<4>(A, W, S, C, M, N, K, lda, ldc, band, stream);
    return launch_units_mmax<8>(A, W, S, C, M, N, K, lda, ldc, band, stream);
  }
  // Activations larger than LDS, and 9..16 rows: segments of K staged once
  // per workgroup for all its tiles, up to 5 tiles (80 rows) per workgroup.
  // For 9..16 rows it beats keeping the activations in registers (measured on
  // MI355X: N = K = 5120 M = 16 11.40 -> 10.08 us, M = 12 10.35 -> 9.97,
  // N = 17408 M = 16 22.7 -> 21.9, N = K = 4096 M = 16 8.11 -> 7.82).
  if (seg_ok) {
    SegGrid sg;
    const hipError_t e = seg_grid(N, band, sg);
    if (e != hipSuccess) return e;
    if (sg.tiles <= 5u) {
      if (M <= 8) return launch_segs<8>(sg, stream, A, W, S, C, M, N, K, lda, ldc, band);
      return launch_segs<16>(sg, stream, A, W, S, C, M, N, K, lda, ldc, band);
    }
    // more than five tiles per workgroup: row ranges (9..16 rows with up to
    // 5 blocks per wave keep the registers kernel below)
    if (band == 0u && !(M > 8 && nbw <= 5u)) {
      if (M <= 8) return launch_segs_ranges<8>(stream, A, W, S, C, M, N, K, lda, ldc);
      return launch_segs_ranges<16>(stream, A, W, S, C, M, N, K, lda, ldc);
    }
  }
  // 9..16 rows over more than five tiles per workgroup with up to 5 blocks per
  // wave (K <= 5120): activations in registers (N = K = 5120, M = 16: 12.7 us
  // against 16.2 us per phase, when it served that shape).
  if (bounded && M > 8 && nbw <= 5u) {
    if (nbw <= 1u) return launch_regs<1>(A, W, S, C, M, N, K, lda, ldc, band, stream);
    if (nbw <= 2u) return launch_regs<2>(A, W, S, C, M, N, K, lda, ldc, band, stream);
    if (nbw <= 4u) return launch_regs<4>(A, W, S, C, M, N, K, lda, ldc, band, stream);
    return launch_regs<5>(A, W, S, C, M, N, K, lda, ldc, band, stream);
  }
  if (M <= 4) return launch_slots<slots_for(4)>(A, W, S, C, M, N, K, lda, ldc, band, stream);
  if (M <= 8) return launch_slots<slots_for(8)>(A, W, S, C, M, N, K, lda, ldc, band, stream);
  return launch_slots<slots_for(16)>(A, W, S, C, M, N, K, lda, ldc, band, stream);
}

}  // namespace wqd
