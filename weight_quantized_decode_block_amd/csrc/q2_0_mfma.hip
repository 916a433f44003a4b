// Q2_0 ternary decode GEMV / batched GEMV on the gfx950 matrix cores.
//
//   C[m,n] = bf16( sum_k A[m,k] * (code[n,k] - 1) * d[n, k/128] ),  m < M <= 8
//
// Operation: page "gemv_q2_vec.rs", docs of q2_0_gemv_vec (M=1, 16 codes per
// 32-bit word, A staged in shared memory, dequant (code-1)*d inside the dot
// product) and q2_0_gemv_vec_batchm (each weight word read once per launch and
// applied to every row of a launch of at most 8 rows; rows bit-identical to
// the M=1 result).  The pages' kernels run the MACs on scalar FMAs; here they
// run on v_mfma_f32_16x16x32_bf16 and the vector ALUs only decode.
//
// Two kernels give the same bits (the same units, seeds, chains and
// reduction order) and are chosen by shape (launch_mmax at the end): the
// pairs kernel described next (activations resident in LDS), and the
// segmented kernel for large activations (described at its definition, with
// its 16-wave two-group form).
//
// Work layout (requires K/128 to be even: whole block pairs)
//   * A tile is 8 weight rows over the whole of K.  One MFMA covers two
//     consecutive 128-k blocks (a block pair) of the tile: its 16 columns are
//     (block half h, weight row r) = column 8h + r, and its 16 rows are (block
//     half h, activation row m) = row 8h + m.  Output (8h+m, 8h+r) is the dot
//     product of activation row m with weight row r over block half h; the
//     two off-diagonal quadrants mix different blocks and are never used.
//     Eight rows per tile (instead of sixteen) gives twice as many tiles,
//     which spreads a matrix far more evenly over 256 compute units, and still
//     leaves room for all 8 activation rows of a batched launch.
//   * A workgroup of 8 waves walks its tiles (blockIdx.x, + gridDim.x, ...).
//     Wave w owns block pairs w, w+8, w+16, ... of every tile and works on
//     its own: for each pair every lane loads the 12-byte window of the 8
//     rows' 68 bytes that holds its own 8 code bytes (one buffer load per
//     lane, straight into the registers the decode reads), and the wave keeps
//     DEPTH pairs in flight.  No barrier separates a wave's loads from its
//     compute; the 8 waves meet once per tile, to add their partial sums.
//   * Activations: all M rows of A are copied into LDS once per workgroup.
//     Each group of four consecutive activations is stored in the order
//     (a0, a2, a1, a3), the order the decode below produces codes in.  Rows
//     m >= M read a zero region.
//   * Decode: for a code word w, u = w & 0x33333333 holds codes 4i and 4i+2
//     in the two nibbles of byte i, v = (w >> 2) & 0x33333333 codes 4i+1 and
//     4i+3.  A 2-bit code zero-extended to a nibble is the FP4 E2M1 value
//     c/2, so the hardware FP4->BF16 conversion with scale 2 gives exact BF16
//     pairs (c_4i, c_4i+2) and (c_4i+1, c_4i+3).
//   * The -1 of (code-1): for every block and activation row, an MFMA chain
//     of the activations against an all -1 operand gives -sum a over the
//     block.  The wave that owns a block pair computes it on its workgroup's
//     first tile and keeps it in LDS for the later ones.  It seeds that
//     block's chain, which then ends at sum a*c - sum a = sum a*(c-1)
//     (products a*c are exact, c in 0..3).
//   * Scale: acc += d[n] * chain once per block (fma), never per element.
//   * At the end of a tile the 16 partial sums of an output (8 waves x 2
//     block halves) are added in LDS in fixed order and rows m < M are stored
//     as BF16, round to nearest even.  The last tile is shifted back to start
//     at N - 8, so every tile holds 8 real weight rows.
//
// Bit-identity across row counts: an output's value depends only on its own
// activation row, its weight row and the fixed block / wave / half order;
// activation row m always sits in MFMA rows m and 8 + m.  So M=1 and every
// batched M give the same bits.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#include "wqd_internal.h"

namespace wqd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));

constexpr int kBlockBytes = 34;
constexpr int kRows = 8;                                  // weight rows per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlots8 = 8;  // accumulation slots of a tile's block pairs
constexpr uint32_t kLdsMax = 160u * 1024u;                // LDS per compute unit on gfx950

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int BYTE>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 2.0f, BYTE));
}

// The 16 codes of word w as two 8-element BF16 operands, in the order
// (c0 c2 c1 c3 c4 c6 c5 c7) and (c8 c10 c9 c11 c12 c14 c13 c15).
__device__ __forceinline__ void decode_word(uint32_t w, bf16x8_t &lo, bf16x8_t &hi) {
  const uint32_t u = w & 0x33333333u;
  const uint32_t v = (w >> 2) & 0x33333333u;
  u32x4_t a, b;
  a.x = fp4x2_to_bf16x2<0>(u);
  a.y = fp4x2_to_bf16x2<0>(v);
  a.z = fp4x2_to_bf16x2<1>(u);
  a.w = fp4x2_to_bf16x2<1>(v);
  b.x = fp4x2_to_bf16x2<2>(u);
  b.y = fp4x2_to_bf16x2<2>(v);
  b.z = fp4x2_to_bf16x2<3>(u);
  b.w = fp4x2_to_bf16x2<3>(v);
  lo = __builtin_bit_cast(bf16x8_t, a);
  hi = __builtin_bit_cast(bf16x8_t, b);
}

// Eight consecutive activations (a0..a7) reordered to (a0 a2 a1 a3 a4 a6 a5 a7).
__device__ __forceinline__ u32x4_t permute_acts(u32x4_t x) {
  u32x4_t y;
  y.x = __builtin_amdgcn_perm(x.y, x.x, 0x05040100u);
  y.y = __builtin_amdgcn_perm(x.y, x.x, 0x07060302u);
  y.z = __builtin_amdgcn_perm(x.w, x.z, 0x05040100u);
  y.w = __builtin_amdgcn_perm(x.w, x.z, 0x07060302u);
  return y;
}

// -sum over a block of each MFMA row's activations, in the MFMA accumulator
// layout (every column holds the same value).
__device__ __forceinline__ f32x4_t neg_sum_chain(const bf16x8_t (&a)[4]) {
  const u32x4_t m1 = {0xbf80bf80u, 0xbf80bf80u, 0xbf80bf80u, 0xbf80bf80u};  // bf16 -1.0
  const bf16x8_t neg1 = __builtin_bit_cast(bf16x8_t, m1);
  f32x4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], neg1, x, 0, 0, 0);
  return x;
}

// One tile's share of a unit of the segmented kernels: the lane's 12-byte
// window w of the block pair, its 16 codes decoded and fed to four MFMA
// seeded with -sum(a), then the product scaled by the block's fp16 scale
// (taken from lane (h, r, 0) of the column) into the tile's accumulator.
template <int NF>
__device__ __forceinline__ void seg_tile(const u32x3_t &w, uint32_t sel, uint32_t i, uint32_t h, const f32x4_t &seed,
                                         const bf16x8_t (&a)[4], f32x4_t &acc) {
  const uint32_t w0 = __builtin_amdgcn_perm(w.y, w.x, sel);
  const uint32_t w1 = __builtin_amdgcn_perm(w.z, w.y, sel);
  const uint32_t own_d = h ? (w.x >> 16) : (w.x & 0xFFFFu);  // meaningful on lanes g = 0
  const uint32_t dbits = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(i << 2), (int)own_d);
  const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)dbits);
  bf16x8_t b0, b1, b2, b3;
  decode_word(w0, b0, b1);
  decode_word(w1, b2, b3);
  f32x4_t x = seed;
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b0, x, 0, 0, 0);
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b1, x, 0, 0, 0);
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], b2, x, 0, 0, 0);
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], b3, x, 0, 0, 0);
#pragma unroll
  for (int rr = 0; rr < NF; ++rr) acc[rr] = __builtin_fmaf((float)d, x[rr], acc[rr]);
}

// ---------------------------------------------------------------------------
// Segmented kernel: for large activations (too large for LDS, or large
// enough that staging them all before the first unit costs more than
// staging them in pieces).  The pairs kernel's units, seeds, chains and
// reduction order, so the same bits.
//   * One workgroup per CU owns rows [r0, r1) (an even split of N) as
//     T <= TMAX 8-row tiles (TMAX up to nine; the launcher splits larger N
//     into launches over row ranges); rows past r1 re-read row r1 - 1 and
//     are never stored.
//   * K is walked in segments of SP block pairs.  A segment of every
//     activation row is staged in LDS once per workgroup (the pairs kernel's
//     permuted order) into one of two buffers: the next segment's loads are
//     in flight while the current one is used, one barrier per segment.
//   * Wave w owns pairs w, w + 8, ...; SP is a multiple of 8, so it meets them
//     in ascending order, segment after segment.  A unit is one pair for all
//     T tiles: the lane's activations are read from LDS and the seed chain is
//     run once, then feed TMAX chains of four MFMA, one per tile, each tile
//     with its own accumulator.
//   * Weights go straight from memory to the lanes (the pairs kernel's 12-byte
//     windows), one segment's units ahead: a wave computes from its ring
//     registers in place and requests the unit DEPTH ahead into them.  A
//     request past the wave's last pair, or for a tile past the workgroup's
//     rows, lies outside the buffer's range and fetches nothing (such a tile
//     computes on zeros and is never stored).
//   * After the last segment the 16 partial sums of each output are added in
//     LDS in the pairs kernel's order and rows m < M are stored.
// Measured on MI355X (graph-replayed, cold weights) against the per-phase
// kernel it replaced (super-tiles of up to four tiles walked in phases of 16
// blocks, weights and activations both staged through LDS, one barrier per
// phase): N = 5120 K = 17408 M = 8 14.7 -> 11.9 us, M = 5 13.3 -> 10.8; and
// against the pairs kernel with the activations resident: K = 17408 M = 4
// 12.7 -> 11.8, M = 3 12.5 -> 11.5, K = 8192 M = 8 9.1 -> 7.8, M = 6 9.1 ->
// 7.5, K = 6144 M = 8 7.4 -> 6.7, K = 12288 M = 4 10.3 -> 9.9.  What did not
// pay: requesting weights and activations two segments ahead (M = 8 11.9 ->
// 13.6 us: more requests in flight, and the compute units' address path is
// already busy most of the kernel with the 278 KB of activations each CU
// stages), and three buffers with a per-wave arrival counter in LDS instead
// of the barrier, so waves may run a segment apart (11.9 -> 12.4).
// LDS: [zero rows: 256][segment buffer 0][segment buffer 1]; the partial sums
// reuse it at the end.
template <int MMAX, int NG = 1>
struct SegShape {
  static constexpr int kSP = MMAX == 4 ? 32 : 16;                // block pairs per segment
  static constexpr int kPitch = kSP * 512 + 16;                  // LDS pitch of an activation row segment
  static constexpr int kBuf = MMAX * kPitch;                     // one segment buffer
  static constexpr int kBuf0 = 256;                              // after the zero rows
  static constexpr int kBytes = kBuf0 + 2 * kBuf;
  static constexpr int kThr = kThreads * NG;                     // threads: NG groups of 8 waves
  static constexpr int kChunks = MMAX * kSP * 32 / kThr;         // 16-byte chunks per thread per segment
  static_assert(kSP % kWaves == 0, "a wave must meet its pairs in ascending order");
  static_assert(MMAX * kSP * 32 % kThr == 0, "whole staging rounds");
  static_assert(kBytes <= (int)kLdsMax, "two segment buffers must fit in LDS");
};
// Buffer offset of a request with nothing to fetch: beyond every weight and
// activation buffer the kernel accepts (under 2^31 bytes), and below 2^32
// after adding a pair offset.
constexpr uint32_t kPastEnd = 0x80000000u;

template <int MMAX, int TMAX, int DEPTH>
__global__ __launch_bounds__(kThreads) void q2_0_segs_kernel(const uint16_t *__restrict__ A,
                                                             const uint8_t *__restrict__ B,
                                                             uint16_t *__restrict__ C, uint32_t N, uint32_t K,
                                                             uint32_t M, uint32_t ldc) {
  using G = SegShape<MMAX>;
  constexpr uint32_t kSP = G::kSP, kUps = kSP / kWaves;  // a wave's units per full segment
  constexpr int NF = MMAX < 4 ? MMAX : 4;                // accumulator rows that can hold outputs
  static_assert(kUps % DEPTH == 0, "the ring holds whole rounds of a segment's units");
  static_assert(TMAX * kSlots8 * 2 * MMAX * kRows * 4 <= G::kBytes, "the partial sums reuse the buffers");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t i = lane & 15u, g = lane >> 4;
  const uint32_t h = i >> 3, rw = i & 7u;  // MFMA column i = (block half h, weight row rw)
  const uint32_t nb = K >> 7, npairs = nb >> 1;
  const uint32_t nseg = (npairs + kSP - 1u) / kSP;

  // Staging: chunk c = u * 512 + tid of a segment is activation row
  // c / (32 SP), 16-byte column c % (32 SP); segment s adds s * 512 SP bytes
  // (a scalar offset).  Rows m >= M fetch nothing (their zeros land in buffer
  // rows no lane reads); columns past K in the last segment fetch the next
  // row's start or nothing, and no lane reads them either.  The first
  // segment's loads go out before any other set-up.
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(A), (short)0, (int)(M * K * 2u), 0x00020000);
  u32x4_t av[G::kChunks];
  uint32_t a_src[G::kChunks], a_dst[G::kChunks];
#pragma unroll
  for (int u = 0; u < G::kChunks; ++u) {
    const uint32_t c = (uint32_t)u * kThreads + tid;
    const uint32_t m = c / (32u * kSP), col = c % (32u * kSP);
    a_src[u] = m < M ? m * 2u * K + 16u * col : kPastEnd;
    a_dst[u] = (uint32_t)G::kBuf0 + m * (uint32_t)G::kPitch + 16u * col;
  }
  auto stage_load = [&](uint32_t s) {
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u)
      av[u] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, a_src[u], s * kSP * 512u, 0);
  };
  auto stage_store = [&](uint32_t s) {
    const uint32_t boff = (s & 1u) * (uint32_t)G::kBuf;
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u) *reinterpret_cast<u32x4_t *>(lds + a_dst[u] + boff) = permute_acts(av[u]);
  };
  stage_load(0u);

  uint32_t r0, r1;
  even_rows(N, blockIdx.x, gridDim.x, r0, r1);
  const uint32_t T = (r1 - r0 + (uint32_t)kRows - 1u) / (uint32_t)kRows;  // <= TMAX (checked by the launcher)
  const uint32_t rb = nb * kBlockBytes;
  const uint32_t nq = npairs > wave ? (npairs - wave + kWaves - 1u) / kWaves : 0u;  // the wave's pairs
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(B), (short)0, (int)(N * rb), 0x00020000);
  uint32_t voff[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    const uint32_t row = min(r0 + (uint32_t)kRows * (uint32_t)t + rw, r1 - 1u);
    voff[t] = (uint32_t)t < T ? row * rb + 32u * h + 8u * g : kPastEnd;
  }

  // unit q of this wave is pair wave + 8 q, for every tile
  struct SegRegs {
    u32x3_t w[TMAX];
  };
  auto issue = [&](uint32_t q) {
    const bool live = q < nq;
    const uint32_t soff = 68u * (wave + kWaves * q);
    SegRegs r;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) r.w[t] = __builtin_amdgcn_raw_buffer_load_b96(wrsrc, live ? voff[t] : kPastEnd, soff, 0);
    return r;
  };

  SegRegs ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) ring[d] = issue((uint32_t)d);
  if (tid < 16u) {  // zero region standing in for activation rows m >= M
    const u32x4_t z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t *>(lds + 16u * tid) = z;
  }
  stage_store(0u);
  __syncthreads();
  stage_load(min(1u, nseg - 1u));  // (a single segment re-reads itself, stored nowhere)

  const bool a_ok = rw < M;
  const uint32_t a_lane = a_ok ? (uint32_t)G::kBuf0 + rw * G::kPitch + h * 256u + 64u * g : 64u * g;
  const uint32_t a_buf = a_ok ? (uint32_t)G::kBuf : 0u;  // per buffer
  const uint32_t a_stride = a_ok ? 512u : 0u;            // per pair
  const uint32_t sel = h ? 0x07060504u : 0x05040302u;    // the 8 code bytes at byte 2 (h = 0) or 4 (h = 1)
  const bool lane_out = (g >> 1) == h;

  f32x4_t acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
  // every tile is computed (a tile past the workgroup's rows sees zero
  // weights and is never stored), so the T chains interleave
  auto unit = [&](const SegRegs &r, uint32_t q, uint32_t s) {
    const uint32_t pl = wave + kWaves * q - s * kSP;  // pair within the segment
    const uint8_t *act = lds + a_lane + (s & 1u) * a_buf + a_stride * pl;
    bf16x8_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const bf16x8_t *>(act + 16 * j);
    const f32x4_t seed = neg_sum_chain(a);
#pragma unroll
    for (int t = 0; t < TMAX; ++t) seg_tile<NF>(r.w[t], sel, i, h, seed, a, acc[t]);
  };

  // Every segment but the last is full (each wave owns kUps of its pairs
  // there) and runs as straight-line code: compute from the ring registers
  // in place and request the unit DEPTH ahead into them (past the wave's last
  // pair: a request that fetches nothing).  The last segment's units were
  // all requested by then.
  const uint32_t nlast = nseg - 1u;
  uint32_t q = 0;
  for (uint32_t s = 0; s < nlast; ++s) {
#pragma unroll
    for (int u = 0; u < (int)kUps; ++u) {
      unit(ring[u % DEPTH], q, s);
      ring[u % DEPTH] = issue(q + DEPTH);
      ++q;
    }
    stage_store(s + 1u);  // that buffer was last read in segment s - 1, before the previous barrier
    __syncthreads();
    stage_load(min(s + 2u, nlast));  // (the last segment re-read at the end, stored nowhere)
  }
#pragma unroll
  for (int u = 0; u < (int)kUps; ++u) {
    if (q < nq) {
      unit(ring[u % DEPTH], q, nlast);
      if (q + DEPTH < nq) ring[u % DEPTH] = issue(q + DEPTH);
    }
    ++q;
  }

  // the 16 partial sums of each output, added in slot and half order
  __syncthreads();  // every wave is done with the segment buffers
  float *part = reinterpret_cast<float *>(lds);  // [tile][slot][half][m][r]
  if (lane_out) {
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if ((uint32_t)t < T) {
#pragma unroll
        for (int rr = 0; rr < NF; ++rr) {
          const uint32_t m = 4u * (g & 1u) + rr;
          if (m < M) part[((((uint32_t)t * kSlots8 + wave) * 2u + h) * MMAX + m) * kRows + rw] = acc[t][rr];
        }
      }
    }
  }
  __syncthreads();
  const uint32_t per = M * (uint32_t)kRows;
  for (uint32_t x = tid; x < T * per; x += kThreads) {  // (more outputs than threads from nine 8-row tiles on)
    const uint32_t t = x / per, lt = x - t * per;
    const uint32_t m = lt >> 3, col = lt & 7u;
    const uint32_t n = r0 + (uint32_t)kRows * t + col;
    if (n < r1) {
      const float *pp = part + ((t * kSlots8 * 2u) * MMAX + m) * kRows + col;
      float v = pp[0];
      for (uint32_t k = 1; k < 2u * kSlots8; ++k) v = v + pp[k * MMAX * kRows];
      store_out(C + (size_t)m * ldc + n, f32_to_bf16_rne(v));
    }
  }
}

// Two-group form of the segmented kernel for five to seven tiles per
// workgroup at six or eight rows: 16 waves, where waves w and w + 8 own the
// same pairs (w, w + 8, ...) and split the tiles, group 0 taking tiles 0, 2,
// 4, ... and group 1 tiles 1, 3, 5, ...; each group runs its own seed chains.
// Every chain, slot and reduction step is that of the 8-wave form, so the
// bits are the same; what changes is four waves per SIMD instead of two
// (each with half the registers, one unit in flight) to hide the latency of
// the decode-MFMA chains.  Measured on MI355X (graph-replayed, cold weights)
// against the 8-wave form: N = 12304 K = 12288 M = 8 (seven tiles) 18.2 ->
// 15.6-15.8 us, N = 12288 K = 17408 M = 8 (six) 20.3 -> 18.5, N = 9216
// K = 17408 M = 8 (five) 17.0 -> 16.3, N = 10496 K = 17408 M = 5 (six, the
// 6-row instance) 18.4 -> 17.5.  At two to four tiles it was mixed within
// 3 %, and at eight or nine (registers) slower or even.  It is a kernel of
// its own rather than a template switch of the 8-wave one because the same
// restructuring applied there changed that kernel's register allocation and
// cost it 3 % (N = 5120 K = 17408 M = 8); the shared per-tile chain
// (seg_tile) leaves its machine code as it was.
template <int MMAX, int TMAX>
__global__ __launch_bounds__(2 * kThreads) void q2_0_segs_groups_kernel(const uint16_t *__restrict__ A,
                                                                       const uint8_t *__restrict__ B,
                                                                       uint16_t *__restrict__ C, uint32_t N,
                                                                       uint32_t K, uint32_t M, uint32_t ldc) {
  constexpr int NG = 2;
  using G = SegShape<MMAX, NG>;
  constexpr uint32_t kSP = G::kSP, kUps = kSP / kWaves;  // a wave's units per full segment
  constexpr uint32_t kThr = G::kThr;
  constexpr int NF = MMAX < 4 ? MMAX : 4;
  static_assert(TMAX * kSlots8 * 2 * MMAX * kRows * 4 <= G::kBytes, "the partial sums reuse the buffers");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t wave = wave_all & (uint32_t)(kWaves - 1);  // owns pairs wave, wave + 8, ...
  const uint32_t grp = wave_all / (uint32_t)kWaves;         // owns tiles grp, grp + 2, ...
  const uint32_t i = lane & 15u, g = lane >> 4;
  const uint32_t h = i >> 3, rw = i & 7u;
  const uint32_t nb = K >> 7, npairs = nb >> 1;
  const uint32_t nseg = (npairs + kSP - 1u) / kSP;

  // staging as in the 8-wave form over twice the threads; each chunk's
  // offsets are recomputed when used (registers are the scarce resource here)
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(A), (short)0, (int)(M * K * 2u), 0x00020000);
  u32x4_t av[G::kChunks];
  auto a_src = [&](int u) {
    const uint32_t c = (uint32_t)u * kThr + tid;
    const uint32_t m = c / (32u * kSP), col = c % (32u * kSP);
    return m < M ? m * 2u * K + 16u * col : kPastEnd;
  };
  auto a_dst = [&](int u) {
    const uint32_t c = (uint32_t)u * kThr + tid;
    const uint32_t m = c / (32u * kSP), col = c % (32u * kSP);
    return (uint32_t)G::kBuf0 + m * (uint32_t)G::kPitch + 16u * col;
  };
  auto stage_load = [&](uint32_t s) {
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u)
      av[u] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, a_src(u), s * kSP * 512u, 0);
  };
  auto stage_store = [&](uint32_t s) {
    const uint32_t boff = (s & 1u) * (uint32_t)G::kBuf;
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u) *reinterpret_cast<u32x4_t *>(lds + a_dst(u) + boff) = permute_acts(av[u]);
  };
  stage_load(0u);

  uint32_t r0, r1;
  even_rows(N, blockIdx.x, gridDim.x, r0, r1);
  const uint32_t T = (r1 - r0 + (uint32_t)kRows - 1u) / (uint32_t)kRows;  // <= TMAX (checked by the launcher)
  const uint32_t rb = nb * kBlockBytes;
  const uint32_t nq = npairs > wave ? (npairs - wave + kWaves - 1u) / kWaves : 0u;  // the wave's pairs
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(B), (short)0, (int)(N * rb), 0x00020000);
  const bool a_ok = rw < M;
  const uint32_t a_lane = a_ok ? (uint32_t)G::kBuf0 + rw * G::kPitch + h * 256u + 64u * g : 64u * g;
  const uint32_t a_buf = a_ok ? (uint32_t)G::kBuf : 0u;
  const uint32_t a_stride = a_ok ? 512u : 0u;
  const uint32_t sel = h ? 0x07060504u : 0x05040302u;
  const bool lane_out = (g >> 1) == h;
  float *part = reinterpret_cast<float *>(lds);  // [tile][slot][half][m][r], after the last segment

  // The group's TG tiles: its own requests, registers and chains; both
  // groups meet the same barriers.
  auto run = [&](auto TGc) {
    constexpr int TG = decltype(TGc)::value;
    uint32_t voff[TG];
#pragma unroll
    for (int k = 0; k < TG; ++k) {
      const uint32_t t = grp + (uint32_t)NG * (uint32_t)k;
      const uint32_t row = min(r0 + (uint32_t)kRows * t + rw, r1 - 1u);
      voff[k] = t < T ? row * rb + 32u * h + 8u * g : kPastEnd;
    }
    struct SegRegs {
      u32x3_t w[TG];
    };
    auto issue = [&](uint32_t q) {  // unit q of this wave: pair wave + 8 q, for the group's tiles
      const bool live = q < nq;
      const uint32_t soff = 68u * (wave + kWaves * q);
      SegRegs r;
#pragma unroll
      for (int k = 0; k < TG; ++k)
        r.w[k] = __builtin_amdgcn_raw_buffer_load_b96(wrsrc, live ? voff[k] : kPastEnd, soff, 0);
      return r;
    };

    SegRegs ring = issue(0u);
    if (tid < 16u) {  // zero region standing in for activation rows m >= M
      const u32x4_t z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t *>(lds + 16u * tid) = z;
    }
    stage_store(0u);
    __syncthreads();
    stage_load(min(1u, nseg - 1u));

    f32x4_t acc[TG];
#pragma unroll
    for (int k = 0; k < TG; ++k) acc[k] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
    auto unit = [&](const SegRegs &r, uint32_t q, uint32_t s) {
      const uint32_t pl = wave + kWaves * q - s * kSP;
      const uint8_t *act = lds + a_lane + (s & 1u) * a_buf + a_stride * pl;
      bf16x8_t a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const bf16x8_t *>(act + 16 * j);
      const f32x4_t seed = neg_sum_chain(a);
#pragma unroll
      for (int k = 0; k < TG; ++k) seg_tile<NF>(r.w[k], sel, i, h, seed, a, acc[k]);
    };

    // full segments straight-line, the last one peeled (as in the 8-wave form)
    const uint32_t nlast = nseg - 1u;
    uint32_t q = 0;
    for (uint32_t s = 0; s < nlast; ++s) {
#pragma unroll
      for (int u = 0; u < (int)kUps; ++u) {
        unit(ring, q, s);
        ring = issue(q + 1u);
        ++q;
      }
      stage_store(s + 1u);
      __syncthreads();
      stage_load(min(s + 2u, nlast));
    }
#pragma unroll
    for (int u = 0; u < (int)kUps; ++u) {
      if (q < nq) {
        unit(ring, q, nlast);
        if (q + 1u < nq) ring = issue(q + 1u);
      }
      ++q;
    }

    __syncthreads();  // every wave is done with the segment buffers
    if (lane_out) {
#pragma unroll
      for (int k = 0; k < TG; ++k) {
        const uint32_t t = grp + (uint32_t)NG * (uint32_t)k;
        if (t < T) {
#pragma unroll
          for (int rr = 0; rr < NF; ++rr) {
            const uint32_t m = 4u * (g & 1u) + rr;
            if (m < M) part[(((t * kSlots8 + wave) * 2u + h) * MMAX + m) * kRows + rw] = acc[k][rr];
          }
        }
      }
    }
  };
  if (grp == 0u)
    run(std::integral_constant<int, (TMAX + 1) / 2>{});
  else
    run(std::integral_constant<int, TMAX / 2>{});

  // the 16 partial sums of each output, added in slot and half order
  __syncthreads();
  const uint32_t per = M * (uint32_t)kRows;
  for (uint32_t x = tid; x < T * per; x += kThr) {
    const uint32_t t = x / per, lt = x - t * per;
    const uint32_t m = lt >> 3, col = lt & 7u;
    const uint32_t n = r0 + (uint32_t)kRows * t + col;
    if (n < r1) {
      const float *pp = part + ((t * kSlots8 * 2u) * MMAX + m) * kRows + col;
      float v = pp[0];
      for (uint32_t k = 1; k < 2u * kSlots8; ++k) v = v + pp[k * MMAX * kRows];
      store_out(C + (size_t)m * ldc + n, f32_to_bf16_rne(v));
    }
  }
}

// ---------------------------------------------------------------------------
// Resident-activation kernel (the usual case): per-wave block pairs.
// ---------------------------------------------------------------------------
// LDS: [zero rows: 256][partial tiles, per subgroup: 2 x 8 slots x 2 x MMAX x 8 floats]
// [seeds, per subgroup: nb x 8 floats][A: M rows, pitch 2K + 16].
template <int MMAX, int SG = 1>
struct PairLayout {
  static constexpr int kZero = 0;
  static constexpr int kPart = kZero + 256;
  static constexpr int kPartBytes = 2 * kSlots8 * 2 * MMAX * kRows * 4;  // one subgroup's
  static constexpr int kFixed = kPart + SG * kPartBytes;
};

template <int MMAX, int SG = 1>
constexpr size_t pair_lds_bytes(uint32_t M, uint32_t K) {
  return (size_t)PairLayout<MMAX, SG>::kFixed + (size_t)SG * (K >> 7) * 32u + (size_t)M * (2u * K + 16u);
}

// f(integral_constant<e>) for the runtime value e in [E, D)
template <int E, int D, typename F>
__device__ __forceinline__ void drain_case(uint32_t e, F &&f) {
  if constexpr (E < D) {
    if (e == (uint32_t)E)
      f(std::integral_constant<int, E>{});
    else
      drain_case<E + 1, D>(e, f);
  }
}

// One block pair's bytes for this lane: the aligned 3-dword window holding
// its 8 code bytes.  The fp16 scale comes from the window of lane g = 0 of
// the same column, which starts at the half's scale (first block) or two
// bytes before it (second block), through one cross-lane permute.
struct PairRegs {
  u32x3_t w;
};

// NW waves per workgroup (4 or 8).  Pair p of a tile belongs to accumulation
// slot p % 8 whatever NW is: wave w owns pairs w, w + NW, ... and keeps one
// accumulator per slot it owns, so the sums are those of the segmented kernel.
// Weight bytes go straight from memory to the lanes that use them (buffer
// loads bounded by the matrix size): lane (h, r, g) reads 12 bytes at
// 68p + 32h + 8g of weight row r; the scale is taken from lane (h, r, 0)'s 12
// bytes.
//
// SG = 2 runs two such groups of NW waves in one workgroup over one LDS copy
// of the activations: subgroup s walks the tiles of virtual workgroup
// 2 blockIdx.x + s of a grid of 2 gridDim.x, with its own partials and
// seeds, so every output is computed as with SG = 1.  The once-per-tile
// barrier is shared, so both subgroups walk as many tiles as subgroup 0; the
// tiles past subgroup 1's own count load in bounds (the last tile) and
// neither compute nor store.
template <int MMAX, int NW, int DEPTH, int UA, int SG = 1, int LATE = 0>
__global__ __launch_bounds__(64 * NW * SG) void q2_0_pairs_kernel(const uint16_t *__restrict__ A,
                                                                  const uint8_t *__restrict__ B,
                                                                  uint16_t *__restrict__ C, uint32_t N, uint32_t K,
                                                                  uint32_t M) {
  using L = PairLayout<MMAX, SG>;
  constexpr int NF = MMAX < 4 ? MMAX : 4;  // accumulator rows that can hold outputs
  constexpr int NACC = kSlots8 / NW;       // accumulation slots per wave
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(SG == 1 || (SG == 2 && NW == 8), "one or two subgroups of 8 waves");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane((tid >> 6) & (uint32_t)(NW - 1));
  const uint32_t sg = SG == 1 ? 0u : __builtin_amdgcn_readfirstlane(tid / (64u * NW));
  const uint32_t ltid = tid - sg * (64u * NW);  // thread index within the subgroup
  const uint32_t i = lane & 15u, g = lane >> 4;
  const uint32_t h = i >> 3, rw = i & 7u;  // MFMA column i = (block half h, weight row rw)
  const uint32_t nb = K >> 7, npairs = nb >> 1;
  const uint32_t a_off = L::kFixed + (uint32_t)SG * nb * 32u;

  // Activation staging, UA chunks per thread per round: the launcher picks UA
  // so that one round usually holds all of A.  Chunk c of A (16 bytes, row
  // c / cpr) goes to LDS byte a_off + 16 * (c + row): rows are 2K + 16 bytes
  // apart.  The row is counted with MMAX - 1 compares (no division).  Idle
  // slots re-read chunk 0 and write into the partials.
  const uint32_t cpr = K >> 3;
  const uint32_t total = M * cpr;
  u32x4_t av[UA];
  uint32_t adst[UA];
  auto a_load = [&](uint32_t base) {
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const uint32_t c = base + (uint32_t)u * (64u * NW * SG) + tid;
      const bool in = c < total;
      const uint32_t cc = in ? c : 0u;
      uint32_t m = 0;
#pragma unroll
      for (int j = 1; j < MMAX; ++j) m += cc >= (uint32_t)j * cpr ? 1u : 0u;
      av[u] = *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const uint8_t *>(A) + (size_t)cc * 16u);
      adst[u] = in ? a_off + 16u * (cc + m) : (uint32_t)L::kPart;
    }
  };
  // The activations' first round is requested before any other set-up (about
  // 100 mostly scalar instructions per wave, which the waves of a CU issue one
  // at a time on its scalar unit); measured on MI355X at N = K = 5120, M = 1:
  // 4.87 -> 4.48 us per call.
  a_load(0u);

  const uint32_t rb = nb * kBlockBytes;
  const uint32_t ntiles = N >= (uint32_t)kRows ? (N + kRows - 1u) / kRows : 1u;
  const uint32_t gx = gridDim.x * (uint32_t)SG, bx = blockIdx.x * (uint32_t)SG + sg;
  const uint32_t b0 = blockIdx.x * (uint32_t)SG;             // subgroup 0's virtual workgroup
  const uint32_t my_tiles = (ntiles - b0 + gx - 1) / gx;     // tiles walked (and barriers) by every wave
  const uint32_t own_tiles = (ntiles - bx + gx - 1) / gx;    // tiles that are this subgroup's own
  // pairs of a tile owned by this wave: wave, wave + NW, ...  A wave that
  // owns none (K = 1024, NW = 8) still runs one unit per tile that computes
  // nothing, so every wave meets the once-per-tile barrier.
  const uint32_t upw = npairs > wave ? (npairs - wave + NW - 1) / NW : 1u;
  const uint32_t nq = my_tiles * upw;
  const uint32_t seed_off = L::kFixed + sg * nb * 32u;
  const uint32_t a_pitch = 2u * K + 16u;

  auto zero_rows = [&]() {
    if (tid < 16u) {  // zero region standing in for activation rows m >= M
      const u32x4_t z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t *>(lds + L::kZero + 16u * tid) = z;
    }
  };
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(B), (short)0, (int)(N * rb), 0x00020000);
  const uint32_t row_off = min(rw, N - 1u) * rb;  // rows past N (N < 8) re-read row N - 1
  const uint32_t w_voff = row_off + 32u * h + 8u * g;
  // Unit q of this wave is pair wave + NW*u of tile j (q = j * upw + u).
  // Two wave-uniform cursors walk the units in order, one for the loads
  // (DEPTH units ahead) and one for the compute, so the per-unit bookkeeping
  // is a few scalar adds.  Past the end the load cursor keeps walking with its
  // tile rows clamped to the last tile, so the load address never waits for
  // the tile count (a division); such loads are never used.  Measured on
  // MI355X against re-reading the wave's first pair past the end: N = 17408
  // K = 5120 M = 1 8.19 -> 8.09 us, N = K = 5120 M = 8 6.44 -> 6.39.
  struct Cursor {
    uint32_t q, u, j, row;  // unit, pair index within the tile, tile index, tile's first row
  };
  const uint32_t row_step = (uint32_t)kRows * gx;
  const uint32_t row_last = N >= (uint32_t)kRows ? N - (uint32_t)kRows : 0u;
  auto first_row = [&]() { return N >= (uint32_t)kRows ? min(bx * (uint32_t)kRows, row_last) : 0u; };
  auto advance = [&](Cursor &c) {
    ++c.q;
    if (++c.u == upw) {
      c.u = 0;
      ++c.j;
      c.row = N >= (uint32_t)kRows ? min(c.row + row_step, row_last) : 0u;
    }
  };
  Cursor ld = {0u, 0u, 0u, first_row()};
  auto issue_next = [&]() {
    const uint32_t p = min(wave + NW * ld.u, npairs - 1u);
    const uint32_t soff = ld.row * rb + 68u * p;
    PairRegs r;
    r.w = __builtin_amdgcn_raw_buffer_load_b96(wrsrc, w_voff, soff, 0);
    advance(ld);
    return r;
  };

  const bool a_ok = rw < M;
  const uint32_t a_lane = a_ok ? a_off + rw * a_pitch + h * 256u + 64u * g : (uint32_t)L::kZero + 64u * g;
  const uint32_t a_stride = a_ok ? 512u : 0u;  // per pair
  // seed of MFMA rows 4g..4g+3 = (half g/2, activation rows 4(g%2)..+3)
  const uint32_t s_lane = seed_off + (g >> 1) * 32u + 16u * (g & 1u);  // + 64 per pair
  // the 8 code bytes sit at byte 2 (h = 0) or 4 (h = 1) of the window
  const uint32_t sel = h ? 0x07060504u : 0x05040302u;
  const bool lane_out = (g >> 1) == h;
  float *part = reinterpret_cast<float *>(lds + L::kPart + sg * (uint32_t)L::kPartBytes);  // [tile parity][slot][half][m][r]

  // ---- prologue: A into LDS (permuted) while the first DEPTH pairs are in flight
  PairRegs ring[DEPTH];
  {
    auto a_store = [&]() {
#pragma unroll
      for (int u = 0; u < UA; ++u) *reinterpret_cast<u32x4_t *>(lds + adst[u]) = permute_acts(av[u]);
    };
    // the first DEPTH - LATE pairs' weights, behind the activations' first round
#pragma unroll
    for (int d = 0; d < DEPTH - LATE; ++d) ring[d] = issue_next();
    zero_rows();
    a_store();
    for (uint32_t base = UA * (64u * NW * SG); base < total; base += UA * (64u * NW * SG)) {
      a_load(base);
      a_store();
    }
    __syncthreads();
    // LATE ring slots are requested only now, so that their requests do not
    // queue ahead of the activation copy
#pragma unroll
    for (int d = DEPTH - LATE; d < DEPTH; ++d) ring[d] = issue_next();
  }

  f32x4_t acc[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k) acc[k] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
  // Pair p of the tile into acc.  On the workgroup's first tile the pair's
  // seeds are computed and kept in LDS (only this wave ever uses them); later
  // tiles read them back.
  auto unit = [&](const PairRegs &r, uint32_t p, bool first, f32x4_t &sum) {
    const uint8_t *act = lds + a_lane + a_stride * p;
    bf16x8_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const bf16x8_t *>(act + 16 * j);
    f32x4_t x;
    if (first) {
      x = neg_sum_chain(a);
      if (i == 0u) *reinterpret_cast<f32x4_t *>(lds + s_lane + 64u * p) = x;
    } else {
      x = *reinterpret_cast<const f32x4_t *>(lds + s_lane + 64u * p);
    }
    const uint32_t w0 = __builtin_amdgcn_perm(r.w.y, r.w.x, sel);
    const uint32_t w1 = __builtin_amdgcn_perm(r.w.z, r.w.y, sel);
    const uint32_t own_d = h ? (r.w.x >> 16) : (r.w.x & 0xFFFFu);  // meaningful on lanes g = 0
    const uint32_t dbits = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(i << 2), (int)own_d);
    const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)dbits);
    bf16x8_t b0, b1, b2, b3;
    decode_word(w0, b0, b1);
    decode_word(w1, b2, b3);
    x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b0, x, 0, 0, 0);
    x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b1, x, 0, 0, 0);
    x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], b2, x, 0, 0, 0);
    x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], b3, x, 0, 0, 0);
#pragma unroll
    for (int rr = 0; rr < NF; ++rr) sum[rr] = __builtin_fmaf((float)d, x[rr], sum[rr]);
  };

  // One unit: compute from its ring registers, then (LD) request the unit
  // DEPTH ahead into the same registers (reusing them in place keeps the ring
  // free of register copies, which would wait for loads still in flight), and
  // after the wave's last pair of the tile add the tile's partial sums.
  Cursor cc = {0u, 0u, 0u, first_row()};
  auto step = [&](PairRegs &r, auto ld_next) {
    const uint32_t j = cc.j, u = cc.u, row = cc.row;
    const uint32_t p = wave + NW * u;
    const bool own = SG == 1 || j < own_tiles;
    if (p < npairs && own) {
      if (NACC == 1 || (u & 1u) == 0u)
        unit(r, p, j == 0u, acc[0]);
      else
        unit(r, p, j == 0u, acc[NACC - 1]);
    }
    if constexpr (decltype(ld_next)::value) r = issue_next();
    advance(cc);
    if (u + 1u == upw) {  // tile done: add the 16 partial sums of each output in fixed order
      const uint32_t par = j & 1u;
      if (lane_out) {
#pragma unroll
        for (int k = 0; k < NACC; ++k) {
          const uint32_t slot = wave + NW * k;
#pragma unroll
          for (int rr = 0; rr < NF; ++rr) {
            const uint32_t m = 4u * (g & 1u) + rr;
            if (m < M) part[(((par * kSlots8 + slot) * 2u + h) * MMAX + m) * kRows + rw] = acc[k][rr];
          }
        }
      }
#pragma unroll
      for (int k = 0; k < NACC; ++k) acc[k] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
      __syncthreads();
      if (ltid < M * (uint32_t)kRows && own) {
        const uint32_t m = ltid >> 3, col = ltid & 7u;
        const uint32_t n = row + col;
        if (n < N) {
          const float *pp = part + (par * kSlots8 * 2u * MMAX + m) * kRows + col;
          float v = pp[0];
          for (uint32_t k = 1; k < 2u * kSlots8; ++k) v = v + pp[k * MMAX * kRows];
          store_out(C + (size_t)m * N + n, f32_to_bf16_rne(v));
        }
      }
      // this parity's partials are next written after the following tile's barrier
    }
  };

  // Only units the wave computes are requested.  The loop runs while all of
  // its requests are, and the DEPTH .. 2 DEPTH - 1 units left after it run as
  // straight-line code with exactly the requests still needed (a request past
  // the wave's last unit occupies the compute unit's address path; one behind
  // a branch makes the compiler wait for every load in flight where the
  // branch rejoins).  Measured on MI355X against a ring that requests units
  // past the end: N = K = 5120 M = 2 4.63 -> 4.52 us, M = 4 5.00 -> 4.87.
  const std::true_type LD;
  const std::false_type NOLD;
  while (cc.q + 2u * DEPTH <= nq) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) step(ring[d], LD);
  }
  const uint32_t rem = nq - cc.q;
  auto drain = [&](auto E) {  // E of the DEPTH ring units still request one more
    constexpr int e = decltype(E)::value;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (d < e)
        step(ring[d], LD);
      else
        step(ring[d], NOLD);
    }
#pragma unroll
    for (int d = 0; d < e; ++d) step(ring[d], NOLD);
  };
  if (rem >= (uint32_t)DEPTH) {
    const uint32_t e = rem - DEPTH;  // < DEPTH
    drain_case<0, DEPTH>(e, drain);
  } else {  // fewer units than the ring (the prologue requested a few past the end)
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if ((uint32_t)d < rem) step(ring[d], NOLD);
  }
}

// Launches KERN as a persistent grid: as many workgroups as fit on the device
// at once, by registers (resolved once per kernel and process), by LDS (per
// call) and at most max_per_cu per compute unit, each walking every
// gridDim.x-th tile.
template <auto KERN>
hipError_t launch_persistent(int threads, size_t lds, int max_per_cu, uint32_t ntiles, hipStream_t stream,
                             const uint16_t *a, const uint8_t *b, uint16_t *c, uint32_t N, uint32_t K, uint32_t M) {
  struct Res {
    hipError_t err = hipSuccess;
    int wg_per_cu = 1, cus = 1;
  };
  static const Res res = [threads] {
    Res r;
    int dev = 0, per_cu = 0;
    if ((r.err = hipFuncSetAttribute(reinterpret_cast<const void *>(KERN),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax)) != hipSuccess)
      return r;
    if ((r.err = hipGetDevice(&dev)) != hipSuccess) return r;
    if ((r.err = hipDeviceGetAttribute(&r.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return r;
    if ((r.err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERN, threads, 0)) != hipSuccess) return r;
    r.wg_per_cu = per_cu > 0 ? per_cu : 1;
    if (r.cus < 1) r.cus = 1;
    return r;
  }();
  if (res.err != hipSuccess) return res.err;
  const int by_lds = (int)(kLdsMax / lds);
  int per_cu = by_lds < res.wg_per_cu ? (by_lds > 0 ? by_lds : 1) : res.wg_per_cu;
  if (per_cu > max_per_cu) per_cu = max_per_cu;
  const uint32_t resident = (uint32_t)(per_cu * res.cus);
  const uint32_t grid = ntiles < resident ? ntiles : resident;
  hipLaunchKernelGGL(KERN, dim3(grid), dim3(threads), lds, stream, a, b, c, N, K, M);
  return hipGetLastError();
}

// The pairs kernel with UA = the activation chunks per thread that cover A in
// one staging round exactly (1 .. 10; larger A is staged in rounds of 10).
// Idle chunk slots (which re-read chunk 0 and are stored nowhere useful) cost
// time: measured on MI355X against the coarser choice of 2, 3, 4, 5 or 10,
// N = K = 5120 M = 5 5.88 -> 5.42 us, M = 6 5.92 -> 5.70, N = K = 4096 M = 1
// 3.55 -> 3.49 (and against 10 everywhere, N = K = 5120 M = 2 4.86 -> 4.71,
// N = 5120 K = 17408 M = 1 9.92 -> 9.33).
template <int MMAX, int NW, int D, int SG, int LATE, int UA = 1>
hipError_t launch_pairs(uint32_t per_thread, int threads, size_t lds, int max_per_cu, uint32_t ntiles,
                        hipStream_t stream, const uint16_t *a, const uint8_t *b, uint16_t *c, uint32_t N, uint32_t K,
                        uint32_t M) {
  if constexpr (UA < 10) {
    if (per_thread > (uint32_t)UA)
      return launch_pairs<MMAX, NW, D, SG, LATE, UA + 1>(per_thread, threads, lds, max_per_cu, ntiles, stream, a, b, c,
                                                          N, K, M);
  }
  return launch_persistent<q2_0_pairs_kernel<MMAX, NW, D, UA, SG, LATE>>(threads, lds, max_per_cu, ntiles, stream, a, b,
                                                                         c, N, K, M);
}

template <auto KERN, uint32_t THREADS, size_t LDS>
hipError_t launch_segs_k(uint32_t grid, hipStream_t stream, const uint16_t *a, const uint8_t *b, uint16_t *c,
                         uint32_t N, uint32_t K, uint32_t M, uint32_t ldc) {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void *>(KERN), hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(KERN, dim3(grid), dim3(THREADS), LDS, stream, a, b, c, N, K, M, ldc);
  return hipGetLastError();
}

template <int MMAX, int TMAX>
hipError_t launch_segs_t(uint32_t grid, hipStream_t stream, const uint16_t *a, const uint8_t *b, uint16_t *c,
                         uint32_t N, uint32_t K, uint32_t M, uint32_t ldc) {
  constexpr size_t lds = SegShape<MMAX>::kBytes;
  if constexpr ((MMAX == 6 || MMAX == 8) && TMAX >= 5 && TMAX <= 7) {  // the two-group form
    return launch_segs_k<q2_0_segs_groups_kernel<MMAX, TMAX>, 2u * kThreads, lds>(grid, stream, a, b, c, N, K, M, ldc);
  } else {
    // one segment's units in flight, or one unit from seven tiles on (two would
    // not fit in registers)
    return launch_segs_k<q2_0_segs_kernel<MMAX, TMAX, TMAX >= 7 ? 1 : SegShape<MMAX>::kSP / kWaves>, kThreads, lds>(
        grid, stream, a, b, c, N, K, M, ldc);
  }
}

// The one-workgroup-per-CU grid of the segmented kernel: the
// rows split evenly over min(CUs, tiles) workgroups, and the tiles of one
// workgroup's share.
struct EvenGrid {
  uint32_t grid, rows, tiles;
};
inline hipError_t even_grid(uint32_t N, EvenGrid &g) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus = n > 0 ? n : 1;
  }
  const uint32_t ntiles = (N + kRows - 1u) / kRows;
  g.grid = ntiles < (uint32_t)cus ? ntiles : (uint32_t)cus;
  g.rows = (N + g.grid - 1u) / g.grid;
  g.tiles = (g.rows + kRows - 1u) / kRows;
  return hipSuccess;
}

// The segmented kernel takes at most nine tiles per workgroup (four for the
// 4-row instance, whose deeper ring would not fit in registers beyond
// that; from seven tiles on one unit is in flight, for the same reason).
// Larger N runs as launches over consecutive row ranges, as few as that
// allows, each a full walk over K (rows are independent, so the bits do not
// change).  Measured on MI355X against the kernel it replaced, which walked
// super-tiles of up to four tiles in phases of 16 blocks through LDS (one
// barrier per phase, activations and weights both staged): N = 9216
// K = 17408 M = 8 25.8 -> 17.1 us, N = 10496 M = 5 23.3 -> 18.2, N = 12288
// M = 8 27.2 -> 20.1, N = 12304 K = 12288 M = 8 23.1 -> 18.2, N = K = 17408
// M = 8 38.4 -> 24.6, N = 5120 M = 8 14.7 -> 11.9.  (With resident
// activations over nine tiles, N = 17408 K = 5120, the two-subgroup pairs
// kernel stays faster: M = 8 10.5 against 11.4 us.)
template <int MMAX>
constexpr uint32_t kSegMaxTiles = MMAX == 4 ? 4u : 9u;

template <int MMAX>
hipError_t launch_segs_range(const EvenGrid &g, hipStream_t stream, const uint16_t *a, const uint8_t *b,
                             uint16_t *c, uint32_t N, uint32_t K, uint32_t M, uint32_t ldc) {
  if (g.tiles <= 1u) return launch_segs_t<MMAX, 1>(g.grid, stream, a, b, c, N, K, M, ldc);
  if (g.tiles <= 2u) return launch_segs_t<MMAX, 2>(g.grid, stream, a, b, c, N, K, M, ldc);
  if (g.tiles <= 3u) return launch_segs_t<MMAX, 3>(g.grid, stream, a, b, c, N, K, M, ldc);
  if constexpr (MMAX == 4) {
    return launch_segs_t<MMAX, 4>(g.grid, stream, a, b, c, N, K, M, ldc);
  } else {
    if (g.tiles <= 4u) return launch_segs_t<MMAX, 4>(g.grid, stream, a, b, c, N, K, M, ldc);
    if (g.tiles <= 5u) return launch_segs_t<MMAX, 5>(g.grid, stream, a, b, c, N, K, M, ldc);
    if (g.tiles <= 6u) return launch_segs_t<MMAX, 6>(g.grid, stream, a, b, c, N, K, M, ldc);
    if (g.tiles <= 7u) return launch_segs_t<MMAX, 7>(g.grid, stream, a, b, c, N, K, M, ldc);
    if (g.tiles <= 8u) return launch_segs_t<MMAX, 8>(g.grid, stream, a, b, c, N, K, M, ldc);
    return launch_segs_t<MMAX, 9>(g.grid, stream, a, b, c, N, K, M, ldc);
  }
}

template <int MMAX>
hipError_t launch_segs(const EvenGrid &g, hipStream_t stream, const uint16_t *a, const uint8_t *b, uint16_t *c,
                       uint32_t N, uint32_t K, uint32_t M) {
  if (g.tiles <= kSegMaxTiles<MMAX>) return launch_segs_range<MMAX>(g, stream, a, b, c, N, K, M, N);
  const size_t rb = (size_t)(K >> 7) * kBlockBytes;
  uint32_t parts = (g.tiles + kSegMaxTiles<MMAX> - 1u) / kSegMaxTiles<MMAX>;
  for (;; ++parts) {  // as few ranges as keep every range within the tile limit
    const uint32_t len = (N + parts - 1u) / parts;
    EvenGrid pg;
    const hipError_t e = even_grid(len, pg);
    if (e != hipSuccess) return e;
    if (pg.tiles <= kSegMaxTiles<MMAX>) break;
  }
  const uint32_t len = (N + parts - 1u) / parts;
  for (uint32_t r = 0; r < N; r += len) {
    const uint32_t n = min(len, N - r);
    EvenGrid pg;
    hipError_t e = even_grid(n, pg);
    if (e != hipSuccess) return e;
    e = launch_segs_range<MMAX>(pg, stream, a, b + (size_t)r * rb, c + r, n, K, M, N);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int MMAX>
hipError_t launch_mmax(const void *A, const void *B, void *C, uint32_t N, uint32_t K, uint32_t M,
                       hipStream_t stream) {
  const uint32_t ntiles = N >= (uint32_t)kRows ? (N + kRows - 1) / kRows : 1u;
  const auto *a = static_cast<const uint16_t *>(A);
  const auto *b = static_cast<const uint8_t *>(B);
  auto *c = static_cast<uint16_t *>(C);
  constexpr int NW = 8;
  const bool big = (uint64_t)N * (K >> 7) * kBlockBytes >= (16ull << 20);
  // Up to two workgroups per compute unit where the LDS allows it (measured
  // on MI355X, graph-replayed, cold weights: M = 1 5.28 -> 4.88 us at
  // N = K = 5120, N = 5120 K = 17408 12.1 -> 10.6; M = 5 6.58 -> 5.91, M = 7
  // 6.70 -> 6.16), except for five to eight rows of a matrix of 16 MB or more.
  const int kMaxPerCu = (MMAX <= 4 || !big) ? 2 : 1;
  // Ring schedules (the same bits whatever the schedule): every launch
  // requests its activations first and drains its ring without requests past
  // a wave's last unit.  A wave keeps DEPTH block pairs in flight, LATE of the
  // first DEPTH requested only after the staging barrier (so that they do not
  // queue ahead of the activation copy).
  //   * One row: three pairs when a wave owns three per tile (K = 4352 ..
  //     6144; the third late on large matrices), else two with the second
  //     late.  Measured against two with a separate scale load and requests
  //     past the end: N = K = 5120 4.48 -> 4.32 us (two-deep drained 4.38,
  //     with the second late 4.35), N = K = 4096 4.02 -> 3.58, N = K = 2048
  //     2.69 -> 2.54, N = 256 K = 1024 2.31 -> 2.26, N = K = 8192 7.23 ->
  //     6.92, N = 17408 K = 5120 8.43 -> 8.16.
  //   * Batched rows with two workgroups per compute unit: two pairs.
  //   * Batched rows with one workgroup per compute unit (matrices of 16 MB or
  //     more, or five to eight rows whose activations leave LDS for one):
  //     three pairs, the third late.  Measured against three with the
  //     weights requested before the activations and requests past the end:
  //     N = K = 5120 M = 8 6.60 -> 6.46 us, N = K = 8192 M = 2 8.25 -> 7.61,
  //     M = 4 9.80 -> 8.87, N = 17408 K = 5120 M = 2 9.40 -> 8.57, M = 3 9.84 ->
  //     9.08, M = 4 10.47 -> 9.59, N = 5120 K = 17408 M = 2 10.77 -> 10.11,
  //     M = 4 12.94 -> 12.53; two subgroups (below) N = 17408 K = 5120 M = 5
  //     11.67 -> 10.97, M = 8 11.30 -> 10.61.
  //
  // Five to eight rows over five to seven tiles per workgroup (from
  // K = 3072): the segmented kernel's two-group form, ahead of both pairs
  // forms.  Measured (graph-replayed, cold weights): N = 12288 K = 5120 M = 8
  // 9.43 -> 8.14 us, N = 9216 M = 8 8.26 -> 7.20, N = 10240 M = 6 7.68 ->
  // 7.16, N = 10240 K = 6144 M = 8 9.67 -> 8.09, N = 12288 K = 4096 M = 5
  // 7.30 -> 6.56, and against the two subgroups at 16 MB or more, N = 14336
  // K = 5120 M = 8 9.26 -> 8.69, M = 6 9.52 -> 8.55 (N = 10240 K = 3072 M = 8
  // even).
  if constexpr (MMAX > 4) {
    if (K >= 3072u) {
      EvenGrid eg;
      const hipError_t e = even_grid(N, eg);
      if (e != hipSuccess) return e;
      if (eg.tiles >= 5u && eg.tiles <= 7u) return launch_segs<MMAX>(eg, stream, a, b, c, N, K, M);
    }
  }
  // Five to eight rows of a matrix of 16 MB or more: two subgroups of 8 waves
  // per workgroup over one copy of the activations (measured on MI355X,
  // N = 17408, K = 5120: M = 8 12.45 -> 11.46 us, M = 5 12.54 -> 11.70; at
  // N = K = 5120 one group stays faster, 6.74 against 7.31).  The 8-row
  // instance serves the 6-row tier here too (the same bits; N = 17408,
  // K = 5120, M = 6: 11.78 against 12.14 us for the 6-row instance).
  if constexpr (MMAX > 4) {
    const size_t lds2 = pair_lds_bytes<8, 2>(M, K);
    if (big && lds2 <= kLdsMax) {
      const uint32_t pt = (M * (K >> 3) + 1023u) / 1024u;
      const uint32_t half = (ntiles + 1u) / 2u;
      return launch_pairs<8, NW, 3, 2, 1>(pt, 1024, lds2, 1, half, stream, a, b, c, N, K, M);
    }
  }
  // Activations of 96 KB or more over two or three tiles per workgroup (four
  // for the 4-row instance): the segmented kernel stages them in pieces
  // behind the first units instead of all before them (measured in its
  // description; at one tile per workgroup, N = 2048 K = 17408 M = 4, the
  // pairs kernel stays faster, 7.0 against 7.5 us, at four tiles, N = K =
  // 8192 M = 8, the two tie, and with smaller activations the pairs kernel is
  // faster: N = 5120 K = 12288 M = 2 8.0 against 8.5, N = K = 8192 M = 4 8.9
  // against 10.0).  Four tiles at three or four rows: N = 8192 K = 17408
  // M = 4 15.75 -> 14.67 us, M = 3 15.52 -> 14.47 (N = 7168 K = 20480 M = 4
  // even).  Five to eight rows from K = 6144 on take it from 60 KB (one pairs
  // workgroup per CU there): N = 5120 K = 7168 M = 6 8.14 -> 6.39 us, K = 6144
  // M = 7 7.64 -> 6.68, K = 8192 M = 5 8.05 -> 7.40, N = 4096 K = 7168 M = 5
  // 6.19 -> 5.45 (K = 6144 M = 5 and N = 6144 M = 6 even), and over four
  // tiles N = 7168 K = 6144 M = 7 8.78 -> 7.72 (N = K = 8192 M = 8 even); at
  // K = 5120 the pairs kernel stays (N = 5120 M = 6 5.68 against 5.93, over
  // four tiles N = 8192 M = 8 7.29 against 7.48).  Three or four
  // rows from 84 KB on: N = 5120 K = 14336 M = 3 11.21 -> 9.61, K = 11264
  // M = 4 9.51 -> 8.99 (at 80 KB, K = 10240 M = 4, the pairs kernel stays:
  // 8.40 against 8.78).
  if constexpr (MMAX >= 4) {
    const uint64_t a_bytes = (uint64_t)M * K * 2u;
    const bool wide = M >= 5u && K >= 6144u && a_bytes >= 60u * 1024u;  // five to eight rows from K = 6144
    if (a_bytes >= (MMAX == 4 ? 84u : 96u) * 1024u || wide) {
      EvenGrid eg;
      const hipError_t e = even_grid(N, eg);
      if (e != hipSuccess) return e;
      if (eg.tiles >= 2u && eg.tiles <= (MMAX == 4 || wide ? 4u : 3u))
        return launch_segs<MMAX>(eg, stream, a, b, c, N, K, M);
    }
  }
  // Two rows of 64 KB or more (K >= 16384) over two to nine tiles per
  // workgroup (one launch): the segmented kernel too.  There a pairs
  // workgroup stages 64 KB or more before its first unit and each of its
  // waves walks eight or more pairs per tile, while the segmented kernel
  // stages in pieces behind its first units and serves all of a workgroup's
  // tiles from each unit's activations and seed.
  // Measured (graph-replayed, cold weights): N = 5120 K = 17408 9.93 -> 8.73
  // us, N = 8192 13.28 -> 11.46, N = 10240 14.62 -> 13.82, N = 14336 18.42
  // -> 17.79, N = 5120 K = 20480 13.12 -> 10.29, N = 12288 K = 20480 23.15
  // -> 19.91, N = K = 17408 21.94 -> 21.88, N = 8192 K = 16384 even; below
  // K = 16384 the pairs kernel stays faster (N = 5120 K = 12288 7.72 against
  // 7.97, K = 8192 6.05 against 6.45), and so it does beyond nine tiles, where
  // the segmented kernel would take two launches (N = 20480 K = 16384 25.8
  // against 30.5).
  if constexpr (MMAX == 2) {
    if ((uint64_t)M * K * 2u >= 64u * 1024u) {
      EvenGrid eg;
      const hipError_t e = even_grid(N, eg);
      if (e != hipSuccess) return e;
      if (eg.tiles >= 2u && eg.tiles <= kSegMaxTiles<MMAX>) return launch_segs<MMAX>(eg, stream, a, b, c, N, K, M);
    }
  }
  const size_t lds = pair_lds_bytes<MMAX>(M, K);
  if (lds <= kLdsMax) {  // activations fit in LDS: the pairs kernel
    const uint32_t per_thread = (M * (K >> 3) + 64 * NW - 1) / (64 * NW);  // staging chunks per thread
#define WQD_PAIRS(D, L) \
  return launch_pairs<MMAX, NW, D, 1, L>(per_thread, 64 * NW, lds, kMaxPerCu, ntiles, stream, a, b, c, N, K, M)
    if constexpr (MMAX == 1) {
      const uint32_t pairs_per_wave = ((K >> 8) + NW - 1u) / NW;
      if (pairs_per_wave == 3u && !big) WQD_PAIRS(3, 0);
      if (pairs_per_wave == 3u) WQD_PAIRS(3, 1);
      WQD_PAIRS(2, 1);
    } else {
      const bool two_per_cu = kMaxPerCu >= 2 && 2u * lds <= kLdsMax;
      if (two_per_cu && !big) WQD_PAIRS(2, 0);
      WQD_PAIRS(3, 1);
    }
#undef WQD_PAIRS
  }
  // else the segmented kernel (same bits)
  EvenGrid eg;
  const hipError_t e = even_grid(N, eg);
  if (e != hipSuccess) return e;
  return launch_segs<MMAX>(eg, stream, a, b, c, N, K, M);
}

}  // namespace

bool q2_0_pairs_supports(uint32_t N, uint32_t K) {
  // whole block pairs, and weights within the buffer loads' 2^31-byte range
  // (which also holds the segmented kernel's requests with nothing to fetch)
  return K >= 1024u && ((K >> 7) % 2u) == 0 && (uint64_t)N * (K >> 7) * kBlockBytes < (1ull << 31);
}

hipError_t launch_q2_0_pairs(const void *A, const void *B, void *C, uint32_t N, uint32_t K, uint32_t m,
                             uint32_t width, hipStream_t stream) {
  if (m == 0 || m > width || !q2_0_pairs_supports(N, K)) return hipErrorInvalidValue;
  switch (width) {
    case 1: return launch_mmax<1>(A, B, C, N, K, m, stream);
    case 2: return launch_mmax<2>(A, B, C, N, K, m, stream);
    case 4: return launch_mmax<4>(A, B, C, N, K, m, stream);
    case 6: return launch_mmax<6>(A, B, C, N, K, m, stream);
    case 8: return launch_mmax<8>(A, B, C, N, K, m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wqd
