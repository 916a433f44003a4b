// Q2_0 ternary decode GEMV / batched GEMV on the gfx950 matrix cores.
//
//   C[m,n] = bf16( sum_k A[m,k] * (code[n,k] - 1) * d[n, k/128] ),  m < M <= 16
//
// Operation: page "gemv_q2_vec.rs", docs of q2_0_gemv_vec (M=1, 16 codes per
// 32-bit word, A staged in shared memory, dequant (code-1)*d inside the dot
// product) and q2_0_gemv_vec_batchm (each weight word read once per launch and
// applied to every row; rows bit-identical to the M=1 result).  The pages'
// batched template is issue-bound on its scalar MACs; here the MACs of all rows
// run on v_mfma_f32_16x16x32_bf16, so the vector ALUs only decode, and M=1 runs
// the same kernel as every other M (which is what makes rows bit-identical).
//
// Work layout (requires K/128 to be a multiple of 8, so that every 8-block run
// of a weight row starts on a 16-byte boundary)
//   * A workgroup of 8 waves owns one tile of 16 weight rows and walks K in
//     phases of up to 16 blocks (2048 k).  Each phase's bytes - the 16 rows'
//     34-byte blocks and the M activation rows - are fetched with 16-byte loads
//     in which consecutive lanes read consecutive addresses (a scalar base per
//     phase plus a fixed per-lane offset), kept two phases ahead in registers
//     and written to one of two LDS buffers; one barrier per phase separates
//     writing a buffer from reading it.  Loads and stores are branch-free, so
//     each store waits only for its own phase's loads: a slot with nothing to
//     fetch re-reads an in-bounds chunk and stores it to a dummy LDS slot.
//   * In a phase, wave w handles blocks w and w+8.  Lane l (i = l%16, g = l/16)
//     reads code words 2g and 2g+1 of weight row i (three aligned dwords and a
//     v_perm per word undo the block's 0/2-byte misalignment) and the 32
//     activations k = 32g..32g+31 of row m = i (a zeroed LDS region stands in
//     for rows m >= M); four v_mfma_f32_16x16x32_bf16, the j-th on
//     k = 32g + 8j .. 32g + 8j + 7 of both operands, cover the block.
//   * Decode: for a code word w, u = (w & 0x03030303) | ((w << 2) & 0x30303030)
//     and v = ((w >> 4) & 0x03030303) | ((w >> 2) & 0x30303030) put codes
//     4i, 4i+1 (u) and 4i+2, 4i+3 (v) in the two nibbles of byte i.  A 2-bit
//     code zero-extended to a nibble is the FP4 E2M1 value c/2, so the hardware
//     FP4->BF16 conversion with scale 2 gives the exact BF16 pair (c_j, c_j+1)
//     in k order, matching the activations' natural order.
//   * The -1 of (code-1): a fifth MFMA chain per block multiplies the
//     activations by an all -1 operand, giving -sum a over the block in the
//     accumulator layout; it seeds the block's chain, which then ends at
//     sum a*c - sum a = sum a*(c-1).  Products a*c are exact (c in 0..3).
//   * Scale: acc += d[n] * chain once per block (fma), never per element.
//   * The 8 waves' partial tiles are added in LDS in fixed wave order and rows
//     m < M are stored as BF16, round to nearest even.
//
// Bit-identity across row counts: an output's value depends only on its own
// activation row, its weight row and the fixed block / wave order; activation
// rows >= M are zero operands.  So M=1 and every batched M give the same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wqd_internal.h"

namespace wqd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBlockBytes = 34;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kPhaseBlocks = 16;                          // blocks per phase
constexpr int kPhaseWBytes = kPhaseBlocks * kBlockBytes;  // 544 bytes of one weight row per phase
constexpr int kWPitch = kPhaseWBytes + 16;                // LDS row pitch (bank spread)
constexpr int kWBytes = 16 * kWPitch;                     // weight part of a buffer
constexpr int kAPhaseBytes = kPhaseBlocks * 256;          // 4096 bytes of one activation row per phase
constexpr int kAPitch = kAPhaseBytes + 16;                // LDS pitch of an activation row
constexpr int kSecond = 8;                                // a wave's second block of a phase: w + 8

// LDS: [buffer 0][buffer 1][zero rows: kAPhaseBytes][partial tiles: kWaves x
// 16 x 16 floats]; a buffer holds 16 weight-row segments, MMAX activation-row
// segments and a 16-byte dummy slot at kDummy (buffer-relative).
template <int MMAX>
struct Layout {
  static constexpr int kSlots = 2 + (MMAX * (kAPhaseBytes / 16) + kThreads - 1) / kThreads;
  static constexpr int kDummy = kWBytes + MMAX * kAPitch;
  static constexpr int kBuf = kDummy + 16;
  static constexpr int kZero = 2 * kBuf;
  static constexpr int kPart = kZero + kAPhaseBytes;
  static constexpr int kTotal = kPart + kWaves * 256 * 4;
};

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

// The 16 codes of word w as two 8-element BF16 operands (codes 0..7, 8..15).
__device__ __forceinline__ void decode_word(uint32_t w, bf16x8_t &lo, bf16x8_t &hi) {
  const uint32_t u = (w & 0x03030303u) | ((w << 2) & 0x30303030u);
  const uint32_t v = ((w >> 4) & 0x03030303u) | ((w >> 2) & 0x30303030u);
  u32x4_t a, b;
  a.x = fp4x2_to_bf16x2<0>(u);  // c0, c1
  a.y = fp4x2_to_bf16x2<0>(v);  // c2, c3
  a.z = fp4x2_to_bf16x2<1>(u);  // c4, c5
  a.w = fp4x2_to_bf16x2<1>(v);  // c6, c7
  b.x = fp4x2_to_bf16x2<2>(u);  // c8, c9
  b.y = fp4x2_to_bf16x2<2>(v);  // c10, c11
  b.z = fp4x2_to_bf16x2<3>(u);  // c12, c13
  b.w = fp4x2_to_bf16x2<3>(v);  // c14, c15
  lo = __builtin_bit_cast(bf16x8_t, a);
  hi = __builtin_bit_cast(bf16x8_t, b);
}

// The 16-byte chunk slots of a thread.  Slots 0-1 carry weight chunks: row
// r = tid/32 of the tile, column col = tid%32 + 32s of the row's phase segment
// (34 columns in a full phase).  Slots 2.. carry activation chunks: c =
// (s-2)*512 + tid, row m = c/256, column c%256 (256 columns in a full phase).
// Every slot keeps two precomputed (source offset, LDS destination) pairs: one
// for full phases and one for the K tail's shorter phase.  A column past a
// phase's end re-reads an in-bounds column and goes to the dummy LDS slot; an
// activation row past M likewise.  A tile always has 16 real rows when N >= 16
// (the last tile is shifted back to start at N - 16); for N < 16 a row past N
// re-reads row N - 1 and its columns are never stored.  Source offsets are
// relative to a per-phase scalar base, so issuing a phase costs one select per
// slot.
template <int S>
struct Slots {
  uint32_t src[2][S];  // [full, tail]
  uint32_t dst[2][S];
};

template <int S>
__device__ __forceinline__ void make_slots(Slots<S> &sl, uint32_t tid, uint32_t N, uint32_t rb, uint32_t K,
                                           uint32_t M, uint32_t tail_blocks, uint32_t dummy) {
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const uint32_t pbn = v == 0 ? (uint32_t)kPhaseBlocks : tail_blocks;
    const uint32_t wcols = pbn * kBlockBytes / 16u, acols = pbn * 16u;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (s < 2) {
        const uint32_t r = tid >> 5, col = (tid & 31u) + 32u * s;
        const uint32_t row = min(r, N - 1u);
        const bool in = col < wcols;
        sl.src[v][s] = row * rb + 16u * (in ? col : 0u);
        sl.dst[v][s] = in ? r * kWPitch + 16u * col : dummy;
      } else {
        const uint32_t c = (uint32_t)(s - 2) * kThreads + tid;
        const uint32_t m = c >> 8, col = c & 255u;
        const bool in = m < M && col < acols;
        sl.src[v][s] = in ? m * K * 2u + 16u * col : 0u;
        sl.dst[v][s] = in ? kWBytes + m * kAPitch + 16u * col : dummy;
      }
    }
  }
}

// One block into acc.  `blk` points at the block in LDS (its fp16 scale),
// `win` at this lane's aligned code window, `act` at its 64 bytes of
// activations (or the zero region); `sel` undoes the block's misalignment.
__device__ __forceinline__ void mac_block(const uint8_t *blk, const uint8_t *win, const uint8_t *act, uint32_t sel,
                                          f32x4_t &acc) {
  const u32x4_t *pa = reinterpret_cast<const u32x4_t *>(act);
  bf16x8_t a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = __builtin_bit_cast(bf16x8_t, pa[j]);
  const u32x4_t m1 = {0xbf80bf80u, 0xbf80bf80u, 0xbf80bf80u, 0xbf80bf80u};  // bf16 -1.0
  const bf16x8_t neg1 = __builtin_bit_cast(bf16x8_t, m1);
  f32x4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], neg1, x, 0, 0, 0);

  const uint32_t *pw = reinterpret_cast<const uint32_t *>(win);
  const uint32_t c0 = pw[0], c1 = pw[1], c2 = pw[2];
  const uint32_t w0 = __builtin_amdgcn_perm(c1, c0, sel);
  const uint32_t w1 = __builtin_amdgcn_perm(c2, c1, sel);
  const float d = (float)*reinterpret_cast<const _Float16 *>(blk);
  bf16x8_t b0, b1, b2, b3;
  decode_word(w0, b0, b1);
  decode_word(w1, b2, b3);
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b0, x, 0, 0, 0);
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b1, x, 0, 0, 0);
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], b2, x, 0, 0, 0);
  x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], b3, x, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(d, x[r], acc[r]);
}

template <int MMAX, int DEPTH>
__global__ __launch_bounds__(kThreads) void q2_0_mfma_kernel(const uint16_t *__restrict__ A,
                                                             const uint8_t *__restrict__ B,
                                                             uint16_t *__restrict__ C, uint32_t N, uint32_t K,
                                                             uint32_t M) {
  using L = Layout<MMAX>;
  constexpr int S = L::kSlots;
  static_assert(DEPTH % 2 == 0, "buffer parity must be a compile-time function of the ring slot");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t i = lane & 15u, g = lane >> 4;
  const uint32_t nb = K >> 7;
  const uint32_t nphase = (nb + kPhaseBlocks - 1) / kPhaseBlocks;
  const uint32_t tail_blocks = nb - (nphase - 1u) * kPhaseBlocks;  // blocks in the last phase of a tile
  const uint32_t rb = nb * kBlockBytes;
  const uint32_t ntiles = (N + 15u) / 16u;
  // This workgroup's tiles are blockIdx.x, blockIdx.x + gridDim.x, ...; its
  // phases form one sequence over them, and the load ring runs across tile
  // boundaries so the next tile's first phases are in flight when a tile ends.
  const uint32_t my_tiles = (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x;
  const uint32_t nq = my_tiles * nphase;

  // zero region standing in for activation rows m >= M (visible after the
  // first phase barrier)
  if (tid < (uint32_t)kAPhaseBytes / 16u) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t *>(lds + L::kZero + 16u * tid) = z;
  }

  Slots<S> sl;
  make_slots<S>(sl, tid, N, rb, K, M, tail_blocks, L::kDummy);
  // First row of this workgroup's j-th tile; the last tile of the matrix is
  // shifted back so that every tile holds 16 real rows (rows it shares with
  // the previous tile are computed with the same arithmetic and rewritten with
  // the same bits).
  auto tile_row = [&](uint32_t j) {
    const uint32_t n0 = (blockIdx.x + j * gridDim.x) * 16u;
    return N >= 16u ? min(n0, N - 16u) : 0u;
  };

  // Sequence element q is phase q % nphase of this workgroup's tile q / nphase.
  // Past the end (q >= nq) it re-reads phase 0 of the first tile, stored nowhere.
  auto issue_q = [&](uint32_t q, u32x4_t(&r)[S]) {
    const bool live = q < nq;
    const uint32_t j = live ? q / nphase : 0u;
    const uint32_t p = live ? q - j * nphase : 0u;
    const bool tail = p + 1u == nphase;
    const uint8_t *wb = B + (size_t)tile_row(j) * rb + (size_t)p * kPhaseWBytes;
    const uint8_t *ab = reinterpret_cast<const uint8_t *>(A) + (size_t)p * kAPhaseBytes;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t off = tail ? sl.src[1][s] : sl.src[0][s];
      r[s] = *reinterpret_cast<const u32x4_t *>((s < 2 ? wb : ab) + off);
    }
  };

  // This lane's read offsets (from the LDS base) for the wave's first block of
  // a phase in buffer 0; buffer 1 adds kBuf, the second block (w + 8) adds
  // 8 blocks.  Blocks w and w+8 have the same 0/2-byte misalignment.
  const uint32_t blk = i * kWPitch + wave * kBlockBytes;
  const uint32_t win = (blk + 8u * g) & ~3u;  // code bytes start at +2 (even block) or +4 (odd)
  const uint32_t sel = (blk & 2u) ? 0x07060504u : 0x05040302u;
  const bool a_ok = i < M;
  const uint32_t act = a_ok ? kWBytes + i * kAPitch + wave * 256u + 64u * g : L::kZero + 64u * g;
  const uint32_t act_buf = a_ok ? (uint32_t)L::kBuf : 0u;  // the zero region is shared by both buffers
  const uint32_t act_second = a_ok ? kSecond * 256u : 0u;
  float *part = reinterpret_cast<float *>(lds + L::kPart);  // [wave][m][n]

  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // One sequence element: store its chunks into buffer `parity`, request the
  // element DEPTH ahead into the same registers, compute, and finish the tile
  // after its last phase.
  auto step = [&](uint32_t q, uint32_t parity, u32x4_t(&r)[S]) {
    uint8_t *buf = lds + parity * L::kBuf;
    const uint32_t j = q / nphase, p = q - j * nphase;
    const bool tail = p + 1u == nphase;
    const uint32_t pbn = tail ? tail_blocks : (uint32_t)kPhaseBlocks;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t dst = tail ? sl.dst[1][s] : sl.dst[0][s];
      *reinterpret_cast<u32x4_t *>(buf + dst) = r[s];
    }
    issue_q(q + DEPTH, r);
    __syncthreads();
    const uint8_t *a0 = lds + act + parity * act_buf;
    if (wave < pbn) mac_block(buf + blk, buf + win, a0, sel, acc);
    if (wave + kSecond < pbn)
      mac_block(buf + blk + kSecond * kBlockBytes, buf + win + kSecond * kBlockBytes, a0 + act_second, sel, acc);
    if (tail) {  // tile done: add the 8 waves' partial tiles in fixed order
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) part[(wave * 16u + 4u * g + rr) * 16u + i] = acc[rr];
      acc = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
      __syncthreads();
      if (tid < 256u) {
        const uint32_t m = tid >> 4, col = tid & 15u;
        const uint32_t n = tile_row(j) + col;
        if (m < M && n < N) {
          float v = part[m * 16u + col];
          for (uint32_t w = 1; w < kWaves; ++w) v = v + part[(w * 16u + m) * 16u + col];
          C[(size_t)m * N + n] = f32_to_bf16_rne(v);
        }
      }
      // the next write of `part` comes after at least one more phase barrier
    }
  };

  u32x4_t ring[DEPTH][S];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) issue_q((uint32_t)d, ring[d]);
  uint32_t q = 0;
  for (; q + DEPTH <= nq; q += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) step(q + d, (uint32_t)(d & 1), ring[d]);
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (q + d < nq) step(q + d, (uint32_t)(d & 1), ring[d]);
}

template <int MMAX, int DEPTH>
hipError_t launch_mmax(const void *A, const void *B, void *C, uint32_t N, uint32_t K, uint32_t M,
                       hipStream_t stream) {
  // Persistent grid: as many workgroups as fit on the device at once, each
  // walking every gridDim.x-th tile.  Resolved once per process.
  static int resident = 0;
  if (resident == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&(q2_0_mfma_kernel<MMAX, DEPTH>)),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Layout<MMAX>::kTotal);
    if (e != hipSuccess) return e;
    int dev = 0, cus = 0, per_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (q2_0_mfma_kernel<MMAX, DEPTH>), kThreads,
                                                          Layout<MMAX>::kTotal)) != hipSuccess)
      return e;
    resident = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  }
  const uint32_t ntiles = (N + 15) / 16;
  const uint32_t grid = ntiles < (uint32_t)resident ? ntiles : (uint32_t)resident;
  hipLaunchKernelGGL((q2_0_mfma_kernel<MMAX, DEPTH>), dim3(grid), dim3(kThreads), Layout<MMAX>::kTotal, stream,
                     static_cast<const uint16_t *>(A), static_cast<const uint8_t *>(B),
                     static_cast<uint16_t *>(C), N, K, M);
  return hipGetLastError();
}

}  // namespace

bool q2_0_mfma_supports(uint32_t K, uint32_t m) { return ((K >> 7) % 8u) == 0 && m >= 1 && m <= 16; }

hipError_t launch_q2_0_mfma(const void *A, const void *B, void *C, uint32_t N, uint32_t K, uint32_t m,
                            hipStream_t stream) {
  if (m <= 2) return launch_mmax<2, 2>(A, B, C, N, K, m, stream);
  if (m <= 4) return launch_mmax<4, 2>(A, B, C, N, K, m, stream);
  if (m <= 8) return launch_mmax<8, 2>(A, B, C, N, K, m, stream);
  return launch_mmax<16, 2>(A, B, C, N, K, m, stream);
}

}  // namespace wqd
