// C-ABI layer of libwqd.so: argument validation, Q2_0 row chunking, device
// checks and launch dispatch.  Every check runs before the first HIP call, so
// argument errors are reported the same way on a machine without a GPU.
//
// Behaviour follows page "gemv_q2_vec.rs" (q2_0_gemv_vec launcher; the
// batched launcher's Q2_BATCHM_MAX_M chunking, batchm_row_chunks and
// batchm_launch_chunks) and page "w8a16_gemm_m16.rs" (the checks of
// w8a16_gemm_m16 and its _n64 and _strided variants).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>

#include "../../include/wqd.h"
#include "wqd_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// 0 = not yet checked, 1 = gfx950, 2 = other architecture.  Written once
// per device (racing writers store the same value), read without a lock.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];

// Confirms a current HIP device exists and is a gfx950 part (the only code
// object this library carries).
int check_device(const char *fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(WQD_ENODEV, "%s: no usable HIP device (%s)", fn, hipGetErrorString(e));
  }
  if (dev >= kMaxDevices) return fail(WQD_ENODEV, "%s: device index %d too large", fn, dev);
  int state = g_dev_state[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(WQD_EHIP, "%s: hipGetDeviceProperties: %s", fn, hipGetErrorString(e));
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(state, std::memory_order_release);
  }
  if (state != 1)
    return fail(WQD_EUNSUPPORTED, "%s: device %d is not gfx950 (this library carries gfx950 code only)", fn, dev);
  return WQD_OK;
}

// Q2_0 matrix-core row tiers (include/wqd.h, WQD_Q2_0_TIER_WIDTHS): widths 1
// and 8 are the base tiers, 2, 4 and 6 the exact-row tiers.
constexpr uint32_t kTierWidths[WQD_Q2_0_TIER_COUNT] = WQD_Q2_0_TIER_WIDTHS;
constexpr bool kTierExact[WQD_Q2_0_TIER_COUNT] = {false, true, true, true, false};
constexpr uint32_t kTiersCompiled = (1u << WQD_Q2_0_TIER_COUNT) - 1u;

// Kernel for Q2_0, chosen from N and K only (never M), so batched rows stay
// bit-identical to M=1 rows: the matrix-core kernels when K is a multiple of
// 256 from 1024 up and the weights are under 2^31 bytes, on the row tier
// q2_0_tier_width(m), else the vector-ALU kernel.  The two families differ
// from each other only by fp32 rounding order; every matrix-core kernel and
// tier gives the same bits.  The presence of WQD_Q2_0_VALU (any value; read
// once per process) forces the vector-ALU kernel everywhere, for A/B runs.
hipError_t launch_q2_0(const void *A, const void *B, void *C, uint32_t N, uint32_t K, uint32_t m,
                       hipStream_t stream) {
  static const bool valu = std::getenv("WQD_Q2_0_VALU") != nullptr;
  const uint32_t width = q2_0_tier_width(m);
  if (!valu && width != 0 && wqd::q2_0_pairs_supports(N, K))
    return wqd::launch_q2_0_pairs(A, B, C, N, K, m, width, stream);
  return wqd::launch_q2_0_valu(A, B, C, N, K, m, stream);
}

int check_launch(const char *fn, hipError_t e) {
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(WQD_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return WQD_OK;
}

int validate_q2_0(const char *fn, const void *A, const void *B, void *C, uint32_t N,
                  uint32_t K, uint32_t group) {
  if (!A || !B || !C) return fail(WQD_ENULL, "%s: A, B and C must be non-NULL", fn);
  if (group != WQD_Q2_0_GROUP) return fail(WQD_EINVAL, "%s: group=%u, only 128 is supported", fn, group);
  if (N == 0) return fail(WQD_EINVAL, "%s: N must be >= 1", fn);
  if (K == 0 || K % WQD_Q2_0_GROUP != 0) return fail(WQD_EINVAL, "%s: K=%u is not a positive multiple of 128", fn, K);
  if (K > WQD_Q2_0_MAX_K) return fail(WQD_EUNSUPPORTED, "%s: K=%u above %u", fn, K, (unsigned)WQD_Q2_0_MAX_K);
  if (!aligned(A, 16)) return fail(WQD_EALIGN, "%s: A must be 16-byte aligned", fn);
  if (!aligned(B, 4)) return fail(WQD_EALIGN, "%s: B must be 4-byte aligned", fn);
  if (!aligned(C, 2)) return fail(WQD_EALIGN, "%s: C must be 2-byte aligned", fn);
  return WQD_OK;
}

// Checks shared by the three W8A16 entry points (page "w8a16_gemm_m16.rs":
// 1 <= m <= 16, K a multiple of 128).
int validate_w8a16(const char *fn, const void *A, const void *W, const float *S, void *C, uint32_t M,
                   uint32_t N, uint32_t K) {
  if (!A || !W || !S || !C) return fail(WQD_ENULL, "%s: A, W, S and C must be non-NULL", fn);
  if (M < 1 || M > WQD_W8A16_MAX_M) return fail(WQD_EINVAL, "%s: m=%u outside 1..16 (the M tile)", fn, M);
  if (K == 0 || K % WQD_W8A16_BLOCK != 0)
    return fail(WQD_EINVAL, "%s: K=%u is not a positive multiple of 128 (block-scale granularity)", fn, K);
  if (N == 0) return fail(WQD_EINVAL, "%s: N must be >= 1", fn);
  if (!aligned(A, 16)) return fail(WQD_EALIGN, "%s: A must be 16-byte aligned", fn);
  if (!aligned(W, 16)) return fail(WQD_EALIGN, "%s: W must be 16-byte aligned", fn);
  if (!aligned(S, 4)) return fail(WQD_EALIGN, "%s: S must be 4-byte aligned", fn);
  if (!aligned(C, 2)) return fail(WQD_EALIGN, "%s: C must be 2-byte aligned", fn);
  return WQD_OK;
}

// Row pitches of the strided entry points (page "w8a16_gemm_m16.rs", doc of
// w8a16_gemm_m16_strided): each covers its row, the activation pitch keeps
// rows 16-byte aligned, and the strided span fits 32-bit element offsets.
int validate_pitches(const char *fn, uint32_t M, uint32_t N, uint32_t K, uint32_t a_row_stride,
                     uint32_t c_row_stride) {
  if (a_row_stride < K || c_row_stride < N)
    return fail(WQD_EINVAL, "%s: row pitches must cover the rows (a_row_stride=%u < K=%u or c_row_stride=%u < N=%u)",
                fn, a_row_stride, K, c_row_stride, N);
  if (a_row_stride % 8 != 0)
    return fail(WQD_EINVAL, "%s: a_row_stride=%u is not a multiple of 8 (16-byte activation rows)", fn, a_row_stride);
  if (static_cast<uint64_t>(M - 1) * a_row_stride + K > 0xFFFFFFFFull ||
      static_cast<uint64_t>(M - 1) * c_row_stride + N > 0xFFFFFFFFull)
    return fail(WQD_EINVAL, "%s: row pitches too large (the strided span exceeds 2^32 elements)", fn);
  return WQD_OK;
}

// 16-row tiles per workgroup in w8a16_gemm_m16_n64: 64 weight rows each.
constexpr uint32_t kN64Band = 4;

}  // namespace

extern "C" {

const char *wqd_last_error(void) { return g_last_error; }

int q2_0_select_tier(uint32_t m, uint32_t present_mask, int exact_m) {
  if (m == 0) return -1;
  for (int i = 0; i < WQD_Q2_0_TIER_COUNT; ++i)
    if (kTierWidths[i] >= m && ((present_mask >> i) & 1u) && (exact_m || !kTierExact[i])) return i;
  return -1;
}

int q2_0_exact_m_tiers_enabled(void) {
  static const int on = std::getenv("WQD_NO_EXACT_M_TIERS") == nullptr ? 1 : 0;
  return on;
}

uint32_t q2_0_tier_width(uint32_t m) {
  const int i = q2_0_select_tier(m, kTiersCompiled, q2_0_exact_m_tiers_enabled());
  return i < 0 ? 0u : kTierWidths[i];
}

size_t q2_0_packed_bytes(uint32_t N, uint32_t K) {
  if (K % WQD_Q2_0_GROUP != 0) return 0;
  return static_cast<size_t>(N) * (K / WQD_Q2_0_GROUP) * WQD_Q2_0_BLOCK_BYTES;
}

uint32_t q2_0_batchm_chunks(uint32_t M, uint32_t K, uint32_t N, uint64_t *out3, uint32_t cap) {
  uint32_t count = 0;
  for (uint32_t r0 = 0; r0 < M; r0 += WQD_Q2_0_BATCHM_MAX_M, ++count) {
    uint32_t rows = (M - r0) < WQD_Q2_0_BATCHM_MAX_M ? (M - r0) : WQD_Q2_0_BATCHM_MAX_M;
    if (out3 && count < cap) {
      out3[3 * count + 0] = static_cast<uint64_t>(r0) * K * 2;
      out3[3 * count + 1] = static_cast<uint64_t>(r0) * N * 2;
      out3[3 * count + 2] = rows;
    }
  }
  return count;
}

int q2_0_gemv(const void *A, const void *B, void *C, uint32_t N, uint32_t K, uint32_t group,
              hipStream_t stream) {
  static const char fn[] = "q2_0_gemv";
  int rc = validate_q2_0(fn, A, B, C, N, K, group);
  if (rc) return rc;
  if ((rc = check_device(fn))) return rc;
  (void)hipGetLastError();
  return check_launch(fn, launch_q2_0(A, B, C, N, K, 1, stream));
}

int q2_0_gemv_batchm(const void *A, const void *B, void *C, uint32_t N, uint32_t K,
                     uint32_t group, uint32_t M, hipStream_t stream) {
  static const char fn[] = "q2_0_gemv_batchm";
  int rc = validate_q2_0(fn, A, B, C, N, K, group);
  if (rc) return rc;
  if (M == 0) return WQD_OK;  // no rows: nothing to launch
  if ((rc = check_device(fn))) return rc;
  (void)hipGetLastError();
  const char *a = static_cast<const char *>(A);
  char *c = static_cast<char *>(C);
  for (uint32_t r0 = 0; r0 < M; r0 += WQD_Q2_0_BATCHM_MAX_M) {
    uint32_t rows = (M - r0) < WQD_Q2_0_BATCHM_MAX_M ? (M - r0) : WQD_Q2_0_BATCHM_MAX_M;
    rc = check_launch(fn, launch_q2_0(a + static_cast<size_t>(r0) * K * 2, B,
                                           c + static_cast<size_t>(r0) * N * 2, N, K, rows, stream));
    if (rc) return rc;
  }
  return WQD_OK;
}

int w8a16_gemm_m16(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                   uint32_t K, hipStream_t stream) {
  static const char fn[] = "w8a16_gemm_m16";
  int rc = validate_w8a16(fn, A, W, S, C, M, N, K);
  if (rc) return rc;
  if ((rc = check_device(fn))) return rc;
  (void)hipGetLastError();
  return check_launch(fn, wqd::launch_w8a16_m16(A, W, S, C, M, N, K, K, N, 0, stream));
}

int w8a16_gemm_m16_n64(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                       uint32_t K, hipStream_t stream) {
  static const char fn[] = "w8a16_gemm_m16_n64";
  int rc = validate_w8a16(fn, A, W, S, C, M, N, K);
  if (rc) return rc;
  if ((rc = check_device(fn))) return rc;
  (void)hipGetLastError();
  return check_launch(fn, wqd::launch_w8a16_m16(A, W, S, C, M, N, K, K, N, kN64Band, stream));
}

int w8a16_gemm_m16_strided(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                           uint32_t K, uint32_t a_row_stride, uint32_t c_row_stride, hipStream_t stream) {
  static const char fn[] = "w8a16_gemm_m16_strided";
  int rc = validate_w8a16(fn, A, W, S, C, M, N, K);
  if (rc) return rc;
  if ((rc = validate_pitches(fn, M, N, K, a_row_stride, c_row_stride))) return rc;
  if ((rc = check_device(fn))) return rc;
  (void)hipGetLastError();
  return check_launch(fn, wqd::launch_w8a16_m16(A, W, S, C, M, N, K, a_row_stride, c_row_stride, 0, stream));
}

int w8a16_gemv_batch16_strided(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N,
                               uint32_t K, uint32_t a_row_stride, uint32_t c_row_stride, hipStream_t stream) {
  static const char fn[] = "w8a16_gemv_batch16_strided";
  int rc = validate_w8a16(fn, A, W, S, C, M, N, K);
  if (rc) return rc;
  if ((rc = validate_pitches(fn, M, N, K, a_row_stride, c_row_stride))) return rc;
  const uint32_t rows = wqd::w8a16_gemv_rows_per_launch(K);
  if (rows == 0)
    return fail(WQD_EUNSUPPORTED, "%s: K=%u above 81920 (one activation row must fit in LDS)", fn, K);
  if ((rc = check_device(fn))) return rc;
  (void)hipGetLastError();
  const uint16_t *a = static_cast<const uint16_t *>(A);
  uint16_t *c = static_cast<uint16_t *>(C);
  for (uint32_t r0 = 0; r0 < M; r0 += rows) {
    const uint32_t m = (M - r0) < rows ? (M - r0) : rows;
    rc = check_launch(fn, wqd::launch_w8a16_gemv(a + static_cast<size_t>(r0) * a_row_stride, W, S,
                                                 c + static_cast<size_t>(r0) * c_row_stride, m, N, K,
                                                 a_row_stride, c_row_stride, stream));
    if (rc) return rc;
  }
  return WQD_OK;
}

int w8a16_gemv_batch16(const void *A, const void *W, const float *S, void *C, uint32_t M, uint32_t N, uint32_t K,
                       hipStream_t stream) {
  return w8a16_gemv_batch16_strided(A, W, S, C, M, N, K, K, N, stream);
}

}  // extern "C"
