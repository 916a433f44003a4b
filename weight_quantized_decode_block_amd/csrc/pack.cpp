// Host packer for the block_q2_0 layout (see include/wqd.h): per 128-weight
// block, the fp16 scale d little-endian in bytes 0-1, then eight little-endian
// 32-bit words, word q holding codes 16q..16q+15 with code i of the word in
// bits 2i..2i+1.  The pages give the inline fp16 scale and the 16-codes-per-
// 32-bit-word packing (page "gemv_q2_vec.rs", module doc and q2_0_gemv_vec
// doc); the field and byte order are this library's fixed reading.
#include <cstring>

#include "../../include/wqd.h"

extern "C" int q2_0_pack(const uint8_t *codes, const uint16_t *d_f16, uint32_t N, uint32_t K,
                         void *out) {
  if (!codes || !d_f16 || !out) return WQD_ENULL;
  if (K == 0 || K % WQD_Q2_0_GROUP != 0) return WQD_EINVAL;
  const size_t nb = K / WQD_Q2_0_GROUP;
  const size_t total = static_cast<size_t>(N) * K;
  for (size_t i = 0; i < total; ++i)
    if (codes[i] > 2) return WQD_EINVAL;
  uint8_t *dst = static_cast<uint8_t *>(out);
  for (size_t n = 0; n < N; ++n) {
    for (size_t b = 0; b < nb; ++b) {
      uint8_t *blk = dst + (n * nb + b) * WQD_Q2_0_BLOCK_BYTES;
      const uint16_t d = d_f16[n * nb + b];
      blk[0] = static_cast<uint8_t>(d & 0xff);
      blk[1] = static_cast<uint8_t>(d >> 8);
      const uint8_t *c = codes + n * K + b * WQD_Q2_0_GROUP;
      for (int q = 0; q < 8; ++q) {
        uint32_t word = 0;
        for (int i = 0; i < 16; ++i) word |= static_cast<uint32_t>(c[16 * q + i]) << (2 * i);
        for (int byte = 0; byte < 4; ++byte)
          blk[2 + 4 * q + byte] = static_cast<uint8_t>(word >> (8 * byte));
      }
    }
  }
  return WQD_OK;
}
