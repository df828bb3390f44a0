// Device code shared by the hash, the gather and the fused hash-gather kernel
// of decode-sized calls: a token's look-back cells, one row id from a mix, and
// the exact E4M3 x E8M0 -> bf16 dequantisation of 8 bytes of a row. Both paths
// call these, so the fused kernel's rows are the separate kernels' bits.
#pragma once

#include "common.h"

namespace engram_rows {

// Value of the cell at chunk position u (u < 0: the history before the chunk):
// a compressed id, or -1 for DEAD.
__device__ __forceinline__ int32_t cell_value(const EngramHashArgs &a,
                                              const int32_t *__restrict__ token_map,
                                              const int32_t *__restrict__ row,
                                              const int32_t *__restrict__ hist, int64_t u) {
  const int H = a.max_ngram - 1;
  if (u >= 0) {
    const int32_t x = row[u];
    if (x < 0 || x >= a.raw_vocab) return -1;
    const int32_t v = token_map[x];
    return (v >= 0 && v < a.compressed_vocab) ? v : -1;
  }
  if (hist != nullptr) {
    const int32_t v = hist[H + u];
    return (v >= 0 && v < a.compressed_vocab) ? v : -1;
  }
  return a.pad_id;
}

// The N cells of the token at position t: vals[i] is the cell i positions back
// (-1 for DEAD), cells[i] what it hashes as. A DEAD cell blocks itself and
// every older cell: they hash as the pad id.
__device__ __forceinline__ void token_cells(const EngramHashArgs &a,
                                            const int32_t *__restrict__ token_map,
                                            const int32_t *__restrict__ row,
                                            const int32_t *__restrict__ hist, int64_t t,
                                            int32_t (&vals)[ENGRAM_MAX_NGRAM],
                                            uint64_t (&cells)[ENGRAM_MAX_NGRAM]) {
  const int N = a.max_ngram;
  bool blocked = false;
#pragma unroll
  for (int i = 0; i < ENGRAM_MAX_NGRAM; ++i) {
    if (i < N) {
      const int32_t v = cell_value(a, token_map, row, hist, t - i);
      vals[i] = v;
      blocked = blocked || (v < 0);
      cells[i] = blocked ? (uint64_t)a.pad_id : (uint64_t)v;
    }
  }
}

// (x mod p) + off with the reciprocal r = floor((2^64 - 1) / p): q = hi64(x r)
// is floor(x / p) or one less for x < 2^63, p < 2^32, so one conditional
// subtraction gives the exact remainder.
__device__ __forceinline__ int64_t row_id(uint64_t x, uint64_t p, uint64_t recip, int64_t off) {
  uint64_t r = x - __umul64hi(x, recip) * p;
  if (r >= p) r -= p;
  return (int64_t)r + off;
}

__device__ __forceinline__ uint32_t dequant_byte_exact(uint32_t byte, uint32_t s) {
  const uint32_t sign = (byte & 0x80u) << 8;
  const uint32_t mag = byte & 0x7Fu;
  if (mag == 0x7Fu || s == 0xFFu) return 0x7FC0u | sign;     // E4M3 NaN, E8M0 NaN
  const float f = ldexpf(__uint_as_float(mag << 20), (int)s - 7);
  return engram::f32_to_bf16_rne(f) | sign;
}

__device__ __forceinline__ uint32_t dequant_pair_fast(uint32_t word, float scale, bool hi) {
  const auto f = hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true)
                    : __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
  const uint32_t lo32 = __float_as_uint(f[0] * scale);
  const uint32_t hi32 = __float_as_uint(f[1] * scale);
  return (lo32 >> 16) | (hi32 & 0xFFFF0000u);
}

// 8 E4M3 bytes under E8M0 scale s as 8 bf16. For scales 10..246 no value can
// leave the bf16 normal range, so the hardware OCP-E4M3 -> f32 conversion, one
// multiply by the power of two 2^(s-127) and truncation to the upper 16 bits
// are exact. Other scales take an integer path: the E4M3 magnitude bits placed
// at the f32 exponent/mantissa position give value * 2^-120 (subnormal codes
// become f32 denormals, kept by the denormal mode), ldexp by s - 7 is exact or
// overflows, and one nearest-even rounding to bf16 handles bf16 subnormals.
__device__ __forceinline__ uint4 dequant8(uint2 q, uint32_t s) {
  uint4 o;
  if (s - 10u <= 236u) {
    const float scale = __uint_as_float(s << 23);
    o.x = dequant_pair_fast(q.x, scale, false);
    o.y = dequant_pair_fast(q.x, scale, true);
    o.z = dequant_pair_fast(q.y, scale, false);
    o.w = dequant_pair_fast(q.y, scale, true);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t word = i < 2 ? q.x : q.y;
      const int sh = (i & 1) * 16;
      w[i] = dequant_byte_exact((word >> sh) & 0xFFu, s) |
             (dequant_byte_exact((word >> (sh + 8)) & 0xFFu, s) << 16);
    }
    o = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return o;
}

}  // namespace engram_rows
