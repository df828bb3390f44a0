// Shared device helpers of the Engram HIP kernels (gfx950, wave64) and the
// argument structs the kernels and their launchers share; the launchers'
// declarations follow in launchers.h, so that this file changes only with code
// the kernels compile in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram.h"

namespace engram {

constexpr int kWave = 64;

// bf16 bit pattern of a float, rounded to nearest with ties to even. Exact for
// subnormals (the encoding is linear there) and rounds finite overflow to inf.
// NaN inputs are handled by the callers that can see them.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Two bf16 (low half = first element) from two floats, nearest-even: one
// v_cvt_pk_bf16_f32. On gfx950 it gives the bits of f32_to_bf16_rne for every
// finite and infinite input (checked on 3.4e7 random and tie patterns); a NaN
// comes out as a quiet NaN.
typedef __bf16 engram_bf16x2 __attribute__((ext_vector_type(2)));
typedef float engram_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const engram_f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, engram_bf16x2));
}

// Where the projection with gate sums leaves token t's key-side sums: float2
// index of kv row t's start (bf16 rows of (hc + 1) * dim, dim a multiple of 4).
// Pair stream * (dim / 128) + block from there holds (sum k^2, sum h q_w k_w k)
// over 128-column block `block` of that stream; these bytes lie in the row's
// key columns, which that projection does not otherwise write.
__device__ __forceinline__ int64_t gate_sums_pairs(int64_t t, int hc, int dim) {
  return t * (int64_t)(hc + 1) * dim / 4;
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Eight consecutive elements of a bf16 (F32 = false) or fp32 row, addressed by
// chunk index: one 16-byte or two 16-byte accesses.
template <bool F32>
struct Chunk8;
template <>
struct Chunk8<false> {
  uint4 v;
  __device__ __forceinline__ void load(const void *p, int64_t i) {
    v = reinterpret_cast<const uint4 *>(p)[i];
  }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void put(void *p, int64_t i) const {
    reinterpret_cast<uint4 *>(p)[i] = v;
  }
  __device__ __forceinline__ float operator[](int e) const {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return bf16_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
  __device__ __forceinline__ static void store(void *p, int64_t i, const float f[8]) {
    uint4 o;
    o.x = pack_bf16x2(f[0], f[1]);
    o.y = pack_bf16x2(f[2], f[3]);
    o.z = pack_bf16x2(f[4], f[5]);
    o.w = pack_bf16x2(f[6], f[7]);
    reinterpret_cast<uint4 *>(p)[i] = o;
  }
  // the same accesses with the nontemporal hint, for data used once
  __device__ __forceinline__ void load_nt(const void *p, int64_t i) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + i);
    v = make_uint4(t.x, t.y, t.z, t.w);
  }
  __device__ __forceinline__ static void store_nt(void *p, int64_t i, const float f[8]) {
    const u32x4 o = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7])};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(p) + i);
  }
};
template <>
struct Chunk8<true> {
  float4 a, b;
  __device__ __forceinline__ void load(const void *p, int64_t i) {
    a = reinterpret_cast<const float4 *>(p)[2 * i];
    b = reinterpret_cast<const float4 *>(p)[2 * i + 1];
  }
  __device__ __forceinline__ void zero() {
    a = make_float4(0.f, 0.f, 0.f, 0.f);
    b = a;
  }
  __device__ __forceinline__ void put(void *p, int64_t i) const {
    reinterpret_cast<float4 *>(p)[2 * i] = a;
    reinterpret_cast<float4 *>(p)[2 * i + 1] = b;
  }
  __device__ __forceinline__ float operator[](int e) const {
    const float4 &q = e < 4 ? a : b;
    const int r = e & 3;
    return r == 0 ? q.x : r == 1 ? q.y : r == 2 ? q.z : q.w;
  }
  __device__ __forceinline__ static void store(void *p, int64_t i, const float f[8]) {
    reinterpret_cast<float4 *>(p)[2 * i] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4 *>(p)[2 * i + 1] = make_float4(f[4], f[5], f[6], f[7]);
  }
  __device__ __forceinline__ void load_nt(const void *p, int64_t i) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + 2 * i);
    const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + 2 * i + 1);
    a = make_float4(x.x, x.y, x.z, x.w);
    b = make_float4(y.x, y.y, y.z, y.w);
  }
  __device__ __forceinline__ static void store_nt(void *p, int64_t i, const float f[8]) {
    const f32x4 x = {f[0], f[1], f[2], f[3]}, y = {f[4], f[5], f[6], f[7]};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p) + 2 * i);
    __builtin_nontemporal_store(y, reinterpret_cast<f32x4 *>(p) + 2 * i + 1);
  }
};

}  // namespace engram

// Kernel arguments shared by the kernels and their launchers.
// Hash setup of `layers` Engram layers sharing one token map; segment j of
// layer l is entry l * segments + j of the per-segment arrays.
struct EngramHashArgs {
  int32_t raw_vocab, compressed_vocab, max_ngram, heads, segments, pad_id, layers;
  uint64_t mult[ENGRAM_MAX_LAYERS][ENGRAM_MAX_NGRAM];
  uint32_t prime[ENGRAM_MAX_TOTAL_SEGMENTS];
  uint64_t recip[ENGRAM_MAX_TOTAL_SEGMENTS];   // floor((2^64 - 1) / prime)
  int64_t offset[ENGRAM_MAX_TOTAL_SEGMENTS];
};

// Which positions are DEAD. A raw id outside [0, raw_vocab) always is; with a
// token map, so is a raw id whose compressed id lies outside
// [0, compressed_vocab), the hash's own rule, so that the gate and the
// convolution of a layer agree with its row ids on every position.
struct EngramDeadRule {
  int32_t raw_vocab;
  int32_t compressed_vocab;
  const int32_t *token_map;   // NULL: the raw id alone decides
};

__device__ __forceinline__ bool engram_dead(const EngramDeadRule &r, int32_t x) {
  if (x < 0 || x >= r.raw_vocab) return true;
  if (r.token_map == nullptr) return false;
  const int32_t v = r.token_map[x];
  return v < 0 || v >= r.compressed_vocab;
}

// The short convolution branch and its history (conv.hip).
struct EngramConvArgs {
  int taps, dilation, history;   // history = (taps - 1) * dilation
  float eps;
  const float *weight;           // [hc, dim, taps]
  const float *norm_weight;      // [hc, dim] or NULL
  const void *state_v_in;        // [batch, history, dim] kv dtype, or NULL
  const float *state_s_in;       // [batch, history, hc + 1]
  void *state_v_out;             // or NULL
  float *state_s_out;
};

#include "launchers.h"
