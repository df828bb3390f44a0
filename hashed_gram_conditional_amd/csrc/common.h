// Shared device helpers of the Engram HIP kernels (gfx950, wave64).
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

// Launchers implemented by the kernel translation units. They validate nothing:
// the C-ABI layer checks every argument first. Each returns hipSuccess or the
// launch error.
// Hash setup of `layers` Engram layers sharing one token map; segment j of
// layer l is entry l * segments + j of the per-segment arrays.
struct EngramHashArgs {
  int32_t raw_vocab, compressed_vocab, max_ngram, heads, segments, pad_id, layers;
  uint64_t mult[ENGRAM_MAX_LAYERS][ENGRAM_MAX_NGRAM];
  uint32_t prime[ENGRAM_MAX_TOTAL_SEGMENTS];
  uint64_t recip[ENGRAM_MAX_TOTAL_SEGMENTS];   // floor((2^64 - 1) / prime)
  int64_t offset[ENGRAM_MAX_TOTAL_SEGMENTS];
};

hipError_t engram_launch_hash(const EngramHashArgs &a, const int32_t *token_map,
                              const int32_t *ids, int64_t batch, int64_t seq,
                              const int32_t *hist_in, int32_t *hist_out,
                              int64_t *row_ids, hipStream_t stream);

// Hash and gather of one Engram layer in one launch, one block per token, for
// decode-sized calls on an HBM-resident E4M3 table: the rows (bf16, [batch *
// seq, S * 256]) of the separate kernels, no row ids written. a.layers must be
// 1, and hist_out NULL or seq 1 (the history committed in place).
hipError_t engram_launch_hash_gather_e4m3(const EngramHashArgs &a, const int32_t *token_map,
                                          const int32_t *ids, int64_t batch, int64_t seq,
                                          const int32_t *hist_in, int32_t *hist_out,
                                          const uint8_t *table, int64_t table_rows,
                                          uint16_t *out, hipStream_t stream);

// host_table: the table is pinned host memory; the gather then runs on a few
// CUs as a grid-strided kernel, leaving the rest to concurrent work.
hipError_t engram_launch_gather_e4m3(const uint8_t *table, int64_t table_rows,
                                     const int64_t *row_ids, int64_t n_ids,
                                     uint16_t *out, bool host_table, hipStream_t stream);

hipError_t engram_launch_gather_rows(const uint8_t *table, int64_t table_rows,
                                     const int64_t *row_ids, int64_t n_ids, uint8_t *out,
                                     bool host_table, hipStream_t stream);

// Rows split into their codes [n_ids, 256] and scales [n_ids, 8].
hipError_t engram_launch_gather_mx(const uint8_t *table, int64_t table_rows,
                                   const int64_t *row_ids, int64_t n_ids, uint8_t *codes,
                                   uint8_t *scales, bool host_table, hipStream_t stream);

hipError_t engram_launch_gather_f32(const float *table, int64_t table_rows,
                                    int32_t row_dim, const int64_t *row_ids,
                                    int64_t n_ids, float *out, hipStream_t stream);

// bf16 projection kv[m, n] = sum_k e[m, k] w[n, k]; w's rows are ldw >= k
// elements apart, e and kv are dense.
hipError_t engram_launch_gemm_bf16(const uint16_t *e, const uint16_t *w, int64_t ldw,
                                   uint16_t *kv, int64_t m, int64_t n, int64_t k, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

// The bf16 projection of hc keys and one value (n = (hc + 1) * dim, dim a
// multiple of 256) over 256 x 256 tiles whatever the token count: value columns
// stored as engram_launch_gemm_bf16's whole-tile kernel stores them, key tiles
// replaced by the gate's sums of each token (engram::gate_sums_pairs), which
// read h [m, hc * dim] and the folded gate weights qk_w [hc * dim].
hipError_t engram_launch_gemm_bf16_sums(const uint16_t *e, const uint16_t *w, int64_t ldw,
                                        const uint16_t *h, const float *qk_w, uint16_t *kv,
                                        int64_t m, int32_t hc, int32_t dim, int64_t k,
                                        hipStream_t stream);

// Whether engram_launch_gemm_bf16 runs this shape as whole 256 x 256 tiles
// (enough of them for every CU, no skinny decode schedule).
hipError_t engram_gemm_bf16_whole_tiles(int64_t m, int64_t n, int64_t k, bool *whole);

// Workspace the bf16 projection uses for a split-K schedule (0 when none).
hipError_t engram_gemm_bf16_workspace(int64_t m, int64_t n, int64_t k, size_t *bytes);

// Block-scaled FP8 projection: W codes [n, 256 S] and scales [n, 8 S], e the
// looked-up 264-byte rows [m, S, 264]; kv bf16 [m, n]. Split-K as for bf16
// when a large enough workspace is given.
hipError_t engram_launch_gemm_mx(const uint8_t *w_codes, const uint8_t *w_scales,
                                 const uint8_t *e_codes, const uint8_t *e_scales,
                                 int32_t segments, uint16_t *kv,
                                 int64_t m, int64_t n, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);
hipError_t engram_gemm_mx_workspace(int64_t m, int64_t n, int32_t segments, size_t *bytes);
// The block-scaled FP8 projection over whole 256 x 256 tiles with the gate's
// sums in the key tiles' epilogue (as engram_launch_gemm_bf16_sums), and
// whether engram_launch_gemm_mx runs a shape as whole tiles.
hipError_t engram_launch_gemm_mx_sums(const uint8_t *w_codes, const uint8_t *w_scales,
                                      const uint8_t *e_codes, const uint8_t *e_scales,
                                      int32_t segments, const uint16_t *h, const float *qk_w,
                                      uint16_t *kv, int64_t m, int32_t hc, int32_t dim,
                                      hipStream_t stream);
hipError_t engram_gemm_mx_whole_tiles(int64_t m, int64_t n, int32_t segments, bool *whole);

hipError_t engram_launch_gemm_f32(const float *e, const float *w, int64_t ldw, float *kv,
                                  int64_t m, int64_t n, int64_t k, hipStream_t stream);

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

// stats == NULL: the gate and the residual update. stats != NULL (float
// [tokens, hc + 1]): gates and the value row's mean square per token, h
// untouched. plain selects sigmoid(s) over the signed root. k_w == NULL: q_w
// holds the folded products q_w * k_w (engram_launch_fold_gate_weights).
hipError_t engram_launch_gate(bool f32, const int32_t *ids, EngramDeadRule dead_rule,
                              const void *kv, const float *q_w, const float *k_w,
                              void *h, float *gate_out, float *stats, int64_t tokens,
                              int32_t hc, int32_t dim, float eps, float clamp, int plain,
                              hipStream_t stream);

// The gate and residual update from the sums engram_launch_gemm_bf16_sums left
// in kv's key columns, the value row of kv and h (bf16; dim a multiple of 256).
// stats != NULL: engram_launch_gate's statistics mode on the sums instead.
hipError_t engram_launch_gate_sums(const int32_t *ids, EngramDeadRule dead_rule, const void *kv,
                                   void *h, float *gate_out, float *stats, int64_t tokens,
                                   int32_t hc, int32_t dim, float eps, float clamp, int plain,
                                   hipStream_t stream);

// qk_w[i] = q_w[i] * k_w[i] over hc * dim fp32 values (dim a multiple of 8).
hipError_t engram_launch_fold_gate_weights(const float *q_w, const float *k_w, float *qk_w,
                                           int32_t hc, int32_t dim, hipStream_t stream);

// Short convolution branch and its history (conv.hip).
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
hipError_t engram_launch_short_conv(bool f32, const EngramConvArgs &c, const int32_t *ids,
                                    EngramDeadRule dead_rule, const void *kv, const float *stats,
                                    void *h, int64_t batch, int64_t seq, int32_t hc,
                                    int32_t dim, hipStream_t stream);

// dst[c * dst_ld + r] = src[r, c] for a row-major [rows, cols] array of 2- or
// 4-byte elements (layout.hip).
hipError_t engram_launch_transpose(const void *src, void *dst, int64_t rows, int64_t cols,
                                   int64_t dst_ld, int elem_bytes, hipStream_t stream);
