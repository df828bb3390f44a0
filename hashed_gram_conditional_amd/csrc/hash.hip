// Steps 1-2 of the Engram layer: compressed ids, multiply-XOR n-gram mixes and
// per-head prime moduli into one offset table.
//
// Pages: "DeepSeek-V4.1 模型结构（5）：记忆，Engram", eq. (H), the items under it
// (orders are computed incrementally; the heads of an order share one mix;
// sequence starts pad), the image-token paragraph (DEAD cascade) and
// "一层只有一张表" (segment offsets); "ds4.c 学习笔记 · Engram", "布局与哈希探测"
// (3-token hash state); "条件记忆：DeepSeek V4.1 Engram 如何用 O(1) 查表换掉一层计算",
// §4.4 (decode fuses the hash with the history commit).
//
// Layout: one block of 256 threads owns TOK consecutive flat tokens (256, or
// 64 for calls of at most 4096 tokens, such as decode steps, so that the work
// spreads over more CUs). Phase 1: one thread per token builds the look-back
// cells once, then each layer's N-1 mixes (its own multipliers) into LDS.
// Phase 2: for each layer the block writes its TOK x S int64 row ids as one
// contiguous, fully coalesced span of that layer's [tokens, S] slice, all 256
// threads reducing mixes modulo the layer's primes. Several layers in one pass follow "条件记忆：DeepSeek V4.1
// Engram 如何用 O(1) 查表换掉一层计算" §2.4 (every layer's ids are known before
// the layer loop) and "DeepSeek-V4.1 模型结构（5）：记忆，Engram", "一层只有一张表"
// (each layer has its own primes and multipliers).
//
// mix < 2^63 and p < 2^32, and gfx950 has no 64-bit integer divide, so
// x mod p uses the precomputed reciprocal r = floor((2^64-1)/p): q = hi64(x r)
// is floor(x/p) or one less (the error term x(1 + (2^64-1) mod p) / (p 2^64)
// is below 1), so one conditional subtraction gives the exact remainder
// (Barrett, "Implementing the RSA public key encryption algorithm on a standard
// digital signal processor", CRYPTO 1986).
#include "row_device.h"

namespace {

constexpr int kThreads = 256;

using engram_rows::cell_value;

template <int L, int TOK>
__global__ __launch_bounds__(kThreads) void hash_kernel(
    EngramHashArgs a, const int32_t *__restrict__ token_map, const int32_t *__restrict__ ids,
    int64_t batch, int64_t seq, const int32_t *hist_in, int32_t *hist_out,
    int64_t *__restrict__ row_ids, int commit_history) {
  constexpr int kSeg = L * ENGRAM_MAX_SEGMENTS < ENGRAM_MAX_TOTAL_SEGMENTS
                           ? L * ENGRAM_MAX_SEGMENTS : ENGRAM_MAX_TOTAL_SEGMENTS;
  __shared__ uint64_t s_mix[L][ENGRAM_MAX_NGRAM - 1][TOK];
  __shared__ uint64_t s_recip[kSeg];
  __shared__ int64_t s_off[kSeg];
  __shared__ uint32_t s_prime[kSeg];

  const int tid = threadIdx.x;
  const int S = a.segments;
  const int N = a.max_ngram;
  const int H = N - 1;
  for (int j = tid; j < L * S; j += kThreads) {
    s_prime[j] = a.prime[j];
    s_recip[j] = a.recip[j];
    s_off[j] = a.offset[j];
  }

  const int64_t ntok = batch * seq;
  const int64_t tok0 = (int64_t)blockIdx.x * TOK;
  const int64_t g = tok0 + tid;
  if (tid < TOK && g < ntok) {
    const int64_t b = g / seq;
    const int64_t t = g - b * seq;
    const int32_t *row = ids + b * seq;
    const int32_t *hist = hist_in ? hist_in + b * H : nullptr;
    int32_t vals[ENGRAM_MAX_NGRAM];
    uint64_t cells[ENGRAM_MAX_NGRAM];
    engram_rows::token_cells(a, token_map, row, hist, t, vals, cells);
#pragma unroll
    for (int l = 0; l < L; ++l) {
      uint64_t mix = 0;
#pragma unroll
      for (int i = 0; i < ENGRAM_MAX_NGRAM; ++i) {
        if (i < N) {
          // Orders build on each other: mix_{n+1} = mix_n ^ x'_{t-n} m_n.
          mix ^= cells[i] * a.mult[l][i];
          if (i >= 1) s_mix[l][i - 1][tid] = mix;
        }
      }
    }
    if (commit_history) {
      // T == 1: this thread is its sequence's only token. Every history read
      // above precedes these writes, so hist_out may alias hist_in.
#pragma unroll
      for (int s = 0; s < ENGRAM_MAX_NGRAM - 1; ++s)
        if (s < H) hist_out[b * H + s] = vals[H - 1 - s];
    }
  }
  __syncthreads();

  const int64_t left = ntok - tok0;
  const int ntb = left < TOK ? (int)left : TOK;
  const int total = ntb * S;
#pragma unroll
  for (int l = 0; l < L; ++l) {
    int64_t *out = row_ids + (int64_t)l * ntok * S + tok0 * S;
    for (int o = tid; o < total; o += kThreads) {
      const int lt = o / S;
      const int j = o - lt * S;
      const int js = l * S + j;
      out[o] = engram_rows::row_id(s_mix[l][j / a.heads][lt], s_prime[js], s_recip[js],
                                   s_off[js]);
    }
  }
}

// History after a chunk of T != 1 tokens, one thread per sequence. Runs after
// hash_kernel on the same stream, so hist_out may alias hist_in.
__global__ void history_kernel(EngramHashArgs a, const int32_t *__restrict__ token_map,
                               const int32_t *__restrict__ ids, int64_t batch, int64_t seq,
                               const int32_t *hist_in, int32_t *hist_out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int H = a.max_ngram - 1;
  const int32_t *row = ids + b * seq;
  const int32_t *hist = hist_in ? hist_in + b * H : nullptr;
  int32_t vals[ENGRAM_MAX_NGRAM - 1];
#pragma unroll
  for (int s = 0; s < ENGRAM_MAX_NGRAM - 1; ++s)
    if (s < H) vals[s] = cell_value(a, token_map, row, hist, seq - H + s);
#pragma unroll
  for (int s = 0; s < ENGRAM_MAX_NGRAM - 1; ++s)
    if (s < H) hist_out[b * H + s] = vals[s];
}

}  // namespace

hipError_t engram_launch_hash(const EngramHashArgs &a, const int32_t *token_map,
                              const int32_t *ids, int64_t batch, int64_t seq,
                              const int32_t *hist_in, int32_t *hist_out, int64_t *row_ids,
                              hipStream_t stream) {
  const int64_t ntok = batch * seq;
  const bool fused = hist_out != nullptr && seq == 1;
  if (ntok > 0) {
    const bool small = ntok <= 4096;
    const int tok = small ? 64 : 256;
    const dim3 grid((unsigned)((ntok + tok - 1) / tok));
    const int commit = fused ? 1 : 0;
#define ENGRAM_HASH_CASE(Lc)                                                                  \
  case Lc:                                                                                  \
    if (small)                                                                              \
      hipLaunchKernelGGL((hash_kernel<Lc, 64>), grid, dim3(kThreads), 0, stream, a, token_map, \
                         ids, batch, seq, hist_in, hist_out, row_ids, commit);              \
    else                                                                                    \
      hipLaunchKernelGGL((hash_kernel<Lc, 256>), grid, dim3(kThreads), 0, stream, a,        \
                         token_map, ids, batch, seq, hist_in, hist_out, row_ids, commit);   \
    break;
    switch (a.layers) {
      ENGRAM_HASH_CASE(1)
      ENGRAM_HASH_CASE(2)
      ENGRAM_HASH_CASE(3)
      ENGRAM_HASH_CASE(4)
      default:
        return hipErrorInvalidValue;
    }
#undef ENGRAM_HASH_CASE
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (hist_out != nullptr && !fused && batch > 0) {
    const int threads = 128;
    const int64_t blocks = (batch + threads - 1) / threads;
    hipLaunchKernelGGL(history_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, a,
                       token_map, ids, batch, seq, hist_in, hist_out);
    return hipGetLastError();
  }
  return hipSuccess;
}
