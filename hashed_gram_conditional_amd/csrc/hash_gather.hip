// Steps 1-3 in one launch for decode-sized calls: each token's row ids are
// formed and its rows gathered and dequantised by one block, so the ids never
// go to memory and the step saves a launch and a dependent round trip.
//
// Pages: as for the hash ("DeepSeek-V4.1 模型结构（5）：记忆，Engram", eq. (H)
// and the image-token paragraph; "ds4.c 学习笔记 · Engram", "布局与哈希探测")
// and the gather ("ds4.c 学习笔记 · Engram", "永不常驻的 I/O 设计";
// "条件记忆：DeepSeek V4.1 Engram 如何用 O(1) 查表换掉一层计算" §五 for
// out-of-range rows); "条件记忆：DeepSeek V4.1 Engram 如何用 O(1) 查表换掉一层计算"
// §4.4 (decode fuses the hash with the history commit).
//
// One block of 128 threads per token. Thread 0 builds the token's cells and
// mixes (engram_rows::token_cells, as the hash kernel does) and commits the
// history of a one-token step; threads j < S form row id j in LDS
// (engram_rows::row_id); then each half-wave owns rows h, h + 4, ... of the
// token, issues all its loads before converting any, and writes each row as
// the gather kernel does (lane l: payload bytes 8l..8l+7 and scale l/4, 8 bf16
// out, engram_rows::dequant8). The rows are the separate kernels' bits. The
// split variant (for the block-scaled FP8 projection) copies each row's codes
// and scales apart instead, as the row-splitting gather does.
#include "row_device.h"

namespace {

constexpr int kThreads = 128;
constexpr int kHalves = kThreads / 32;
constexpr int kMaxRowsPerHalf = (ENGRAM_MAX_SEGMENTS + kHalves - 1) / kHalves;

template <bool SPLIT>
__global__ __launch_bounds__(kThreads) void hash_gather_e4m3_kernel(
    EngramHashArgs a, const int32_t *__restrict__ token_map, const int32_t *__restrict__ ids,
    int64_t seq, const int32_t *hist_in, int32_t *hist_out, int commit_history,
    const uint8_t *__restrict__ table, int64_t table_rows, uint16_t *__restrict__ out,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  __shared__ uint64_t s_mix[ENGRAM_MAX_NGRAM - 1];
  __shared__ int64_t s_rid[ENGRAM_MAX_SEGMENTS];
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int S = a.segments;
  const int N = a.max_ngram;
  const int H = N - 1;
  const int64_t b = g / seq;
  const int64_t t = g - b * seq;
  if (tid == 0) {
    const int32_t *row = ids + b * seq;
    const int32_t *hist = hist_in ? hist_in + b * H : nullptr;
    int32_t vals[ENGRAM_MAX_NGRAM];
    uint64_t cells[ENGRAM_MAX_NGRAM];
    engram_rows::token_cells(a, token_map, row, hist, t, vals, cells);
    uint64_t mix = 0;
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_NGRAM; ++i) {
      if (i < N) {
        mix ^= cells[i] * a.mult[0][i];
        if (i >= 1) s_mix[i - 1] = mix;
      }
    }
    if (commit_history) {
      // one token per sequence: every history read above precedes these writes
#pragma unroll
      for (int s = 0; s < ENGRAM_MAX_NGRAM - 1; ++s)
        if (s < H) hist_out[b * H + s] = vals[H - 1 - s];
    }
  }
  __syncthreads();
  if (tid < S)
    s_rid[tid] = engram_rows::row_id(s_mix[tid / a.heads], a.prime[tid], a.recip[tid],
                                     a.offset[tid]);
  __syncthreads();

  const int half = tid >> 5;
  const int l = tid & 31;
  uint2 q[kMaxRowsPerHalf];
  uint32_t sc[kMaxRowsPerHalf];
  bool in[kMaxRowsPerHalf];
#pragma unroll
  for (int k = 0; k < kMaxRowsPerHalf; ++k) {
    const int j = half + k * kHalves;
    in[k] = false;
    if (j < S) {
      const int64_t r = s_rid[j];
      in[k] = (uint64_t)r < (uint64_t)table_rows;
      if (in[k]) {
        const uint8_t *row = table + r * ENGRAM_ROW_BYTES;
        q[k] = *reinterpret_cast<const uint2 *>(row + 8 * l);
        sc[k] = row[ENGRAM_ROW_DIM_E4M3 + (l >> 2)];
      }
    }
  }
  if constexpr (SPLIT) {
    // row j of the token: its 256 codes and its 8 scales, bytes unchanged
#pragma unroll
    for (int k = 0; k < kMaxRowsPerHalf; ++k) {
      const int j = half + k * kHalves;
      if (j < S) {
        const int64_t r = g * (int64_t)S + j;
        *reinterpret_cast<uint2 *>(codes + r * ENGRAM_ROW_DIM_E4M3 + 8 * l) =
            in[k] ? q[k] : make_uint2(0u, 0u);
        // lane l holds scale byte l / 4
        if ((l & 3) == 0) scales[r * 8 + (l >> 2)] = in[k] ? (uint8_t)sc[k] : (uint8_t)0;
      }
    }
  } else {
    uint16_t *dst = out + g * (int64_t)S * ENGRAM_ROW_DIM_E4M3;
#pragma unroll
    for (int k = 0; k < kMaxRowsPerHalf; ++k) {
      const int j = half + k * kHalves;
      if (j < S) {
        const uint4 o = in[k] ? engram_rows::dequant8(q[k], sc[k]) : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4 *>(dst + j * ENGRAM_ROW_DIM_E4M3 + 8 * l) = o;
      }
    }
  }
}

}  // namespace

hipError_t engram_launch_hash_gather_e4m3(const EngramHashArgs &a, const int32_t *token_map,
                                          const int32_t *ids, int64_t batch, int64_t seq,
                                          const int32_t *hist_in, int32_t *hist_out,
                                          const uint8_t *table, int64_t table_rows,
                                          uint16_t *out, hipStream_t stream) {
  const int64_t ntok = batch * seq;
  if (ntok <= 0) return hipSuccess;
  if (a.layers != 1 || (hist_out != nullptr && seq != 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(hash_gather_e4m3_kernel<false>, dim3((unsigned)ntok), dim3(kThreads), 0,
                     stream, a, token_map, ids, seq, hist_in, hist_out,
                     hist_out != nullptr ? 1 : 0, table, table_rows, out, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t engram_launch_hash_gather_mx(const EngramHashArgs &a, const int32_t *token_map,
                                        const int32_t *ids, int64_t batch, int64_t seq,
                                        const int32_t *hist_in, int32_t *hist_out,
                                        const uint8_t *table, int64_t table_rows, uint8_t *codes,
                                        uint8_t *scales, hipStream_t stream) {
  const int64_t ntok = batch * seq;
  if (ntok <= 0) return hipSuccess;
  if (a.layers != 1 || (hist_out != nullptr && seq != 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(hash_gather_e4m3_kernel<true>, dim3((unsigned)ntok), dim3(kThreads), 0,
                     stream, a, token_map, ids, seq, hist_in, hist_out,
                     hist_out != nullptr ? 1 : 0, table, table_rows, nullptr, codes, scales);
  return hipGetLastError();
}
