// Step 3 of the Engram layer: gather table rows and dequantise them to bf16
// (or copy them unchanged for the block-scaled FP8 projection).
//
// Pages: "ds4.c 学习笔记 · Engram", "布局与哈希探测" (264-byte rows) and
// "永不常驻的 I/O 设计" (256 E4M3 bytes + 8 E8M0 scales, 32 values per scale);
// "DeepSeek-V4.1 模型结构（5）：记忆，Engram", "196B 参数怎么存、怎么取" (rows
// dequantise independently); "条件记忆：DeepSeek V4.1 Engram 如何用 O(1) 查表换掉一层计算",
// §2.3 (bf16 output) and §五 (out-of-range rows read as zeros).
//
// E4M3 rows: a half-wave (32 lanes) owns one row; lane l reads payload bytes
// 8l..8l+7 (one dwordx2; rows start 8-byte aligned because 264 = 8 * 33) and
// the scale byte l/4, and writes 8 bf16 (one dwordx4), so each half-wave reads
// 256 contiguous bytes and writes 512 contiguous bytes. A wave keeps 16 rows in
// flight (8 row pairs) before converting any of them, to cover HBM latency on
// random rows.
//
// Dequantisation is exact. For scales 10..246 no value can leave the bf16
// normal range, so the hardware OCP-E4M3 -> f32 conversion, one multiply by the
// power of two 2^(s-127) and truncation to the upper 16 bits are exact. Other
// scales take an integer path: the E4M3 magnitude bits placed at the f32
// exponent/mantissa position give value * 2^-120 (subnormal codes become f32
// denormals, kept by the denormal mode), ldexp by s - 7 is exact or overflows,
// and one nearest-even rounding to bf16 handles bf16 subnormals.
#include "row_device.h"

namespace {

constexpr int kSlots = 8;                 // row pairs per wave
constexpr int kRowsPerWave = 2 * kSlots;
constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kRowsPerWave * (kThreads / engram::kWave);

using engram_rows::dequant8;

template <int NT>
__global__ __launch_bounds__(NT) void gather_e4m3_kernel(
    const uint8_t *__restrict__ table, int64_t table_rows, const int64_t *__restrict__ row_ids,
    int64_t n, uint16_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int l = lane & 31;
  const int64_t waves = (int64_t)gridDim.x * (NT >> 6);
  for (int64_t wave = ((int64_t)blockIdx.x * NT + threadIdx.x) >> 6;
       wave * kRowsPerWave < n; wave += waves) {
  const int64_t base = wave * kRowsPerWave;

  int64_t r[kSlots];
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int64_t idx = base + 2 * s + half;
    r[s] = idx < n ? row_ids[idx] : -1;
  }
  uint2 q[kSlots];
  uint32_t sc[kSlots];
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    if ((uint64_t)r[s] < (uint64_t)table_rows) {
      const uint8_t *row = table + r[s] * ENGRAM_ROW_BYTES;
      q[s] = *reinterpret_cast<const uint2 *>(row + 8 * l);
      sc[s] = row[ENGRAM_ROW_DIM_E4M3 + (l >> 2)];
    } else {
      q[s] = make_uint2(0u, 0u);
      sc[s] = 0u;
    }
  }
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int64_t idx = base + 2 * s + half;
    if (idx < n) {
      const uint4 o = ((uint64_t)r[s] < (uint64_t)table_rows) ? dequant8(q[s], sc[s])
                                                               : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4 *>(out + idx * ENGRAM_ROW_DIM_E4M3 + 8 * l) = o;
    }
  }
  }
}

__global__ __launch_bounds__(kThreads) void gather_f32_kernel(
    const float *__restrict__ table, int64_t table_rows, int32_t row_dim,
    const int64_t *__restrict__ row_ids, int64_t n, float *__restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int cpr = row_dim >> 2;
  const int64_t i = g / cpr;
  const int c = (int)(g - i * cpr);
  if (i >= n) return;
  const int64_t r = row_ids[i];
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if ((uint64_t)r < (uint64_t)table_rows)
    v = reinterpret_cast<const float4 *>(table + r * row_dim)[c];
  reinterpret_cast<float4 *>(out + i * row_dim)[c] = v;
}

// Rows copied unchanged (the block-scaled FP8 projection consumes them as
// they are): one thread per 8-byte word, 33 words per 264-byte row, so
// consecutive threads cover a row's contiguous bytes. Ids outside [0, rows)
// give zero rows.
constexpr int kRowWords = ENGRAM_ROW_BYTES / 8;

// U words per thread per pass, kept in flight together: a pass of the whole grid
// covers U * threads words, then the grid strides on.
template <int NT, int U>
__global__ __launch_bounds__(NT) void gather_rows_kernel(
    const uint8_t *__restrict__ table, int64_t table_rows, const int64_t *__restrict__ row_ids,
    int64_t n_ids, uint8_t *__restrict__ out) {
  const int64_t total = n_ids * kRowWords;
  const int64_t threads = (int64_t)gridDim.x * NT;
  for (int64_t g0 = (int64_t)blockIdx.x * NT + threadIdx.x; g0 < total; g0 += U * threads) {
    uint2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + u * threads;
      v[u] = make_uint2(0u, 0u);
      if (g < total) {
        const int64_t i = g / kRowWords;
        const int w = (int)(g - i * kRowWords);
        const int64_t r = row_ids[i];
        if (r >= 0 && r < table_rows)
          v[u] = *reinterpret_cast<const uint2 *>(table + r * ENGRAM_ROW_BYTES + (int64_t)w * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + u * threads;
      if (g < total) *reinterpret_cast<uint2 *>(out + g * 8) = v[u];
    }
  }
}

// The same rows split for the block-scaled FP8 projection: words 0-31 of row i
// (its 256 codes) go to codes[i * 256 ..], word 32 (its 8 scales) to
// scales[i * 8]. With the S rows of a token side by side, codes is the token's
// K-long row of E4M3 inputs and scales its K/32 block scales.
template <int NT, int U>
__global__ __launch_bounds__(NT) void gather_mx_kernel(
    const uint8_t *__restrict__ table, int64_t table_rows, const int64_t *__restrict__ row_ids,
    int64_t n_ids, uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  const int64_t total = n_ids * kRowWords;
  const int64_t threads = (int64_t)gridDim.x * NT;
  for (int64_t g0 = (int64_t)blockIdx.x * NT + threadIdx.x; g0 < total; g0 += U * threads) {
    uint2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + u * threads;
      v[u] = make_uint2(0u, 0u);
      if (g < total) {
        const int64_t i = g / kRowWords;
        const int w = (int)(g - i * kRowWords);
        const int64_t r = row_ids[i];
        if (r >= 0 && r < table_rows)
          v[u] = *reinterpret_cast<const uint2 *>(table + r * ENGRAM_ROW_BYTES + (int64_t)w * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + u * threads;
      if (g < total) {
        const int64_t i = g / kRowWords;
        const int w = (int)(g - i * kRowWords);
        uint8_t *dst = w < kRowWords - 1 ? codes + i * ENGRAM_ROW_DIM_E4M3 + (int64_t)w * 8
                                         : scales + i * 8;
        *reinterpret_cast<uint2 *>(dst) = v[u];
      }
    }
  }
}

// Grid of the gathers from a host-resident table: one 1024-thread block per XCD
// fills one CU each, so a fetch running beside the projection takes 8 of the
// 256 CUs, while keeping about half a megabyte of reads in flight over the
// host link.
constexpr int kHostThreads = 1024;
constexpr int kHostBlocks = 8;
constexpr int kHostUnroll = 8;

}  // namespace

hipError_t engram_launch_gather_rows(const uint8_t *table, int64_t table_rows,
                                     const int64_t *row_ids, int64_t n_ids, uint8_t *out,
                                     bool host_table, hipStream_t stream) {
  if (n_ids <= 0) return hipSuccess;
  if (host_table) {
    hipLaunchKernelGGL((gather_rows_kernel<kHostThreads, kHostUnroll>), dim3(kHostBlocks),
                       dim3(kHostThreads), 0, stream, table, table_rows, row_ids, n_ids, out);
    return hipGetLastError();
  }
  const int64_t blocks = (n_ids * kRowWords + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((gather_rows_kernel<kThreads, 1>), dim3((unsigned)blocks), dim3(kThreads),
                     0, stream, table, table_rows, row_ids, n_ids, out);
  return hipGetLastError();
}

hipError_t engram_launch_gather_mx(const uint8_t *table, int64_t table_rows,
                                   const int64_t *row_ids, int64_t n_ids, uint8_t *codes,
                                   uint8_t *scales, bool host_table, hipStream_t stream) {
  if (n_ids <= 0) return hipSuccess;
  if (host_table) {
    hipLaunchKernelGGL((gather_mx_kernel<kHostThreads, kHostUnroll>), dim3(kHostBlocks),
                       dim3(kHostThreads), 0, stream, table, table_rows, row_ids, n_ids, codes,
                       scales);
    return hipGetLastError();
  }
  const int64_t blocks = (n_ids * kRowWords + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((gather_mx_kernel<kThreads, 1>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, table, table_rows, row_ids, n_ids, codes, scales);
  return hipGetLastError();
}

hipError_t engram_launch_gather_e4m3(const uint8_t *table, int64_t table_rows,
                                     const int64_t *row_ids, int64_t n_ids, uint16_t *out,
                                     bool host_table, hipStream_t stream) {
  if (n_ids <= 0) return hipSuccess;
  if (host_table) {
    hipLaunchKernelGGL(gather_e4m3_kernel<kHostThreads>, dim3(kHostBlocks), dim3(kHostThreads),
                       0, stream, table, table_rows, row_ids, n_ids, out);
    return hipGetLastError();
  }
  const int64_t blocks = (n_ids + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(gather_e4m3_kernel<kThreads>, dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, table, table_rows, row_ids, n_ids, out);
  return hipGetLastError();
}

hipError_t engram_launch_gather_f32(const float *table, int64_t table_rows, int32_t row_dim,
                                    const int64_t *row_ids, int64_t n_ids, float *out,
                                    hipStream_t stream) {
  if (n_ids <= 0) return hipSuccess;
  const int64_t work = n_ids * (row_dim / 4);
  const int64_t blocks = (work + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(gather_f32_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     table, table_rows, row_dim, row_ids, n_ids, out);
  return hipGetLastError();
}
