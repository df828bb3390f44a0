// Step 4 of the Engram layer: the fused key/value projection kv = e W.
//
// Pages: "DeepSeek-V4.1 模型结构（5）：记忆，Engram", "每条流一个 key 的设计沿用自原版"
// (hc keys and one value as one 6144 x 25600 matrix, the layer's only dense
// compute per "196B 参数怎么存、怎么取"); "ds4.c 学习笔记 · Engram", "消费" (the
// weight is stored with the 6144 inputs innermost).
//
// bf16 path: C[m, n] = sum_k E[m, k] W[n, k]; both operands are K-contiguous.
// One block of 4 waves computes a 256 (n) x 256 (m) tile; each wave a 128 x 128
// quarter as 4 x 4 v_mfma_f32_32x32x16_bf16 tiles with fp32 accumulators.
// W rows feed the MFMA's first operand and E rows the second, so each lane's
// accumulator holds 4 consecutive output columns of one token and the epilogue
// writes 8-byte bf16 quads.
//
// The K loop stages 256 x 64 tiles of both operands in LDS, double-buffered
// (2 x 64 KiB): global loads of step k+1 are in flight while step k's MFMAs run.
// Each LDS row is 128 bytes (8 chunks of 16 bytes); chunk c of row r is stored
// at slot c ^ (r & 7), so the 16-byte fragment reads of 8 consecutive rows hit
// 8 different bank groups.
//
// Blocks are renumbered so that the blocks the hardware places on one XCD (it
// deals block ids round-robin over 8 XCDs) form one contiguous range, and tiles
// are walked in groups of 8 token-tiles sharing weight tiles, for L2 reuse.
#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256;       // tokens per tile
constexpr int BN = 256;       // output columns per tile
constexpr int BK = 64;        // K per stage
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int kChunks = BK / 8;                       // 16-byte chunks per LDS row
constexpr int kLoads = BM * kChunks / kThreads;       // 16-byte loads per thread per operand

// Buffer resource word 3 for gfx9-family raw buffers (no format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(
    const uint16_t *__restrict__ E, const uint16_t *__restrict__ W, uint16_t *__restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n) {
  __shared__ __align__(16) uint16_t sW[2 * BN * BK];   // [2][BN][BK]
  __shared__ __align__(16) uint16_t sE[2 * BM * BK];   // [2][BM][BK]

  // ---- tile assignment ----
  const int nblocks = tiles_m * tiles_n;
  int bid = blockIdx.x;
  const int full = (nblocks / kXcds) * kXcds;
  if (bid < full) bid = (bid % kXcds) * (full / kXcds) + bid / kXcds;
  const int in_group = kGroupM * tiles_n;
  const int group = bid / in_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int local = bid - group * in_group;
  const int tile_m = first_m + local % gsize;
  const int tile_n = local / gsize;
  const int m0 = tile_m * BM;
  const int n0 = tile_n * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave >> 1;     // which 128 output columns
  const int wm = wave & 1;      // which 128 tokens

  // ---- global -> register staging through buffer loads ----
  // One buffer resource per operand panel (its 256 rows x K); loads past the
  // panel's last valid row return zeros, which covers the M and N edges. Thread
  // tid stages 16-byte chunk c = tid % 8 of rows tid / 8 + 32 i, i < 8; the
  // K step advances the uniform offset only.
  const int rows_w = min(BN, N - n0);
  const int rows_e = min(BM, M - m0);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(W + (int64_t)n0 * K), 0, rows_w * K * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsE = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(E + (int64_t)m0 * K), 0, rows_e * K * 2, kBufferFlags);
  const int lrow = tid / kChunks;
  const int lchunk = tid % kChunks;
  const int voff = (lrow * K + lchunk * 8) * 2;
  const int row_stride = (kThreads / kChunks) * K * 2;     // 32 rows, bytes
  const int lds_off = swz(lrow, lchunk);                   // + i * 32 rows
  uint4 rW[kLoads], rE[kLoads];

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / BK;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    rW[i] = load16(rsW, voff, i * row_stride);
    rE[i] = load16(rsE, voff, i * row_stride);
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    *reinterpret_cast<uint4 *>(sW + lds_off + i * 32 * BK) = rW[i];
    *reinterpret_cast<uint4 *>(sE + lds_off + i * 32 * BK) = rE[i];
  }
  __syncthreads();

  const int frow = lane & 31;       // row within a 32-row MFMA tile
  const int fk = lane >> 5;         // which 8-wide K half of a 16-wide step

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
      const int koff = (kt + 1) * BK * 2;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        rW[i] = load16(rsW, voff, koff + i * row_stride);
        rE[i] = load16(rsE, voff, koff + i * row_stride);
      }
    }
    const uint16_t *cW = sW + cur * BN * BK;
    const uint16_t *cE = sE + cur * BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wn * 128 + i * 32 + frow;
        a[i] = *reinterpret_cast<const bf16x8 *>(cW + swz(row, kk * 2 + fk));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wm * 128 + j * 32 + frow;
        b[j] = *reinterpret_cast<const bf16x8 *>(cE + swz(row, kk * 2 + fk));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      uint16_t *nW = sW + (cur ^ 1) * BN * BK;
      uint16_t *nE = sE + (cur ^ 1) * BM * BK;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        *reinterpret_cast<uint4 *>(nW + lds_off + i * 32 * BK) = rW[i];
        *reinterpret_cast<uint4 *>(nE + lds_off + i * 32 * BK) = rE[i];
      }
    }
    __syncthreads();
  }

  // ---- epilogue: accumulator r of tile (i, j) is output column
  // n0 + wn*128 + i*32 + (r/4)*8 + (lane/32)*4 + r%4 of token m0 + wm*128 + j*32 + lane%32.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 128 + j * 32 + frow;
    if (m >= M) continue;
    uint16_t *crow = C + (int64_t)m * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 128 + i * 32 + g * 8 + fk * 4;
        if (n < N) {
          uint2 v;
          v.x = engram::pack_bf16x2(acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1]);
          v.y = engram::pack_bf16x2(acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]);
          *reinterpret_cast<uint2 *>(crow + n) = v;
        }
      }
    }
  }
}

// fp32 path for small fp32 layers: one thread per output, sequential K.
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *__restrict__ E,
                                                       const float *__restrict__ W,
                                                       float *__restrict__ C, int64_t M,
                                                       int64_t N, int64_t K) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= M * N) return;
  const int64_t m = g / N;
  const int64_t n = g - m * N;
  const float *e = E + m * K;
  const float *w = W + n * K;
  float acc = 0.f;
  for (int64_t k = 0; k < K; ++k) acc = fmaf(e[k], w[k], acc);
  C[g] = acc;
}

}  // namespace

hipError_t engram_launch_gemm_bf16(const uint16_t *e, const uint16_t *w, uint16_t *kv,
                                   int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  if (m <= 0 || n <= 0) return hipSuccess;
  const int tiles_m = (int)((m + BM - 1) / BM);
  const int tiles_n = (int)((n + BN - 1) / BN);
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads),
                     0, stream, e, w, kv, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t engram_launch_gemm_f32(const float *e, const float *w, float *kv, int64_t m,
                                  int64_t n, int64_t k, hipStream_t stream) {
  if (m <= 0 || n <= 0) return hipSuccess;
  const int64_t blocks = (m * n + 255) / 256;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, e, w, kv,
                     m, n, k);
  return hipGetLastError();
}
