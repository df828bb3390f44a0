// Tiling shared by the wide projection kernels (bf16 in gemm.hip, block-scaled
// FP8 in gemm_mx.hip): 256 x 256 output tiles, the XCD-aware tile order, the
// bf16 epilogue of a tile's accumulators and the stream-K schedule with its
// fixup for calls with fewer tiles than CUs.
#pragma once

#include "common.h"

namespace engram_gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define ENGRAM_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int BM = 256;       // tokens per tile
constexpr int kWideThreads = 256;
constexpr int kNarrowThreads = 512;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
// Buffer resource word 3 for gfx9-family raw buffers (no format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

// Tile origin of this block: block ids are renumbered so that each XCD's
// blocks are contiguous, then walked in groups of kGroupM token-tiles.
__device__ __forceinline__ void tile_origin(int tiles_m, int tiles_n, int bn, int &m0, int &n0) {
  const int nblocks = tiles_m * tiles_n;
  int bid = blockIdx.x;
  const int full = (nblocks / kXcds) * kXcds;
  if (bid < full) bid = (bid % kXcds) * (full / kXcds) + bid / kXcds;
  const int in_group = kGroupM * tiles_n;
  const int group = bid / in_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int local = bid - group * in_group;
  m0 = (first_m + local % gsize) * BM;
  n0 = (local / gsize) * bn;
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

constexpr int BN = 256;          // wide tile width
constexpr int kWideOutputs = 256; // accumulators per thread of a wide tile

// bf16 store of a finished wide tile. Accumulator r of tile (i, j) is output
// column n0 + wn*128 + i*32 + (r/4)*8 + (lane/32)*4 + r%4 of token
// m0 + wm*128 + j*32 + lane%32.
__device__ __forceinline__ void wide_store_bf16(const f32x16 (&acc)[4][4],
                                                uint16_t *__restrict__ C, int M, int N, int m0,
                                                int n0) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int frow = lane & 31, fk = lane >> 5;
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

// Epilogue of a finished key tile (all its columns in stream n0 / dim, dim a
// multiple of 256): in place of the bf16 keys, each token's two sums over the
// 128 columns of each wave's half, sum k^2 and sum h q_w k_w k, with k the
// accumulator rounded to bf16 as the stored key would be, h the token's stream
// (bf16 [M, hc * dim], read here) and qk_w the folded weights [hc * dim]. They
// go to kv row m's key columns (engram::gate_sums_pairs), which the gate then
// reads instead of the keys. Lanes l and l + 32 hold the same token and
// alternating quads of 4 columns; their sums meet in one exchange.
__device__ __forceinline__ void wide_store_gate_sums(const f32x16 (&acc)[4][4],
                                                     const uint16_t *__restrict__ h,
                                                     const float *__restrict__ qk_w,
                                                     uint16_t *__restrict__ kv, int M, int m0,
                                                     int n0, int hc, int dim) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int frow = lane & 31, fk = lane >> 5;
  const int key_cols = hc * dim;
  const int stream = n0 / dim;
  const int block = (n0 - stream * dim) / 128 + wn;
  const int nb = n0 + wn * 128 + fk * 4;
  // All 64 pieces of h this lane needs are requested before any arithmetic, so
  // the tile waits for HBM once (the registers that staged the operands are
  // free by now); rows past M read row m0's stream (in bounds) and store nothing.
  uint2 hv[4][4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 128 + j * 32 + frow;
    const uint16_t *hrow = h + (int64_t)(m < M ? m : m0) * key_cols + nb;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        hv[j][i][g] = *reinterpret_cast<const uint2 *>(hrow + i * 32 + g * 8);
  }
  float4 w[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) w[i][g] = *reinterpret_cast<const float4 *>(qk_w + nb + i * 32 + g * 8);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 128 + j * 32 + frow;
    const bool ok = m < M;
    float skk = 0.f, shk = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t k01 = engram::pack_bf16x2(acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1]);
        const uint32_t k23 = engram::pack_bf16x2(acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]);
        const float k[4] = {__uint_as_float(k01 << 16), __uint_as_float(k01 & 0xFFFF0000u),
                            __uint_as_float(k23 << 16), __uint_as_float(k23 & 0xFFFF0000u)};
        const float hh[4] = {__uint_as_float(hv[j][i][g].x << 16),
                             __uint_as_float(hv[j][i][g].x & 0xFFFF0000u),
                             __uint_as_float(hv[j][i][g].y << 16),
                             __uint_as_float(hv[j][i][g].y & 0xFFFF0000u)};
        const float ww[4] = {w[i][g].x, w[i][g].y, w[i][g].z, w[i][g].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          skk = fmaf(k[c], k[c], skk);
          shk = fmaf(hh[c] * ww[c], k[c], shk);
        }
      }
    skk += __shfl_xor(skk, 32, engram::kWave);
    shk += __shfl_xor(shk, 32, engram::kWave);
    if (fk == 0 && ok)
      reinterpret_cast<float2 *>(kv)[engram::gate_sums_pairs(m, hc, dim) + stream * (dim / 128) +
                                     block] = make_float2(skk, shk);
  }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// ---- stream-K schedule for calls with fewer wide tiles than CUs ----------------
// The (tile, K-step) units, tile-major, are dealt to G persistent blocks in
// equal contiguous ranges: block b owns units [floor(b U / G), floor((b+1) U / G)).
// A tile a block covers whole is stored as bf16 at once. A tile split between
// blocks leaves one fp32 piece per block: a block's first piece goes to its
// slot 0 and its last to slot 1 (the pieces between are whole tiles). The
// fixup kernel then sums a tile's pieces in block order, so every result is
// reproducible for a given shape and CU count.
struct StreamK {
  int64_t units;      // tiles * KT
  int blocks;         // G
  int kt;             // K-steps per tile
  int tiles_m;
  __device__ __forceinline__ int64_t start(int b) const { return (int64_t)b * units / blocks; }
  // the block owning unit x: the largest b with start(b) <= x
  __device__ __forceinline__ int owner(int64_t x) const {
    const int64_t b = ((x + 1) * blocks + units - 1) / units - 1;
    return (int)(b < blocks - 1 ? b : blocks - 1);
  }
};

// Partial accumulators, thread-major per register so that one store
// instruction of a wave covers 256 contiguous bytes: value r of thread t of
// slot s of block b sits at ws[((b * 2 + s) * kWideOutputs + r) * kWideThreads + t].
__device__ __forceinline__ float *piece_slot(float *ws, int b, int s) {
  return ws + ((int64_t)(b * 2 + s) * kWideOutputs) * kWideThreads;
}

constexpr int kFixupRegs = 16;
constexpr int kFixupParts = kWideOutputs / kFixupRegs;

inline hipError_t cu_count(int &cus) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return err;
}

// The stream-K schedule of a call, or blocks = 0 when whole wide tiles fill the CUs.
inline hipError_t plan_streamk(int64_t m, int64_t n, int64_t kt, StreamK &sk) {
  int cus = 0;
  const hipError_t err = cu_count(cus);
  if (err != hipSuccess) return err;
  const int64_t tiles_m = (m + BM - 1) / BM;
  const int64_t tiles = tiles_m * ((n + BN - 1) / BN);
  sk.tiles_m = (int)tiles_m;
  sk.kt = (int)kt;
  sk.units = tiles * sk.kt;
  sk.blocks = tiles >= cus ? 0 : (int)(sk.units < cus ? sk.units : cus);
  return hipSuccess;
}

// Sums the split tiles' pieces in block order and stores them as bf16 (defined
// in gemm.hip): one launch of tiles * kFixupParts blocks.
hipError_t launch_streamk_fixup(const float *ws, uint16_t *kv, int64_t m, int64_t n,
                                const StreamK &sk, hipStream_t stream);

}  // namespace engram_gemm
