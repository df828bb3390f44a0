// Step 4 of the Engram layer: the fused key/value projection kv = e W.
//
// Pages: "DeepSeek-V4.1 模型结构（5）：记忆，Engram", "每条流一个 key 的设计沿用自原版"
// (hc keys and one value as one 6144 x 25600 matrix, the layer's only dense
// compute per "196B 参数怎么存、怎么取"); "ds4.c 学习笔记 · Engram", "消费" (the
// weight is stored with the 6144 inputs innermost).
//
// bf16 path: C[m, n] = sum_k E[m, k] W[n, k]; both operands are K-contiguous,
// fp32 accumulation in v_mfma_f32_32x32x16_bf16, one bf16 rounding at the end.
// W rows feed the MFMA's first operand and E rows the second, so each lane's
// accumulator holds 4 consecutive output columns of one token and the epilogue
// writes 8-byte bf16 quads. K advances in steps of 64 through two LDS stages.
// In LDS, 16-byte chunk c of a 128-byte row r sits in slot
// c ^ (r & 7) ^ ((r >> 3) & 1): the fragment reads of any 16 consecutive rows
// (one b128 read phase) then touch 16 distinct bank groups, and so do the
// stores of two consecutive rows.
//
// Two kernels, both over 256-token tiles:
//
// gemm_bf16_kernel (256 x 256 tiles, enough tiles to fill the chip). 4 waves,
// one per SIMD, each owning a 128 x 128 block of outputs (16 MFMA tiles, 256
// accumulator registers). Operands move global -> VGPR -> LDS: the loads of
// step k+2 are issued during step k, and the LDS stores of step k+1 happen
// during step k, so every load has one full step to arrive. Both are spread
// evenly over the step's four 16-deep sub-steps (4 loads and 4 stores among
// 16 MFMAs each); issuing a step's 64 KiB of loads in one burst stalls MFMA
// issue while every CU's requests queue in L2 at the same moment. Each
// sub-step first reads the next sub-step's fragments, so their LDS latency is
// hidden behind 16 MFMAs. One barrier per step (LDS counter only; the loads in
// flight stay in flight) sits before the step's last 8 MFMAs.
//
// gemm_bf16_narrow_kernel (128 x 256 tiles, used when 256-wide tiles would
// leave CUs idle: small token counts, decode). 8 waves (2 per SIMD), each a
// 64 x 64 block; operand tiles go global -> LDS by direct buffer loads one
// step ahead, with one barrier per step. Halving the tile width doubles the
// tile count without splitting K, so both kernels give the same bits.
//
// Buffer loads past an operand panel's last valid row return zeros, which
// covers the M and N edges. Blocks are renumbered so that the blocks the
// hardware places on one XCD (it deals block ids round-robin over 8 XCDs) form
// one contiguous range, and tiles are walked in groups of 8 token-tiles
// sharing weight tiles, for L2 reuse.
#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define ENGRAM_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int BM = 256;       // tokens per tile
constexpr int BK = 64;        // K per stage
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

struct WideLds {
  uint16_t w[2][BN * BK];
  uint16_t e[2][BM * BK];
};

// K-steps [ks, ke) of the wide tile at (m0, n0), accumulated into acc (which
// the caller zeroes). Starts with a block barrier, so the LDS stages may be
// reused from a previous tile. Loads of steps at or past ke read other rows of
// the panel or zeros and are never used.
__device__ __forceinline__ void wide_tile(const uint16_t *__restrict__ E,
                                          const uint16_t *__restrict__ W, int M, int N, int K,
                                          int m0, int n0, int ks, int ke, f32x16 (&acc)[4][4],
                                          WideLds &lds) {
  uint16_t (*sW)[BN * BK] = lds.w;
  uint16_t (*sE)[BM * BK] = lds.e;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0..3
  const int wn = wave >> 1;        // which 128 output columns
  const int wm = wave & 1;         // which 128 tokens

  const int rows_w = min(BN, N - n0);
  const int rows_e = min(BM, M - m0);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(W + (int64_t)n0 * K), 0, rows_w * K * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsE = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(E + (int64_t)m0 * K), 0, rows_e * K * 2, kBufferFlags);
  // A step's operands are 16 chunks of 16 bytes per thread: chunk i < 8 is W
  // row i*32 + t/8, chunk i >= 8 is E row (i-8)*32 + t/8, 16-byte column t%8 of
  // the step's 128-byte K slice. Its LDS slot follows the swizzle; since i*32
  // is a multiple of 16, the slot depends on t only.
  const int g_row = tid >> 3;
  const int g_chunk = tid & 7;
  const int g_voff = (g_row * K + g_chunk * 8) * 2;
  const int g_rstride = 32 * K * 2;
  const int s_off = g_row * BK + ((g_chunk ^ (g_row & 7) ^ ((g_row >> 3) & 1)) << 3);
  // Fragment reads: lane l reads row (base + l % 32), K-chunk 2 kk + l / 32.
  const int frow = lane & 31;
  const int fk = lane >> 5;
  const int fsw = (frow & 7) ^ ((frow >> 3) & 1);
  const int a_base = (wn * 128 + frow) * BK;
  const int b_base = (wm * 128 + frow) * BK;

  uint4 g0[16], g1[16];

// Quarter q of a step's chunks: loads, then LDS stores.
#define ENGRAM_LOADQ(g, kt_, q)                                                               \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                           \
    if ((q) < 2)                                                                            \
      g[(q) * 4 + i] = load16(rsW, g_voff, ((q) * 4 + i) * g_rstride + (kt_) * BK * 2);     \
    else                                                                                    \
      g[(q) * 4 + i] = load16(rsE, g_voff, ((q) * 4 + i - 8) * g_rstride + (kt_) * BK * 2); \
  }
#define ENGRAM_STOREQ(g, st, q)                                                               \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                           \
    if ((q) < 2)                                                                            \
      *reinterpret_cast<uint4 *>(&sW[st][s_off + ((q) * 4 + i) * 32 * BK]) = g[(q) * 4 + i]; \
    else                                                                                    \
      *reinterpret_cast<uint4 *>(&sE[st][s_off + ((q) * 4 + i - 8) * 32 * BK]) =           \
          g[(q) * 4 + i];                                                                   \
  }
#define ENGRAM_FRAGS(st, kk, dst_a, dst_b)                                                    \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) dst_a[i] = *reinterpret_cast<const bf16x8 *>( \
      &sW[st][a_base + i * 32 * BK + ((((kk) * 2 + fk) ^ fsw) << 3)]);                      \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) dst_b[j] = *reinterpret_cast<const bf16x8 *>( \
      &sE[st][b_base + j * 32 * BK + ((((kk) * 2 + fk) ^ fsw) << 3)]);
#define ENGRAM_MMA(A, B, I0, I1)                                                              \
  _Pragma("unroll") for (int i = I0; i < I1; ++i)                                           \
  _Pragma("unroll") for (int j = 0; j < 4; ++j)                                             \
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], B[j], acc[i][j], 0, 0, 0);
// The barrier waits for this wave's LDS traffic only; the global loads of the
// next steps stay in flight (their users wait for them individually).
#define ENGRAM_LDS_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
#define ENGRAM_FENCE() __builtin_amdgcn_sched_barrier(0)
#define ENGRAM_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
// Sub-step order: 8 fragment reads each after an MFMA, then loads (0x020) and
// LDS stores (0x200) alternating with the remaining MFMAs.
#define ENGRAM_SUBSTEP_ORDER()                                                                \
  for (int s_ = 0; s_ < 8; ++s_) { ENGRAM_GROUP(0x100, 1); ENGRAM_GROUP(0x008, 1); }         \
  for (int s_ = 0; s_ < 4; ++s_) {                                                          \
    ENGRAM_GROUP(0x020, 1); ENGRAM_GROUP(0x008, 1); ENGRAM_GROUP(0x200, 1); ENGRAM_GROUP(0x008, 1); \
  }

  bf16x8 a0[4], b0[4], a1[4], b1[4];
  // Prologue: step ks into stage 0, step ks+1 in flight; every wave is done
  // with the stages first.
  __syncthreads();
  ENGRAM_LOADQ(g0, ks, 0) ENGRAM_LOADQ(g0, ks, 1) ENGRAM_LOADQ(g0, ks, 2) ENGRAM_LOADQ(g0, ks, 3)
  ENGRAM_LOADQ(g1, ks + 1, 0) ENGRAM_LOADQ(g1, ks + 1, 1) ENGRAM_LOADQ(g1, ks + 1, 2)
  ENGRAM_LOADQ(g1, ks + 1, 3)
  ENGRAM_STOREQ(g0, 0, 0) ENGRAM_STOREQ(g0, 0, 1) ENGRAM_STOREQ(g0, 0, 2) ENGRAM_STOREQ(g0, 0, 3)
  ENGRAM_LDS_BARRIER();
  ENGRAM_FRAGS(0, 0, a0, b0);

// Step kt computes from stage P, loads step kt+2 into gP and stores step kt+1
// (held in gQ) into stage Q. Stage Q was last read in step kt-1, which every
// wave finished before the previous barrier. Stores past the last step land in
// a stage that is never read again.
#define ENGRAM_STEP(P, Q, gP, gQ)                                                             \
  {                                                                                         \
    ENGRAM_FRAGS(P, 1, a1, b1);                                                             \
    ENGRAM_LOADQ(gP, kt + 2, 0);                                                            \
    ENGRAM_STOREQ(gQ, Q, 0);                                                                \
    ENGRAM_MMA(a0, b0, 0, 4);                                                               \
    ENGRAM_SUBSTEP_ORDER();                                                                 \
    ENGRAM_FENCE();                                                                         \
    ENGRAM_FRAGS(P, 2, a0, b0);                                                             \
    ENGRAM_LOADQ(gP, kt + 2, 1);                                                            \
    ENGRAM_STOREQ(gQ, Q, 1);                                                                \
    ENGRAM_MMA(a1, b1, 0, 4);                                                               \
    ENGRAM_SUBSTEP_ORDER();                                                                 \
    ENGRAM_FENCE();                                                                         \
    ENGRAM_FRAGS(P, 3, a1, b1);                                                             \
    ENGRAM_LOADQ(gP, kt + 2, 2);                                                            \
    ENGRAM_STOREQ(gQ, Q, 2);                                                                \
    ENGRAM_MMA(a0, b0, 0, 4);                                                               \
    ENGRAM_SUBSTEP_ORDER();                                                                 \
    ENGRAM_FENCE();                                                                         \
    ENGRAM_LOADQ(gP, kt + 2, 3);                                                            \
    ENGRAM_STOREQ(gQ, Q, 3);                                                                \
    ENGRAM_MMA(a1, b1, 0, 2);                                                               \
    for (int s_ = 0; s_ < 4; ++s_) {                                                        \
      ENGRAM_GROUP(0x020, 1); ENGRAM_GROUP(0x008, 1); ENGRAM_GROUP(0x200, 1); ENGRAM_GROUP(0x008, 1); \
    }                                                                                       \
    ENGRAM_FENCE();                                                                         \
    ENGRAM_LDS_BARRIER();                                                                   \
    ENGRAM_FENCE();                                                                         \
    ENGRAM_FRAGS(Q, 0, a0, b0);                                                             \
    ENGRAM_MMA(a1, b1, 2, 4);                                                               \
    for (int s_ = 0; s_ < 8; ++s_) { ENGRAM_GROUP(0x100, 1); ENGRAM_GROUP(0x008, 1); }       \
    ENGRAM_FENCE();                                                                         \
  }
  // Two steps per iteration keep the register double buffers g0 / g1 static.
  int kt = ks;
  for (; kt + 1 < ke; kt += 2) {
    ENGRAM_STEP(0, 1, g0, g1);
    ++kt;
    ENGRAM_STEP(1, 0, g1, g0);
    --kt;
  }
  if (kt < ke) ENGRAM_STEP(0, 1, g0, g1);
#undef ENGRAM_STEP
#undef ENGRAM_SUBSTEP_ORDER
#undef ENGRAM_GROUP
#undef ENGRAM_FENCE
#undef ENGRAM_LDS_BARRIER
#undef ENGRAM_MMA
#undef ENGRAM_FRAGS
#undef ENGRAM_STOREQ
#undef ENGRAM_LOADQ

}

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

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint16_t *__restrict__ E, const uint16_t *__restrict__ W,
                      uint16_t *__restrict__ C, int M, int N, int K, int tiles_m, int tiles_n) {
  __shared__ __align__(1024) WideLds lds;
  int m0, n0;
  tile_origin(tiles_m, tiles_n, BN, m0, n0);
  f32x16 acc[4][4];
  zero_acc(acc);
  wide_tile(E, W, M, N, K, m0, n0, 0, K / BK, acc, lds);
  wide_store_bf16(acc, C, M, N, m0, n0);
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

__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_streamk_kernel(const uint16_t *__restrict__ E, const uint16_t *__restrict__ W,
                              uint16_t *__restrict__ C, float *__restrict__ ws, int M, int N,
                              int K, StreamK sk) {
  __shared__ __align__(1024) WideLds lds;
  const int b = blockIdx.x;
  const int64_t u0 = sk.start(b), u1 = sk.start(b + 1);
  const int tid = threadIdx.x;
  f32x16 acc[4][4];
  for (int64_t u = u0; u < u1;) {
    const int64_t tile = u / sk.kt;
    const int ks = (int)(u - tile * sk.kt);
    const int ke = (int)min((int64_t)sk.kt, (int64_t)ks + (u1 - u));
    const int m0 = (int)(tile % sk.tiles_m) * BM;
    const int n0 = (int)(tile / sk.tiles_m) * BN;
    zero_acc(acc);
    wide_tile(E, W, M, N, K, m0, n0, ks, ke, acc, lds);
    if (ks == 0 && ke == sk.kt) {
      wide_store_bf16(acc, C, M, N, m0, n0);
    } else {
      float *dst = piece_slot(ws, b, u == u0 ? 0 : 1) + tid;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[((i * 4 + j) * 16 + r) * kWideThreads] = acc[i][j][r];
    }
    u += ke - ks;
  }
}

// Sums the pieces of a split tile in block order and stores bf16. Block
// (tile, part) handles accumulator registers [part * 16, part * 16 + 16) of
// all 256 threads of the tile: four quads of consecutive output columns per
// thread, loads coalesced across threads. Tiles one block finished whole exit
// at once.
constexpr int kFixupRegs = 16;
constexpr int kFixupParts = kWideOutputs / kFixupRegs;

__global__ __launch_bounds__(kWideThreads) void gemm_streamk_fixup_kernel(
    const float *__restrict__ ws, uint16_t *__restrict__ C, int M, int N, StreamK sk) {
  const int64_t tile = blockIdx.x / kFixupParts;
  const int part = blockIdx.x % kFixupParts;
  const int first = sk.owner(tile * sk.kt);
  const int last = sk.owner((tile + 1) * sk.kt - 1);
  if (first == last) return;
  const int t = threadIdx.x;
  float v[kFixupRegs];
#pragma unroll
  for (int q = 0; q < kFixupRegs; ++q) v[q] = 0.f;
  for (int b = first; b <= last; ++b) {
    // block b's piece of this tile is its first one iff its range starts here
    const int slot = (sk.start(b) / sk.kt == tile) ? 0 : 1;
    const float *src = piece_slot(const_cast<float *>(ws), b, slot) +
                       (int64_t)part * kFixupRegs * kWideThreads + t;
#pragma unroll
    for (int q = 0; q < kFixupRegs; ++q) v[q] += src[q * kWideThreads];
  }
  // register index (i*4 + j)*16 + r, r in [0, 16): part = i*4 + j
  const int i = part >> 2, j = part & 3;
  const int lane = t & 63, wave = t >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int m = (int)(tile % sk.tiles_m) * BM + wm * 128 + j * 32 + (lane & 31);
  if (m >= M) return;
  uint16_t *crow = C + (int64_t)m * N;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int n = (int)(tile / sk.tiles_m) * BN + wn * 128 + i * 32 + g * 8 + (lane >> 5) * 4;
    if (n < N) {
      uint2 o;
      o.x = engram::pack_bf16x2(v[g * 4 + 0], v[g * 4 + 1]);
      o.y = engram::pack_bf16x2(v[g * 4 + 2], v[g * 4 + 3]);
      *reinterpret_cast<uint2 *>(crow + n) = o;
    }
  }
}

// ---- block-scaled FP8 (MX) projection --------------------------------------------
// kv = e W with both operands in the table's block encoding: E4M3 values with one
// E8M0 scale per 32 inputs. W is codes [N, K] plus scales [N, K/32]; e is the
// looked-up rows themselves, [tokens, S, 264] (256 codes then 8 scales per
// segment), so no dequantisation happens at all: v_mfma_scale_f32_32x32x64_f8f6f4
// multiplies E4M3 pairs exactly, applies both 2^(scale - 127) factors per 32-input
// block and accumulates in fp32.
//
// Lane layout of that MFMA (measured on gfx950 with single-instruction probes):
// lane l of half h = l / 32 holds row l % 32; its bytes 0-15 are inputs
// [16h, 16h + 16) of the 64 and bytes 16-31 inputs [32 + 16h, 32 + 16h + 16);
// the scale of row r for inputs [0, 32) comes from lane r's scale operand and
// for [32, 64) from lane r + 32's. The output layout is that of the bf16 MFMA,
// so the epilogues are shared.
//
// Tiles and schedule follow gemm_bf16_kernel: 256 x 256 outputs, 4 waves of
// 128 x 128, a K-step of 128 inputs (128 bytes per row, the same LDS rows and
// swizzle as the bf16 kernel), two 64-input MFMA sub-steps per K-step. Each
// thread stages one step of loads in registers: it stores quarter q of step k+1
// to LDS before reloading that quarter with step k+2, so every load has a step to
// arrive. Scales travel as one dword (4 blocks) per row per step.

struct MxOperands {
  const uint8_t *w_codes;    // [N, K]
  const uint8_t *w_scales;   // [N, K / 32]
  const uint8_t *e_rows;     // [M, S, 264]
  int segments;              // S; K = 256 S
};

constexpr int kMxBk = 128;            // inputs per K-step
constexpr int kRowBytes = 264;

struct MxLds {
  uint8_t w[2][BN * kMxBk];
  uint8_t e[2][BM * kMxBk];
  uint32_t ws[2][BN];
  uint32_t es[2][BM];
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 join16(uint4 lo, uint4 hi) {
  i32x8 v;
  v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
  v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
  return v;
}

__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
}

// K-steps [ks, ke) of the MX tile at (m0, n0) into acc (zeroed by the caller).
// Registers: the B fragments of a 64-input chunk are double-buffered, the A
// fragments stream one tile ahead (both A fragments the MFMAs after the barrier
// need are read before it, as other waves then start refilling the stage).
__device__ __forceinline__ void wide_tile_mx(
    const MxOperands &op, int M, int N, int m0, int n0, int ks, int ke, f32x16 (&acc)[4][4],
    uint8_t *__restrict__ w0, uint8_t *__restrict__ w1, uint8_t *__restrict__ e0,
    uint8_t *__restrict__ e1, uint32_t *__restrict__ ws0, uint32_t *__restrict__ ws1,
    uint32_t *__restrict__ es0, uint32_t *__restrict__ es1) {
  const int K = op.segments * 256;
  const int KB = K / 32;                       // scale bytes per W row
  const int RS = op.segments * kRowBytes;      // bytes per e row
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int rows_w = min(BN, N - n0), rows_e = min(BM, M - m0);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(op.w_codes + (int64_t)n0 * K), 0, rows_w * K, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsWs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(op.w_scales + (int64_t)n0 * KB), 0, rows_w * KB, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsE = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(op.e_rows + (int64_t)m0 * RS), 0, rows_e * RS, kBufferFlags);
  // code chunk i of this thread: row (i % 8) * 32 + t / 8, 16-byte column t % 8
  const int g_row = tid >> 3, g_chunk = tid & 7;
  const int ge_voff = g_row * RS + g_chunk * 16;
  const int s_off = g_row * kMxBk + ((g_chunk ^ (g_row & 7) ^ ((g_row >> 3) & 1)) << 4);
  const int frow = lane & 31, h = lane >> 5;
  const int fsw = (frow & 7) ^ ((frow >> 3) & 1);
  const int a_base = (wn * 128 + frow) * kMxBk;
  const int b_base = (wm * 128 + frow) * kMxBk;
  const int a_srow = wn * 128 + frow, b_srow = wm * 128 + frow;
  // fragment chunk offsets within a row for 64-input chunk c: 4c + h and 4c + 2 + h
  const int f0lo = ((0 + h) ^ fsw) << 4, f0hi = ((2 + h) ^ fsw) << 4;
  const int f1lo = ((4 + h) ^ fsw) << 4, f1hi = ((6 + h) ^ fsw) << 4;

  // W codes and scales go global -> LDS by direct loads: instruction i of wave w
  // fills rows (8 w + i) * 8 + p / 8 (lane p), slot p % 8, so lane p fetches
  // logical chunk (p % 8) ^ (row & 7) ^ ((row >> 3) & 1) = (p % 8) ^ (p / 8) ^ (i & 1).
  const int dl_row = (wave * 8) * 8 + (lane >> 3);
  const int dl_c0 = (lane & 7) ^ (lane >> 3);
  const int dl_v0 = dl_row * K + dl_c0 * 16;
  const int dl_v1 = dl_row * K + (dl_c0 ^ 1) * 16;
  uint4 g[8];
  uint32_t ges = 0;
// Stage buffers are distinct restrict pointers, so the compiler can tell the
// direct loads into one stage from reads of the other and waits for nothing.
#define MX_W(st) ((st) ? w1 : w0)
#define MX_E(st) ((st) ? e1 : e0)
#define MX_WS(st) ((st) ? ws1 : ws0)
#define MX_ES(st) ((st) ? es1 : es0)
#define MX_WOFF(kt_) ((kt_) * kMxBk)
#define MX_EOFF(kt_) (((kt_) >> 1) * kRowBytes + ((kt_) & 1) * kMxBk)
#define MX_ESOFF(kt_) (((kt_) >> 1) * kRowBytes + 256 + ((kt_) & 1) * 4)
// Half q of a step: q = 0 the W codes and scales, q = 1 the e codes and scales.
// Direct loads of W: code chunk i (i < 8) or the scales (i = 8) of step kt_ into stage st.
#define MX_DMAW1(kt_, st, i)                                                                  \
  if ((i) < 8)                                                                              \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(                                               \
        rsW, (__attribute__((address_space(3))) void *)&MX_W(st)[(wave * 8 + (i)) * 1024],  \
        16, ((i) & 1) ? dl_v1 : dl_v0, (i) * 8 * K + MX_WOFF(kt_), 0, 0);                   \
  else                                                                                      \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(                                               \
        rsWs, (__attribute__((address_space(3))) void *)&MX_WS(st)[wave * 64], 4, tid * KB, \
        (kt_) * 4, 0, 0);
// e chunk i (i < 8) or the scales (i = 8): store the staged step into stage st,
// then reload the register with step kt_.
#define MX_EPAIR(st, i, kt_)                                                                  \
  if ((i) < 8) {                                                                            \
    *reinterpret_cast<uint4 *>(&MX_E(st)[s_off + (i) * 32 * kMxBk]) = g[i];                 \
    g[i] = load16(rsE, ge_voff, (i) * 32 * RS + MX_EOFF(kt_));                              \
  } else {                                                                                  \
    MX_ES(st)[tid] = ges;                                                                   \
    ges = load4(rsE, tid * RS, MX_ESOFF(kt_));                                              \
  }
// W copies of a step are issued right after the previous barrier; the 9 e
// reloads that follow them may stay in flight across the next barrier.
#define MX_BARRIER() asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory")
#define MX_FRAG(buf, base, c, t)                                                              \
  join16(*reinterpret_cast<const uint4 *>(&(buf)[(base) + (t) * 32 * kMxBk + ((c) ? f1lo : f0lo)]), \
         *reinterpret_cast<const uint4 *>(&(buf)[(base) + (t) * 32 * kMxBk + ((c) ? f1hi : f0hi)]))
#define MX_FRAGA(st, c, t) MX_FRAG(MX_W(st), a_base, c, t)
#define MX_FRAGSB(st, c, dst)                                                                 \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) dst[j] = MX_FRAG(MX_E(st), b_base, c, j);
#define MX_SCALES(st, sA, sB)                                                                 \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) sA[i] = MX_WS(st)[a_srow + i * 32];         \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) sB[j] = MX_ES(st)[b_srow + j * 32];
// scale byte of 32-input block 2c + h of the step
#define MX_SB(word, c) ((int)(((word) >> (8 * (2 * (c) + h))) & 0xFFu))
#define MX_TILE(i, afrag, bfr, sbv, sa_in)                                                    \
  {                                                                                         \
    const int sa_ = (sa_in);                                                                \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                           \
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afrag, bfr[j], acc[i][j], 0, \
                                                                  0, 0, sa_, 0, sbv[j]);    \
  }
#define MX_FENCE() __builtin_amdgcn_sched_barrier(0)
#define MX_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

  i32x8 bC[4], bN[4], aC, aN;
  uint32_t aS[4], bS[4];
  int sbv[4], sa2, sa3;
  // Prologue: W of steps ks and ks+1 by direct loads, e of step ks into stage 0,
  // e of step ks+1 staged in registers.
  __syncthreads();
  _Pragma("unroll") for (int i = 0; i < 9; ++i) { MX_DMAW1(ks, 0, i) }
  _Pragma("unroll") for (int i = 0; i < 8; ++i)
    g[i] = load16(rsE, ge_voff, i * 32 * RS + MX_EOFF(ks));
  ges = load4(rsE, tid * RS, MX_ESOFF(ks));
  _Pragma("unroll") for (int i = 0; i < 9; ++i) { MX_EPAIR(0, i, ks + 1) }
  _Pragma("unroll") for (int i = 0; i < 9; ++i) { MX_DMAW1(ks + 1, 1, i) }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  MX_FRAGSB(0, 0, bC)
  aC = MX_FRAGA(0, 0, 0);
  MX_SCALES(0, aS, bS)

// Step kt reads stage P. Before its barrier it stores the staged e of step
// kt+1 into stage Q and restages e of step kt+2 (9 pairs over the first five
// tiles); after the barrier stage P is free and takes W of step kt+2.
#define MX_STEP(P, Q)                                                                         \
  {                                                                                         \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) sbv[j] = MX_SB(bS[j], 0);                 \
    MX_FRAGSB(P, 1, bN)                                                                     \
    MX_EPAIR(Q, 0, kt + 2) MX_EPAIR(Q, 1, kt + 2)                                           \
    aN = MX_FRAGA(P, 0, 1);                                                                 \
    MX_TILE(0, aC, bC, sbv, MX_SB(aS[0], 0))                                                \
    for (int s_ = 0; s_ < 2; ++s_) {                                                        \
      MX_GROUP(0x100, 4); MX_GROUP(0x008, 1); MX_GROUP(0x200, 1); MX_GROUP(0x020, 1);       \
      MX_GROUP(0x008, 1);                                                                   \
    }                                                                                       \
    MX_FENCE();                                                                             \
    MX_EPAIR(Q, 2, kt + 2) MX_EPAIR(Q, 3, kt + 2)                                           \
    aC = MX_FRAGA(P, 0, 2);                                                                 \
    MX_TILE(1, aN, bC, sbv, MX_SB(aS[1], 0))                                                \
    for (int s_ = 0; s_ < 2; ++s_) {                                                        \
      MX_GROUP(0x100, 1); MX_GROUP(0x008, 1); MX_GROUP(0x200, 1); MX_GROUP(0x020, 1);       \
      MX_GROUP(0x008, 1);                                                                   \
    }                                                                                       \
    MX_FENCE();                                                                             \
    MX_EPAIR(Q, 4, kt + 2) MX_EPAIR(Q, 5, kt + 2)                                           \
    aN = MX_FRAGA(P, 0, 3);                                                                 \
    MX_TILE(2, aC, bC, sbv, MX_SB(aS[2], 0))                                                \
    for (int s_ = 0; s_ < 2; ++s_) {                                                        \
      MX_GROUP(0x100, 1); MX_GROUP(0x008, 1); MX_GROUP(0x200, 1); MX_GROUP(0x020, 1);       \
      MX_GROUP(0x008, 1);                                                                   \
    }                                                                                       \
    MX_FENCE();                                                                             \
    MX_EPAIR(Q, 6, kt + 2) MX_EPAIR(Q, 7, kt + 2)                                           \
    aC = MX_FRAGA(P, 1, 0);                                                                 \
    MX_TILE(3, aN, bC, sbv, MX_SB(aS[3], 0))                                                \
    for (int s_ = 0; s_ < 2; ++s_) {                                                        \
      MX_GROUP(0x100, 1); MX_GROUP(0x008, 1); MX_GROUP(0x200, 1); MX_GROUP(0x020, 1);       \
      MX_GROUP(0x008, 1);                                                                   \
    }                                                                                       \
    MX_FENCE();                                                                             \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) sbv[j] = MX_SB(bS[j], 1);                 \
    MX_EPAIR(Q, 8, kt + 2)                                                                  \
    aN = MX_FRAGA(P, 1, 1);                                                                 \
    MX_TILE(0, aC, bN, sbv, MX_SB(aS[0], 1))                                                \
    MX_FENCE();                                                                             \
    MX_TILE(1, aN, bN, sbv, MX_SB(aS[1], 1))                                                \
    aC = MX_FRAGA(P, 1, 2);                                                                 \
    aN = MX_FRAGA(P, 1, 3);                                                                 \
    sa2 = MX_SB(aS[2], 1);                                                                  \
    sa3 = MX_SB(aS[3], 1);                                                                  \
    for (int s_ = 0; s_ < 2; ++s_) { MX_GROUP(0x008, 1); MX_GROUP(0x100, 1); MX_GROUP(0x008, 1); } \
    MX_FENCE();                                                                             \
    MX_BARRIER();                                                                           \
    MX_FENCE();                                                                             \
    /* stage Q (step kt+1): its fragments and scales; stage P takes W of step kt+2 */       \
    MX_FRAGSB(Q, 0, bC)                                                                     \
    MX_SCALES(Q, aS, bS)                                                                    \
    MX_DMAW1(kt + 2, P, 0) MX_DMAW1(kt + 2, P, 1) MX_DMAW1(kt + 2, P, 2)                    \
    MX_DMAW1(kt + 2, P, 3) MX_DMAW1(kt + 2, P, 4)                                           \
    MX_TILE(2, aC, bN, sbv, sa2)                                                            \
    for (int s_ = 0; s_ < 4; ++s_) { MX_GROUP(0x100, 3); MX_GROUP(0x008, 1); MX_GROUP(0x020, 1); } \
    MX_FENCE();                                                                             \
    MX_DMAW1(kt + 2, P, 5) MX_DMAW1(kt + 2, P, 6) MX_DMAW1(kt + 2, P, 7)                    \
    MX_DMAW1(kt + 2, P, 8)                                                                  \
    MX_TILE(3, aN, bN, sbv, sa3)                                                            \
    aC = MX_FRAGA(Q, 0, 0);                                                                 \
    for (int s_ = 0; s_ < 4; ++s_) { MX_GROUP(0x100, 1); MX_GROUP(0x008, 1); MX_GROUP(0x020, 1); } \
    MX_FENCE();                                                                             \
  }
  int kt = ks;
  for (; kt + 1 < ke; kt += 2) {
    MX_STEP(0, 1)
    ++kt;
    MX_STEP(1, 0)
    --kt;
  }
  if (kt < ke) MX_STEP(0, 1)
  // Direct loads issued for steps past ke must land before the stages are reused.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef MX_STEP
#undef MX_GROUP
#undef MX_FENCE
#undef MX_TILE
#undef MX_SB
#undef MX_SCALES
#undef MX_FRAGSB
#undef MX_FRAGA
#undef MX_FRAG
#undef MX_BARRIER
#undef MX_EPAIR
#undef MX_DMAW1
#undef MX_ESOFF
#undef MX_EOFF
#undef MX_WOFF
#undef MX_W
#undef MX_E
#undef MX_WS
#undef MX_ES
}

__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mx_kernel(MxOperands op, uint16_t *__restrict__ C, int M, int N, int tiles_m,
                    int tiles_n) {
  __shared__ __align__(1024) MxLds lds;
  int m0, n0;
  tile_origin(tiles_m, tiles_n, BN, m0, n0);
  f32x16 acc[4][4];
  zero_acc(acc);
  wide_tile_mx(op, M, N, m0, n0, 0, op.segments * 256 / kMxBk, acc, lds.w[0], lds.w[1],
               lds.e[0], lds.e[1], lds.ws[0], lds.ws[1], lds.es[0], lds.es[1]);
  wide_store_bf16(acc, C, M, N, m0, n0);
}

__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mx_streamk_kernel(MxOperands op, uint16_t *__restrict__ C, float *__restrict__ ws,
                            int M, int N, StreamK sk) {
  __shared__ __align__(1024) MxLds lds;
  const int b = blockIdx.x;
  const int64_t u0 = sk.start(b), u1 = sk.start(b + 1);
  const int tid = threadIdx.x;
  f32x16 acc[4][4];
  for (int64_t u = u0; u < u1;) {
    const int64_t tile = u / sk.kt;
    const int ks = (int)(u - tile * sk.kt);
    const int ke = (int)min((int64_t)sk.kt, (int64_t)ks + (u1 - u));
    const int m0 = (int)(tile % sk.tiles_m) * BM;
    const int n0 = (int)(tile / sk.tiles_m) * BN;
    zero_acc(acc);
    wide_tile_mx(op, M, N, m0, n0, ks, ke, acc, lds.w[0], lds.w[1], lds.e[0], lds.e[1],
                 lds.ws[0], lds.ws[1], lds.es[0], lds.es[1]);
    if (ks == 0 && ke == sk.kt) {
      wide_store_bf16(acc, C, M, N, m0, n0);
    } else {
      float *dst = piece_slot(ws, b, u == u0 ? 0 : 1) + tid;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[((i * 4 + j) * 16 + r) * kWideThreads] = acc[i][j][r];
    }
    u += ke - ks;
  }
}

template <int TN>
__global__ __launch_bounds__(kNarrowThreads) void gemm_bf16_narrow_kernel(
    const uint16_t *__restrict__ E, const uint16_t *__restrict__ W, uint16_t *__restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr int TI = TN / 64;          // 32-row MFMA tiles per wave along n
  constexpr int WR = TN / 64;          // W-panel direct loads per wave per stage
  __shared__ __align__(1024) uint16_t sW0[TN * BK];
  __shared__ __align__(1024) uint16_t sW1[TN * BK];
  __shared__ __align__(1024) uint16_t sE0[BM * BK];
  __shared__ __align__(1024) uint16_t sE1[BM * BK];

  int m0, n0;
  tile_origin(tiles_m, tiles_n, TN, m0, n0);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 0..7
  const int wn = wave >> 2;        // which TN/2 output columns
  const int wm = wave & 3;         // which 64 tokens

  const int rows_w = min(TN, N - n0);
  const int rows_e = min(BM, M - m0);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(W + (int64_t)n0 * K), 0, rows_w * K * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsE = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(E + (int64_t)m0 * K), 0, rows_e * K * 2, kBufferFlags);
  // Direct loads: row (R w + i) * 8 + p / 8 has (row & 7) = p / 8 and, R being
  // even, ((row >> 3) & 1) = i & 1, so lane p fetches logical chunk
  // (p % 8) ^ (p / 8) ^ (i & 1) of its row.
  const int dl_c0 = (lane & 7) ^ (lane >> 3);
  const int dl_rw = wave * WR * 8 + (lane >> 3);
  const int dl_re = wave * 32 + (lane >> 3);
  const int dl_w0 = (dl_rw * K + dl_c0 * 8) * 2;
  const int dl_w1 = (dl_rw * K + (dl_c0 ^ 1) * 8) * 2;
  const int dl_e0 = (dl_re * K + dl_c0 * 8) * 2;
  const int dl_e1 = (dl_re * K + (dl_c0 ^ 1) * 8) * 2;
  const int rstride8 = 8 * K * 2;
  // Fragment reads: lane l reads row (base + l % 32), K-chunk 2 kk + l / 32.
  const int frow = lane & 31;
  const int fk = lane >> 5;
  const int fsw = (frow & 7) ^ ((frow >> 3) & 1);
  const int a_base = (wn * (TN / 2) + frow) * BK;
  const int b_base = (wm * 64 + frow) * BK;

  f32x16 acc[TI][2];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int KT = K / BK;

#define ENGRAM_ISSUE(kt_, dW, dE)                                                             \
  _Pragma("unroll") for (int i = 0; i < WR; ++i) {                                          \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, ENGRAM_LDS((dW) + (wave * WR + i) * 512), \
                                             16, (i & 1) ? dl_w1 : dl_w0,                   \
                                             i * rstride8 + (kt_) * BK * 2, 0, 0);          \
  }                                                                                         \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                           \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsE, ENGRAM_LDS((dE) + (wave * 4 + i) * 512),  \
                                             16, (i & 1) ? dl_e1 : dl_e0,                   \
                                             i * rstride8 + (kt_) * BK * 2, 0, 0);          \
  }
#define ENGRAM_FRAGS(buf_w, buf_e, kk, dst_a, dst_b)                                          \
  _Pragma("unroll") for (int i = 0; i < TI; ++i) dst_a[i] =                                 \
      *reinterpret_cast<const bf16x8 *>((buf_w) + a_base + i * 32 * BK +                    \
                                        ((((kk) * 2 + fk) ^ fsw) << 3));                     \
  _Pragma("unroll") for (int j = 0; j < 2; ++j) dst_b[j] =                                  \
      *reinterpret_cast<const bf16x8 *>((buf_e) + b_base + j * 32 * BK +                    \
                                        ((((kk) * 2 + fk) ^ fsw) << 3));
#define ENGRAM_MMA(A, B, I0, I1)                                                              \
  _Pragma("unroll") for (int i = I0; i < I1; ++i)                                           \
  _Pragma("unroll") for (int j = 0; j < 2; ++j)                                             \
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], B[j], acc[i][j], 0, 0, 0);
// Per 16-byte fragment step: issue the TI + 2 reads of the next step, then the
// 2 TI MFMAs.
#define ENGRAM_SCHED(id)                                                                      \
  __builtin_amdgcn_sched_group_barrier(0x100, TI + 2, id);                                  \
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * TI, id);

  ENGRAM_ISSUE(0, sW0, sE0);
  __syncthreads();
  bf16x8 a0[TI], b0[2], a1[TI], b1[2];
  ENGRAM_FRAGS(sW0, sE0, 0, a0, b0);
  for (int kt = 0; kt < KT; ++kt) {
    const bool odd = kt & 1;
    const uint16_t *cW = odd ? sW1 : sW0;
    const uint16_t *cE = odd ? sE1 : sE0;
    uint16_t *nW = odd ? sW0 : sW1;
    uint16_t *nE = odd ? sE0 : sE1;
    // Stage kt+1 refills the buffer last read in step kt-1; every wave finished
    // those reads before the previous barrier.
    if (kt + 1 < KT) {
      ENGRAM_ISSUE(kt + 1, nW, nE);
    }
    ENGRAM_FRAGS(cW, cE, 1, a1, b1);
    ENGRAM_MMA(a0, b0, 0, TI);
    ENGRAM_SCHED(0);
    ENGRAM_FRAGS(cW, cE, 2, a0, b0);
    ENGRAM_MMA(a1, b1, 0, TI);
    ENGRAM_SCHED(1);
    ENGRAM_FRAGS(cW, cE, 3, a1, b1);
    ENGRAM_MMA(a0, b0, 0, TI);
    ENGRAM_SCHED(2);
    ENGRAM_MMA(a1, b1, 0, TI / 2);
    // Stage kt+1 has landed in every wave's view, and every read of stage kt
    // has completed, once all waves pass here.
    __syncthreads();
    if (kt + 1 < KT) {
      ENGRAM_FRAGS(nW, nE, 0, a0, b0);
    }
    ENGRAM_MMA(a1, b1, TI / 2, TI);
  }
#undef ENGRAM_ISSUE
#undef ENGRAM_FRAGS
#undef ENGRAM_MMA
#undef ENGRAM_SCHED

  // ---- epilogue: accumulator r of tile (i, j) is output column
  // n0 + wn*TN/2 + i*32 + (r/4)*8 + (lane/32)*4 + r%4 of token m0 + wm*64 + j*32 + lane%32.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wm * 64 + j * 32 + frow;
    if (m >= M) continue;
    uint16_t *crow = C + (int64_t)m * N;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * (TN / 2) + i * 32 + g * 8 + fk * 4;
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

namespace {

hipError_t cu_count(int &cus) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return err;
}

// The stream-K schedule of a call, or blocks = 0 when whole wide tiles fill the CUs.
hipError_t plan_streamk(int64_t m, int64_t n, int64_t kt, StreamK &sk) {
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

}  // namespace

hipError_t engram_gemm_bf16_workspace(int64_t m, int64_t n, int64_t k, size_t *bytes) {
  *bytes = 0;
  if (m <= 0 || n <= 0) return hipSuccess;
  StreamK sk;
  const hipError_t err = plan_streamk(m, n, k / BK, sk);
  if (err != hipSuccess) return err;
  *bytes = (size_t)sk.blocks * 2 * kWideOutputs * kWideThreads * sizeof(float);
  return hipSuccess;
}

hipError_t engram_launch_gemm_bf16(const uint16_t *e, const uint16_t *w, uint16_t *kv,
                                   int64_t m, int64_t n, int64_t k, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  if (m <= 0 || n <= 0) return hipSuccess;
  StreamK sk;
  hipError_t err = plan_streamk(m, n, k / BK, sk);
  if (err != hipSuccess) return err;
  const int tiles_m = sk.tiles_m;
  const int tiles_n256 = (int)((n + BN - 1) / BN);
  if (sk.blocks == 0) {
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)(tiles_m * tiles_n256)),
                       dim3(kWideThreads), 0, stream, e, w, kv, (int)m, (int)n, (int)k, tiles_m,
                       tiles_n256);
    return hipGetLastError();
  }
  const size_t need = (size_t)sk.blocks * 2 * kWideOutputs * kWideThreads * sizeof(float);
  if (workspace != nullptr && workspace_bytes >= need) {
    hipLaunchKernelGGL(gemm_bf16_streamk_kernel, dim3((unsigned)sk.blocks), dim3(kWideThreads), 0,
                       stream, e, w, kv, (float *)workspace, (int)m, (int)n, (int)k, sk);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(gemm_streamk_fixup_kernel,
                       dim3((unsigned)(tiles_m * tiles_n256 * kFixupParts)), dim3(kWideThreads),
                       0, stream, (const float *)workspace, kv, (int)m, (int)n, sk);
    return hipGetLastError();
  }
  // No workspace: 128-wide tiles over the whole K.
  const int tiles_n128 = (int)((n + 127) / 128);
  hipLaunchKernelGGL(gemm_bf16_narrow_kernel<128>, dim3((unsigned)(tiles_m * tiles_n128)),
                     dim3(kNarrowThreads), 0, stream, e, w, kv, (int)m, (int)n, (int)k, tiles_m,
                     tiles_n128);
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

hipError_t engram_launch_gemm_mx(const uint8_t *w_codes, const uint8_t *w_scales,
                                 const uint8_t *e_rows, int32_t segments, uint16_t *kv,
                                 int64_t m, int64_t n, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (m <= 0 || n <= 0) return hipSuccess;
  const MxOperands op{w_codes, w_scales, e_rows, segments};
  StreamK sk;
  hipError_t err = plan_streamk(m, n, (int64_t)segments * 256 / kMxBk, sk);
  if (err != hipSuccess) return err;
  const int tiles_m = sk.tiles_m;
  const int tiles_n = (int)((n + BN - 1) / BN);
  const size_t need = (size_t)sk.blocks * 2 * kWideOutputs * kWideThreads * sizeof(float);
  if (sk.blocks == 0 || workspace == nullptr || workspace_bytes < need) {
    hipLaunchKernelGGL(gemm_mx_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kWideThreads),
                       0, stream, op, kv, (int)m, (int)n, tiles_m, tiles_n);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(gemm_mx_streamk_kernel, dim3((unsigned)sk.blocks), dim3(kWideThreads), 0,
                     stream, op, kv, (float *)workspace, (int)m, (int)n, sk);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gemm_streamk_fixup_kernel, dim3((unsigned)(tiles_m * tiles_n * kFixupParts)),
                     dim3(kWideThreads), 0, stream, (const float *)workspace, kv, (int)m, (int)n,
                     sk);
  return hipGetLastError();
}

hipError_t engram_gemm_mx_workspace(int64_t m, int64_t n, int32_t segments, size_t *bytes) {
  *bytes = 0;
  if (m <= 0 || n <= 0) return hipSuccess;
  StreamK sk;
  const hipError_t err = plan_streamk(m, n, (int64_t)segments * 256 / kMxBk, sk);
  if (err != hipSuccess) return err;
  *bytes = (size_t)sk.blocks * 2 * kWideOutputs * kWideThreads * sizeof(float);
  return hipSuccess;
}
