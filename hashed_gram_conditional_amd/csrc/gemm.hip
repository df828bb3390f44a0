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
// W's rows sit ldw >= K elements apart (E's are dense). With rows a multiple of
// 4 KiB apart (K = 6144: 12 KiB), a K-step's loads from all CUs fall at the
// same offset within a memory page, and a call that streams W from HBM once
// (the decode schedule below) loses ~10 % to it. A row stride of 128 bytes
// more spreads them; the products and their bits do not depend on ldw.
// In LDS, 16-byte chunk c of a 128-byte row r sits in slot
// c ^ (r & 7) ^ ((r >> 3) & 1): the fragment reads of any 16 consecutive rows
// (one b128 read phase) then touch 16 distinct bank groups, and so do the
// stores of two consecutive rows.
//
// Three kernels, all over 256-token tiles:
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
// gemm_bf16_sums_kernel (the same tiles, order and loop) ends a key tile by
// forming the gate's two key-side sums per token in place of storing its keys
// (wide_store_gate_sums in gemm_tiles.h); value tiles are stored as above.
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
#include "gemm_tiles.h"

using namespace engram_gemm;

namespace {

constexpr int BK = 64;        // K per stage

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
                                          int ldw, int m0, int n0, int ks, int ke,
                                          f32x16 (&acc)[4][4],
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
      const_cast<uint16_t *>(W + (int64_t)n0 * ldw), 0, rows_w * ldw * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsE = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(E + (int64_t)m0 * K), 0, rows_e * K * 2, kBufferFlags);
  // A step's operands are 16 chunks of 16 bytes per thread: chunk i < 8 is W
  // row i*32 + t/8, chunk i >= 8 is E row (i-8)*32 + t/8, 16-byte column t%8 of
  // the step's 128-byte K slice. Its LDS slot follows the swizzle; since i*32
  // is a multiple of 16, the slot depends on t only.
  const int g_row = tid >> 3;
  const int g_chunk = tid & 7;
  const int g_voff_w = (g_row * ldw + g_chunk * 8) * 2, g_voff_e = (g_row * K + g_chunk * 8) * 2;
  const int g_rstride_w = 32 * ldw * 2, g_rstride_e = 32 * K * 2;
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
      g[(q) * 4 + i] =                                                                      \
          load16(rsW, g_voff_w, ((q) * 4 + i) * g_rstride_w + (kt_) * BK * 2);              \
    else                                                                                    \
      g[(q) * 4 + i] =                                                                      \
          load16(rsE, g_voff_e, ((q) * 4 + i - 8) * g_rstride_e + (kt_) * BK * 2);          \
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

__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint16_t *__restrict__ E, const uint16_t *__restrict__ W,
                      uint16_t *__restrict__ C, int M, int N, int K, int ldw, int tiles_m,
                      int tiles_n) {
  __shared__ __align__(1024) WideLds lds;
  int m0, n0;
  tile_origin(tiles_m, tiles_n, BN, m0, n0);
  f32x16 acc[4][4];
  zero_acc(acc);
  wide_tile(E, W, M, N, K, ldw, m0, n0, 0, K / BK, acc, lds);
  wide_store_bf16(acc, C, M, N, m0, n0);
}

// The same tiles and order, with key tiles (columns below hc * dim) ending in
// the gate's sums instead of bf16 keys. Their epilogue reads 128 KiB of h and
// writes 2 KiB where the plain kernel writes 128 KiB of keys, and the gate
// then reads 1.3 KB of sums per token instead of hc * dim keys.
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_sums_kernel(const uint16_t *__restrict__ E, const uint16_t *__restrict__ W,
                           uint16_t *__restrict__ C, int M, int N, int K, int ldw, int tiles_m,
                           int tiles_n, const uint16_t *__restrict__ h,
                           const float *__restrict__ qk_w, int hc, int dim) {
  __shared__ __align__(1024) WideLds lds;
  int m0, n0;
  tile_origin(tiles_m, tiles_n, BN, m0, n0);
  f32x16 acc[4][4];
  zero_acc(acc);
  wide_tile(E, W, M, N, K, ldw, m0, n0, 0, K / BK, acc, lds);
  if (n0 < hc * dim)
    wide_store_gate_sums(acc, h, qk_w, C, M, m0, n0, hc, dim);
  else
    wide_store_bf16(acc, C, M, N, m0, n0);
}

// ---- skinny calls: one token tile, columns dealt to every CU ----------------------
// With at most 256 tokens (decode) the 256 x 256 tiles number fewer than the
// CUs. Here block b takes all tokens and its own slice of 32 * NT output columns
// (96 or 128 for 25600 columns over 256 CUs: 224 x 96 + 32 x 128), so the blocks
// cover N once with no K split and no partial sums. The weight streams from
// HBM once, kSkRing - 1 K-steps ahead of use through a register ring; every
// block reads the same E, which the L2 holds, 2 steps ahead. Both pass through
// two LDS stages laid out as in the wide kernel (128-byte rows, the same
// swizzle and fragment reads). Wave w owns tokens [64 w, 64 w + 64) against all
// the block's columns. A step's E loads are issued before its weight loads, so
// waiting for E (one step old) never waits for the weight's HBM latency. Each
// output sums its K16 chunks in increasing order in one MFMA accumulator, as
// the wide kernel does, so both give the same bits.
constexpr int kSkMaxCols = 128;
constexpr int kSkRing = 6;                // weight steps in registers

struct SkinnyLds {
  uint16_t w[2][kSkMaxCols * BK];
  uint16_t e[2][BM * BK];
};

template <int NT>
__device__ __forceinline__ void skinny_block(const uint16_t *__restrict__ E,
                                             const uint16_t *__restrict__ W,
                                             uint16_t *__restrict__ C, int M, int N, int K,
                                             int ldw, int c0, SkinnyLds &lds) {
  const int KT = K / BK;                    // multiple of kSkRing (checked by the launcher)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cols = min(32 * NT, N - c0);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(W + (int64_t)c0 * ldw), 0, cols * ldw * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsE = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(E), 0, min(M, BM) * K * 2, kBufferFlags);
  // chunk q of a step: row q * 32 + t / 8, 16-byte column t % 8 (as in the wide kernel)
  const int g_row = tid >> 3, g_chunk = tid & 7;
  const int g_voff_w = (g_row * ldw + g_chunk * 8) * 2, g_voff_e = (g_row * K + g_chunk * 8) * 2;
  const int g_rstride_w = 32 * ldw * 2, g_rstride_e = 32 * K * 2;
  const int s_off = g_row * BK + ((g_chunk ^ (g_row & 7) ^ ((g_row >> 3) & 1)) << 3);
  const int frow = lane & 31, fk = lane >> 5;
  const int fsw = (frow & 7) ^ ((frow >> 3) & 1);
  const int e_base = (wave * 64 + frow) * BK;

  uint4 wr[kSkRing][4], er[2][8];
  f32x16 acc[NT][2];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8 a0[NT], b0[2], a1[NT], b1[2];

#define SK_KOFF(kt_) (((kt_) < KT ? (kt_) : KT - 1) * BK * 2)
#define SK_LOADE(slot, kt_, q0, q1)                                                           \
  _Pragma("unroll") for (int q = q0; q < q1; ++q)                                           \
    er[slot][q] = load16(rsE, g_voff_e, q * g_rstride_e + SK_KOFF(kt_));
#define SK_LOADW(slot, kt_, q0, q1)                                                           \
  _Pragma("unroll") for (int q = q0; q < q1; ++q)                                           \
    wr[slot][q] = load16(rsW, g_voff_w, q * g_rstride_w + SK_KOFF(kt_));
#define SK_STOREE(st, slot, q0, q1)                                                           \
  _Pragma("unroll") for (int q = q0; q < q1; ++q)                                           \
    *reinterpret_cast<uint4 *>(&lds.e[st][s_off + q * 32 * BK]) = er[slot][q];
#define SK_STOREW(st, slot, q0, q1)                                                           \
  _Pragma("unroll") for (int q = q0; q < q1; ++q)                                           \
    *reinterpret_cast<uint4 *>(&lds.w[st][s_off + q * 32 * BK]) = wr[slot][q];
#define SK_FRAGS(st, kk, dst_a, dst_b)                                                        \
  _Pragma("unroll") for (int i = 0; i < NT; ++i) dst_a[i] = *reinterpret_cast<const bf16x8 *>( \
      &lds.w[st][(i * 32 + frow) * BK + ((((kk) * 2 + fk) ^ fsw) << 3)]);                   \
  _Pragma("unroll") for (int j = 0; j < 2; ++j) dst_b[j] = *reinterpret_cast<const bf16x8 *>( \
      &lds.e[st][e_base + j * 32 * BK + ((((kk) * 2 + fk) ^ fsw) << 3)]);
#define SK_MMA(A, B)                                                                          \
  _Pragma("unroll") for (int i = 0; i < NT; ++i)                                            \
  _Pragma("unroll") for (int j = 0; j < 2; ++j)                                             \
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], B[j], acc[i][j], 0, 0, 0);
#define SK_FENCE() __builtin_amdgcn_sched_barrier(0)
// Step kt (ring slot s = kt % kSkRing) computes from stage s & 1. It loads E of
// step kt + 2 into E slot s & 1 (stored to LDS during step kt - 1) and the
// weight of step kt + kSkRing - 1 into the ring slot of step kt - 1 (stored
// during step kt - 2), and stores step kt + 1 into the other stage, which every
// wave finished reading before the previous barrier.
#define SK_STEP(s)                                                                            \
  {                                                                                         \
    const int P = (s) & 1, Q = P ^ 1;                                                       \
    const int ws_ = ((s) + 1) % kSkRing, wl_ = ((s) + kSkRing - 1) % kSkRing;               \
    SK_FRAGS(P, 1, a1, b1);                                                                 \
    SK_LOADE(P, kt + (s) + 2, 0, 3);                                                        \
    SK_STOREE(Q, Q, 0, 4);                                                                  \
    SK_MMA(a0, b0);                                                                         \
    SK_FENCE();                                                                             \
    SK_FRAGS(P, 2, a0, b0);                                                                 \
    SK_LOADE(P, kt + (s) + 2, 3, 6);                                                        \
    SK_STOREE(Q, Q, 4, 8);                                                                  \
    SK_MMA(a1, b1);                                                                         \
    SK_FENCE();                                                                             \
    SK_FRAGS(P, 3, a1, b1);                                                                 \
    SK_LOADE(P, kt + (s) + 2, 6, 8);                                                        \
    SK_LOADW(wl_, kt + (s) + kSkRing - 1, 0, 2);                                            \
    SK_STOREW(Q, ws_, 0, 2);                                                                \
    SK_MMA(a0, b0);                                                                         \
    SK_FENCE();                                                                             \
    SK_LOADW(wl_, kt + (s) + kSkRing - 1, 2, 4);                                            \
    SK_STOREW(Q, ws_, 2, 4);                                                                \
    SK_MMA(a1, b1);                                                                         \
    SK_FENCE();                                                                             \
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                       \
    SK_FENCE();                                                                             \
    SK_FRAGS(Q, 0, a0, b0);                                                                 \
  }

  // prologue: weight of steps 0 .. kSkRing - 2, E of steps 0 and 1; step 0 into stage 0
#pragma unroll
  for (int s = 0; s < kSkRing - 1; ++s) SK_LOADW(s, s, 0, 4);
  SK_LOADE(0, 0, 0, 8);
  SK_LOADE(1, 1, 0, 8);
  SK_STOREW(0, 0, 0, 4);
  SK_STOREE(0, 0, 0, 8);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  SK_FRAGS(0, 0, a0, b0);
  for (int kt = 0; kt < KT; kt += kSkRing) {
    SK_STEP(0) SK_STEP(1) SK_STEP(2) SK_STEP(3) SK_STEP(4) SK_STEP(5)
  }
#undef SK_STEP
#undef SK_FENCE
#undef SK_MMA
#undef SK_FRAGS
#undef SK_STOREW
#undef SK_STOREE
#undef SK_LOADW
#undef SK_LOADE
#undef SK_KOFF

  // accumulator r of (i, j): column c0 + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4,
  // token 64 wave + 32 j + lane % 32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = wave * 64 + j * 32 + frow;
    if (m >= M) continue;
    uint16_t *crow = C + (int64_t)m * N;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = c0 + i * 32 + g * 8 + fk * 4;
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

// Block b: columns [b w_lo + min(b, wide) 32, ...), 32 more than w_lo for the
// first `wide` blocks.
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_skinny_kernel(const uint16_t *__restrict__ E, const uint16_t *__restrict__ W,
                             uint16_t *__restrict__ C, int M, int N, int K, int ldw, int w_lo,
                             int wide) {
  __shared__ __align__(1024) SkinnyLds lds;
  const int b = blockIdx.x;
  const int c0 = b * w_lo + min(b, wide) * 32;
  if (c0 >= N) return;
  const int nt = (w_lo + (b < wide ? 32 : 0)) / 32;
  if (nt == 4)
    skinny_block<4>(E, W, C, M, N, K, ldw, c0, lds);
  else if (nt == 3)
    skinny_block<3>(E, W, C, M, N, K, ldw, c0, lds);
  else
    skinny_block<2>(E, W, C, M, N, K, ldw, c0, lds);
}

__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_streamk_kernel(const uint16_t *__restrict__ E, const uint16_t *__restrict__ W,
                              uint16_t *__restrict__ C, float *__restrict__ ws, int M, int N,
                              int K, int ldw, StreamK sk) {
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
    wide_tile(E, W, M, N, K, ldw, m0, n0, ks, ke, acc, lds);
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

template <int TN>
__global__ __launch_bounds__(kNarrowThreads) void gemm_bf16_narrow_kernel(
    const uint16_t *__restrict__ E, const uint16_t *__restrict__ W, uint16_t *__restrict__ C,
    int M, int N, int K, int ldw, int tiles_m, int tiles_n) {
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
      const_cast<uint16_t *>(W + (int64_t)n0 * ldw), 0, rows_w * ldw * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsE = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(E + (int64_t)m0 * K), 0, rows_e * K * 2, kBufferFlags);
  // Direct loads: row (R w + i) * 8 + p / 8 has (row & 7) = p / 8 and, R being
  // even, ((row >> 3) & 1) = i & 1, so lane p fetches logical chunk
  // (p % 8) ^ (p / 8) ^ (i & 1) of its row.
  const int dl_c0 = (lane & 7) ^ (lane >> 3);
  const int dl_rw = wave * WR * 8 + (lane >> 3);
  const int dl_re = wave * 32 + (lane >> 3);
  const int dl_w0 = (dl_rw * ldw + dl_c0 * 8) * 2;
  const int dl_w1 = (dl_rw * ldw + (dl_c0 ^ 1) * 8) * 2;
  const int dl_e0 = (dl_re * K + dl_c0 * 8) * 2;
  const int dl_e1 = (dl_re * K + (dl_c0 ^ 1) * 8) * 2;
  const int rstride8_w = 8 * ldw * 2, rstride8_e = 8 * K * 2;
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
                                             i * rstride8_w + (kt_) * BK * 2, 0, 0);        \
  }                                                                                         \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                           \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsE, ENGRAM_LDS((dE) + (wave * 4 + i) * 512),  \
                                             16, (i & 1) ? dl_e1 : dl_e0,                   \
                                             i * rstride8_e + (kt_) * BK * 2, 0, 0);        \
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
                                                       int64_t N, int64_t K, int64_t ldw) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= M * N) return;
  const int64_t m = g / N;
  const int64_t n = g - m * N;
  const float *e = E + m * K;
  const float *w = W + n * ldw;
  float acc = 0.f;
  for (int64_t k = 0; k < K; ++k) acc = fmaf(e[k], w[k], acc);
  C[g] = acc;
}

// The skinny schedule, when it applies: at most one token tile, K a multiple of
// 8 steps, and 64-128 columns per CU. w_lo = 32 floor(n / (32 G)); the first
// `wide` blocks take 32 columns more.
hipError_t plan_skinny(int64_t m, int64_t n, int64_t k, int &w_lo, int &wide, int &blocks) {
  blocks = 0;
  if (m > BM || k % (BK * kSkRing) != 0 || n > INT32_MAX) return hipSuccess;
  int cus = 0;
  const hipError_t err = cu_count(cus);
  if (err != hipSuccess) return err;
  const int64_t lo = (n / cus) / 32 * 32;
  if (lo < 64 || lo + 32 > kSkMaxCols) return hipSuccess;
  w_lo = (int)lo;
  wide = (int)((n - (int64_t)cus * lo + 31) / 32);
  blocks = cus;
  return hipSuccess;
}

}  // namespace

hipError_t engram_gemm_bf16_workspace(int64_t m, int64_t n, int64_t k, size_t *bytes) {
  *bytes = 0;
  if (m <= 0 || n <= 0) return hipSuccess;
  int w_lo = 0, wide = 0, sk_blocks = 0;
  hipError_t e0 = plan_skinny(m, n, k, w_lo, wide, sk_blocks);
  if (e0 != hipSuccess) return e0;
  if (sk_blocks > 0) return hipSuccess;
  StreamK sk;
  const hipError_t err = plan_streamk(m, n, k / BK, sk);
  if (err != hipSuccess) return err;
  *bytes = (size_t)sk.blocks * 2 * kWideOutputs * kWideThreads * sizeof(float);
  return hipSuccess;
}

hipError_t engram_launch_gemm_bf16(const uint16_t *e, const uint16_t *w, int64_t ldw,
                                   uint16_t *kv, int64_t m, int64_t n, int64_t k, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  if (m <= 0 || n <= 0) return hipSuccess;
  int w_lo = 0, wide = 0, sk_blocks = 0;
  hipError_t err = plan_skinny(m, n, k, w_lo, wide, sk_blocks);
  if (err != hipSuccess) return err;
  if (sk_blocks > 0) {
    hipLaunchKernelGGL(gemm_bf16_skinny_kernel, dim3((unsigned)sk_blocks), dim3(kWideThreads), 0,
                       stream, e, w, kv, (int)m, (int)n, (int)k, (int)ldw, w_lo, wide);
    return hipGetLastError();
  }
  StreamK sk;
  err = plan_streamk(m, n, k / BK, sk);
  if (err != hipSuccess) return err;
  const int tiles_m = sk.tiles_m;
  const int tiles_n256 = (int)((n + BN - 1) / BN);
  if (sk.blocks == 0) {
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)(tiles_m * tiles_n256)),
                       dim3(kWideThreads), 0, stream, e, w, kv, (int)m, (int)n, (int)k, (int)ldw,
                       tiles_m, tiles_n256);
    return hipGetLastError();
  }
  const size_t need = (size_t)sk.blocks * 2 * kWideOutputs * kWideThreads * sizeof(float);
  if (workspace != nullptr && workspace_bytes >= need) {
    hipLaunchKernelGGL(gemm_bf16_streamk_kernel, dim3((unsigned)sk.blocks), dim3(kWideThreads), 0,
                       stream, e, w, kv, (float *)workspace, (int)m, (int)n, (int)k, (int)ldw,
                       sk);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    return engram_gemm::launch_streamk_fixup((const float *)workspace, kv, m, n, sk, stream);
  }
  // No workspace: 128-wide tiles over the whole K.
  const int tiles_n128 = (int)((n + 127) / 128);
  hipLaunchKernelGGL(gemm_bf16_narrow_kernel<128>, dim3((unsigned)(tiles_m * tiles_n128)),
                     dim3(kNarrowThreads), 0, stream, e, w, kv, (int)m, (int)n, (int)k, (int)ldw,
                     tiles_m, tiles_n128);
  return hipGetLastError();
}

hipError_t engram_gemm_bf16_whole_tiles(int64_t m, int64_t n, int64_t k, bool *whole) {
  *whole = false;
  if (m <= 0 || n <= 0) return hipSuccess;
  int w_lo = 0, wide = 0, sk_blocks = 0;
  hipError_t err = plan_skinny(m, n, k, w_lo, wide, sk_blocks);
  if (err != hipSuccess || sk_blocks > 0) return err;
  StreamK sk;
  err = plan_streamk(m, n, k / BK, sk);
  if (err != hipSuccess) return err;
  *whole = sk.blocks == 0;
  return hipSuccess;
}

hipError_t engram_launch_gemm_bf16_sums(const uint16_t *e, const uint16_t *w, int64_t ldw,
                                        const uint16_t *h, const float *qk_w, uint16_t *kv,
                                        int64_t m, int32_t hc, int32_t dim, int64_t k,
                                        hipStream_t stream) {
  if (m <= 0) return hipSuccess;
  const int64_t n = (int64_t)(hc + 1) * dim;
  const int tiles_m = (int)((m + BM - 1) / BM);
  const int tiles_n = (int)(n / BN);
  hipLaunchKernelGGL(gemm_bf16_sums_kernel, dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(kWideThreads), 0, stream, e, w, kv, (int)m, (int)n, (int)k, (int)ldw,
                     tiles_m, tiles_n, h, qk_w, (int)hc, (int)dim);
  return hipGetLastError();
}

hipError_t engram_launch_gemm_f32(const float *e, const float *w, int64_t ldw, float *kv,
                                  int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  if (m <= 0 || n <= 0) return hipSuccess;
  const int64_t blocks = (m * n + 255) / 256;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, e, w, kv,
                     m, n, k, ldw);
  return hipGetLastError();
}

hipError_t engram_gemm::launch_streamk_fixup(const float *ws, uint16_t *kv, int64_t m, int64_t n,
                                             const StreamK &sk, hipStream_t stream) {
  const int64_t tiles = (int64_t)sk.tiles_m * ((n + BN - 1) / BN);
  hipLaunchKernelGGL(gemm_streamk_fixup_kernel, dim3((unsigned)(tiles * kFixupParts)),
                     dim3(kWideThreads), 0, stream, ws, kv, (int)m, (int)n, sk);
  return hipGetLastError();
}
