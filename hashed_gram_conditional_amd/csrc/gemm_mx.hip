// Step 4 with the projection weight in block-scaled FP8: kv = e W on the
// looked-up rows' own codes and scales.
//
// Pages: "条件记忆：DeepSeek V4.1 Engram 如何用 O(1) 查表换掉一层计算" §2.3 (the
// weight is block-FP8; the table holds fp8 e4m3 payloads with e8m0 block
// scales); "DeepSeek Engram 详解：把静态知识从计算里拆出来" §4.3 (the key and
// value projections fused into one product).
//
// kv = e W with both operands in the table's block encoding: E4M3 values with one
// E8M0 scale per 32 inputs. W is codes [N, K] plus scales [N, K/32], and so is e:
// the looked-up rows' codes [tokens, K] (the S rows of a token side by side) and
// scales [tokens, K/32], split apart by the gather so that every 128-byte K
// slice of an e row is line-aligned (a 264-byte row stride put each slice across
// two cache lines and cost 7 % of the kernel). No dequantisation happens at
// all: v_mfma_scale_f32_32x32x64_f8f6f4
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
// swizzle as the bf16 kernel), two 64-input MFMA sub-steps per K-step. W goes
// global -> LDS by direct buffer loads, issued right after a step's barrier for
// the step after next, into the stage that barrier has just freed. e rows are
// staged in registers: during step k each thread stores its 9 pieces of step
// k+1 to LDS and at once reloads each with step k+2, spread over the step's
// first tiles, so every load has a full step to arrive. Scales travel as one
// dword (4 blocks) per row per step.
//
// Calls of at most 256 tokens (decode) run gemm_mx_skinny_kernel: every CU takes
// all tokens against its own weight rows, with no split of K (below).

#include "gemm_tiles.h"

using namespace engram_gemm;

namespace {

struct MxOperands {
  const uint8_t *w_codes;    // [N, K]
  const uint8_t *w_scales;   // [N, K / 32]
  const uint8_t *e_codes;    // [M, K]
  const uint8_t *e_scales;   // [M, K / 32]
  int segments;              // S; K = 256 S
};

constexpr int kMxBk = 128;            // inputs per K-step

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
      const_cast<uint8_t *>(op.e_codes + (int64_t)m0 * K), 0, rows_e * K, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsEs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(op.e_scales + (int64_t)m0 * KB), 0, rows_e * KB, kBufferFlags);
  // code chunk i of this thread: row (i % 8) * 32 + t / 8, 16-byte column t % 8
  const int g_row = tid >> 3, g_chunk = tid & 7;
  const int ge_voff = g_row * K + g_chunk * 16;
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
#define MX_EOFF(kt_) ((kt_) * kMxBk)
#define MX_ESOFF(kt_) ((kt_) * 4)
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
    g[i] = load16(rsE, ge_voff, (i) * 32 * K + MX_EOFF(kt_));                               \
  } else {                                                                                  \
    MX_ES(st)[tid] = ges;                                                                   \
    ges = load4(rsEs, tid * KB, MX_ESOFF(kt_));                                             \
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
    g[i] = load16(rsE, ge_voff, i * 32 * K + MX_EOFF(ks));
  ges = load4(rsEs, tid * KB, MX_ESOFF(ks));
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

// The same tiles with the key tiles' epilogue forming the gate's sums in place
// of the keys (wide_store_gate_sums), as gemm_bf16_sums_kernel does.
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mx_sums_kernel(MxOperands op, uint16_t *__restrict__ C, int M, int N, int tiles_m,
                         int tiles_n, const uint16_t *__restrict__ h,
                         const float *__restrict__ qk_w, int hc, int dim) {
  __shared__ __align__(1024) MxLds lds;
  int m0, n0;
  tile_origin(tiles_m, tiles_n, BN, m0, n0);
  f32x16 acc[4][4];
  zero_acc(acc);
  wide_tile_mx(op, M, N, m0, n0, 0, op.segments * 256 / kMxBk, acc, lds.w[0], lds.w[1],
               lds.e[0], lds.e[1], lds.ws[0], lds.ws[1], lds.es[0], lds.es[1]);
  if (n0 < hc * dim)
    wide_store_gate_sums(acc, h, qk_w, C, M, m0, n0, hc, dim);
  else
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

// ---- skinny calls: one token tile, columns dealt to every CU ----------------------
// gemm_bf16_skinny_kernel's schedule on the block-scaled operands. With at most
// 256 tokens (decode) block b takes every token against its own 32 * NT weight
// rows (96 or 128 for 25600 rows over 256 CUs), so the weight crosses HBM once
// and nothing is split over K. The weight streams kMsRing - 1 K-steps ahead
// through a register ring, e (the same for every block, from L2) 2 steps ahead;
// both pass through two LDS stages in gemm_mx_kernel's layout and fragment order.
// Wave w owns tokens [64 w, 64 w + 64). Each output sums its 64-input chunks in
// increasing order in one accumulator with the same MFMA and scale bytes as
// gemm_mx_kernel, so the two give the same bits. Every thread loads a weight
// row's scale dword (threads 128-255 repeat rows 0-127 into spare LDS words), so
// no thread-dependent branch splits the loop.
constexpr int kMsMaxCols = 128;
constexpr int kMsRing = 6;
struct MxSkLds {
  uint8_t w[2][kMsMaxCols * kMxBk];
  uint8_t e[2][BM * kMxBk];
  uint32_t ws[2][2 * kMsMaxCols];   // entries 128-255 repeat 0-127
  uint32_t es[2][BM];
};

template <int NT>
__device__ __forceinline__ void mx_skinny_block(const MxOperands &op, uint16_t *__restrict__ C, int M,
                                                int N, int c0, MxSkLds &lds) {
  const int K = op.segments * 256;
  const int KB = K / 32;
  const int KT = K / kMxBk;                 // a multiple of kMsRing (checked by the launcher)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cols = min(32 * NT, N - c0);
  const int toks = min(M, BM);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(op.w_codes + (int64_t)c0 * K), 0, cols * K, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsWs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(op.w_scales + (int64_t)c0 * KB), 0, cols * KB, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsE = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(op.e_codes), 0, toks * K, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsEs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(op.e_scales), 0, toks * KB, kBufferFlags);
  // code chunk q of a step: row q * 32 + t / 8, 16-byte column t % 8
  const int g_row = tid >> 3, g_chunk = tid & 7;
  const int g_voff = g_row * K + g_chunk * 16;
  const int s_off = g_row * kMxBk + ((g_chunk ^ (g_row & 7) ^ ((g_row >> 3) & 1)) << 4);
  const int frow = lane & 31, h = lane >> 5;
  const int fsw = (frow & 7) ^ ((frow >> 3) & 1);
  const int b_base = (wave * 64 + frow) * kMxBk;
  const int f0lo = ((0 + h) ^ fsw) << 4, f0hi = ((2 + h) ^ fsw) << 4;
  const int f1lo = ((4 + h) ^ fsw) << 4, f1hi = ((6 + h) ^ fsw) << 4;

  uint4 wr[kMsRing][4], er[2][8];
  uint32_t wsr[kMsRing], esr[2];
  f32x16 acc[NT][2];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  i32x8 b0[2], b1[2], aC, aN;
  uint32_t aS[NT], bS[2];

#define MS_KT(kt_) ((kt_) < KT ? (kt_) : KT - 1)
#define MS_LOADE(slot, kt_, q0, q1)                                                           \
  _Pragma("unroll") for (int q = q0; q < q1; ++q)                                           \
    er[slot][q] = load16(rsE, g_voff, q * 32 * K + MS_KT(kt_) * kMxBk);
#define MS_LOADES(slot, kt_) esr[slot] = load4(rsEs, tid * KB, MS_KT(kt_) * 4);
#define MS_LOADW(slot, kt_)                                                                   \
  _Pragma("unroll") for (int q = 0; q < 4; ++q)                                             \
    wr[slot][q] = load16(rsW, g_voff, q * 32 * K + MS_KT(kt_) * kMxBk);                     \
  wsr[slot] = load4(rsWs, (tid & 127) * KB, MS_KT(kt_) * 4);
#define MS_STOREE(st, slot, q0, q1)                                                           \
  _Pragma("unroll") for (int q = q0; q < q1; ++q)                                           \
    *reinterpret_cast<uint4 *>(&lds.e[st][s_off + q * 32 * kMxBk]) = er[slot][q];
#define MS_STOREES(st, slot) lds.es[st][tid] = esr[slot];
#define MS_STOREW(st, slot)                                                                   \
  _Pragma("unroll") for (int q = 0; q < 4; ++q)                                             \
    *reinterpret_cast<uint4 *>(&lds.w[st][s_off + q * 32 * kMxBk]) = wr[slot][q];           \
  lds.ws[st][tid] = wsr[slot];
#define MS_FRAG(buf, base, c)                                                                 \
  join16(*reinterpret_cast<const uint4 *>(&(buf)[(base) + ((c) ? f1lo : f0lo)]),            \
         *reinterpret_cast<const uint4 *>(&(buf)[(base) + ((c) ? f1hi : f0hi)]))
#define MS_FRAGA(st, c, i) MS_FRAG(lds.w[st], ((i) * 32 + frow) * kMxBk, c)
#define MS_FRAGSB(st, c, dst_b)                                                               \
  _Pragma("unroll") for (int j = 0; j < 2; ++j)                                             \
    dst_b[j] = MS_FRAG(lds.e[st], b_base + j * 32 * kMxBk, c);
#define MS_SCALES(st)                                                                         \
  _Pragma("unroll") for (int i = 0; i < NT; ++i) aS[i] = lds.ws[st][i * 32 + frow];         \
  _Pragma("unroll") for (int j = 0; j < 2; ++j) bS[j] = lds.es[st][wave * 64 + j * 32 + frow];
#define MS_SB(word, c) ((int)(((word) >> (8 * (2 * (c) + h))) & 0xFFu))
#define MS_TILE(i, A, B, c)                                                                   \
  _Pragma("unroll") for (int j = 0; j < 2; ++j)                                             \
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                            \
        A, B[j], acc[i][j], 0, 0, 0, MS_SB(aS[i], c), 0, MS_SB(bS[j], c));
#define MS_FENCE() __builtin_amdgcn_sched_barrier(0)
// Step kt (ring slot s = kt % kMsRing) computes from stage s & 1: its first
// 64-input chunk over the tiles, with the A fragment of the next tile read ahead,
// then the second. Spread over the first chunk's tiles it stores e and the
// weight of step kt + 1 (loaded earlier) into the other stage, and loads e of
// step kt + 2 and the weight of step kt + kMsRing - 1.
#define MS_STEP(s)                                                                            \
  {                                                                                         \
    const int P = (s) & 1, Q = P ^ 1;                                                       \
    const int ws_ = ((s) + 1) % kMsRing, wl_ = ((s) + kMsRing - 1) % kMsRing;               \
    _Pragma("unroll") for (int i = 0; i < NT; ++i) {                                        \
      aN = i + 1 < NT ? MS_FRAGA(P, 0, i + 1) : MS_FRAGA(P, 1, 0);                          \
      if (i == 0) { MS_FRAGSB(P, 1, b1) }                                                   \
      if (i == 0) { MS_LOADE(P, kt + (s) + 2, 0, 4) MS_STOREE(Q, Q, 0, 4) }                 \
      if (i == 1) { MS_LOADE(P, kt + (s) + 2, 4, 8) MS_LOADES(P, kt + (s) + 2)              \
                    MS_STOREE(Q, Q, 4, 8) MS_STOREES(Q, Q) }                                \
      if (i == (NT > 2 ? 2 : NT - 1)) { MS_LOADW(wl_, kt + (s) + kMsRing - 1) MS_STOREW(Q, ws_) } \
      MS_TILE(i, aC, b0, 0)                                                                 \
      aC = aN;                                                                              \
      MS_FENCE();                                                                           \
    }                                                                                       \
    _Pragma("unroll") for (int i = 0; i < NT; ++i) {                                        \
      if (i + 1 < NT) aN = MS_FRAGA(P, 1, i + 1);                                           \
      MS_TILE(i, aC, b1, 1)                                                                 \
      if (i + 1 < NT) aC = aN;                                                              \
      MS_FENCE();                                                                           \
    }                                                                                       \
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                       \
    MS_FENCE();                                                                             \
    MS_FRAGSB(Q, 0, b0)                                                                     \
    aC = MS_FRAGA(Q, 0, 0);                                                                 \
    MS_SCALES(Q)                                                                            \
  }
  // prologue: the weight of steps 0 .. kMsRing - 2, E of steps 0 and 1; step 0 into stage 0
#pragma unroll
  for (int s = 0; s < kMsRing - 1; ++s) { MS_LOADW(s, s) }
  MS_LOADE(0, 0, 0, 8)
  MS_LOADES(0, 0)
  MS_LOADE(1, 1, 0, 8)
  MS_LOADES(1, 1)
  MS_STOREW(0, 0)
  MS_STOREE(0, 0, 0, 8)
  MS_STOREES(0, 0)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  MS_FRAGSB(0, 0, b0)
  aC = MS_FRAGA(0, 0, 0);
  MS_SCALES(0)
  for (int kt = 0; kt < KT; kt += kMsRing) {
    MS_STEP(0) MS_STEP(1) MS_STEP(2) MS_STEP(3) MS_STEP(4) MS_STEP(5)
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef MS_STEP
#undef MS_FENCE
#undef MS_TILE
#undef MS_FRAGA
#undef MS_FRAGSB
#undef MS_SB
#undef MS_SCALES
#undef MS_FRAG
#undef MS_STOREW
#undef MS_STOREES
#undef MS_STOREE
#undef MS_LOADW
#undef MS_LOADES
#undef MS_LOADE
#undef MS_KT
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
        const int n = c0 + i * 32 + g * 8 + h * 4;
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

__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mx_skinny_kernel(MxOperands op, uint16_t *__restrict__ C, int M, int N, int w_lo, int wide) {
  __shared__ __align__(1024) MxSkLds lds;
  const int b = blockIdx.x;
  const int c0 = b * w_lo + min(b, wide) * 32;
  if (c0 >= N) return;
  const int nt = (w_lo + (b < wide ? 32 : 0)) / 32;
  if (nt == 4) mx_skinny_block<4>(op, C, M, N, c0, lds);
  else if (nt == 3) mx_skinny_block<3>(op, C, M, N, c0, lds);
  else mx_skinny_block<2>(op, C, M, N, c0, lds);
}

// The skinny schedule, when it applies: at most one token tile, whole rings of
// K-steps, and 64-128 weight rows per CU. w_lo = 32 floor(n / (32 G)); the first
// `wide` blocks take 32 rows more.
hipError_t plan_mx_skinny(int64_t m, int64_t n, int32_t segments, int &w_lo, int &wide,
                          int &blocks) {
  blocks = 0;
  const int64_t kt = (int64_t)segments * 256 / kMxBk;
  if (m > BM || kt % kMsRing != 0 || n > INT32_MAX) return hipSuccess;
  int cus = 0;
  const hipError_t err = cu_count(cus);
  if (err != hipSuccess) return err;
  const int64_t lo = (n / cus) / 32 * 32;
  if (lo < 64 || lo + 32 > kMsMaxCols) return hipSuccess;
  w_lo = (int)lo;
  wide = (int)((n - (int64_t)cus * lo + 31) / 32);
  blocks = cus;
  return hipSuccess;
}

}  // namespace

hipError_t engram_launch_gemm_mx(const uint8_t *w_codes, const uint8_t *w_scales,
                                 const uint8_t *e_codes, const uint8_t *e_scales,
                                 int32_t segments, uint16_t *kv,
                                 int64_t m, int64_t n, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (m <= 0 || n <= 0) return hipSuccess;
  const MxOperands op{w_codes, w_scales, e_codes, e_scales, segments};
  int w_lo = 0, wide = 0, sk_blocks = 0;
  hipError_t err = plan_mx_skinny(m, n, segments, w_lo, wide, sk_blocks);
  if (err != hipSuccess) return err;
  if (sk_blocks > 0) {
    hipLaunchKernelGGL(gemm_mx_skinny_kernel, dim3((unsigned)sk_blocks), dim3(kWideThreads), 0,
                       stream, op, kv, (int)m, (int)n, w_lo, wide);
    return hipGetLastError();
  }
  StreamK sk;
  err = plan_streamk(m, n, (int64_t)segments * 256 / kMxBk, sk);
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
  return engram_gemm::launch_streamk_fixup((const float *)workspace, kv, m, n, sk, stream);
}

hipError_t engram_launch_gemm_mx_sums(const uint8_t *w_codes, const uint8_t *w_scales,
                                      const uint8_t *e_codes, const uint8_t *e_scales,
                                      int32_t segments, const uint16_t *h, const float *qk_w,
                                      uint16_t *kv, int64_t m, int32_t hc, int32_t dim,
                                      hipStream_t stream) {
  if (m <= 0) return hipSuccess;
  const MxOperands op{w_codes, w_scales, e_codes, e_scales, segments};
  const int64_t n = (int64_t)(hc + 1) * dim;
  const int tiles_m = (int)((m + BM - 1) / BM);
  const int tiles_n = (int)(n / BN);
  hipLaunchKernelGGL(gemm_mx_sums_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kWideThreads),
                     0, stream, op, kv, (int)m, (int)n, tiles_m, tiles_n, h, qk_w, (int)hc,
                     (int)dim);
  return hipGetLastError();
}

hipError_t engram_gemm_mx_whole_tiles(int64_t m, int64_t n, int32_t segments, bool *whole) {
  *whole = false;
  if (m <= 0 || n <= 0) return hipSuccess;
  StreamK sk;
  const hipError_t err = plan_streamk(m, n, (int64_t)segments * 256 / kMxBk, sk);
  if (err != hipSuccess) return err;
  *whole = sk.blocks == 0;
  return hipSuccess;
}

hipError_t engram_gemm_mx_workspace(int64_t m, int64_t n, int32_t segments, size_t *bytes) {
  *bytes = 0;
  if (m <= 0 || n <= 0) return hipSuccess;
  int w_lo = 0, wide = 0, sk_blocks = 0;
  hipError_t err = plan_mx_skinny(m, n, segments, w_lo, wide, sk_blocks);
  if (err != hipSuccess) return err;
  if (sk_blocks > 0) return hipSuccess;
  StreamK sk;
  err = plan_streamk(m, n, (int64_t)segments * 256 / kMxBk, sk);
  if (err != hipSuccess) return err;
  *bytes = (size_t)sk.blocks * 2 * kWideOutputs * kWideThreads * sizeof(float);
  return hipSuccess;
}
