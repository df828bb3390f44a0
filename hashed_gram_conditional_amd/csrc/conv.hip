// The short convolution branch after the gate, and its history across chunks.
//
// Pages: "DeepSeek Engram 详解：把静态知识从计算里拆出来" §4.2 (Y = SiLU(Conv1D(
// RMSNorm(V~))) + V~ on the gated values V~ = alpha v, depthwise and causal,
// kernel size 4 at dilation 3 so that position t reads t, t-3, t-6, t-9, filters
// starting at zero, H += Y) and §9.5 (decode and chunked prefill keep the past 9
// positions); "条件记忆：DeepSeek V4.1 Engram 如何用 O(1) 查表换掉一层计算" §三
// (output = value + short_conv(value)); "DeepSeek-V4.1 模型结构（5）：记忆，Engram",
// "V4.1 相对原版的两处改动" (the branch the original design had after the gate).
//
// The gate kernel has already stored, per token, the hc gates and the mean
// square of the value row v. The gated value of stream m is alpha_m v, so its
// RMS is |alpha_m| rms(v): the normalised input is
//   n = alpha_m v / sqrt(alpha_m^2 mean(v^2) + eps) * g_m
// and no (token, stream) vector has to be reduced again. Each thread owns one
// stream and 8 channels, keeps their filters (8 x taps) and norm weights in
// registers, and walks a run of consecutive tokens, so the filters are read once
// per run. The value rows a token reaches lie at most (taps - 1) dilation rows
// back and are shared by the hc streams and the run's neighbours: they come from
// the L2. h is read and written once. Arithmetic is fp32; h is rounded once.
//
// The history of a sequence is the last L = (taps - 1) dilation positions in
// factored form: their value rows (kv's dtype) and [alpha_0..alpha_{hc-1},
// mean(v^2)] (fp32), which rebuild V~ exactly as the chunk's own positions do.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8;
constexpr int kMaxHcConv = 8;
constexpr int kWindowTokens = 12;   // 228 VGPRs, 2 waves per SIMD (16 tokens: 256 and 1 wave)

// The kernels issue few memory operations per arithmetic one, so they use the
// hardware's exp2, reciprocal and reciprocal square root (about 1 ulp each)
// instead of the correctly rounded library sequences, which would make them
// bound by VALU issue.
// SiLU(u) = u sigmoid(u) = u / (1 + 2^(-u log2(e))).
__device__ __forceinline__ float silu(float u) {
  return u * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-u * 1.4426950408889634f));
}

// 1 / RMS of the gated value alpha v, times alpha: alpha / sqrt(alpha^2 mean(v^2) + eps).
__device__ __forceinline__ float norm_factor(float a, float ms, float eps) {
  return a * __builtin_amdgcn_rsqf(fmaf(a * a, ms, eps));
}

template <bool F32, int TAPS>
__global__ __launch_bounds__(kThreads) void short_conv_kernel(
    EngramConvArgs c, const int32_t *__restrict__ ids, EngramDeadRule dead_rule,
    const void *__restrict__ kv, const float *__restrict__ stats, void *__restrict__ h,
    int64_t ntok, int64_t seq, int hc, int dim, int tpb) {
  const int cps = dim / kChunk;
  const int p = blockIdx.y * kThreads + threadIdx.x;
  if (p >= hc * cps) return;
  const int m = p / cps;
  const int ci = p - m * cps;

  float w[kChunk][TAPS];
  {
    const float4 *wp =
        reinterpret_cast<const float4 *>(c.weight + ((int64_t)m * dim + ci * kChunk) * TAPS);
#pragma unroll
    for (int q = 0; q < 2 * TAPS; ++q) {
      const float4 f = wp[q];
      const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) w[(4 * q + r) / TAPS][(4 * q + r) % TAPS] = fv[r];
    }
  }
  float g[kChunk];
  if (c.norm_weight != nullptr) {
    const float4 *gp = reinterpret_cast<const float4 *>(c.norm_weight + (int64_t)m * dim) + 2 * ci;
    const float4 g0 = gp[0], g1 = gp[1];
    g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
    g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
  } else {
#pragma unroll
    for (int e = 0; e < kChunk; ++e) g[e] = 1.f;
  }

  // the norm weight multiplies each filter tap of its channel
#pragma unroll
  for (int e = 0; e < kChunk; ++e)
#pragma unroll
    for (int j = 0; j < TAPS; ++j) w[e][j] *= g[e];

  const int64_t kv_row = (int64_t)(hc + 1) * cps;   // chunks per kv row
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  const int64_t t1 = t0 + tpb < ntok ? t0 + tpb : ntok;
  for (int64_t t = t0; t < t1; ++t) {
    if (engram_dead(dead_rule, ids[t])) continue;   // DEAD: streams untouched
    const int64_t b = t / seq;
    const int64_t s = t - b * seq;
    float u[kChunk], vt[kChunk];
#pragma unroll
    for (int e = 0; e < kChunk; ++e) {
      u[e] = 0.f;
      vt[e] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < TAPS; ++j) {
      const int64_t back = (int64_t)(TAPS - 1 - j) * c.dilation;
      engram::Chunk8<F32> v;
      float a, ms;
      if (s >= back) {                                // inside the chunk
        const int64_t row = t - back;
        v.load(kv, row * kv_row + (int64_t)hc * cps + ci);
        a = stats[row * (hc + 1) + m];
        ms = stats[row * (hc + 1) + hc];
      } else if (c.state_v_in != nullptr) {           // the sequence's history
        const int64_t srow = b * c.history + c.history + (s - back);
        v.load(c.state_v_in, srow * cps + ci);
        a = c.state_s_in[srow * (hc + 1) + m];
        ms = c.state_s_in[srow * (hc + 1) + hc];
      } else {
        continue;                                     // before the sequence start: zero
      }
      const float r = norm_factor(a, ms, c.eps);
#pragma unroll
      for (int e = 0; e < kChunk; ++e) u[e] = fmaf(w[e][j], r * v[e], u[e]);
      if (j == TAPS - 1) {
#pragma unroll
        for (int e = 0; e < kChunk; ++e) vt[e] = a * v[e];
      }
    }
    const int64_t hi = (t * hc + m) * (int64_t)cps + ci;
    engram::Chunk8<F32> hh;
    hh.load_nt(h, hi);
    float o[kChunk];
#pragma unroll
    for (int e = 0; e < kChunk; ++e) o[e] = hh[e] + (silu(u[e]) + vt[e]);
    engram::Chunk8<F32>::store_nt(h, hi, o);
  }
}

// The papers' configuration (TAPS taps at dilation DIL known at compile time,
// bf16 rows) for calls with enough tokens: a block owns TB consecutive flat
// tokens and 256 (stream, 8-channel) pairs. The value chunks of the rows
// [t0 - L, t0 + TB) are loaded once into a register window (each tap of each
// token then indexes it statically), the rows' gates and mean squares once into
// LDS, and the run's h chunks are requested with them, so the fully unrolled
// token loop waits for memory once. A tap whose row lies before its sequence's
// start reads the history (or zero) instead of the window.
template <int TAPS, int DIL, int TB>
__global__ __launch_bounds__(kThreads) void short_conv_window_kernel(
    EngramConvArgs c, const int32_t *__restrict__ ids, EngramDeadRule dead_rule,
    const void *__restrict__ kv, const float *__restrict__ stats, void *__restrict__ h,
    int64_t ntok, int64_t seq, int hc, int dim) {
  constexpr int L = (TAPS - 1) * DIL;
  constexpr int R = TB + L;                       // window rows
  static_assert(R * (kMaxHcConv + 1) <= kThreads && TB <= kThreads,
                "one shared element per thread");
  __shared__ float s_stat[R][kMaxHcConv + 1];
  __shared__ int32_t s_ids[TB];
  const int cps = dim / kChunk;
  // Channel segments vary fastest over the grid, so the blocks of one token
  // group run together and share their value rows in the L2.
  const int segs = (hc * cps + kThreads - 1) / kThreads;
  const int64_t group = blockIdx.x / segs;
  const int seg = (int)(blockIdx.x - group * segs);
  const int64_t t0 = group * TB;
  const int tid = threadIdx.x;
  const int p = seg * kThreads + tid;
  const bool live = p < hc * cps;
  const int pp = live ? p : 0;                    // idle threads load pair 0 and store nothing
  const int m = pp / cps;
  const int ci = pp - m * cps;
  const int64_t kv_row = (int64_t)(hc + 1) * cps;

  // The gates, mean squares and ids the block shares go first (one element per
  // thread, branch-free with clamped addresses): the loads complete in order,
  // so storing them to LDS then waits for nothing issued after them. Then every
  // other global load of the thread is issued before the block's barrier:
  // filters, norm weights and the value window.
  const int nstat = R * (hc + 1);
  const int sr = tid / (hc + 1), scol = tid - sr * (hc + 1);
  const int64_t srow_g = t0 - L + sr;
  const bool stat_ok = tid < nstat && srow_g >= 0 && srow_g < ntok;
  const float stat_v = stats[stat_ok ? srow_g * (hc + 1) + scol : 0];
  const int64_t tid_tok = t0 + (tid < TB ? tid : 0);
  const int32_t id_v = ids[tid_tok < ntok ? tid_tok : ntok - 1];
  float4 wq[2 * TAPS];
  {
    const float4 *wp =
        reinterpret_cast<const float4 *>(c.weight + ((int64_t)m * dim + ci * kChunk) * TAPS);
#pragma unroll
    for (int q = 0; q < 2 * TAPS; ++q) wq[q] = wp[q];
  }
  float4 g0 = make_float4(1.f, 1.f, 1.f, 1.f), g1 = g0;
  if (c.norm_weight != nullptr) {
    const float4 *gp = reinterpret_cast<const float4 *>(c.norm_weight + (int64_t)m * dim) + 2 * ci;
    g0 = gp[0];
    g1 = gp[1];
  }
  engram::Chunk8<false> win[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t row = t0 - L + r;
    row = row < 0 ? 0 : row >= ntok ? ntok - 1 : row;
    win[r].load(kv, row * kv_row + (int64_t)hc * cps + ci);
  }
  // The run's h chunks as well: the loop below stores to h, so a load left in
  // it could not be issued before the previous token's store and each token
  // would wait for HBM in turn. Rows past the chunk read its last token's row.
  const int64_t h_step = (int64_t)hc * cps;
  engram::Chunk8<false> hh[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    const int64_t row = t0 + i < ntok ? t0 + i : ntok - 1;
    hh[i].load_nt(h, (row * hc + m) * (int64_t)cps + ci);
  }

  if (tid < nstat) s_stat[sr][scol] = stat_ok ? stat_v : 0.f;
  if (tid < TB) s_ids[tid] = (t0 + tid < ntok && !engram_dead(dead_rule, id_v)) ? id_v : -1;
  __syncthreads();
  if (!live) return;

  float w[kChunk][TAPS];
#pragma unroll
  for (int q = 0; q < 2 * TAPS; ++q) {
    const float fv[4] = {wq[q].x, wq[q].y, wq[q].z, wq[q].w};
#pragma unroll
    for (int r = 0; r < 4; ++r) w[(4 * q + r) / TAPS][(4 * q + r) % TAPS] = fv[r];
  }
  const float g[kChunk] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
  for (int e = 0; e < kChunk; ++e)
#pragma unroll
    for (int j = 0; j < TAPS; ++j) w[e][j] *= g[e];
  // normalisation factor of each window row
  float rs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rs[r] = norm_factor(s_stat[r][m], s_stat[r][hc], c.eps);
  // Sequence and position of the run's tokens: one division per block, then
  // stepped (token counts fit in 32 bits, which the API checks).
  const int seq32 = (int)seq;
  int b = (int)(t0 / seq32);
  int s = (int)(t0 - (int64_t)b * seq32) - 1;
  const int64_t h_base = (t0 * hc + m) * (int64_t)cps + ci;
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    if (++s == seq32) {
      s = 0;
      ++b;
    }
    const int32_t x = s_ids[i];
    if (x < 0) continue;          // DEAD (or past the last token): streams untouched
    float u[kChunk];
#pragma unroll
    for (int e = 0; e < kChunk; ++e) u[e] = 0.f;
#pragma unroll
    for (int j = 0; j < TAPS; ++j) {
      const int back = (TAPS - 1 - j) * DIL;
      const int r = i + L - back;                  // window row of this tap
      if (s >= back) {
#pragma unroll
        for (int e = 0; e < kChunk; ++e) u[e] = fmaf(w[e][j], rs[r] * win[r][e], u[e]);
      } else if (c.state_v_in != nullptr) {
        const int64_t srow = (int64_t)b * c.history + c.history + (s - back);
        engram::Chunk8<false> v;
        v.load(c.state_v_in, srow * cps + ci);
        const float a = c.state_s_in[srow * (hc + 1) + m];
        const float ms = c.state_s_in[srow * (hc + 1) + hc];
        const float rr = norm_factor(a, ms, c.eps);
#pragma unroll
        for (int e = 0; e < kChunk; ++e) u[e] = fmaf(w[e][j], rr * v[e], u[e]);
      }
    }
    const float a_t = s_stat[i + L][m];
    float o[kChunk];
#pragma unroll
    for (int e = 0; e < kChunk; ++e) o[e] = hh[i][e] + fmaf(a_t, win[i + L][e], silu(u[e]));
    engram::Chunk8<false>::store_nt(h, h_base + i * h_step, o);
  }
}

// History after the chunk: position q of the new history is entry q + T of
// [old history (L) ; chunk (T)]. One block column per sequence; each thread
// owns one 8-element column of the value rows (and the first hc + 1 threads of
// the first block one column of the scalars) and walks q upwards, so a read
// never meets an entry this call has already overwritten: the output may alias
// the input. Runs after the convolution on the same stream.
template <bool F32>
__global__ __launch_bounds__(kThreads) void conv_state_kernel(
    EngramConvArgs c, const void *__restrict__ kv, const float *__restrict__ stats,
    int64_t seq, int hc, int dim) {
  const int64_t b = blockIdx.x;
  const int cps = dim / kChunk;
  const int ci = blockIdx.y * kThreads + threadIdx.x;
  const int L = c.history;
  const int64_t kv_row = (int64_t)(hc + 1) * cps;
  if (ci < cps) {
    for (int q = 0; q < L; ++q) {
      const int64_t x = q + seq;
      engram::Chunk8<F32> v;
      if (x >= L)
        v.load(kv, (b * seq + x - L) * kv_row + (int64_t)hc * cps + ci);
      else if (c.state_v_in != nullptr)
        v.load(c.state_v_in, (b * L + x) * cps + ci);
      else
        v.zero();
      v.put(c.state_v_out, (b * L + q) * cps + ci);
    }
  }
  if (blockIdx.y == 0 && (int)threadIdx.x <= hc) {
    const int col = threadIdx.x;
    for (int q = 0; q < L; ++q) {
      const int64_t x = q + seq;
      float f = 0.f;
      if (x >= L)
        f = stats[(b * seq + x - L) * (hc + 1) + col];
      else if (c.state_s_in != nullptr)
        f = c.state_s_in[(b * L + x) * (hc + 1) + col];
      c.state_s_out[(b * L + q) * (hc + 1) + col] = f;
    }
  }
}

// The convolution over the chunk's tokens.
template <bool F32>
hipError_t launch_conv(const EngramConvArgs &c, const int32_t *ids, EngramDeadRule dead_rule,
                       const void *kv, const float *stats, void *h, int64_t ntok, int64_t seq,
                       int hc, int dim, hipStream_t stream) {
  int dev = 0, cus = 256;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess)
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  const int cps = dim / kChunk;
  const int gy = (hc * cps + kThreads - 1) / kThreads;
  const int64_t window_blocks = (ntok + kWindowTokens - 1) / kWindowTokens * gy;
  if (!F32 && c.taps == 4 && c.dilation == 3 && ntok >= (int64_t)kWindowTokens * cus &&
      window_blocks <= INT32_MAX) {
    const dim3 grid((unsigned)window_blocks);
    hipLaunchKernelGGL((short_conv_window_kernel<4, 3, kWindowTokens>), grid, dim3(kThreads), 0,
                       stream, c, ids, dead_rule, kv, stats, h, ntok, seq, hc, dim);
    return hipGetLastError();
  }
  // Runs of up to 16 tokens per thread while that still leaves about 8 blocks
  // per CU; one token per run for decode-sized calls.
  int64_t tpb = ntok * gy / (8 * (int64_t)cus);
  tpb = tpb < 1 ? 1 : tpb > 16 ? 16 : tpb;
  const dim3 grid((unsigned)((ntok + tpb - 1) / tpb), (unsigned)gy);
#define ENGRAM_CONV_CASE(N)                                                                 \
  case N:                                                                                   \
    hipLaunchKernelGGL((short_conv_kernel<F32, N>), grid, dim3(kThreads), 0, stream, c, ids, \
                       dead_rule, kv, stats, h, ntok, seq, hc, dim, (int)tpb);              \
    break;
  switch (c.taps) {
    ENGRAM_CONV_CASE(1)
    ENGRAM_CONV_CASE(2)
    ENGRAM_CONV_CASE(3)
    ENGRAM_CONV_CASE(4)
    ENGRAM_CONV_CASE(5)
    ENGRAM_CONV_CASE(6)
    ENGRAM_CONV_CASE(7)
    ENGRAM_CONV_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef ENGRAM_CONV_CASE
  return hipGetLastError();
}

template <bool F32>
hipError_t launch(const EngramConvArgs &c, const int32_t *ids, EngramDeadRule dead_rule,
                  const void *kv,
                  const float *stats, void *h, int64_t batch, int64_t seq, int hc, int dim,
                  hipStream_t stream) {
  const int64_t ntok = batch * seq;
  if (ntok > 0) {
    const hipError_t err =
        launch_conv<F32>(c, ids, dead_rule, kv, stats, h, ntok, seq, hc, dim, stream);
    if (err != hipSuccess) return err;
  }
  if (c.state_v_out != nullptr && batch > 0 && c.history > 0) {
    const int cps = dim / kChunk;
    const int cols = cps > hc + 1 ? cps : hc + 1;
    const dim3 grid((unsigned)batch, (unsigned)((cols + kThreads - 1) / kThreads));
    hipLaunchKernelGGL((conv_state_kernel<F32>), grid, dim3(kThreads), 0, stream, c, kv, stats,
                       seq, hc, dim);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t engram_launch_short_conv(bool f32, const EngramConvArgs &c, const int32_t *ids,
                                    EngramDeadRule dead_rule, const void *kv, const float *stats,
                                    void *h, int64_t batch, int64_t seq, int32_t hc,
                                    int32_t dim, hipStream_t stream) {
  return f32 ? launch<true>(c, ids, dead_rule, kv, stats, h, batch, seq, hc, dim, stream)
             : launch<false>(c, ids, dead_rule, kv, stats, h, batch, seq, hc, dim, stream);
}
