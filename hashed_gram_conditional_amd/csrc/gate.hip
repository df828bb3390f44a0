// Step 5 of the Engram layer: context gate per hyper-connection stream and the
// residual update.
//
// Pages: "DeepSeek-V4.1 模型结构（5）：记忆，Engram", "门控：用当前的上下文决定查到的向量用多少"
// (s^(m) = RMSNorm(h^(m)) . RMSNorm(k^(m)) / sqrt(d), h^(m) += alpha^(m) v, one
// shared v for all streams), "sigmoid 之前多一步带符号的平方根" (the signed
// square root before the sigmoid, with a clamp on |s|, and the papers' plain
// sigmoid(s) it departs from, also "DeepSeek Engram 详解：把静态知识从计算里拆出来"
// §4.1) and the image-token paragraph (gate 0 at DEAD positions); "ds4.c 学习笔记 · Engram", "消费：学习投影 +
// 余弦门控" (the learned scales q_w * k_w inside the dot, eps inside the
// reciprocal roots of the mean squares, the update rounded to bf16 once) and
// "布局与哈希探测" item 4 (masked rows are left untouched).
//
// gate_kernel: one block per token, 256 threads when there are enough tokens
// to fill the chip (512 for few tokens whose streams are too wide for
// gate_stream_kernel, below). Each thread owns CPT chunks of 8
// elements per stream (16-byte bf16 accesses). Streams are handled one after
// another: the three reductions of stream m (sum h^2, sum k^2, sum h q_w k_w k)
// need only its own h and k, so after one barrier its gate is known and its h,
// still in registers, is updated and stored before the next stream is read. h
// is read from HBM once (updating all streams after all reductions re-read it,
// and the L2 had often dropped it by then). All arithmetic is fp32.
//
// Few tokens (decode, up to 2 chunks per thread): gate_stream_kernel gives every
// (token, stream) pair a block of its own, 4 per CU at 256 tokens x 4 streams,
// so a stream's loads, its one barrier and its update overlap the other
// streams' instead of queueing behind them in one block. Its thread count,
// chunk ownership and reduction order are the per-token kernel's, so the bits
// are too; the block of stream 0 also forms the statistics mode's mean square
// of the value row.
//
// With a stats buffer the kernel is the first half of the short-convolution
// variant: it stores each token's gates and the mean square of its value row
// (the factors of the gated value's RMS) and leaves h to the convolution.
//
// gate_sums_kernel is the second half of the projection that computes the key
// side of the gate in its epilogue (the pages' "上下文门控 + 单次 GEMM 融合" in
// "条件记忆：DeepSeek V4.1 Engram 如何用 O(1) 查表换掉一层计算" §2.3): it reads
// each token's sums of k^2 and h q_w k_w k per 128-column block instead of
// the keys: 93 KB per token at hc 4 x 5120 against 133 KB (52 KB against
// 92 KB in the statistics mode).
#include "common.h"

namespace {

constexpr int kMaxThreads = 512;
constexpr int kMaxHc = 8;
constexpr int kChunk = 8;        // elements per chunk

template <bool F32>
using Chunk = engram::Chunk8<F32>;

// Every byte the gate touches is used once, so its loads and stores carry the
// nontemporal hint (5 % faster at 32768 tokens than cached accesses).

template <bool F32, int CPT>
__global__ __launch_bounds__(kMaxThreads) void gate_kernel(
    const int32_t *__restrict__ ids, EngramDeadRule dead_rule, const void *__restrict__ kv,
    const float *__restrict__ q_w, const float *__restrict__ k_w, void *__restrict__ h,
    float *__restrict__ gate_out, float *__restrict__ stats, int hc, int dim, float eps,
    float clamp, int plain) {
  // one slot per (wave, stream): every stream's partial sums have their own
  // place, so one barrier per stream orders writes before reads
  __shared__ float red[kMaxThreads / engram::kWave][kMaxHc + 1][3];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  if (engram_dead(dead_rule, ids[t])) {   // DEAD: gate 0, streams untouched
    if (gate_out != nullptr && tid < hc) gate_out[t * hc + tid] = 0.f;
    if (stats != nullptr && tid <= hc) stats[t * (hc + 1) + tid] = 0.f;
    return;
  }
  const int cps = dim / kChunk;                   // chunks per stream
  const int64_t kv_row = t * (int64_t)(hc + 1) * cps;
  const int64_t h_row = t * (int64_t)hc * cps;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int nwaves = nthreads >> 6;
  const float inv_d = 1.0f / (float)dim;
  const float inv_sqrt_d = 1.0f / sqrtf((float)dim);

  Chunk<F32> vv[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = tid + c * nthreads;
    if (ci < cps) vv[c].load_nt(kv, kv_row + (int64_t)hc * cps + ci);
  }
  if (stats != nullptr) {
    float svv = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + c * nthreads;
      if (ci < cps) {
#pragma unroll
        for (int e = 0; e < 8; ++e) svv = fmaf(vv[c][e], vv[c][e], svv);
      }
    }
    svv = engram::warp_sum(svv);
    if (lane == 0) red[wave][kMaxHc][0] = svv;
  }

  // The weights q_w * k_w of chunk ci of stream m, one fp32 product each; with
  // k_w == NULL, q_w already holds those products (folded once per call).
  auto scales = [&](int m, int ci, float (&w)[8]) {
    const float4 *qp = reinterpret_cast<const float4 *>(q_w + (int64_t)m * dim) + 2 * ci;
    const float4 q0 = qp[0], q1 = qp[1];
    if (k_w == nullptr) {
      w[0] = q0.x; w[1] = q0.y; w[2] = q0.z; w[3] = q0.w;
      w[4] = q1.x; w[5] = q1.y; w[6] = q1.z; w[7] = q1.w;
    } else {
      const float4 *kp = reinterpret_cast<const float4 *>(k_w + (int64_t)m * dim) + 2 * ci;
      const float4 k0 = kp[0], k1 = kp[1];
      w[0] = q0.x * k0.x; w[1] = q0.y * k0.y; w[2] = q0.z * k0.z; w[3] = q0.w * k0.w;
      w[4] = q1.x * k1.x; w[5] = q1.y * k1.y; w[6] = q1.z * k1.z; w[7] = q1.w * k1.w;
    }
  };
  {
    // Stream by stream: the gate of stream m depends on its own h and k only, so
    // its h is reduced, gated and updated from registers before the next stream
    // is read; h crosses HBM once in each direction.
#pragma unroll
    for (int m = 0; m < kMaxHc; ++m) {
      if (m >= hc) break;
      Chunk<F32> hh[CPT];
      float shh = 0.f, skk = 0.f, shk = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int ci = tid + c * nthreads;
        if (ci < cps) {
          Chunk<F32> kc;
          hh[c].load_nt(h, h_row + (int64_t)m * cps + ci);
          kc.load_nt(kv, kv_row + (int64_t)m * cps + ci);
          float w[8];
          scales(m, ci, w);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float he = hh[c][e];
            const float ke = kc[e];
            shh = fmaf(he, he, shh);
            skk = fmaf(ke, ke, skk);
            shk = fmaf(he * w[e], ke, shk);
          }
        }
      }
      shh = engram::warp_sum(shh);
      skk = engram::warp_sum(skk);
      shk = engram::warp_sum(shk);
      if (lane == 0) {
        red[wave][m][0] = shh;
        red[wave][m][1] = skk;
        red[wave][m][2] = shk;
      }
      __syncthreads();
      float a = 0.f, b = 0.f, c2 = 0.f;
      for (int w = 0; w < nwaves; ++w) {
        a += red[w][m][0];
        b += red[w][m][1];
        c2 += red[w][m][2];
      }
      const float rh = 1.0f / sqrtf(a * inv_d + eps);
      const float rk = 1.0f / sqrtf(b * inv_d + eps);
      const float sc = c2 * rh * rk * inv_sqrt_d;
      const float z = plain ? sc : copysignf(sqrtf(fmaxf(fabsf(sc), clamp)), sc);
      const float alpha = 1.0f / (1.0f + expf(-z));
      if (tid == 0) {
        if (gate_out != nullptr) gate_out[t * hc + m] = alpha;
        if (stats != nullptr) stats[t * (hc + 1) + m] = alpha;
      }
      if (stats == nullptr) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int ci = tid + c * nthreads;
          if (ci < cps) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(alpha, vv[c][e], hh[c][e]);
            Chunk<F32>::store_nt(h, h_row + (int64_t)m * cps + ci, o);
          }
        }
      }
    }
  }
  if (stats != nullptr && tid == 0) {
    // the value row's partial sums were published before the first barrier
    float svv = 0.f;
    for (int w = 0; w < nwaves; ++w) svv += red[w][kMaxHc][0];
    stats[t * (hc + 1) + hc] = svv * inv_d;
  }
}

// One (token, stream) pair per block, blockIdx.x the token and blockIdx.y the
// stream: gate_kernel's arithmetic for that stream (the same chunks per thread,
// fma order, wave sums and order of the waves' partial sums). With a stats
// buffer the block stores the stream's gate there instead of updating h, and
// the block of stream 0 also stores the value row's mean square.
template <bool F32, int CPT>
__global__ __launch_bounds__(kMaxThreads) void gate_stream_kernel(
    const int32_t *__restrict__ ids, EngramDeadRule dead_rule, const void *__restrict__ kv,
    const float *__restrict__ q_w, const float *__restrict__ k_w, void *__restrict__ h,
    float *__restrict__ gate_out, float *__restrict__ stats, int hc, int dim, float eps,
    float clamp, int plain) {
  __shared__ float red[kMaxThreads / engram::kWave][3];
  __shared__ float red_v[kMaxThreads / engram::kWave];
  const int64_t t = blockIdx.x;
  const int m = blockIdx.y;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  if (engram_dead(dead_rule, ids[t])) {   // DEAD: gate 0, the stream untouched
    if (tid == 0) {
      if (gate_out != nullptr) gate_out[t * hc + m] = 0.f;
      if (stats != nullptr) {
        stats[t * (hc + 1) + m] = 0.f;
        if (m == 0) stats[t * (hc + 1) + hc] = 0.f;
      }
    }
    return;
  }
  const int cps = dim / kChunk;
  const int64_t kv_row = t * (int64_t)(hc + 1) * cps;
  const int64_t h_row = (t * (int64_t)hc + m) * cps;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int nwaves = nthreads >> 6;
  Chunk<F32> vv[CPT], hh[CPT], kk[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = tid + c * nthreads;
    if (ci < cps) {
      vv[c].load_nt(kv, kv_row + (int64_t)hc * cps + ci);
      hh[c].load_nt(h, h_row + ci);
      kk[c].load_nt(kv, kv_row + (int64_t)m * cps + ci);
    }
  }
  const bool value_stats = stats != nullptr && m == 0;
  if (value_stats) {
    float svv = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + c * nthreads;
      if (ci < cps) {
#pragma unroll
        for (int e = 0; e < 8; ++e) svv = fmaf(vv[c][e], vv[c][e], svv);
      }
    }
    svv = engram::warp_sum(svv);
    if (lane == 0) red_v[wave] = svv;
  }
  float shh = 0.f, skk = 0.f, shk = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = tid + c * nthreads;
    if (ci < cps) {
      // q_w * k_w of the chunk (with k_w == NULL, q_w holds the products)
      const float4 *qp = reinterpret_cast<const float4 *>(q_w + (int64_t)m * dim) + 2 * ci;
      const float4 q0 = qp[0], q1 = qp[1];
      float w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      if (k_w != nullptr) {
        const float4 *kp = reinterpret_cast<const float4 *>(k_w + (int64_t)m * dim) + 2 * ci;
        const float4 k0 = kp[0], k1 = kp[1];
        w[0] *= k0.x; w[1] *= k0.y; w[2] *= k0.z; w[3] *= k0.w;
        w[4] *= k1.x; w[5] *= k1.y; w[6] *= k1.z; w[7] *= k1.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float he = hh[c][e];
        const float ke = kk[c][e];
        shh = fmaf(he, he, shh);
        skk = fmaf(ke, ke, skk);
        shk = fmaf(he * w[e], ke, shk);
      }
    }
  }
  shh = engram::warp_sum(shh);
  skk = engram::warp_sum(skk);
  shk = engram::warp_sum(shk);
  if (lane == 0) {
    red[wave][0] = shh;
    red[wave][1] = skk;
    red[wave][2] = shk;
  }
  __syncthreads();
  float a = 0.f, b = 0.f, c2 = 0.f;
  for (int w = 0; w < nwaves; ++w) {
    a += red[w][0];
    b += red[w][1];
    c2 += red[w][2];
  }
  const float inv_d = 1.0f / (float)dim;
  const float inv_sqrt_d = 1.0f / sqrtf((float)dim);
  const float rh = 1.0f / sqrtf(a * inv_d + eps);
  const float rk = 1.0f / sqrtf(b * inv_d + eps);
  const float sc = c2 * rh * rk * inv_sqrt_d;
  const float z = plain ? sc : copysignf(sqrtf(fmaxf(fabsf(sc), clamp)), sc);
  const float alpha = 1.0f / (1.0f + expf(-z));
  if (tid == 0) {
    if (gate_out != nullptr) gate_out[t * hc + m] = alpha;
    if (stats != nullptr) stats[t * (hc + 1) + m] = alpha;
    if (value_stats) {
      float svv = 0.f;
      for (int w = 0; w < nwaves; ++w) svv += red_v[w];
      stats[t * (hc + 1) + hc] = svv * inv_d;
    }
  }
  if (stats != nullptr) return;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = tid + c * nthreads;
    if (ci < cps) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(alpha, vv[c][e], hh[c][e]);
      Chunk<F32>::store_nt(h, h_row + ci, o);
    }
  }
}

// Threads per token block for the gate kernels: 128 when there are enough
// tokens to keep HBM busy (about 8 per CU), up to 512 below that (few); never
// more threads than a stream has 8-element chunks, rounded up to whole waves.
hipError_t gate_threads(int64_t tokens, int dim, int &threads, int &cpt, bool &few) {
  int dev = 0, cus = 256;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  const int cps = dim / kChunk;
  few = tokens < 8 * (int64_t)cus;
  threads = few ? kMaxThreads : 256;
  const int needed = ((cps + engram::kWave - 1) / engram::kWave) * engram::kWave;
  if (threads > needed) threads = needed;
  cpt = (cps + threads - 1) / threads;
  return hipSuccess;
}

template <bool F32>
hipError_t launch(int cpt, int threads, bool few, const int32_t *ids,
                  EngramDeadRule dead_rule,
                  const void *kv, const float *q_w, const float *k_w, void *h, float *gate_out,
                  float *stats, int64_t tokens, int hc, int dim, float eps, float clamp,
                  int plain, hipStream_t stream) {
#define ENGRAM_GATE_CASE(N)                                                                 \
  hipLaunchKernelGGL((gate_kernel<F32, N>), dim3((unsigned)tokens), dim3(threads), 0,       \
                     stream, ids, dead_rule, kv, q_w, k_w, h, gate_out, stats, hc, dim,     \
                     eps, clamp, plain)
  if (few && cpt <= 2) {
#define ENGRAM_GATE_STREAM_CASE(N)                                                          \
  hipLaunchKernelGGL((gate_stream_kernel<F32, N>), dim3((unsigned)tokens, (unsigned)hc),     \
                     dim3(threads), 0, stream, ids, dead_rule, kv, q_w, k_w, h, gate_out,    \
                     stats, hc, dim, eps, clamp, plain)
    if (cpt == 1)
      ENGRAM_GATE_STREAM_CASE(1);
    else
      ENGRAM_GATE_STREAM_CASE(2);
#undef ENGRAM_GATE_STREAM_CASE
    return hipGetLastError();
  }
  switch (cpt) {
    case 1: ENGRAM_GATE_CASE(1); break;
    case 2: ENGRAM_GATE_CASE(2); break;
    case 3: ENGRAM_GATE_CASE(3); break;
    case 4: ENGRAM_GATE_CASE(4); break;
    case 5: ENGRAM_GATE_CASE(5); break;
    case 6: ENGRAM_GATE_CASE(6); break;
    case 7: ENGRAM_GATE_CASE(7); break;
    case 8: ENGRAM_GATE_CASE(8); break;
    default:
      return hipErrorInvalidValue;
  }
#undef ENGRAM_GATE_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t engram_launch_gate(bool f32, const int32_t *ids, EngramDeadRule dead_rule,
                              const void *kv,
                              const float *q_w, const float *k_w, void *h, float *gate_out,
                              float *stats, int64_t tokens, int32_t hc, int32_t dim, float eps,
                              float clamp, int plain, hipStream_t stream) {
  if (tokens <= 0) return hipSuccess;
  int threads = 0, cpt = 0;
  bool few = false;
  const hipError_t err = gate_threads(tokens, dim, threads, cpt, few);
  if (err != hipSuccess) return err;
  // few tokens: a block per (token, stream)
  return f32 ? launch<true>(cpt, threads, few, ids, dead_rule, kv, q_w, k_w, h, gate_out, stats,
                            tokens, hc, dim, eps, clamp, plain, stream)
             : launch<false>(cpt, threads, few, ids, dead_rule, kv, q_w, k_w, h, gate_out, stats,
                             tokens, hc, dim, eps, clamp, plain, stream);
}

namespace {

// The gate from the key-side sums the projection left in kv's key columns
// (engram::gate_sums_pairs): per stream, sum h^2 from h, which is read for
// the update anyway, and the sums of its dim / 128 column blocks, added in
// block order within each wave and then over the waves. The value row and h
// are read, h is written, as in gate_kernel; the keys are never read. With a
// stats buffer it is gate_kernel's statistics mode on the sums: gates and the
// value row's mean square per token, h only read.
template <int CPT>
__global__ __launch_bounds__(kMaxThreads) void gate_sums_kernel(
    const int32_t *__restrict__ ids, EngramDeadRule dead_rule, const uint16_t *__restrict__ kv,
    void *__restrict__ h, float *__restrict__ gate_out, float *__restrict__ stats, int hc,
    int dim, float eps, float clamp, int plain) {
  __shared__ float red[kMaxThreads / engram::kWave][kMaxHc + 1][3];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  if (engram_dead(dead_rule, ids[t])) {   // DEAD: gate 0, streams untouched
    if (gate_out != nullptr && tid < hc) gate_out[t * hc + tid] = 0.f;
    if (stats != nullptr && tid <= hc) stats[t * (hc + 1) + tid] = 0.f;
    return;
  }
  const int cps = dim / kChunk;
  const int blocks = dim / 128;
  const int64_t kv_row = t * (int64_t)(hc + 1) * cps;
  const int64_t h_row = t * (int64_t)hc * cps;
  const float2 *sums = reinterpret_cast<const float2 *>(kv) + engram::gate_sums_pairs(t, hc, dim);
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int nwaves = nthreads >> 6;
  const float inv_d = 1.0f / (float)dim;
  const float inv_sqrt_d = 1.0f / sqrtf((float)dim);

  Chunk<false> vv[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = tid + c * nthreads;
    if (ci < cps) vv[c].load_nt(kv, kv_row + (int64_t)hc * cps + ci);
  }
  if (stats != nullptr) {
    float svv = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + c * nthreads;
      if (ci < cps) {
#pragma unroll
        for (int e = 0; e < 8; ++e) svv = fmaf(vv[c][e], vv[c][e], svv);
      }
    }
    svv = engram::warp_sum(svv);
    if (lane == 0) red[wave][kMaxHc][0] = svv;
  }
#pragma unroll
  for (int m = 0; m < kMaxHc; ++m) {
    if (m >= hc) break;
    Chunk<false> hh[CPT];
    float shh = 0.f, skk = 0.f, shk = 0.f;
    for (int b = tid; b < blocks; b += nthreads) {
      const float2 s = sums[m * blocks + b];
      skk += s.x;
      shk += s.y;
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + c * nthreads;
      if (ci < cps) {
        hh[c].load_nt(h, h_row + (int64_t)m * cps + ci);
#pragma unroll
        for (int e = 0; e < 8; ++e) shh = fmaf(hh[c][e], hh[c][e], shh);
      }
    }
    shh = engram::warp_sum(shh);
    skk = engram::warp_sum(skk);
    shk = engram::warp_sum(shk);
    if (lane == 0) {
      red[wave][m][0] = shh;
      red[wave][m][1] = skk;
      red[wave][m][2] = shk;
    }
    __syncthreads();
    float a = 0.f, b = 0.f, c2 = 0.f;
    for (int w = 0; w < nwaves; ++w) {
      a += red[w][m][0];
      b += red[w][m][1];
      c2 += red[w][m][2];
    }
    const float rh = 1.0f / sqrtf(a * inv_d + eps);
    const float rk = 1.0f / sqrtf(b * inv_d + eps);
    const float sc = c2 * rh * rk * inv_sqrt_d;
    const float z = plain ? sc : copysignf(sqrtf(fmaxf(fabsf(sc), clamp)), sc);
    const float alpha = 1.0f / (1.0f + expf(-z));
    if (tid == 0) {
      if (gate_out != nullptr) gate_out[t * hc + m] = alpha;
      if (stats != nullptr) stats[t * (hc + 1) + m] = alpha;
    }
    if (stats != nullptr) continue;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + c * nthreads;
      if (ci < cps) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(alpha, vv[c][e], hh[c][e]);
        Chunk<false>::store_nt(h, h_row + (int64_t)m * cps + ci, o);
      }
    }
  }
  if (stats != nullptr && tid == 0) {
    // the value row's partial sums were published before the first barrier
    float svv = 0.f;
    for (int w = 0; w < nwaves; ++w) svv += red[w][kMaxHc][0];
    stats[t * (hc + 1) + hc] = svv * inv_d;
  }
}

}  // namespace

hipError_t engram_launch_gate_sums(const int32_t *ids, EngramDeadRule dead_rule, const void *kv,
                                   void *h, float *gate_out, float *stats, int64_t tokens,
                                   int32_t hc, int32_t dim, float eps, float clamp, int plain,
                                   hipStream_t stream) {
  if (tokens <= 0) return hipSuccess;
  int threads = 0, cpt = 0;
  bool few = false;
  const hipError_t err = gate_threads(tokens, dim, threads, cpt, few);
  if (err != hipSuccess) return err;
#define ENGRAM_GATE_SUMS_CASE(N)                                                              \
  hipLaunchKernelGGL((gate_sums_kernel<N>), dim3((unsigned)tokens), dim3(threads), 0, stream,  \
                     ids, dead_rule, (const uint16_t *)kv, h, gate_out, stats, hc, dim, eps,  \
                     clamp, plain)
  switch (cpt) {
    case 1: ENGRAM_GATE_SUMS_CASE(1); break;
    case 2: ENGRAM_GATE_SUMS_CASE(2); break;
    case 3: ENGRAM_GATE_SUMS_CASE(3); break;
    case 4: ENGRAM_GATE_SUMS_CASE(4); break;
    case 5: ENGRAM_GATE_SUMS_CASE(5); break;
    case 6: ENGRAM_GATE_SUMS_CASE(6); break;
    case 7: ENGRAM_GATE_SUMS_CASE(7); break;
    case 8: ENGRAM_GATE_SUMS_CASE(8); break;
    default:
      return hipErrorInvalidValue;
  }
#undef ENGRAM_GATE_SUMS_CASE
  return hipGetLastError();
}

namespace {

__global__ void fold_kernel(const float4 *__restrict__ q_w, const float4 *__restrict__ k_w,
                            float4 *__restrict__ qk_w, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) {
    const float4 q = q_w[i], k = k_w[i];
    qk_w[i] = make_float4(q.x * k.x, q.y * k.y, q.z * k.z, q.w * k.w);
  }
}

}  // namespace

hipError_t engram_launch_fold_gate_weights(const float *q_w, const float *k_w, float *qk_w,
                                           int32_t hc, int32_t dim, hipStream_t stream) {
  const int64_t n4 = (int64_t)hc * dim / 4;
  if (n4 <= 0) return hipSuccess;
  const int threads = 256;
  hipLaunchKernelGGL(fold_kernel, dim3((unsigned)((n4 + threads - 1) / threads)), dim3(threads), 0,
                     stream, reinterpret_cast<const float4 *>(q_w),
                     reinterpret_cast<const float4 *>(k_w), reinterpret_cast<float4 *>(qk_w), n4);
  return hipGetLastError();
}
