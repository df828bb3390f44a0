// Measurement aid for the benchmark, not part of the layer (libengram_calibrate.so).
//
// A stream of v_mfma_f32_32x32x16_bf16, the projection's instruction (or of
// v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 codes with E8M0 scales, the FP8
// projection's), on operand fragments taken from caller data: one wave per SIMD
// on every CU, 16 independent accumulators per wave, each step's A and B
// fragments cycling through 8 of each held in registers, and no memory traffic
// inside the loop. Its rate is what the chip sustains on those operand bits: on
// constant operands the bf16 stream runs at the published peak, on random ones
// the power limit holds the clock well below it. Taken on the projection's own
// operands, it is the ceiling of any kernel computing that product.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kFrags = 8;

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_stream_kernel(const uint4 *__restrict__ a_src, const uint4 *__restrict__ b_src,
                        int64_t n_frag, float *__restrict__ out, int iters) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a[kFrags], b[kFrags];
#pragma unroll
  for (int i = 0; i < kFrags; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, a_src[(g * kFrags + i) % n_frag]);
    b[i] = __builtin_bit_cast(bf16x8, b_src[(g * kFrags + i) % n_frag]);
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kFrags; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a[(s + i) % kFrags], b[(s + 3 * j) % kFrags], acc[i][j], 0, 0, 0);
  }
  // one value per thread keeps every accumulator live
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) t += acc[i][j][r];
  out[g] = t;
}

// The FP8 stream: 32-byte code fragments (64 E4M3 inputs per lane) and one
// E8M0 scale byte per lane and fragment, both operands scaled.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_fp8_stream_kernel(const i32x8 *__restrict__ a_src, const i32x8 *__restrict__ b_src,
                            int64_t n_frag, const uint8_t *__restrict__ sa_src,
                            const uint8_t *__restrict__ sb_src, int64_t n_scale,
                            float *__restrict__ out, int iters) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  i32x8 a[kFrags], b[kFrags];
  int sa[kFrags], sb[kFrags];
#pragma unroll
  for (int i = 0; i < kFrags; ++i) {
    a[i] = a_src[(g * kFrags + i) % n_frag];
    b[i] = b_src[(g * kFrags + i) % n_frag];
    sa[i] = sa_src[(g * kFrags + i) % n_scale];
    sb[i] = sb_src[(g * kFrags + i) % n_scale];
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kFrags; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[(s + i) % kFrags], b[(s + 3 * j) % kFrags], acc[i][j], 0, 0, 0,
              sa[(s + i) % kFrags], 0, sb[(s + 3 * j) % kFrags]);
  }
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) t += acc[i][j][r];
  out[g] = t;
}

}  // namespace

extern "C" {

// FLOP one FP8 call performs: blocks * 4 waves * iters * 128 MFMAs * 131072.
double engram_calibrate_mfma_fp8_flop(int32_t blocks, int32_t iters) {
  return (double)blocks * 4.0 * (double)iters * 128.0 * 131072.0;
}

// a, b: device, 32-byte aligned, at least n_frag 32-byte fragments of E4M3 codes;
// sa, sb: device, at least n_scale E8M0 bytes; out: device float [blocks * 256].
// Returns 0, -1 on bad arguments, or the HIP error code.
int engram_calibrate_mfma_fp8(const void *a, const void *b, int64_t n_frag, const void *sa,
                              const void *sb, int64_t n_scale, float *out, int32_t blocks,
                              int32_t iters, hipStream_t stream) {
  if (a == nullptr || b == nullptr || sa == nullptr || sb == nullptr || out == nullptr ||
      n_frag < kFrags || n_scale < 1 || blocks < 1 || iters < 1 ||
      ((uintptr_t)a % 32) != 0 || ((uintptr_t)b % 32) != 0)
    return -1;
  hipLaunchKernelGGL(mfma_fp8_stream_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     (const i32x8 *)a, (const i32x8 *)b, n_frag, (const uint8_t *)sa,
                     (const uint8_t *)sb, n_scale, out, iters);
  return (int)hipGetLastError();
}

// FLOP one call performs: blocks * 4 waves * iters * 128 MFMAs * 32768.
double engram_calibrate_mfma_flop(int32_t blocks, int32_t iters) {
  return (double)blocks * 4.0 * (double)iters * 128.0 * 32768.0;
}

// a, b: device, 16-byte aligned, at least n_frag 16-byte fragments of bf16 each
// (a for the first MFMA operand, b for the second); out: device float
// [blocks * 256]. Returns 0, -1 on bad arguments, or the HIP error code.
int engram_calibrate_mfma_bf16(const void *a, const void *b, int64_t n_frag, float *out,
                               int32_t blocks, int32_t iters, hipStream_t stream) {
  if (a == nullptr || b == nullptr || out == nullptr || n_frag < kFrags || blocks < 1 ||
      iters < 1 || ((uintptr_t)a % 16) != 0 || ((uintptr_t)b % 16) != 0)
    return -1;
  hipLaunchKernelGGL(mfma_stream_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     (const uint4 *)a, (const uint4 *)b, n_frag, out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
