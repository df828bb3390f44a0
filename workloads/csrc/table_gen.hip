// Device twin of the counter-based table generator in workloads/gen.py
// (table_rows). Byte b of row r is derived from the SplitMix64 state
// seed + (r * 264 + b + 1) * 0x9E3779B97F4A7C15 (Steele, Lea & Flood,
// OOPSLA 2014) through its output finaliser; payload bytes map a draw
// u in [0, 254) to the E4M3 codes other than 0x7F and 0xFF, scale bytes are
// 120 + u for u in [0, 15). Input generation only: nothing of the layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t gen_byte(uint64_t seed, uint64_t row, uint32_t b) {
  const uint64_t ctr = row * 264ull + b + 1ull;
  const uint64_t hi = mix64(seed + ctr * 0x9E3779B97F4A7C15ull) >> 32;
  if (b < 256) {
    const uint32_t u = (uint32_t)((hi * 254ull) >> 32);
    return u + (u >= 127u ? 1u : 0u);
  }
  return 120u + (uint32_t)((hi * 15ull) >> 32);
}

// One thread per 8-byte word of a row (33 words per 264-byte row).
__global__ void fill_table_kernel(uint8_t *__restrict__ dst, int64_t rows, int64_t row_begin,
                                  uint64_t seed) {
  const int64_t words = rows * 33;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = w / 33;
    const uint32_t b0 = (uint32_t)(w - r * 33) * 8u;
    const uint64_t row = (uint64_t)(row_begin + r);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= gen_byte(seed, row, b0 + i) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= gen_byte(seed, row, b0 + 4 + i) << (8 * i);
    *reinterpret_cast<uint2 *>(dst + w * 8) = make_uint2(lo, hi);
  }
}

}  // namespace

// Fills dst (device, 8-byte aligned, rows * 264 bytes) with rows
// [row_begin, row_begin + rows) of the table of `seed`. Returns a hipError_t.
extern "C" int workloads_fill_table(void *dst, int64_t rows, int64_t row_begin, uint64_t seed,
                                    hipStream_t stream) {
  if (rows <= 0) return 0;
  if (dst == nullptr || ((uintptr_t)dst & 7) != 0 || row_begin < 0) return (int)hipErrorInvalidValue;
  const int threads = 256;
  const int64_t words = rows * 33;
  int64_t blocks = (words + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_table_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (uint8_t *)dst, rows, row_begin, seed);
  return (int)hipGetLastError();
}
