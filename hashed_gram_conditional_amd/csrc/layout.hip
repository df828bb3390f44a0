// Re-layout of caller buffers: a tiled transpose, so that weights held with the
// other dimension innermost (the wkv matrix as [inputs, outputs], the gate
// scales as [dim, hc]) can be turned once into the layout the kernels read.
// Not on the per-step path.
#include "common.h"

namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;

// Each block moves one 64 x 64 tile through LDS: reads along the source rows,
// writes along the destination rows (dst_ld elements apart), both coalesced. The extra column keeps
// the transposed LDS reads off a single bank.
template <typename T>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const T *__restrict__ src,
                                                             T *__restrict__ dst, int64_t rows,
                                                             int64_t cols, int64_t dst_ld,
                                                             int64_t tiles_c) {
  __shared__ T tile[kTile][kTile + 1];
  const int64_t b = blockIdx.x;
  const int64_t tr = b / tiles_c;
  const int64_t r0 = tr * kTile, c0 = (b - tr * tiles_c) * kTile;
  const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
  for (int i = ty; i < kTile; i += kThreads / kTile) {
    const int64_t r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < kTile; i += kThreads / kTile) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) dst[c * dst_ld + r] = tile[tx][i];
  }
}

}  // namespace

hipError_t engram_launch_transpose(const void *src, void *dst, int64_t rows, int64_t cols,
                                   int64_t dst_ld, int elem_bytes, hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t tiles_c = (cols + kTile - 1) / kTile;
  const int64_t blocks = ((rows + kTile - 1) / kTile) * tiles_c;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, (const uint16_t *)src, (uint16_t *)dst, rows, cols, dst_ld,
                       tiles_c);
  else
    hipLaunchKernelGGL(transpose_kernel<uint32_t>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, (const uint32_t *)src, (uint32_t *)dst, rows, cols, dst_ld,
                       tiles_c);
  return hipGetLastError();
}
