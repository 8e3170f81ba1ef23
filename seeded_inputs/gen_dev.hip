/*
 * gen_dev.hip -- device build of the seeded input generator (zs_gen.h).
 * Fills HBM with windows of keyed tensors, bit-identical to the host build.
 * Not part of the shard-step library: it only prepares inputs.
 */
#include <hip/hip_runtime.h>

#include "zs_gen.h"

namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
fill_f32(float *out, int64_t n, uint64_t h, int64_t i0, float sigma, int outliers, int kind) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x; j < n; j += stride)
    out[j] = zsg_value(h, uint64_t(i0 + j), sigma, outliers, kind);
}

__global__ void __launch_bounds__(kThreads)
fill_bf16(uint16_t *out, int64_t n, uint64_t h, int64_t i0, float sigma, int outliers) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x; j < n; j += stride)
    out[j] = zsg_to_bf16(zsg_value(h, uint64_t(i0 + j), sigma, outliers, ZSG_KIND_NORMAL));
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + kThreads - 1) / kThreads;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return unsigned(b);
}

}  // namespace

extern "C" {

int zsg_dev_fill_f32(void *out, int64_t n, uint64_t seed, uint32_t tid, uint32_t step,
                     uint32_t rank, int64_t i0, float sigma, int outliers, int kind,
                     void *stream) {
  if (n <= 0) return 0;
  if (!out) return -1;
  const uint64_t h = zsg_key(seed, tid, step, rank);
  hipLaunchKernelGGL(fill_f32, dim3(grid_for(n)), dim3(kThreads), 0, hipStream_t(stream),
                     static_cast<float *>(out), n, h, i0, sigma, outliers, kind);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int zsg_dev_fill_bf16(void *out, int64_t n, uint64_t seed, uint32_t tid, uint32_t step,
                      uint32_t rank, int64_t i0, float sigma, int outliers, void *stream) {
  if (n <= 0) return 0;
  if (!out) return -1;
  const uint64_t h = zsg_key(seed, tid, step, rank);
  hipLaunchKernelGGL(fill_bf16, dim3(grid_for(n)), dim3(kThreads), 0, hipStream_t(stream),
                     static_cast<uint16_t *>(out), n, h, i0, sigma, outliers);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

/* Gradient contributions of one step: row k (rank k) of n elements at
 * out + k*row_stride (elements), shard-local indices [i0, i0+n). */
int zsg_dev_fill_contrib(void *out, int32_t n_d, int64_t row_stride, int64_t n,
                         uint64_t seed, uint32_t step, int64_t i0, float sigma,
                         int outliers, void *stream) {
  for (int32_t k = 0; k < n_d; ++k) {
    const int rc = zsg_dev_fill_bf16(static_cast<uint16_t *>(out) + k * row_stride, n, seed,
                                     ZSG_GRAD, step, uint32_t(k), i0, sigma, outliers, stream);
    if (rc) return rc;
  }
  return 0;
}

}  // extern "C"
