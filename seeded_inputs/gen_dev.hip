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

__global__ void __launch_bounds__(kThreads)
fill_code(int8_t *out, int64_t n, uint64_t h, int64_t i0) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x; j < n; j += stride)
    out[j] = zsg_code(h, uint64_t(i0 + j));
}

// Stands for the time a bucket of inputs takes to arrive over a link whose
// traffic does not touch this GPU's memory: one wave waits on the
// constant-rate wall clock for `ticks`, sleeping between reads.  The loop
// is bounded (at most 2^28 sleeps of 8 x 64 cycles).
__global__ void __launch_bounds__(64) delay_kernel(uint64_t ticks) {
  const uint64_t t0 = wall_clock64();
  for (uint32_t it = 0; it < (1u << 28); ++it) {
    if (wall_clock64() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(8);
  }
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

/* Int8 contributions of one step (see the host build): rank k's codes at
 * codes + k*code_stride, its block scales at scales + k*scale_stride. */
int zsg_dev_fill_contrib_q8(void *codes, void *scales, int32_t n_d, int64_t code_stride,
                            int64_t scale_stride, int64_t n, uint64_t seed, uint32_t step,
                            int64_t i0, int32_t block, float scale_sigma, void *stream) {
  if (n <= 0) return 0;
  if (!codes || !scales || block < 1 || i0 % block) return -1;
  const int64_t b0 = i0 / block;
  const int64_t nb = (i0 + n - 1) / block - b0 + 1;
  for (int32_t k = 0; k < n_d; ++k) {
    const uint64_t hc = zsg_key(seed, ZSG_GRAD, step, uint32_t(k));
    const uint64_t hs = zsg_key(seed, ZSG_GRAD_SCALE, step, uint32_t(k));
    hipLaunchKernelGGL(fill_code, dim3(grid_for(n)), dim3(kThreads), 0, hipStream_t(stream),
                       static_cast<int8_t *>(codes) + k * code_stride, n, hc, i0);
    hipLaunchKernelGGL(fill_f32, dim3(grid_for(nb)), dim3(kThreads), 0, hipStream_t(stream),
                       static_cast<float *>(scales) + k * scale_stride, nb, hs, b0, scale_sigma,
                       0, int(ZSG_KIND_ABS));
    if (hipGetLastError() != hipSuccess) return -4;
  }
  return 0;
}

/* Queue a wait of `usec` microseconds (0 < usec <= 1e6) on `stream`. */
int zsg_dev_delay(double usec, void *stream) {
  if (!(usec > 0.0) || usec > 1e6) return -1;
  int dev = -1, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -4;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    return -4;
  const uint64_t ticks = uint64_t(usec * double(khz) / 1000.0);
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, hipStream_t(stream), ticks);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
