/*
 * gen_host.cpp -- host build of the seeded input generator (zs_gen.h).
 * Fills host arrays with windows [i0, i0+n) of a keyed tensor.  Threads
 * split the window into contiguous pieces; every element depends only on
 * its key and index, so the thread count does not change the values.
 */
#include <thread>
#include <vector>

#include "zs_gen.h"

namespace {

template <class F>
void parallel(int64_t n, int threads, F body) {
  if (threads < 1) threads = 1;
  const int64_t min_piece = 1 << 16;
  if (n < min_piece * 2 || threads == 1) {
    body(0, n);
    return;
  }
  if (threads > n / min_piece) threads = int(n / min_piece);
  std::vector<std::thread> pool;
  const int64_t piece = (n + threads - 1) / threads;
  for (int w = 0; w < threads; ++w) {
    const int64_t lo = w * piece;
    const int64_t hi = lo + piece < n ? lo + piece : n;
    if (lo >= hi) break;
    pool.emplace_back([=] { body(lo, hi); });
  }
  for (auto &t : pool) t.join();
}

}  // namespace

extern "C" {

uint64_t zsg_host_key(uint64_t seed, uint32_t tid, uint32_t step, uint32_t rank) {
  return zsg_key(seed, tid, step, rank);
}

void zsg_host_fill_f32(float *out, int64_t n, uint64_t seed, uint32_t tid,
                       uint32_t step, uint32_t rank, int64_t i0, float sigma,
                       int outliers, int kind, int threads) {
  const uint64_t h = zsg_key(seed, tid, step, rank);
  parallel(n, threads, [=](int64_t lo, int64_t hi) {
    for (int64_t j = lo; j < hi; ++j)
      out[j] = zsg_value(h, uint64_t(i0 + j), sigma, outliers, kind);
  });
}

void zsg_host_fill_bf16(uint16_t *out, int64_t n, uint64_t seed, uint32_t tid,
                        uint32_t step, uint32_t rank, int64_t i0, float sigma,
                        int outliers, int threads) {
  const uint64_t h = zsg_key(seed, tid, step, rank);
  parallel(n, threads, [=](int64_t lo, int64_t hi) {
    for (int64_t j = lo; j < hi; ++j)
      out[j] = zsg_to_bf16(zsg_value(h, uint64_t(i0 + j), sigma, outliers, ZSG_KIND_NORMAL));
  });
}

/* Rows k = 0..n_d-1 of one step's gradient contributions, row k at
 * out + k*row_stride, elements [i0, i0+n) of each rank's shard slice.
 * With many rows the threads take whole rows; with few, each row is split. */
void zsg_host_fill_contrib(uint16_t *out, int32_t n_d, int64_t row_stride,
                           int64_t n, uint64_t seed, uint32_t step, int64_t i0,
                           float sigma, int outliers, int threads) {
  if (threads < 1) threads = 1;
  if (n_d >= threads || n < (int64_t(1) << 17)) {
    const int t = threads < n_d ? threads : n_d;
    std::vector<std::thread> pool;
    for (int w = 0; w < t; ++w)
      pool.emplace_back([=] {
        for (int32_t k = w; k < n_d; k += t)
          zsg_host_fill_bf16(out + k * row_stride, n, seed, ZSG_GRAD, step, uint32_t(k), i0,
                             sigma, outliers, 1);
      });
    for (auto &th : pool) th.join();
    return;
  }
  for (int32_t k = 0; k < n_d; ++k)
    zsg_host_fill_bf16(out + k * row_stride, n, seed, ZSG_GRAD, step, uint32_t(k), i0, sigma,
                       outliers, threads);
}

/* Int8 contributions of one step: codes of rank k at codes + k*code_stride
 * (elements [i0, i0+n) of the shard), and the scales of the blocks those
 * elements fall in, blocks [i0/block, (i0+n-1)/block], at scales +
 * k*scale_stride.  i0 must be a multiple of block. */
void zsg_host_fill_contrib_q8(int8_t *codes, float *scales, int32_t n_d, int64_t code_stride,
                              int64_t scale_stride, int64_t n, uint64_t seed, uint32_t step,
                              int64_t i0, int32_t block, float scale_sigma, int threads) {
  const int64_t b0 = i0 / block;
  const int64_t nb = n > 0 ? (i0 + n - 1) / block - b0 + 1 : 0;
  if (threads < 1) threads = 1;
  const int t = threads < n_d ? threads : n_d;
  std::vector<std::thread> pool;
  for (int w = 0; w < t; ++w)
    pool.emplace_back([=] {
      for (int32_t k = w; k < n_d; k += t) {
        const uint64_t hc = zsg_key(seed, ZSG_GRAD, step, uint32_t(k));
        const uint64_t hs = zsg_key(seed, ZSG_GRAD_SCALE, step, uint32_t(k));
        int8_t *c = codes + k * code_stride;
        float *sc = scales + k * scale_stride;
        for (int64_t j = 0; j < n; ++j) c[j] = zsg_code(hc, uint64_t(i0 + j));
        for (int64_t b = 0; b < nb; ++b)
          sc[b] = zsg_value(hs, uint64_t(b0 + b), scale_sigma, 0, ZSG_KIND_ABS);
      }
    });
  for (auto &th : pool) th.join();
}

}  // extern "C"
