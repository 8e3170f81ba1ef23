// zs_host.h -- internal to the library (not part of the C ABI): the host
// update of zero_shard_host_step with optional per-chunk hooks, through
// which the offload pipeline streams its copies around the update.

#pragma once

#include <cstdint>

#include "zero_shard.h"

namespace zs_host {

// Hooks around the update's chunks of `chunk` shard elements (a multiple of
// 2^18, the update's own work unit): ready(ctx, c) returns once chunk c's
// averaged gradient is in host memory (nonzero: an error, and the update
// stops taking chunks); done(ctx, c) is called once, by one thread, when
// every output of chunk c (master, m, v, the bf16 copy, int8 codes and
// scales) has been written.  Both are called from the update's threads.
struct Hooks {
  int64_t chunk;
  void *ctx;
  int (*ready)(void *ctx, int64_t c);
  int (*done)(void *ctx, int64_t c);
};

// zero_shard_host_step's update; with hooks (may be null) the chunks are
// gated and reported as above.  Returns ZS_EHIP when a hook failed.
__attribute__((visibility("hidden"))) int step(const zs_desc *d, const float *gbar, float lr,
                                               int64_t t, double global_sumsq, int32_t threads,
                                               const Hooks *hooks);

}  // namespace zs_host
