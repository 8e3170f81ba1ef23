// zs_args.h -- argument checks shared by the library's host-side entry
// points (internal; the contract is in include/zero_shard.h).
#ifndef ZS_ARGS_H
#define ZS_ARGS_H

#include <cmath>
#include <cstdint>

#include "zero_shard.h"

namespace zs_args {

// A partition of phi parameters over n_d ranks as zero_shard_init accepts it:
// partition r, or r == 0 over the whole buffer (the unpartitioned update).
inline bool geometry_ok(const zs_desc &d) {
  if (d.n_d < 1 || d.n_d > ZS_MAX_ND || d.r < 0 || d.r >= d.n_d || d.phi < 0) return false;
  const int64_t want = zero_shard_len(d.phi, d.n_d, d.r);
  return d.shard_len == want || (d.r == 0 && d.shard_len == d.phi);
}

// The optimizer's hyper-parameters and the int8 block: beta in [0, 1),
// eps > 0, weight decay >= 0, all finite; bias_correction 0 or 1; a finite
// max_norm; quant_block 0 or one of the supported blocks.
inline bool hyper_ok(const zs_desc &d) {
  if (!(d.beta1 >= 0.0f && d.beta1 < 1.0f && d.beta2 >= 0.0f && d.beta2 < 1.0f)) return false;
  if (!(d.eps > 0.0f) || !std::isfinite(d.eps)) return false;
  if (!(d.weight_decay >= 0.0f) || !std::isfinite(d.weight_decay)) return false;
  if (d.bias_correction != 0 && d.bias_correction != 1) return false;
  if (!std::isfinite(d.max_norm)) return false;
  const int32_t qb = d.quant_block;
  return qb == 0 || qb == 32 || qb == 64 || qb == 128 || qb == 256 || qb == 512;
}

// One step's learning rate and 1-based step counter.
inline bool step_ok(float lr, int64_t t) { return lr >= 0.0f && std::isfinite(lr) && t >= 1; }

}  // namespace zs_args

#endif  // ZS_ARGS_H
