// zero_shard_host.cpp -- the library's host-only code (declared in
// include/zero_shard.h): the ZeRO-Offload host step zero_shard_host_step,
// and the partition geometry zero_shard_len.
//
// ZeRO-Offload keeps the optimizer states in host memory and runs the
// update on the CPU ("ZeRO (딥 러닝)", follow-ups table "후속 기법":
// optimizer states and the update moved to CPU memory and the CPU, with an
// optimized CPU Adam and a one-step delayed update).  This is that CPU
// update for one rank's shard: a3 + a4 (+ a5) from the averaged gradient
// the GPU produced (the norm pass's fp32 spill, copied to the host), with
// exactly the arithmetic of the GPU step -- binary64 from the binary32
// state, each stored value rounded once, IEEE division and square root --
// so an offloaded step and an on-device step give the same bits.
//
// Built with g++ -O3 -march=x86-64-v3 -ffp-contract=off -fno-math-errno:
// the element loop vectorizes to binary64 AVX2, or AVX-512 where the host
// has it (vdivpd and vsqrtpd are correctly rounded, no contraction, so both
// give the same bits), and the shard is split over a pool of host threads
// that take contiguous, quantizer-block-aligned chunks in turn.

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <memory>
#include <new>
#include <thread>
#include <vector>

#include "zero_shard.h"
#include "zs_args.h"
#include "zs_host.h"

namespace {

struct HostConst {
  double b1, omb1, b2, omb2, bc1, bc2, lr, decay, eps, coef;
};

// Nearest-even bf16 of a binary32 (bias-and-truncate form); NaN stays NaN.
inline uint16_t to_bf16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

inline float from_bf16(uint16_t b) {
  const uint32_t u = uint32_t(b) << 16;
  float x;
  std::memcpy(&x, &u, sizeof x);
  return x;
}

// a3 + a4 over elements [lo, hi): the same expression, in the same order, as
// the device step.  Inlined into one body per instruction set below.
__attribute__((always_inline)) inline void adam_range_body(
    const float *__restrict gbar, float *__restrict th, float *__restrict mo,
    float *__restrict va, uint16_t *__restrict p, int64_t lo, int64_t hi, const HostConst &k) {
  for (int64_t i = lo; i < hi; ++i) {
    const double g = k.coef * static_cast<double>(gbar[i]);
    const double m1 = k.b1 * static_cast<double>(mo[i]) + k.omb1 * g;
    const double v1 = k.b2 * static_cast<double>(va[i]) + k.omb2 * (g * g);
    const double mhat = m1 / k.bc1;
    const double vhat = v1 / k.bc2;
    const double t0 = static_cast<double>(th[i]);
    const double t1 = t0 - k.decay * t0 - k.lr * mhat / (std::sqrt(vhat) + k.eps);
    mo[i] = static_cast<float>(m1);
    va[i] = static_cast<float>(v1);
    th[i] = static_cast<float>(t1);
  }
  for (int64_t i = lo; i < hi; ++i) p[i] = to_bf16(th[i]);
}

// a5 over blocks [b_lo, b_hi) of a shard of n elements.  The block absmax is
// taken on the bf16 bit patterns: with the sign cleared, the order of the
// patterns is the order of the magnitudes, any pattern above 0x7f80 is a NaN
// (and then the scale is NaN and every code 0), 0x7f80 is infinity.
__attribute__((always_inline)) inline void quant_blocks_body(
    const uint16_t *__restrict p, int8_t *__restrict codes, float *__restrict scales,
    int64_t b_lo, int64_t b_hi, int64_t n, int64_t block) {
  for (int64_t b = b_lo; b < b_hi; ++b) {
    const int64_t lo = b * block, hi = lo + block < n ? lo + block : n;
    uint16_t amax = 0;
    for (int64_t i = lo; i < hi; ++i) {
      const uint16_t a = p[i] & 0x7fffu;
      amax = a > amax ? a : amax;
    }
    const float a = amax > 0x7f80u ? std::numeric_limits<float>::quiet_NaN() : from_bf16(amax);
    const float s = a / 127.0f;
    scales[b] = s;
    if (!(s != 0.0f) || s != s) {  // zero block, or a NaN in it: all codes 0
      for (int64_t i = lo; i < hi; ++i) codes[i] = 0;
      continue;
    }
    for (int64_t i = lo; i < hi; ++i) {
      float r = from_bf16(p[i]) / s;
      // |r| <= 127 (1 + 2^-24) for finite p; inf / inf is NaN and inf / s
      // (s infinite only with an infinite element) cannot happen when s is
      // finite -- both non-finite cases give code 0
      r = (r - r == 0.0f) ? std::nearbyint(r) : 0.0f;  // default mode: ties to even
      r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
      codes[i] = static_cast<int8_t>(static_cast<int>(r));
    }
  }
}

void adam_range_avx2(const float *gbar, float *th, float *mo, float *va, uint16_t *p, int64_t lo,
                     int64_t hi, const HostConst &k) {
  adam_range_body(gbar, th, mo, va, p, lo, hi, k);
}
void quant_blocks_avx2(const uint16_t *p, int8_t *codes, float *scales, int64_t b_lo,
                       int64_t b_hi, int64_t n, int64_t block) {
  quant_blocks_body(p, codes, scales, b_lo, b_hi, n, block);
}

#define ZS_AVX512 __attribute__((target("avx512f,avx512vl,avx512bw,avx512dq")))
ZS_AVX512 void adam_range_avx512(const float *gbar, float *th, float *mo, float *va, uint16_t *p,
                                 int64_t lo, int64_t hi, const HostConst &k) {
  adam_range_body(gbar, th, mo, va, p, lo, hi, k);
}
ZS_AVX512 void quant_blocks_avx512(const uint16_t *p, int8_t *codes, float *scales, int64_t b_lo,
                                   int64_t b_hi, int64_t n, int64_t block) {
  quant_blocks_body(p, codes, scales, b_lo, b_hi, n, block);
}

// The 512-bit bodies where the host has them (same IEEE operations, so the
// same bits), else the 256-bit ones.
bool have_avx512() {
  static const bool yes = __builtin_cpu_supports("avx512f") &&
                          __builtin_cpu_supports("avx512vl") &&
                          __builtin_cpu_supports("avx512bw") &&
                          __builtin_cpu_supports("avx512dq");
  return yes;
}

}  // namespace

// Partition geometry (declared in include/zero_shard.h): ceil(phi / n_d)
// elements per rank, the last partitions shorter or empty.
extern "C" int64_t zero_shard_len(int64_t phi, int32_t n_d, int32_t r) {
  if (phi < 0 || n_d < 1 || r < 0 || r >= n_d) return -1;
  const int64_t per = phi / n_d + (phi % n_d != 0);
  const int64_t rest = phi - int64_t(r) * per;
  if (rest <= 0) return 0;
  return rest < per ? rest : per;
}

int zs_host::step(const zs_desc *d, const float *gbar, float lr, int64_t t, double global_sumsq,
                  int32_t threads, const Hooks *hooks) {
  if (!d) return ZS_EINVAL;
  if (!zs_args::geometry_ok(*d) || !zs_args::hyper_ok(*d) || !zs_args::step_ok(lr, t))
    return ZS_EINVAL;
  const int32_t qb = d->quant_block;
  const int64_t n = d->shard_len;
  if (n == 0) return ZS_OK;
  if (!gbar || !d->master || !d->m || !d->v || !d->param_out) return ZS_EINVAL;
  if (qb && (!d->q_codes || !d->q_scales)) return ZS_EINVAL;

  HostConst k;
  const double b1 = d->beta1, b2 = d->beta2;
  k.b1 = b1;
  k.omb1 = 1.0 - b1;
  k.b2 = b2;
  k.omb2 = 1.0 - b2;
  k.bc1 = d->bias_correction ? 1.0 - std::pow(b1, double(t)) : 1.0;
  k.bc2 = d->bias_correction ? 1.0 - std::pow(b2, double(t)) : 1.0;
  k.lr = double(lr);
  k.decay = double(lr) * double(d->weight_decay);
  k.eps = double(d->eps);
  k.coef = 1.0;
  if (d->max_norm > 0.0f) {
    const double c = double(d->max_norm) / (std::sqrt(global_sumsq) + 1e-6);
    k.coef = (c != c) ? c : (c < 1.0 ? c : 1.0);
  }

  // Chunks of kChunk elements (a multiple of every quantizer block, so each
  // block is quantized by the thread that produced its bf16 values), handed
  // out in order from a shared counter: a thread that the host deschedules
  // (the cores are shared with the HIP runtime's copy threads when the
  // update runs inside the offload pipeline) holds up one chunk, not a
  // fixed 1/threads of the shard.  Every element's arithmetic is its own,
  // so the split changes no bit.
  constexpr int64_t kChunk = int64_t(1) << 18;
  static_assert(kChunk % 512 == 0, "chunks hold whole quantizer blocks");
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  int64_t nt = threads < 1 ? 1 : threads;
  const int64_t min_piece = int64_t(1) << 16;
  if (nt > (n + min_piece - 1) / min_piece) nt = (n + min_piece - 1) / min_piece;
  if (nt > nchunks) nt = nchunks;
  const bool wide = have_avx512() && std::getenv("ZS_HOST_NO_AVX512") == nullptr;
  auto work = [&](int64_t lo, int64_t hi) {
    const int64_t b_lo = qb ? lo / qb : 0, b_hi = qb ? (hi + qb - 1) / qb : 0;
    if (wide) {
      adam_range_avx512(gbar, d->master, d->m, d->v, d->param_out, lo, hi, k);
      if (qb) quant_blocks_avx512(d->param_out, d->q_codes, d->q_scales, b_lo, b_hi, n, qb);
    } else {
      adam_range_avx2(gbar, d->master, d->m, d->v, d->param_out, lo, hi, k);
      if (qb) quant_blocks_avx2(d->param_out, d->q_codes, d->q_scales, b_lo, b_hi, n, qb);
    }
  };
  // with hooks: hook chunk h covers update chunks [h*per, (h+1)*per); left[h]
  // counts its update chunks still to finish, and the thread that finishes
  // the last one reports it
  const int64_t per = hooks ? hooks->chunk / kChunk : 1;
  const int64_t nhook = hooks ? (nchunks + per - 1) / per : 0;
  std::unique_ptr<std::atomic<int64_t>[]> left;
  if (hooks) {
    if (hooks->chunk < kChunk || hooks->chunk % kChunk) return ZS_EINVAL;
    left.reset(new (std::nothrow) std::atomic<int64_t>[nhook]);
    if (!left) return ZS_ENOMEM;
    for (int64_t h = 0; h < nhook; ++h)
      left[h].store(nchunks - h * per < per ? nchunks - h * per : per, std::memory_order_relaxed);
  }
  std::atomic<int64_t> next{0};
  std::atomic<int> failed{0};
  auto run = [&]() {
    int64_t seen = -1;  // the last hook chunk this thread saw ready (chunks come in order)
    for (int64_t c = next.fetch_add(1, std::memory_order_relaxed);
         c < nchunks && !failed.load(std::memory_order_relaxed);
         c = next.fetch_add(1, std::memory_order_relaxed)) {
      const int64_t h = c / per;
      if (hooks && h > seen) {
        if (hooks->ready(hooks->ctx, h)) {
          failed.store(1);
          break;
        }
        seen = h;
      }
      const int64_t lo = c * kChunk;
      work(lo, lo + kChunk < n ? lo + kChunk : n);
      if (hooks && left[h].fetch_sub(1, std::memory_order_acq_rel) == 1 &&
          hooks->done(hooks->ctx, h))
        failed.store(1);
    }
  };
  std::vector<std::thread> pool;
  for (int64_t i = 1; i < nt; ++i) {
    try {
      pool.emplace_back(run);
    } catch (...) {  // no thread to be had: the running ones take its chunks
      break;
    }
  }
  run();
  for (auto &th : pool) th.join();
  return failed.load() ? ZS_EHIP : ZS_OK;
}

extern "C" int zero_shard_host_step(const zs_desc *d, const float *gbar, float lr, int64_t t,
                                    double global_sumsq, int32_t threads) {
  return zs_host::step(d, gbar, lr, t, global_sumsq, threads, nullptr);
}
