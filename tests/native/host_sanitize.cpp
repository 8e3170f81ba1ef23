// host_sanitize.cpp -- CPU test driver for the host-only library code and
// the oracle under AddressSanitizer / UndefinedBehaviorSanitizer or
// ThreadSanitizer (built and run by tests/test_host_sanitize.py with g++).
//
// For ragged shard lengths, every quantizer block, clipping on and off and
// 1..5 threads it runs three steps of the oracle (orc_step) and of the
// ZeRO-Offload host update (zero_shard_host_step, fed the oracle's averaged
// gradient and S) on the same seeded inputs and requires identical bits.
// It also runs the update with the per-chunk hooks the offload pipeline
// streams its copies through (zs_host::step): each chunk's gradient lands
// only when the chunk is first reported ready, every chunk is reported done
// exactly once with its final outputs, and the bits equal the update
// without hooks.
// Exit status 0 when every case matches.
#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "zero_shard.h"
#include "zs_host.h"
#include "zs_oracle.h"

namespace {

uint16_t bf16_rne(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

double f32(double x) { return double(float(x)); }

struct Case {
  int64_t n;
  int32_t nd, qb;
  float clip;
  int32_t threads;
};

// An empty shard: the host update accepts it and touches nothing.
bool run_empty(const Case &c) {
  zs_desc d;
  std::memset(&d, 0, sizeof d);
  d.phi = 3;
  d.n_d = c.nd;
  d.r = c.nd - 1;  // ceil(3 / n_d) per rank leaves the last rank empty
  d.shard_len = zero_shard_len(d.phi, d.n_d, d.r);
  d.beta1 = 0.9f;
  d.beta2 = 0.999f;
  d.eps = 1e-8f;
  d.bias_correction = 1;
  d.max_norm = c.clip;
  d.quant_block = c.qb;
  return d.shard_len == 0 && zero_shard_host_step(&d, nullptr, 1e-3f, 1, 0.0, c.threads) == ZS_OK;
}

bool run(const Case &c, std::mt19937_64 &rng) {
  if (c.n == 0) return run_empty(c);
  std::normal_distribution<float> g(0.0f, 1e-3f), w(0.0f, 0.02f);
  const int64_t n = c.n;
  std::vector<float> th(n), mo(n, 0.0f), va(n, 0.0f);
  for (auto &x : th) x = w(rng);
  std::vector<float> th2 = th, mo2 = mo, va2 = va;
  const int64_t nb = c.qb ? (n + c.qb - 1) / c.qb : 0;
  std::vector<uint16_t> p1(n), p2(n);
  std::vector<int8_t> q1(n), q2(n);
  std::vector<float> s1(nb), s2(nb), gbar(n);
  const float lr = 1e-3f, b1 = 0.9f, b2 = 0.999f, eps = 1e-8f, wd = 0.1f;
  zs_desc d;
  std::memset(&d, 0, sizeof d);
  d.phi = n;
  d.n_d = c.nd;
  d.r = 0;
  d.shard_len = n;
  d.beta1 = b1;
  d.beta2 = b2;
  d.eps = eps;
  d.weight_decay = wd;
  d.bias_correction = 1;
  d.max_norm = c.clip;
  d.quant_block = c.qb;
  d.master = th2.data();
  d.m = mo2.data();
  d.v = va2.data();
  d.param_out = p2.data();
  d.q_codes = c.qb ? q2.data() : nullptr;
  d.q_scales = c.qb ? s2.data() : nullptr;
  for (int64_t t = 1; t <= 3; ++t) {
    std::vector<std::vector<uint16_t>> rows(c.nd, std::vector<uint16_t>(n));
    std::vector<const uint16_t *> rp(c.nd);
    for (int k = 0; k < c.nd; ++k) {
      for (auto &x : rows[k]) x = bf16_rne(g(rng));
      rp[k] = rows[k].data();
    }
    orc_hyper h;
    std::memset(&h, 0, sizeof h);
    h.lr = f32(lr);
    h.beta1 = f32(b1);
    h.beta2 = f32(b2);
    h.eps = f32(eps);
    h.weight_decay = f32(wd);
    h.bias_correction = 1;
    h.quant_block = c.qb;
    h.t = t;
    h.max_norm = f32(c.clip);
    h.s_other = 0.0;
    double sumsq = 0.0;
    if (orc_step(rp.data(), c.nd, n, th.data(), mo.data(), va.data(), p1.data(),
                 c.qb ? q1.data() : nullptr, c.qb ? s1.data() : nullptr, &h, &sumsq,
                 c.threads) != 0)
      return false;
    const double S = orc_gbar_sumsq(rp.data(), c.nd, n, gbar.data(), c.threads);
    if (zero_shard_host_step(&d, gbar.data(), lr, t, S, c.threads) != ZS_OK) return false;
  }
  const bool same = std::memcmp(th.data(), th2.data(), n * 4) == 0 &&
                    std::memcmp(mo.data(), mo2.data(), n * 4) == 0 &&
                    std::memcmp(va.data(), va2.data(), n * 4) == 0 &&
                    std::memcmp(p1.data(), p2.data(), n * 2) == 0 &&
                    (!c.qb || (std::memcmp(q1.data(), q2.data(), n) == 0 &&
                               std::memcmp(s1.data(), s2.data(), nb * 4) == 0));
  return same;
}

// The hooks' view of one run: the real gradient is copied into the update's
// gradient buffer (poisoned with NaN until then) chunk by chunk, once, when
// the chunk is first reported ready.
struct HookRun {
  int64_t n, chunk;
  const float *grad;  // the gradient to land
  float *landing;     // the buffer the update reads
  const float *ref_master;
  const float *master;
  std::once_flag landed[64];
  std::atomic<int> done[64];
  std::atomic<int> bad{0};
  int64_t fail_at = -1;  // a ready hook that reports an error
};

int hook_ready(void *ctx, int64_t h) {
  HookRun *r = static_cast<HookRun *>(ctx);
  if (h == r->fail_at) return 1;
  std::call_once(r->landed[h], [r, h] {
    const int64_t lo = h * r->chunk, hi = lo + r->chunk < r->n ? lo + r->chunk : r->n;
    std::memcpy(r->landing + lo, r->grad + lo, size_t(hi - lo) * 4);
  });
  return 0;
}

int hook_done(void *ctx, int64_t h) {
  HookRun *r = static_cast<HookRun *>(ctx);
  const int64_t lo = h * r->chunk, hi = lo + r->chunk < r->n ? lo + r->chunk : r->n;
  if (r->done[h].fetch_add(1) != 0 ||
      std::memcmp(r->master + lo, r->ref_master + lo, size_t(hi - lo) * 4) != 0)
    r->bad.store(1);
  return 0;
}

bool run_hooks(int64_t n, int64_t chunk, int32_t qb, float clip, int32_t threads,
               std::mt19937_64 &rng) {
  std::normal_distribution<float> g(0.0f, 1e-3f), w(0.0f, 0.02f);
  std::vector<float> grad(n), th(n), mo(n), va(n);
  for (int64_t i = 0; i < n; ++i) {
    grad[i] = g(rng);
    th[i] = w(rng);
    mo[i] = 1e-4f * g(rng);
    va[i] = std::fabs(1e-3f * g(rng));
  }
  const int64_t nb = qb ? (n + qb - 1) / qb : 0;
  zs_desc d;
  std::memset(&d, 0, sizeof d);
  d.phi = n;
  d.n_d = 1;
  d.shard_len = n;
  d.beta1 = 0.9f;
  d.beta2 = 0.999f;
  d.eps = 1e-8f;
  d.weight_decay = 0.1f;
  d.bias_correction = 1;
  d.max_norm = clip;
  d.quant_block = qb;
  const double S = 3.0;
  // reference: the update without hooks
  std::vector<float> th1 = th, mo1 = mo, va1 = va, s1(nb);
  std::vector<uint16_t> p1(n);
  std::vector<int8_t> q1(n);
  d.master = th1.data();
  d.m = mo1.data();
  d.v = va1.data();
  d.param_out = p1.data();
  d.q_codes = qb ? q1.data() : nullptr;
  d.q_scales = qb ? s1.data() : nullptr;
  if (zero_shard_host_step(&d, grad.data(), 1e-3f, 7, S, threads) != ZS_OK) return false;
  // with hooks, on a gradient buffer that holds NaN until each chunk lands
  std::vector<float> th2 = th, mo2 = mo, va2 = va, s2(nb), landing(n, std::nanf(""));
  std::vector<uint16_t> p2(n);
  std::vector<int8_t> q2(n);
  d.master = th2.data();
  d.m = mo2.data();
  d.v = va2.data();
  d.param_out = p2.data();
  d.q_codes = qb ? q2.data() : nullptr;
  d.q_scales = qb ? s2.data() : nullptr;
  HookRun r;
  r.n = n;
  r.chunk = chunk;
  r.grad = grad.data();
  r.landing = landing.data();
  r.ref_master = th1.data();
  r.master = th2.data();
  for (auto &x : r.done) x.store(0);
  const zs_host::Hooks hooks{chunk, &r, hook_ready, hook_done};
  if (zs_host::step(&d, landing.data(), 1e-3f, 7, S, threads, &hooks) != ZS_OK) return false;
  const int64_t nh = (n + chunk - 1) / chunk;
  for (int64_t h = 0; h < nh; ++h)
    if (r.done[h].load() != 1) return false;
  if (r.bad.load()) return false;
  const bool same = std::memcmp(th1.data(), th2.data(), n * 4) == 0 &&
                    std::memcmp(mo1.data(), mo2.data(), n * 4) == 0 &&
                    std::memcmp(va1.data(), va2.data(), n * 4) == 0 &&
                    std::memcmp(p1.data(), p2.data(), n * 2) == 0 &&
                    (!qb || (std::memcmp(q1.data(), q2.data(), n) == 0 &&
                             std::memcmp(s1.data(), s2.data(), nb * 4) == 0));
  if (!same) return false;
  // a hook chunk that is not a whole number of the update's chunks is refused
  const zs_host::Hooks odd{chunk + 512, &r, hook_ready, hook_done};
  if (zs_host::step(&d, landing.data(), 1e-3f, 8, S, threads, &odd) != ZS_EINVAL) return false;
  // a ready hook that fails stops the update with ZS_EHIP
  if (nh > 1) {
    HookRun f;
    f.n = n;
    f.chunk = chunk;
    f.grad = grad.data();
    f.landing = landing.data();
    f.ref_master = th1.data();
    f.master = th2.data();
    f.fail_at = 1;
    for (auto &x : f.done) x.store(0);
    const zs_host::Hooks fh{chunk, &f, hook_ready, hook_done};
    if (zs_host::step(&d, landing.data(), 1e-3f, 9, S, threads, &fh) != ZS_EHIP) return false;
  }
  return true;
}

}  // namespace

int main() {
  std::mt19937_64 rng(20261202);
  const Case cases[] = {
      {0, 4, 256, 1.0f, 2},        {1, 1, 0, 0.0f, 1},          {7, 3, 32, 0.0f, 2},
      {1000, 4, 64, 0.05f, 3},     {100003, 8, 256, 1.0f, 5},   {196625, 16, 512, 0.01f, 4},
      {131072, 2, 128, 0.0f, 3},   {65537, 64, 256, 0.02f, 2},
  };
  int bad = 0;
  for (const Case &c : cases) {
    const bool ok = run(c, rng);
    std::printf("n=%lld nd=%d qb=%d clip=%g threads=%d: %s\n", (long long)c.n, c.nd, c.qb,
                double(c.clip), c.threads, ok ? "ok" : "MISMATCH");
    bad += !ok;
  }
  const struct {
    int64_t n, chunk;
    int32_t qb;
    float clip;
    int32_t threads;
  } hook_cases[] = {
      {(int64_t(3) << 18) + 1234, int64_t(1) << 18, 256, 1.0f, 3},
      {int64_t(1) << 18, int64_t(1) << 18, 0, 0.0f, 2},
      {(int64_t(5) << 18) + 7, int64_t(1) << 19, 512, 0.5f, 4},
  };
  for (const auto &c : hook_cases) {
    const bool ok = run_hooks(c.n, c.chunk, c.qb, c.clip, c.threads, rng);
    std::printf("hooks n=%lld chunk=%lld qb=%d clip=%g threads=%d: %s\n", (long long)c.n,
                (long long)c.chunk, c.qb, double(c.clip), c.threads, ok ? "ok" : "MISMATCH");
    bad += !ok;
  }
  return bad ? 1 : 0;
}
