/*
 * zs_oracle.cpp -- CPU oracle for one rank's ZeRO-1/2 shard optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY (see zs_oracle.h).  Built with
 * -ffp-contract=off and without fast-math: every + - * / sqrt below is one
 * IEEE binary64 operation, in the order written.
 */
#include "zs_oracle.h"

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

const int64_t kChunk = int64_t(1) << 20;  // fixed chunk for threaded driving

float bits_to_f32(uint32_t u) {
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

uint32_t f32_to_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return u;
}

// Run body(c) for every chunk c of [0, n) on `threads` threads.
template <class F>
void for_chunks(int64_t n, int32_t threads, F body) {
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  if (threads < 1) threads = 1;
  if (threads > nchunks) threads = int32_t(nchunks > 0 ? nchunks : 1);
  if (threads == 1) {
    for (int64_t c = 0; c < nchunks; ++c) body(c);
    return;
  }
  std::vector<std::thread> pool;
  for (int32_t w = 0; w < threads; ++w)
    pool.emplace_back([=] {
      for (int64_t c = w; c < nchunks; c += threads) body(c);
    });
  for (auto &th : pool) th.join();
}

}  // namespace

extern "C" {

/* Stage table of WIKI ("ZeRO-DP의 세 단계"): with K bytes of optimizer
 * state per parameter,
 *   stage 0  (2+2+K) Psi          stage 1  4 Psi + K Psi / N_d
 *   stage 2  2 Psi + (2+K) Psi / N_d
 *   stage 3  (2+2+K) Psi / N_d
 * The same model-state accounting is in DP, "Memory Consumption Analysis"
 * and the ZeRO-1/2/3 memory-savings formulas.  Returns bytes. */
double orc_model_state_bytes(double psi, double nd, int32_t stage, double k) {
  switch (stage) {
    case 0: return (2.0 + 2.0 + k) * psi;
    case 1: return 4.0 * psi + k * psi / nd;
    case 2: return 2.0 * psi + (2.0 + k) * psi / nd;
    case 3: return (2.0 + 2.0 + k) * psi / nd;
    default: return -1.0;
  }
}

/* bf16 is the upper half of a binary32 pattern (BIMU "精度混合训练" names
 * bf16 as the 2-byte half-precision alternative). */
float orc_bf16_to_f32(uint16_t b) { return bits_to_f32(uint32_t(b) << 16); }

/* Round a binary32 to the nearest bf16, ties to the even pattern.  The
 * dropped 16 bits are compared with the halfway point 0x8000; a carry out
 * of the mantissa moves to the next binade (and past the largest finite
 * value to infinity), which is what nearest rounding does.  NaN stays NaN
 * (quiet bit set, sign kept). */
uint16_t orc_f32_to_bf16(float x) {
  const uint32_t u = f32_to_bits(x);
  if ((u & 0x7fffffffu) > 0x7f800000u)
    return uint16_t((u >> 16) | 0x0040u);
  uint32_t hi = u >> 16;
  const uint32_t lo = u & 0xffffu;
  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1;
  return uint16_t(hi);
}

void orc_cast_bf16(const float *x, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(x[i]);
}

/* a1.  The owner of a slice sums the other ranks' gradients for that slice
 * (BIMU "优化状态与梯度分割", step 2; DP "ZeRO-2": reduce-scatter hands rank
 * r the averaged slice).  Sum in rank order k = 0..n_d-1 in binary64: each
 * addend has 8 significant bits, so the sum is exact unless the addends
 * span more than ~45 binades. */
void orc_reduce_sum(const uint16_t *const *rows, int32_t nd, int64_t n,
                    double *sums) {
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0;
    for (int32_t k = 0; k < nd; ++k) s += double(orc_bf16_to_f32(rows[k][i]));
    sums[i] = s;
  }
}

/* Average over the data-parallel ranks (DP, AllReduce step: the mean of the
 * N per-rank gradients), delivered as binary32: the reduction dtype of the
 * FSDP mixed-precision policy in WIKI "FSDP와의 관계".  One rounding: the
 * exact mean to the nearest binary32. */
void orc_reduce_average(const uint16_t *const *rows, int32_t nd, int64_t n,
                        float *gbar) {
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0;
    for (int32_t k = 0; k < nd; ++k) s += double(orc_bf16_to_f32(rows[k][i]));
    gbar[i] = float(s / double(nd));
  }
}

/* a1 with quantized contributions.  ZeRO++ qgZ ("ZeRO (딥 러닝)", follow-ups
 * table "후속 기법") sends each rank's gradient as quantized blocks that are
 * averaged after the all-to-all.  The pages give no format; reading: int8
 * codes with one binary32 scale per block of `block` shard elements, value
 * = code * scale.  Each product is exact in binary64 (8 + 24 bits); the
 * products are summed in rank order and the mean is rounded once to
 * binary32, exactly as for bf16 contributions. */
void orc_reduce_sum_q8(const int8_t *const *codes, const float *const *scales, int32_t nd,
                       int64_t n, int32_t block, double *sums) {
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0;
    for (int32_t k = 0; k < nd; ++k)
      s += double(codes[k][i]) * double(scales[k][i / block]);
    sums[i] = s;
  }
}

void orc_reduce_average_q8(const int8_t *const *codes, const float *const *scales,
                           int32_t nd, int64_t n, int32_t block, float *gbar) {
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0;
    for (int32_t k = 0; k < nd; ++k)
      s += double(codes[k][i]) * double(scales[k][i / block]);
    gbar[i] = float(s / double(nd));
  }
}

/* a2.  Global-norm clipping at gradient_clipping = 1.0 (WIKI "DeepSpeed에서
 * 쓰기").  The pages give no formula; reading: the L2 norm of the averaged
 * gradient, coef = min(1, max_norm / (norm + 1e-6)).  Each square of a
 * binary32 is exact in binary64; the sum runs in index order. */
double orc_sumsq(const float *gbar, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double g = double(gbar[i]);
    s += g * g;
  }
  return s;
}

double orc_clip_coef(double sumsq, double max_norm) {
  const double c = max_norm / (std::sqrt(sumsq) + 1e-6);
  if (std::isnan(c)) return c;  // NaN propagates: no step skipping
  return c < 1.0 ? c : 1.0;
}

/* a3.  Mixed-precision Adam: fp32 master weights, momentum and variance are
 * the optimizer state (DP "Memory Consumption Analysis"; WIKI memory table;
 * BIMU "精度混合训练": half-precision gradients update the fp32 states).
 * The pages name Adam/AdamW without equations.  Reading: Kingma & Ba
 * (bias-corrected moments, eps added to the square root of the corrected
 * variance) with decoupled weight decay (Loshchilov & Hutter), the
 * torch.optim.AdamW update that the FSDP example instantiates:
 *   m' = b1 m + (1-b1) g          v' = b2 v + (1-b2) g^2
 *   theta' = theta - lr wd theta - lr (m'/bc1) / (sqrt(v'/bc2) + eps)
 * evaluated in binary64 from the stored binary32 state and rounded once to
 * binary32 on store. */
void orc_adam(float *master, float *m, float *v, const float *gbar,
              double coef, int64_t n, const orc_hyper *h) {
  const double b1 = h->beta1, b2 = h->beta2;
  double bc1 = 1.0, bc2 = 1.0;
  if (h->bias_correction) {
    bc1 = 1.0 - std::pow(b1, double(h->t));
    bc2 = 1.0 - std::pow(b2, double(h->t));
  }
  for (int64_t i = 0; i < n; ++i) {
    const double g = coef * double(gbar[i]);  // coef = 1 when not clipping
    const double m1 = b1 * double(m[i]) + (1.0 - b1) * g;
    const double v1 = b2 * double(v[i]) + (1.0 - b2) * (g * g);
    const double mhat = m1 / bc1;
    const double vhat = v1 / bc2;
    const double th = double(master[i]);
    const double th1 =
        th - h->lr * h->weight_decay * th - h->lr * mhat / (std::sqrt(vhat) + h->eps);
    m[i] = float(m1);
    v[i] = float(v1);
    master[i] = float(th1);
  }
}

/* a5.  qwZ: block-quantized weights for the all-gather (WIKI "후속 기법",
 * ZeRO++).  The pages say only "block quantization".  Reading, as the
 * 13B-model ZeRO-2 workload fixes it: blocks of `block` contiguous shard
 * elements from element 0, the last one partial; symmetric int8 with
 *   a = max |p|,  s = a / 127 (binary32),  q = round_half_even(p / s)
 * clamped to [-127, 127]; a block of zeros has s = 0 and q = 0.  Both
 * divisions are binary64 divides of binary32 operands rounded once to
 * binary32, which equals the correctly rounded binary32 quotient (53 >=
 * 2*24+2).  A NaN element makes the block's scale NaN; a non-finite
 * quotient gives code 0. */
void orc_quant_int8(const uint16_t *p, int64_t n, int32_t block,
                    int8_t *codes, float *scales) {
  const int64_t nb = (n + block - 1) / block;
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t lo = b * block;
    const int64_t hi = lo + block < n ? lo + block : n;
    float a = 0.0f;
    for (int64_t i = lo; i < hi; ++i) {
      const float x = std::fabs(orc_bf16_to_f32(p[i]));
      if (x > a || std::isnan(x)) a = std::isnan(a) ? a : x;
    }
    const float s = float(double(a) / 127.0);
    scales[b] = s;
    for (int64_t i = lo; i < hi; ++i) {
      int8_t q = 0;
      if (s != 0.0f) {
        const float ratio = float(double(orc_bf16_to_f32(p[i])) / double(s));
        if (std::isfinite(ratio)) {
          double r = std::nearbyint(double(ratio));  // default mode: ties to even
          if (r > 127.0) r = 127.0;
          if (r < -127.0) r = -127.0;
          q = int8_t(r);
        }
      }
      codes[i] = q;
    }
  }
}

/* qwZ receive side.  After the all-gather each rank holds every shard's
 * int8 codes and block scales (WIKI "후속 기법", ZeRO++ qwZ) and rebuilds
 * the half-precision parameters for its forward pass.  Reading: dequantize
 * to binary32 (the product code * scale rounded once; exact in binary64
 * first), then round to the nearest bf16, ties to even. */
void orc_dequant_bf16(const int8_t *const *codes, const float *const *scales, int32_t nd,
                      int64_t phi, int32_t block, uint16_t *out) {
  const int64_t per = phi / nd + (phi % nd != 0);
  for (int32_t r = 0; r < nd; ++r) {
    const int64_t base = int64_t(r) * per;
    const int64_t len = base >= phi ? 0 : (phi - base < per ? phi - base : per);
    for (int64_t j = 0; j < len; ++j) {
      const float x = float(double(codes[r][j]) * double(scales[r][j / block]));
      out[base + j] = orc_f32_to_bf16(x);
    }
  }
}

double orc_gbar_sumsq(const uint16_t *const *rows, int32_t nd, int64_t n,
                      float *gbar, int32_t threads) {
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  std::vector<double> part(size_t(nchunks > 0 ? nchunks : 1), 0.0);
  for_chunks(n, threads, [&](int64_t c) {
    const int64_t lo = c * kChunk;
    const int64_t len = lo + kChunk < n ? kChunk : n - lo;
    std::vector<const uint16_t *> r(static_cast<size_t>(nd), nullptr);
    for (int32_t k = 0; k < nd; ++k) r[size_t(k)] = rows[k] + lo;
    orc_reduce_average(r.data(), nd, len, gbar + lo);
    part[size_t(c)] = orc_sumsq(gbar + lo, len);
  });
  double s = 0.0;
  for (int64_t c = 0; c < nchunks; ++c) s += part[size_t(c)];
  return s;
}

double orc_gbar_sumsq_q8(const int8_t *const *codes, const float *const *scales, int32_t nd,
                         int64_t n, int32_t block, float *gbar, int32_t threads) {
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  std::vector<double> part(size_t(nchunks > 0 ? nchunks : 1), 0.0);
  for_chunks(n, threads, [&](int64_t c) {
    const int64_t lo = c * kChunk;
    const int64_t len = lo + kChunk < n ? kChunk : n - lo;
    std::vector<const int8_t *> cr(static_cast<size_t>(nd), nullptr);
    std::vector<const float *> sr(static_cast<size_t>(nd), nullptr);
    for (int32_t k = 0; k < nd; ++k) {
      cr[size_t(k)] = codes[k] + lo;
      sr[size_t(k)] = scales[k] + lo / block;
    }
    orc_reduce_average_q8(cr.data(), sr.data(), nd, len, block, gbar + lo);
    part[size_t(c)] = orc_sumsq(gbar + lo, len);
  });
  double s = 0.0;
  for (int64_t c = 0; c < nchunks; ++c) s += part[size_t(c)];
  return s;
}

namespace {

/* a2 (apply) .. a5 from the averaged gradient of the whole shard. */
int finish_step(const float *gbar, double p, int64_t n, float *master, float *m, float *v,
                uint16_t *p_out, int8_t *codes, float *scales, const orc_hyper *h,
                double *sumsq_out, int32_t threads) {
  double coef = 1.0;
  if (h->max_norm > 0.0) coef = orc_clip_coef(p + h->s_other, h->max_norm);
  if (sumsq_out) *sumsq_out = p;
  for_chunks(n, threads, [&](int64_t c) {
    const int64_t lo = c * kChunk;
    const int64_t len = lo + kChunk < n ? kChunk : n - lo;
    orc_adam(master + lo, m + lo, v + lo, gbar + lo, coef, len, h);
    orc_cast_bf16(master + lo, len, p_out + lo);
  });
  if (h->quant_block > 0) orc_quant_int8(p_out, n, h->quant_block, codes, scales);
  return 0;
}

bool bad_args(int32_t nd, int64_t n, const orc_hyper *h, const int8_t *codes,
              const float *scales) {
  if (nd < 1 || n < 0 || !h || h->t < 1) return true;
  return h->quant_block < 0 || (h->quant_block > 0 && (!codes || !scales));
}

}  // namespace

/* The shard step in the order the pages give it: the slice owner reduces
 * and averages its slice, updates its own fp32 states with it, and emits the
 * half-precision copy that the all-gather distributes (BIMU
 * "优化状态与梯度分割" steps 2-3; DP "ZeRO-1"/"ZeRO-2"; WIKI
 * "왜 통신량이 늘지 않는가": the update sits between reduce-scatter and
 * all-gather).  Clipping needs the norm of the whole averaged gradient, so
 * it is a separate sweep before any update. */
int orc_step(const uint16_t *const *rows, int32_t nd, int64_t n, float *master,
             float *m, float *v, uint16_t *p_out, int8_t *codes, float *scales,
             const orc_hyper *h, double *sumsq_out, int32_t threads) {
  if (bad_args(nd, n, h, codes, scales)) return -1;
  if (n == 0) {
    if (sumsq_out) *sumsq_out = 0.0;
    return 0;
  }
  float *gbar = static_cast<float *>(std::malloc(size_t(n) * sizeof(float)));
  if (!gbar) return -1;
  const double p = orc_gbar_sumsq(rows, nd, n, gbar, threads);
  const int rc = finish_step(gbar, p, n, master, m, v, p_out, codes, scales, h, sumsq_out,
                             threads);
  std::free(gbar);
  return rc;
}

int orc_step_q8(const int8_t *const *qc, const float *const *qs, int32_t nd, int64_t n,
                int32_t block, float *master, float *m, float *v, uint16_t *p_out,
                int8_t *codes, float *scales, const orc_hyper *h, double *sumsq_out,
                int32_t threads) {
  if (bad_args(nd, n, h, codes, scales) || block < 1 || kChunk % block != 0) return -1;
  if (n == 0) {
    if (sumsq_out) *sumsq_out = 0.0;
    return 0;
  }
  float *gbar = static_cast<float *>(std::malloc(size_t(n) * sizeof(float)));
  if (!gbar) return -1;
  const double p = orc_gbar_sumsq_q8(qc, qs, nd, n, block, gbar, threads);
  const int rc = finish_step(gbar, p, n, master, m, v, p_out, codes, scales, h, sumsq_out,
                             threads);
  std::free(gbar);
  return rc;
}

}  // extern "C"
