// zero_shard.hip -- MI355X (gfx950) kernels and C ABI of the ZeRO-1/2 shard
// optimizer step (declarations and the contract: include/zero_shard.h).
//
// The step is HBM-bound elementwise work, so there is no MFMA here.  Design
// for CDNA4:
//  * the step lays each wave's 512-element chunk out so that every access
//    instruction covers one contiguous run (lane l owns 4 elements at 4l and
//    4 at 256 + 4l), which keeps the fp32 state accesses dense; in the norm
//    pass one lane owns 8 consecutive elements, each contribution row one
//    128-bit load, a wave64 touching 1 KiB of every row per access;
//  * the rank-order sum of the bf16 contributions runs in binary64 registers
//    (binary64 adds issue at the unpacked-binary32 rate on CDNA4, half its
//    packed peak), exact unless the addends span some 45 binades; the
//    average is rounded once to binary32, the precision the reduce-scatter
//    delivers;
//  * rows are loaded in groups of kRowGroup so that many 16-byte loads per
//    lane are in flight while the sum keeps its fixed k order;
//  * the AdamW update runs in binary64 from the binary32 state with every
//    result rounded once on store (IEEE division and square root), the bf16
//    cast uses the gfx950 v_cvt_pk_bf16_f32 conversion (nearest even);
//  * the int8 block quantizer is fused into the same pass: a block of B
//    elements is B/8 adjacent lanes of one wave, its absmax a lane-shuffle
//    reduction, so quantization adds only the code and scale writes;
//  * the global norm is a fixed-grid, fixed-order two-kernel reduction
//    (fp64 block partials, then one block) with no atomics, so identical
//    inputs give identical bits.
// All arithmetic is exactly as written (built with -ffp-contract=off, no
// fast-math, denormals preserved).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>

#include "zero_shard.h"
#include "zs_args.h"

namespace {

using u32x4 = unsigned int __attribute__((ext_vector_type(4)));
using u32x2 = unsigned int __attribute__((ext_vector_type(2)));
using f32x4 = float __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;    // 4 waves per workgroup
constexpr int kVec = 8;          // shard elements per lane
#ifndef ZS_ROW_GROUP
#define ZS_ROW_GROUP 8
#endif
constexpr int kRowGroup = ZS_ROW_GROUP;  // contribution rows loaded together (update)
#ifndef ZS_WIDE_ROW_GROUP
#define ZS_WIDE_ROW_GROUP 4
#endif
#ifndef ZS_WIDE_UNROLL
#define ZS_WIDE_UNROLL 8
#endif
#ifndef ZS_NORM_ROW_GROUP
#define ZS_NORM_ROW_GROUP 4
#endif

#ifndef ZS_NORM_UNROLL
#define ZS_NORM_UNROLL 8
#endif

#ifndef ZS_BLOCKS_PER_CU
#define ZS_BLOCKS_PER_CU 0
#endif
#ifndef ZS_NT_STATE
#define ZS_NT_STATE 0
#endif
#ifndef ZS_DENSE_NT
#define ZS_DENSE_NT 1
#endif
// Nontemporal state loads and stores in the step's dense layout.
constexpr bool kDenseNt = ZS_DENSE_NT;
#ifndef ZS_DENSE_Q_LDS
#define ZS_DENSE_Q_LDS (48 * 1024)
#endif
// LDS reserved (and unused) by each workgroup of the quantizing U = 1 step
// over bf16 rows: at most 3 workgroups per CU (160 KiB each).
constexpr size_t kDenseQLds = ZS_DENSE_Q_LDS;
#ifndef ZS_NT_SPILL
#define ZS_NT_SPILL 1
#endif
#ifndef ZS_NT_OUT
#define ZS_NT_OUT 1
#endif
constexpr bool kNtOut = ZS_NT_OUT;  // nontemporal stores for bf16 / int8 outputs

// Contribution sources: row k is rank k's gradient for this shard.
struct Bf16Rows {
  const u32x4 *p[ZS_MAX_ND];  // bf16: 8 elements per 16-byte load
};
struct Q8Rows {
  const u32x2 *c[ZS_MAX_ND];  // int8 codes: 8 elements per 8-byte load
  const float *s[ZS_MAX_ND];  // one fp32 scale per block of the row
  int32_t shift;              // log2(lane-vectors per block)
};

#ifndef ZS_Q8_WIDE_UNROLL
#define ZS_Q8_WIDE_UNROLL 2
#endif
#ifndef ZS_Q8_WIDE_GROUP
#define ZS_Q8_WIDE_GROUP 4
#endif
#ifndef ZS_Q8_NORM_UNROLL
#define ZS_Q8_NORM_UNROLL 2
#endif
#ifndef ZS_Q8_NORM_GROUP
#define ZS_Q8_NORM_GROUP 4
#endif

// Launch shape per contribution format: lane-vectors per wave sweep and rows
// loaded together, for the wide update and for the norm pass.
template <class Src>
struct Tune;
template <>
struct Tune<Bf16Rows> {
  static constexpr int wide_unroll = ZS_WIDE_UNROLL, wide_group = ZS_WIDE_ROW_GROUP;
  static constexpr int norm_unroll = ZS_NORM_UNROLL, norm_group = ZS_NORM_ROW_GROUP;
};
template <>
struct Tune<Q8Rows> {
  static constexpr int wide_unroll = ZS_Q8_WIDE_UNROLL, wide_group = ZS_Q8_WIDE_GROUP;
  static constexpr int norm_unroll = ZS_Q8_NORM_UNROLL, norm_group = ZS_Q8_NORM_GROUP;
};

struct AdamConst {
  double b1, omb1;  // beta1, 1 - beta1
  double b2, omb2;  // beta2, 1 - beta2
  double bc1, bc2;  // bias corrections (1 when off)
  double lr, decay, eps;  // lr, lr * weight_decay, eps
};

struct Avg {
  int32_t nd;
  int32_t pow2;     // n_d is a power of two: s / n_d == s * (1 / n_d)
  double nd_f, inv_nd;
};

template <class Src>
struct StepArgs {
  Src src;
  Avg avg;
  AdamConst k;
  const double *dyn;    // iff non-null: lr, lr*wd, bc1, bc2 read from here at run time
  int64_t n;
  const double *sumsq;  // clip by this global sum of squares iff non-null
  double max_norm;
  const float *gbar;    // read the averaged gradient from here iff non-null
  float *master, *m, *v;
  uint16_t *pout;
  int8_t *codes;
  float *scales;
};

template <class Src>
struct NormArgs {
  Src src;
  Avg avg;
  int64_t n;
  float *gbar_out;   // store the averaged gradient iff non-null
  double *partials;  // one per block
};

struct DequantArgs {
  const u32x2 *c[ZS_MAX_ND];  // shard r's int8 codes
  const float *s[ZS_MAX_ND];  // shard r's block scales
  int32_t shift;              // log2(lane-vectors per block)
  int64_t per;                // elements per shard (the last may be shorter)
  int64_t phi;
  uint16_t *out;              // bf16[phi]
};

struct QuantArgs {
  const uint16_t *p;
  int64_t n;
  int8_t *codes;
  float *scales;
};

// ------------------------------------------------------------ device helpers

template <bool NT, class T>
__device__ __forceinline__ T ld(const T *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT, class T>
__device__ __forceinline__ void st(T v, T *p) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Nearest-even bf16 of two floats, packed (lo in bits 0..15): one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  const unsigned a = __builtin_bit_cast(unsigned short, static_cast<__bf16>(lo));
  const unsigned b = __builtin_bit_cast(unsigned short, static_cast<__bf16>(hi));
  return a | (b << 16);
}

__device__ __forceinline__ void add_row(double (&s)[kVec], const u32x4 r) {
  s[0] += static_cast<double>(bf16_lo(r.x));
  s[1] += static_cast<double>(bf16_hi(r.x));
  s[2] += static_cast<double>(bf16_lo(r.y));
  s[3] += static_cast<double>(bf16_hi(r.y));
  s[4] += static_cast<double>(bf16_lo(r.z));
  s[5] += static_cast<double>(bf16_hi(r.z));
  s[6] += static_cast<double>(bf16_lo(r.w));
  s[7] += static_cast<double>(bf16_hi(r.w));
}

// One full lane-vector of row k, and its addition into the per-element
// binary64 sums.  bf16: the value itself; int8: code * scale, an exact
// product in binary64.
struct Bf16Frag {
  u32x4 r;
};
struct Q8Frag {
  u32x2 c;
  float s;
};

__device__ __forceinline__ Bf16Frag fetch(const Bf16Rows &src, int k, int64_t vec) {
  return {__builtin_nontemporal_load(src.p[k] + vec)};
}

__device__ __forceinline__ Q8Frag fetch(const Q8Rows &src, int k, int64_t vec) {
  return {__builtin_nontemporal_load(src.c[k] + vec), src.s[k][vec >> src.shift]};
}

__device__ __forceinline__ void accum(double (&s)[kVec], const Bf16Frag &f) { add_row(s, f.r); }

// s + code * scale.  The product of an int8 and a binary32 is exact in
// binary64, so one fused multiply-add rounds exactly as the product followed
// by the addition does, with one instruction instead of two.
__device__ __forceinline__ double add_dequant(double s, unsigned w, int byte, double scale) {
  return __builtin_fma(static_cast<double>(static_cast<int8_t>(w >> (8 * byte))), scale, s);
}

__device__ __forceinline__ void accum(double (&s)[kVec], const Q8Frag &f) {
  const double sc = static_cast<double>(f.s);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s[e] = add_dequant(s[e], f.c.x, e, sc);
    s[e + 4] = add_dequant(s[e + 4], f.c.y, e, sc);
  }
}

// The first nvalid elements of lane-vector vec of row k (the shard's last,
// partial vector), element by element.
__device__ __forceinline__ void accum_partial(double (&s)[kVec], const Bf16Rows &src, int k,
                                              int64_t vec, int nvalid) {
  const uint16_t *row = reinterpret_cast<const uint16_t *>(src.p[k]) + vec * kVec;
#pragma unroll
  for (int e = 0; e < kVec; ++e)
    if (e < nvalid) s[e] += static_cast<double>(__uint_as_float(unsigned(row[e]) << 16));
}

__device__ __forceinline__ void accum_partial(double (&s)[kVec], const Q8Rows &src, int k,
                                              int64_t vec, int nvalid) {
  const int8_t *row = reinterpret_cast<const int8_t *>(src.c[k]) + vec * kVec;
  const double sc = static_cast<double>(src.s[k][vec >> src.shift]);
#pragma unroll
  for (int e = 0; e < kVec; ++e)
    if (e < nvalid) s[e] = __builtin_fma(static_cast<double>(row[e]), sc, s[e]);
}

__device__ __forceinline__ float average(double s, const Avg &a) {
  return a.pow2 ? static_cast<float>(s * a.inv_nd) : static_cast<float>(s / a.nd_f);
}

// Averaged gradient of the 8 elements of lane-vector `vec`.  Full vectors
// take one vector load per row, rows in groups of kRowGroup; a partial
// vector (the shard's last, nvalid < 8) loads element by element.  The
// additions are the same in both cases: k = 0..nd-1 into a binary64
// accumulator per element.
template <class Src>
__device__ __forceinline__ void reduce_average(const Src &src, const Avg &avg, int64_t vec,
                                               int nvalid, float (&g)[kVec]) {
  using Frag = decltype(fetch(src, 0, 0));
  double s[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) s[e] = 0.0;
  if (nvalid == kVec) {
    for (int k0 = 0; k0 < avg.nd; k0 += kRowGroup) {
      Frag r[kRowGroup];
#pragma unroll
      for (int j = 0; j < kRowGroup; ++j)
        if (k0 + j < avg.nd) r[j] = fetch(src, k0 + j, vec);
#pragma unroll
      for (int j = 0; j < kRowGroup; ++j)
        if (k0 + j < avg.nd) accum(s, r[j]);
    }
  } else {
    for (int k = 0; k < avg.nd; ++k) accum_partial(s, src, k, vec, nvalid);
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) g[e] = average(s[e], avg);
}

__device__ __forceinline__ double clip_coef(double sumsq, double max_norm) {
  const double c = max_norm / (sqrt(sumsq) + 1e-6);
  if (c != c) return c;  // NaN propagates
  return c < 1.0 ? c : 1.0;
}

// AdamW on one element: binary64 from the binary32 state, one rounding per
// stored value.  The expression order is the contract's.
__device__ __forceinline__ void adam(double g, float &th, float &mo, float &va,
                                     const AdamConst &k) {
  const double m1 = k.b1 * static_cast<double>(mo) + k.omb1 * g;
  const double v1 = k.b2 * static_cast<double>(va) + k.omb2 * (g * g);
  const double mhat = m1 / k.bc1;
  const double vhat = v1 / k.bc2;
  const double t0 = static_cast<double>(th);
  const double t1 = t0 - k.decay * t0 - k.lr * mhat / (sqrt(vhat) + k.eps);
  mo = static_cast<float>(m1);
  va = static_cast<float>(v1);
  th = static_cast<float>(t1);
}

__device__ __forceinline__ float nanmax(float a, float b) {
  if (a != a) return a;
  return (b > a || b != b) ? b : a;
}

// int8 code of x with scale s (binary32 quotient, ties to even, +-127).
__device__ __forceinline__ int quant_code(float x, float s) {
  if (s == 0.0f) return 0;
  float r = x / s;
  if (!__builtin_isfinite(r)) return 0;
  r = __builtin_rintf(r);
  r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
  return static_cast<int>(r);
}

// Quantize the 8 bf16 values of lane-vector `vec` as part of a block of
// QL adjacent lanes (block = 8*QL elements).  Every lane of the wave must
// call this (the absmax is a shuffle reduction); lanes past the end pass
// nvalid = 0.
template <int QL>
__device__ __forceinline__ void quant_lane(const float (&p)[kVec], int nvalid, int64_t vec,
                                           int8_t *codes, float *scales) {
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < kVec; ++e)
    if (e < nvalid) a = nanmax(a, __builtin_fabsf(p[e]));
#pragma unroll
  for (int off = QL / 2; off >= 1; off >>= 1) a = nanmax(a, __shfl_xor(a, off));
  const float s = a / 127.0f;
  if (nvalid == kVec) {
    unsigned lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= (unsigned(quant_code(p[e], s)) & 0xffu) << (8 * e);
      hi |= (unsigned(quant_code(p[e + 4], s)) & 0xffu) << (8 * e);
    }
    u32x2 q;
    q.x = lo;
    q.y = hi;
    st<kNtOut>(q, reinterpret_cast<u32x2 *>(codes) + vec);
  } else {
#pragma unroll
    for (int e = 0; e < kVec; ++e)
      if (e < nvalid) codes[vec * kVec + e] = static_cast<int8_t>(quant_code(p[e], s));
  }
  if (nvalid > 0 && (vec % QL) == 0) scales[vec / QL] = s;
}

// ------------------------------------------------------------------ kernels

// Averaged gradient of the U full lane-vectors v0, v0+64, .., v0+64(U-1)
// (one per wave-sweep of 64 lanes): U*kRowGroup 16-byte loads in flight per
// lane; per element the same k-ordered binary64 sum as reduce_average.
template <int U, int G, class Src>
__device__ __forceinline__ void reduce_average_wave(const Src &src, const Avg &avg, int64_t v0,
                                                    float (&g)[U][kVec]) {
  using Frag = decltype(fetch(src, 0, 0));
  double s[U][kVec];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < kVec; ++e) s[u][e] = 0.0;
  for (int k0 = 0; k0 < avg.nd; k0 += G) {
    Frag r[U][G];
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (k0 + j < avg.nd)
#pragma unroll
        for (int u = 0; u < U; ++u) r[u][j] = fetch(src, k0 + j, v0 + 64 * u);
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (k0 + j < avg.nd)
#pragma unroll
        for (int u = 0; u < U; ++u) accum(s[u], r[u][j]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < kVec; ++e) g[u][e] = average(s[u][e], avg);
}

// One lane-vector (8 elements) of the update, any fill level: nvalid = 0..8
// valid elements.  Every lane of the wave calls it together (the quantizer
// reduces across lanes); lanes past the end pass a vector with nvalid 0.
template <int QL, class Src>
__device__ __forceinline__ void step_vec(const StepArgs<Src> &A, const AdamConst &k, int64_t vec,
                                         double coef) {
    const int64_t e0 = vec * kVec;
    const int nvalid = e0 + kVec <= A.n ? kVec : (e0 < A.n ? int(A.n - e0) : 0);
    float th[kVec], mo[kVec], va[kVec], g[kVec], p[kVec];
    if (nvalid == kVec) {
      const f32x4 *t4 = reinterpret_cast<const f32x4 *>(A.master) + 2 * vec;
      const f32x4 *m4 = reinterpret_cast<const f32x4 *>(A.m) + 2 * vec;
      const f32x4 *v4 = reinterpret_cast<const f32x4 *>(A.v) + 2 * vec;
      constexpr bool nt = ZS_NT_STATE;
      const f32x4 ta = ld<nt>(t4), tb = ld<nt>(t4 + 1), ma = ld<nt>(m4), mb = ld<nt>(m4 + 1),
                  vx = ld<nt>(v4), vy = ld<nt>(v4 + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        th[e] = ta[e]; th[e + 4] = tb[e];
        mo[e] = ma[e]; mo[e + 4] = mb[e];
        va[e] = vx[e]; va[e + 4] = vy[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const bool ok = e < nvalid;
        th[e] = ok ? A.master[e0 + e] : 0.0f;
        mo[e] = ok ? A.m[e0 + e] : 0.0f;
        va[e] = ok ? A.v[e0 + e] : 0.0f;
      }
    }
    if (nvalid > 0) {
      if (A.gbar) {
        if (nvalid == kVec) {
          const f32x4 *g4 = reinterpret_cast<const f32x4 *>(A.gbar) + 2 * vec;
          const f32x4 ga = __builtin_nontemporal_load(g4), gb = __builtin_nontemporal_load(g4 + 1);
#pragma unroll
          for (int e = 0; e < 4; ++e) { g[e] = ga[e]; g[e + 4] = gb[e]; }
        } else {
#pragma unroll
          for (int e = 0; e < kVec; ++e) g[e] = e < nvalid ? A.gbar[e0 + e] : 0.0f;
        }
      } else {
        reduce_average(A.src, A.avg, vec, nvalid, g);
      }
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        adam(coef * static_cast<double>(g[e]), th[e], mo[e], va[e], k);
      }
    }
    unsigned pb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pb[e] = pack_bf16(th[2 * e], th[2 * e + 1]);
      p[2 * e] = bf16_lo(pb[e]);
      p[2 * e + 1] = bf16_hi(pb[e]);
    }
    if (nvalid == kVec) {
      f32x4 *t4 = reinterpret_cast<f32x4 *>(A.master) + 2 * vec;
      f32x4 *m4 = reinterpret_cast<f32x4 *>(A.m) + 2 * vec;
      f32x4 *v4 = reinterpret_cast<f32x4 *>(A.v) + 2 * vec;
      f32x4 o[6];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[0][e] = th[e]; o[1][e] = th[e + 4];
        o[2][e] = mo[e]; o[3][e] = mo[e + 4];
        o[4][e] = va[e]; o[5][e] = va[e + 4];
      }
      constexpr bool nt = ZS_NT_STATE;
      st<nt>(o[0], t4); st<nt>(o[1], t4 + 1);
      st<nt>(o[2], m4); st<nt>(o[3], m4 + 1);
      st<nt>(o[4], v4); st<nt>(o[5], v4 + 1);
      u32x4 pv;
      pv.x = pb[0]; pv.y = pb[1]; pv.z = pb[2]; pv.w = pb[3];
      st<kNtOut>(pv, reinterpret_cast<u32x4 *>(A.pout) + vec);
    } else if (nvalid > 0) {
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        if (e < nvalid) {
          A.master[e0 + e] = th[e];
          A.m[e0 + e] = mo[e];
          A.v[e0 + e] = va[e];
          A.pout[e0 + e] = static_cast<uint16_t>(pb[e / 2] >> (16 * (e & 1)));
        }
      }
    }
    if constexpr (QL > 0) quant_lane<QL>(p, nvalid, vec, A.codes, A.scales);
}

// Dense element layout for one full 512-element chunk c of a wave.  Lane l
// owns elements 512c + 4l + {0..3} (half 0) and 512c + 256 + 4l + {0..3}
// (half 1), so that every access instruction of the wave covers one
// contiguous run: 1 KiB of an fp32 array, 512 B of a bf16 one, 256 B of
// int8 codes.  (In the per-vector layout a lane owns 8 consecutive elements
// and each fp32 array takes two 16-byte accesses at a 32-byte lane stride,
// half of every run per instruction; measured, that pattern loses
// bandwidth, and with nontemporal accesses loses much more.)  The
// arithmetic per element is the same, so results are bit-identical.
//
// One row's 4 elements at e of a dense chunk: 8 bytes of bf16, or 4 int8
// codes and the scale of their block.
struct Bf16Half {
  u32x2 r;
};
struct Q8Half {
  unsigned c;
  float s;
};
__device__ __forceinline__ Bf16Half fetch_half(const Bf16Rows &src, int k, int64_t e) {
  return {__builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(src.p[k]) + e / 4)};
}
__device__ __forceinline__ Q8Half fetch_half(const Q8Rows &src, int k, int64_t e) {
  return {__builtin_nontemporal_load(reinterpret_cast<const unsigned *>(src.c[k]) + e / 4),
          src.s[k][e >> (src.shift + 3)]};
}
__device__ __forceinline__ void accum_half(double (&s)[kVec], int h, const Bf16Half &f) {
  s[4 * h + 0] += static_cast<double>(bf16_lo(f.r.x));
  s[4 * h + 1] += static_cast<double>(bf16_hi(f.r.x));
  s[4 * h + 2] += static_cast<double>(bf16_lo(f.r.y));
  s[4 * h + 3] += static_cast<double>(bf16_hi(f.r.y));
}
__device__ __forceinline__ void accum_half(double (&s)[kVec], int h, const Q8Half &f) {
  const double sc = static_cast<double>(f.s);
#pragma unroll
  for (int e = 0; e < 4; ++e) s[4 * h + e] = add_dequant(s[4 * h + e], f.c, e, sc);
}

// a5 on a dense chunk: p[0..3] are elements e0..e0+3, p[4..7] the same 256
// elements later.  A block of B <= 256 elements is B/4 adjacent lanes of one
// half, its absmax a lane-shuffle reduction per half; B = 512 is the whole
// chunk.  Every lane of the wave calls this.
template <int QL>
__device__ __forceinline__ void quant_dense(const float (&p)[kVec], int64_t e0, int lane,
                                            int8_t *codes, float *scales) {
  constexpr int B = 8 * QL;
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a0 = nanmax(a0, __builtin_fabsf(p[e]));
    a1 = nanmax(a1, __builtin_fabsf(p[e + 4]));
  }
  if constexpr (B <= 256) {
#pragma unroll
    for (int off = B / 8; off >= 1; off >>= 1) {
      a0 = nanmax(a0, __shfl_xor(a0, off));
      a1 = nanmax(a1, __shfl_xor(a1, off));
    }
  } else {
    a0 = nanmax(a0, a1);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a0 = nanmax(a0, __shfl_xor(a0, off));
    a1 = a0;
  }
  const float s0 = a0 / 127.0f, s1 = a1 / 127.0f;
  unsigned c0 = 0, c1 = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c0 |= (unsigned(quant_code(p[e], s0)) & 0xffu) << (8 * e);
    c1 |= (unsigned(quant_code(p[e + 4], s1)) & 0xffu) << (8 * e);
  }
  st<kNtOut>(c0, reinterpret_cast<unsigned *>(codes + e0));
  st<kNtOut>(c1, reinterpret_cast<unsigned *>(codes + e0 + 256));
  if constexpr (B <= 256) {
    if ((lane % (B / 4)) == 0) {
      scales[e0 / B] = s0;
      scales[(e0 + 256) / B] = s1;
    }
  } else {
    if (lane == 0) scales[e0 / B] = s0;
  }
}

// a1 on the U full chunks c0, c0+1, ... in the dense layout: the rows are
// loaded G at a time for all U chunks (2U loads per row in flight) and
// summed in rank order in binary64, then averaged.
template <int U, int G, class Src>
__device__ __forceinline__ void reduce_dense(const Src &src, const Avg &avg, int64_t c0, int lane,
                                             float (&g)[U][kVec]) {
  using Half = decltype(fetch_half(src, 0, 0));
  double s[U][kVec];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < kVec; ++e) s[u][e] = 0.0;
  for (int k0 = 0; k0 < avg.nd; k0 += G) {
    Half r[U][G][2];
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (k0 + j < avg.nd)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t e0 = (c0 + u) * 512 + 4 * lane;
          r[u][j][0] = fetch_half(src, k0 + j, e0);
          r[u][j][1] = fetch_half(src, k0 + j, e0 + 256);
        }
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (k0 + j < avg.nd)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          accum_half(s[u], 0, r[u][j][0]);
          accum_half(s[u], 1, r[u][j][1]);
        }
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < kVec; ++e) g[u][e] = average(s[u][e], avg);
}

// The fp32 state of a lane's 8 elements of a dense chunk (e0 = its first):
// master, m and v, one 16-byte vector per half each, nontemporal.
struct DenseState {
  f32x4 t[2], m[2], v[2];
};

template <class Src>
__device__ __forceinline__ void load_dense(const StepArgs<Src> &A, int64_t e0, DenseState &s) {
  constexpr bool nt = kDenseNt;
  const f32x4 *t4 = reinterpret_cast<const f32x4 *>(A.master + e0);
  const f32x4 *m4 = reinterpret_cast<const f32x4 *>(A.m + e0);
  const f32x4 *v4 = reinterpret_cast<const f32x4 *>(A.v + e0);
  s.t[0] = ld<nt>(t4); s.t[1] = ld<nt>(t4 + 64);
  s.m[0] = ld<nt>(m4); s.m[1] = ld<nt>(m4 + 64);
  s.v[0] = ld<nt>(v4); s.v[1] = ld<nt>(v4 + 64);
}

// a2 (apply) + a3 + a4 (+ a5) on a lane's 8 elements of a dense chunk,
// given their averaged gradient g and state s.  Every lane of the wave
// calls it together (the quantizer's shuffles).
template <int QL, class Src>
__device__ __forceinline__ void update_dense(const StepArgs<Src> &A, const AdamConst &k,
                                             int64_t e0, int lane, double coef,
                                             const float (&g)[kVec], const DenseState &s) {
  constexpr bool nt = kDenseNt;
  float th[kVec], mo[kVec], va[kVec];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    th[e] = s.t[0][e]; th[e + 4] = s.t[1][e];
    mo[e] = s.m[0][e]; mo[e + 4] = s.m[1][e];
    va[e] = s.v[0][e]; va[e + 4] = s.v[1][e];
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) adam(coef * static_cast<double>(g[e]), th[e], mo[e], va[e], k);
  unsigned pb[4];
  float p[kVec];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pb[e] = pack_bf16(th[2 * e], th[2 * e + 1]);
    p[2 * e] = bf16_lo(pb[e]);
    p[2 * e + 1] = bf16_hi(pb[e]);
  }
  f32x4 o0, o1;
  f32x4 *t4 = reinterpret_cast<f32x4 *>(A.master + e0);
  f32x4 *m4 = reinterpret_cast<f32x4 *>(A.m + e0);
  f32x4 *v4 = reinterpret_cast<f32x4 *>(A.v + e0);
#pragma unroll
  for (int e = 0; e < 4; ++e) { o0[e] = th[e]; o1[e] = th[e + 4]; }
  st<nt>(o0, t4); st<nt>(o1, t4 + 64);
#pragma unroll
  for (int e = 0; e < 4; ++e) { o0[e] = mo[e]; o1[e] = mo[e + 4]; }
  st<nt>(o0, m4); st<nt>(o1, m4 + 64);
#pragma unroll
  for (int e = 0; e < 4; ++e) { o0[e] = va[e]; o1[e] = va[e + 4]; }
  st<nt>(o0, v4); st<nt>(o1, v4 + 64);
  u32x2 q0, q1;
  q0.x = pb[0]; q0.y = pb[1];
  q1.x = pb[2]; q1.y = pb[3];
  st<kNtOut>(q0, reinterpret_cast<u32x2 *>(A.pout + e0));
  st<kNtOut>(q1, reinterpret_cast<u32x2 *>(A.pout + e0 + 256));
  if constexpr (QL > 0) quant_dense<QL>(p, e0, lane, A.codes, A.scales);
}

// a1 (rows) or the spilled gradient, then the update, on the full chunk c in
// the dense layout, one chunk per wave.  The state is loaded after the
// gradient is formed: held across the row loop it would not fit the 96
// registers of the 5-wave form (the compiler spills it to scratch).
template <int QL, class Src>
__device__ __forceinline__ void step_chunk_dense(const StepArgs<Src> &A, const AdamConst &k,
                                                 int64_t c, int lane, double coef) {
  const int64_t e0 = c * 512 + 4 * lane;
  float g[1][kVec];
  if (A.gbar) {
    const f32x4 *g4 = reinterpret_cast<const f32x4 *>(A.gbar + e0);
    const f32x4 ga = __builtin_nontemporal_load(g4);
    const f32x4 gb = __builtin_nontemporal_load(g4 + 64);
#pragma unroll
    for (int e = 0; e < 4; ++e) { g[0][e] = ga[e]; g[0][e + 4] = gb[e]; }
  } else {
    reduce_dense<1, kRowGroup>(A.src, A.avg, c, lane, g);
  }
  DenseState s;
  load_dense(A, e0, s);
  update_dense<QL>(A, k, e0, lane, coef, g[0], s);
}

// The step's constants: fixed at the call, or read from the caller's device
// array when the launch carries one (a graph replayed at every step).
template <class Src>
__device__ __forceinline__ AdamConst step_consts(const StepArgs<Src> &A) {
  AdamConst k = A.k;
  if (A.dyn) {
    k.lr = A.dyn[0];
    k.decay = A.dyn[1];
    k.bc1 = A.dyn[2];
    k.bc2 = A.dyn[3];
  }
  return k;
}

// a1 + a2 (apply) + a3 + a4 (+ a5 when QL > 0).  Each wave owns U
// consecutive 512-element chunks per iteration, in the dense layout.  U = 1:
// one chunk, state, gradient and outputs together.  U > 1 (many
// contribution rows): the rows of all U chunks are reduced first, so that
// every wave reads U runs of 512 B (bf16) of each row with 2*U*G loads in
// flight, then each chunk's state is updated in turn.  The shard's last,
// partial chunk goes vector by vector (lane l takes lane-vectors wb + l,
// wb + 64 + l, ...).  The loop condition is uniform across the wave, as the
// quantizer's shuffles need.
//
// The unquantized U = 1 form over bf16 rows is compiled for 5 waves per
// SIMD, which it fits in 96 VGPRs, and the quantizing U = 1 forms over bf16
// rows run at most 3 workgroups per CU (an LDS reservation made at launch).
// The other forms would spill at the 5-wave target and keep the compiler's
// default.
template <class Src>
constexpr bool kBf16Src = false;
template <>
constexpr bool kBf16Src<Bf16Rows> = true;

template <int QL, int U, class Src>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(QL == 0 && U == 1 && kBf16Src<Src> ? 5 : 1)))
    step_kernel(const StepArgs<Src> A) {
  constexpr int64_t span = 64 * U;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nvec = (A.n + kVec - 1) / kVec;
  const int64_t nfull = A.n / kVec;
  const int64_t stride = int64_t(gridDim.x) * (kThreads / 64) * span;
  const double coef = A.sumsq ? clip_coef(*A.sumsq, A.max_norm) : 1.0;
  const AdamConst k = step_consts(A);
  for (int64_t wb = (int64_t(blockIdx.x) * (kThreads / 64) + wave) * span; wb < nvec;
       wb += stride) {
    if (wb + span > nfull) {
#pragma unroll
      for (int u = 0; u < U; ++u) step_vec<QL, Src>(A, k, wb + 64 * u + lane, coef);
      continue;
    }
    if constexpr (U == 1) {
      step_chunk_dense<QL>(A, k, wb / 64, lane, coef);
    } else {
      float g[U][kVec];  // launched only without a spill: the rows are read
      reduce_dense<U, Tune<Src>::wide_group>(A.src, A.avg, wb / 64, lane, g);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t e0 = (wb / 64 + u) * 512 + 4 * lane;
        DenseState s;
        load_dense(A, e0, s);
        update_dense<QL>(A, k, e0, lane, coef, g[u], s);
      }
    }
  }
}

__device__ __forceinline__ void store_gbar(float *out, int64_t vec, int nvalid,
                                           const float (&g)[kVec]) {
  if (nvalid == kVec) {
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) { a[e] = g[e]; b[e] = g[e + 4]; }
    f32x4 *o = reinterpret_cast<f32x4 *>(out) + 2 * vec;
    st<ZS_NT_SPILL>(a, o);
    st<ZS_NT_SPILL>(b, o + 1);
  } else {
#pragma unroll
    for (int e = 0; e < kVec; ++e)
      if (e < nvalid) out[vec * kVec + e] = g[e];
  }
}

// a2, first kernel: block partial sums of gbar^2 (binary64).  The grid is
// fixed by n alone: one pass, each block 4 waves x one sweep of 64*U
// (U per contribution format) consecutive lane-vectors (lane l takes
// v0+l, v0+64+l, ...), block b the b-th stretch of the launch.  A lane's
// sum runs over its vectors in sweep order, then a fixed butterfly over the
// wave and the 4 wave sums in order; partial b belongs to block b, and the
// launches of a part write consecutive runs of partials, so the partials
// (and S) are in shard order however the part is split into launches.
template <class Src>
__global__ void __launch_bounds__(kThreads) gnorm_partial_kernel(const NormArgs<Src> A) {
  constexpr int U = Tune<Src>::norm_unroll;
  constexpr int64_t span = 64 * U;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nvec = (A.n + kVec - 1) / kVec;
  const int64_t nfull = A.n / kVec;
  const int64_t wb = (int64_t(blockIdx.x) * (kThreads / 64) + wave) * span;
  double acc = 0.0;
  if (wb < nvec) {
    if (wb + span <= nfull) {
      float g[U][kVec];
      reduce_average_wave<U, Tune<Src>::norm_group>(A.src, A.avg, wb + lane, g);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (A.gbar_out) store_gbar(A.gbar_out, wb + 64 * u + lane, kVec, g[u]);
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
          const double x = static_cast<double>(g[u][e]);
          acc += x * x;
        }
      }
    } else {
      for (int u = 0; u < U; ++u) {
        const int64_t vec = wb + 64 * u + lane;
        if (vec >= nvec) break;
        const int64_t e0 = vec * kVec;
        const int nvalid = e0 + kVec <= A.n ? kVec : int(A.n - e0);
        float g[kVec];
        reduce_average(A.src, A.avg, vec, nvalid, g);
        if (A.gbar_out) store_gbar(A.gbar_out, vec, nvalid, g);
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
          if (e < nvalid) {
            const double x = static_cast<double>(g[e]);
            acc += x * x;
          }
        }
      }
    }
  }
  // wave: butterfly over 64 lanes; block: the 4 wave sums in wave order
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  __shared__ double wsum[kThreads / 64];
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) t += wsum[w];
    A.partials[blockIdx.x] = t;
  }
}

// a2, second kernel: one block of 1024 reduces the partials in a fixed
// order (each thread a strided run, then an LDS tree).
constexpr int kFinalThreads = 1024;

__global__ void __launch_bounds__(kFinalThreads) gnorm_final_kernel(const double *partials,
                                                                    int np, double *out) {
  __shared__ double buf[kFinalThreads];
  double s = 0.0;
  for (int i = threadIdx.x; i < np; i += kFinalThreads) s += partials[i];
  buf[threadIdx.x] = s;
  __syncthreads();
  for (int half = kFinalThreads / 2; half >= 1; half >>= 1) {
    if (threadIdx.x < half) buf[threadIdx.x] += buf[threadIdx.x + half];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = buf[0];
}

// a5 as its own pass over the bf16 shard.
template <int QL>
__global__ void __launch_bounds__(kThreads) quant_kernel(const QuantArgs A) {
  const int lane = threadIdx.x & 63;
  const int64_t nvec = (A.n + kVec - 1) / kVec;
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t base = int64_t(blockIdx.x) * kThreads + (threadIdx.x & ~63); base < nvec;
       base += stride) {
    const int64_t vec = base + lane;
    const int64_t e0 = vec * kVec;
    const int nvalid = e0 + kVec <= A.n ? kVec : (e0 < A.n ? int(A.n - e0) : 0);
    float p[kVec];
    if (nvalid == kVec) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(A.p) + vec);
      p[0] = bf16_lo(w.x); p[1] = bf16_hi(w.x); p[2] = bf16_lo(w.y); p[3] = bf16_hi(w.y);
      p[4] = bf16_lo(w.z); p[5] = bf16_hi(w.z); p[6] = bf16_lo(w.w); p[7] = bf16_hi(w.w);
    } else {
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        p[e] = e < nvalid ? __uint_as_float(unsigned(A.p[e0 + e]) << 16) : 0.0f;
    }
    quant_lane<QL>(p, nvalid, vec, A.codes, A.scales);
  }
}

#ifndef ZS_DQ_UNROLL
#define ZS_DQ_UNROLL 1
#endif
#ifndef ZS_DQ_BLOCKS
#define ZS_DQ_BLOCKS 4194304
#endif
constexpr int kDqUnroll = ZS_DQ_UNROLL;  // lane-vectors per lane per wave sweep
constexpr int kDqBlocks = ZS_DQ_BLOCKS;  // workgroups over all shards (at most)

// Dequantize one lane-vector: 8 codes times the block's scale, each product
// a correctly rounded binary32 multiply (the exact product rounded once),
// then 4 v_cvt_pk_bf16_f32.
__device__ __forceinline__ u32x4 dequant_vec(u32x2 c, float sc) {
  float x[kVec];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = static_cast<float>(static_cast<int8_t>(c.x >> (8 * e))) * sc;
    x[e + 4] = static_cast<float>(static_cast<int8_t>(c.y >> (8 * e))) * sc;
  }
  u32x4 pv;
  pv.x = pack_bf16(x[0], x[1]);
  pv.y = pack_bf16(x[2], x[3]);
  pv.z = pack_bf16(x[4], x[5]);
  pv.w = pack_bf16(x[6], x[7]);
  return pv;
}

// Store 8 bf16 values (16 bytes) at o with the widest stores its alignment
// allows: `align` is 16, 8, 4 or 2 bytes, uniform across the grid's shard.
template <bool NT>
__device__ __forceinline__ void store_bf16x8(uint16_t *o, const u32x4 v, int align) {
  if (align >= 16) {
    st<NT>(v, reinterpret_cast<u32x4 *>(o));
  } else if (align == 8) {
    u32x2 a, b;
    a.x = v.x; a.y = v.y;
    b.x = v.z; b.y = v.w;
    st<NT>(a, reinterpret_cast<u32x2 *>(o));
    st<NT>(b, reinterpret_cast<u32x2 *>(o) + 1);
  } else if (align == 4) {
    unsigned *w = reinterpret_cast<unsigned *>(o);
    st<NT>(v.x, w); st<NT>(v.y, w + 1); st<NT>(v.z, w + 2); st<NT>(v.w, w + 3);
  } else {
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < kVec; ++e) o[e] = static_cast<uint16_t>(w[e / 2] >> (16 * (e & 1)));
  }
}

// qwZ receive side: shard blockIdx.y of the all-gathered int8 shards back to
// its slice of the bf16 parameter vector, bf16(binary32(code * scale)).
// Lane-vectors are counted from the shard's own element 0, so code loads and
// block scales are aligned; the slice of the output starts wherever
// r*ceil(phi/n_d) falls, so each lane stores its 16 bytes with the widest
// stores that alignment allows.  Each wave sweeps U*64 consecutive
// lane-vectors per iteration (lane l takes v0+l, v0+64+l, ...); the shard's
// last partial vector goes element by element.
__global__ void __launch_bounds__(kThreads) dequant_kernel(const DequantArgs A) {
  constexpr int U = kDqUnroll;
  constexpr int64_t span = 64 * U;
  const int r = blockIdx.y;
  const int64_t base = int64_t(r) * A.per;
  if (base >= A.phi) return;
  const int64_t len = A.phi - base < A.per ? A.phi - base : A.per;
  const int64_t off = (base * 2) & 15;  // byte offset of the slice mod 16
  const int align = off == 0 ? 16 : (off & 7) == 0 ? 8 : (off & 3) == 0 ? 4 : 2;
  const int64_t nvec = (len + kVec - 1) / kVec;
  const int64_t nfull = len / kVec;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t stride = int64_t(gridDim.x) * (kThreads / 64) * span;
  uint16_t *out = A.out + base;
  for (int64_t wb = (int64_t(blockIdx.x) * (kThreads / 64) + wave) * span; wb < nvec;
       wb += stride) {
    if (wb + span <= nfull) {
      u32x2 c[U];
      float sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t vec = wb + 64 * u + lane;
        c[u] = __builtin_nontemporal_load(A.c[r] + vec);
        sc[u] = A.s[r][vec >> A.shift];
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        store_bf16x8<kNtOut>(out + (wb + 64 * u + lane) * kVec, dequant_vec(c[u], sc[u]), align);
      continue;
    }
    for (int u = 0; u < U; ++u) {
      const int64_t vec = wb + 64 * u + lane;
      if (vec >= nvec) break;
      const int64_t j0 = vec * kVec;
      const int nvalid = j0 + kVec <= len ? kVec : int(len - j0);
      const float sc = A.s[r][vec >> A.shift];
      if (nvalid == kVec) {
        store_bf16x8<kNtOut>(out + j0, dequant_vec(A.c[r][vec], sc), align);
        continue;
      }
      const int8_t *row = reinterpret_cast<const int8_t *>(A.c[r]) + j0;
#pragma unroll
      for (int e = 0; e < kVec; e += 2) {
        if (e < nvalid) {
          const float x0 = static_cast<float>(row[e]) * sc;
          const float x1 = e + 1 < nvalid ? static_cast<float>(row[e + 1]) * sc : 0.0f;
          const unsigned pb = pack_bf16(x0, x1);
          out[j0 + e] = static_cast<uint16_t>(pb);
          if (e + 1 < nvalid) out[j0 + e + 1] = static_cast<uint16_t>(pb >> 16);
        }
      }
    }
  }
}

// --------------------------------------------------------------- host side

constexpr uint32_t kMagic = 0x5a534831u;

}  // namespace

// The block partials of the allocation-free norm pass
// (zero_shard_gnorm_noalloc): a device array of the library itself, one copy
// on every GPU the library runs on, held until the process ends.  Host code
// never names it for its memory: it uses the device address that
// hipGetSymbolAddress returns for the current GPU (scratch_address below).
constexpr int64_t kStaticPartials = 65536;  // 512 KiB: shards up to 2^30 bf16-row elements
static __device__ __align__(256) double scratch[kStaticPartials];

namespace {

std::mutex g_scratch_mu;
double *g_scratch_dev[64] = {};  // device address of `scratch` per device ordinal

// This GPU's copy of `scratch`, resolved once per device with that device
// current (at zero_shard_init, or at the first allocation-free call).
int scratch_address(double **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ZS_EDEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ZS_EHIP;
    g_scratch_dev[dev] = static_cast<double *>(p);
  }
  *out = g_scratch_dev[dev];
  return ZS_OK;
}

}  // namespace

constexpr int kMaxBucketStreams = 4;  // worker streams of the bucketed calls
constexpr int64_t kBucketAlign = 512;  // bucket lengths are multiples of this

struct zs_handle {
  uint32_t magic;
  zs_desc d;
  int device;
  int cus;
  double *partials;   // norm_partials(shard_len) fp64, library-owned scratch
  bool spill_valid;   // gbar_ws holds the gradient of the pending step
  // bucketed calls, created on first use: worker streams (default
  // priority), their norm partials, one fp64 sum per bucket, fork/join events
  int nworkers;
  hipStream_t workers[kMaxBucketStreams];
  hipEvent_t ev_fork, ev_join[kMaxBucketStreams];
  double *bucket_partials;  // kMaxBucketStreams * bucket_part_len
  int64_t bucket_part_len;
  double *bucket_sums;
  int64_t bucket_cap;
};

namespace {

std::mutex g_live_mu;
std::unordered_set<zs_handle *> g_live;

bool live(zs_handle *h) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  return h && g_live.count(h) && h->magic == kMagic;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int quant_lanes(int32_t block) {
  switch (block) {
    case 32: return 4;
    case 64: return 8;
    case 128: return 16;
    case 256: return 32;
    case 512: return 64;
    default: return -1;
  }
}

int64_t grid_blocks(const zs_handle *h, int64_t nvec, int unroll) {
  const int64_t per_block = int64_t(kThreads) * unroll;
  int64_t need = (nvec + per_block - 1) / per_block;
  if (need < 1) need = 1;
  const int64_t per_cu = ZS_BLOCKS_PER_CU;
  if (per_cu <= 0) return need > 0x7fffffff ? 0x7fffffff : need;  // one-shot grid
  const int64_t cap = int64_t(h->cus) * per_cu;
  return need < cap ? need : cap;
}

// Blocks of the norm pass over n elements: one per 4*64*U lane-vectors.
template <class Src>
int64_t norm_blocks(int64_t n) {
  const int64_t nvec = (n + kVec - 1) / kVec;
  const int64_t per_block = int64_t(kThreads) * Tune<Src>::norm_unroll;
  const int64_t b = (nvec + per_block - 1) / per_block;
  return b < 1 ? 1 : b;
}

// Partials a norm pass over n elements needs, for either contribution format.
int64_t norm_partials(int64_t n) {
  const int64_t a = norm_blocks<Bf16Rows>(n), b = norm_blocks<Q8Rows>(n);
  return a > b ? a : b;
}

Avg make_avg(int32_t nd) {
  Avg a;
  a.nd = nd;
  a.pow2 = (nd & (nd - 1)) == 0;
  a.nd_f = double(nd);
  a.inv_nd = 1.0 / double(nd);
  return a;
}

// A contiguous part [off, off + len) of the shard, launched on `st`; the
// norm pass of a part uses its own partials.  The whole shard is the part
// [0, shard_len) on the handle's stream.
struct Part {
  int64_t off, len;
  hipStream_t st;
  double *partials;
};

Part whole(const zs_handle *h) {
  return Part{0, h->d.shard_len, static_cast<hipStream_t>(h->d.stream), h->partials};
}

// Row pointers advanced to shard element `off` (a multiple of the block of
// any contribution scale and of the 8-element lane vector).
Bf16Rows shifted(const Bf16Rows &s, int nd, int64_t off) {
  Bf16Rows r = s;
  for (int k = 0; k < nd; ++k) r.p[k] = s.p[k] + off / kVec;
  return r;
}
Q8Rows shifted(const Q8Rows &s, int nd, int64_t off) {
  Q8Rows r = s;
  for (int k = 0; k < nd; ++k) {
    r.c[k] = s.c[k] + off / kVec;
    r.s[k] = s.s[k] + ((off / kVec) >> s.shift);
  }
  return r;
}

int check_rows(int nd, const zs_bf16 *const *contrib, Bf16Rows *src) {
  if (!contrib) return ZS_EINVAL;
  for (int k = 0; k < nd; ++k) {
    if (!contrib[k]) return ZS_EINVAL;
    if (!aligned(contrib[k], 16)) return ZS_EALIGN;
    src->p[k] = reinterpret_cast<const u32x4 *>(contrib[k]);
  }
  return ZS_OK;
}

int check_q8(const zs_handle *h, const int8_t *const *codes, const float *const *scales,
             int32_t block, Q8Rows *src) {
  const int lanes = quant_lanes(block);
  if (lanes < 0 || !codes || !scales) return ZS_EINVAL;
  src->shift = 0;
  while ((1 << src->shift) < lanes) ++src->shift;
  for (int k = 0; k < h->d.n_d; ++k) {
    if (!codes[k] || !scales[k]) return ZS_EINVAL;
    if (!aligned(codes[k], 8) || !aligned(scales[k], 4)) return ZS_EALIGN;
    src->c[k] = reinterpret_cast<const u32x2 *>(codes[k]);
    src->s[k] = scales[k];
  }
  return ZS_OK;
}

int current_device_ok(const zs_handle *h) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ZS_EHIP;
  return dev == h->device ? ZS_OK : ZS_EDEVICE;
}

int launched() { return hipGetLastError() == hipSuccess ? ZS_OK : ZS_EHIP; }

// The current device is a gfx950 (checked once per device, then cached).
int device_is_gfx950() {
  static std::mutex mu;
  static int state[64] = {0};  // 0 unknown, 1 gfx950, -1 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ZS_EDEVICE;
  std::lock_guard<std::mutex> lk(mu);
  if (dev < 64 && state[dev]) return state[dev] > 0 ? ZS_OK : ZS_EDEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ZS_EHIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) state[dev] = ok ? 1 : -1;
  return ok ? ZS_OK : ZS_EDEVICE;
}

int gnorm_args_ok(zs_handle *h, double *sumsq_dev) {
  if (!live(h)) return ZS_ESTATE;
  if (!sumsq_dev) return ZS_EINVAL;
  if (!aligned(sumsq_dev, 8)) return ZS_EALIGN;
  return ZS_OK;
}

// a2, first sweep over one part, after the contributions were checked:
// block partials, then the fixed-order final reduction into *sumsq_dev.
// Launch length of the norm pass and of the wide update, in shard elements
// (the values zero_shard.h documents): a one-shot grid over a long shard
// streams slower than the same work split into launches of this many
// elements on the same stream (measured: the 812.5M-element norm pass
// 5.07 -> 4.78 ms in launches of 2^26, the N_d = 64 update over 117M
// elements 3.06 -> 2.90 ms in launches of 2^25).  Both are multiples of
// every block span, so only a part's last launch is ragged; the one-vector
// update gains nothing and stays one launch.
constexpr int64_t kNormLaunchLen = ZS_NORM_LAUNCH_LEN;
constexpr int64_t kWideLaunchLen = ZS_WIDE_LAUNCH_LEN;
static_assert(kNormLaunchLen % (int64_t(kThreads) * kVec * ZS_NORM_UNROLL) == 0 &&
                  kWideLaunchLen % (int64_t(512) * ZS_WIDE_UNROLL) == 0,
              "launch lengths must be whole blocks");

// a2, first sweep over one part, after the contributions were checked:
// block partials (launches of kNormLaunchLen elements, partials in shard
// order), then the fixed-order final reduction into *sumsq_dev.
template <class Src>
int launch_gnorm(int nd, float *gbar_ws, const Src &src, const Part &part, double *sumsq_dev) {
  const int64_t n = part.len;
  const hipStream_t st = part.st;
  int64_t off = 0, nblocks = 0;
  do {  // once for an empty part: its partials are zeros
    const int64_t len = n - off < kNormLaunchLen ? n - off : kNormLaunchLen;
    const int64_t blocks = norm_blocks<Src>(len);
    NormArgs<Src> A;
    A.src = len > 0 ? shifted(src, nd, part.off + off) : src;
    A.avg = make_avg(nd);
    A.n = len;
    A.gbar_out = gbar_ws ? gbar_ws + part.off + off : nullptr;
    A.partials = part.partials + nblocks;
    hipLaunchKernelGGL(gnorm_partial_kernel<Src>, dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                       A);
    if (int rc = launched()) return rc;
    nblocks += blocks;
    off += len;
  } while (off < n);
  hipLaunchKernelGGL(gnorm_final_kernel, dim3(1), dim3(kFinalThreads), 0, st,
                     static_cast<const double *>(part.partials), int(nblocks), sumsq_dev);
  return launched();
}

template <class Src>
int run_gnorm(zs_handle *h, const Src &src, double *sumsq_dev) {
  int rc = current_device_ok(h);
  if (rc) return rc;
  if ((rc = launch_gnorm(h->d.n_d, h->d.gbar_ws, src, whole(h), sumsq_dev))) return rc;
  h->spill_valid = h->d.gbar_ws != nullptr;
  return ZS_OK;
}

int step_args_ok(zs_handle *h, float lr, int64_t t, const double *global_sumsq_dev,
                 bool *use_spill);

// The checks of a step whose constants the device reads from consts_dev.
int step_dev_args_ok(zs_handle *h, const double *consts_dev, const double *global_sumsq_dev,
                     bool *use_spill) {
  if (!consts_dev) return live(h) ? ZS_EINVAL : ZS_ESTATE;
  if (!aligned(consts_dev, 8)) return live(h) ? ZS_EALIGN : ZS_ESTATE;
  return step_args_ok(h, 0.0f, 1, global_sumsq_dev, use_spill);
}

int step_args_ok(zs_handle *h, float lr, int64_t t, const double *global_sumsq_dev,
                 bool *use_spill) {
  if (!live(h)) return ZS_ESTATE;
  const zs_desc &d = h->d;
  if (d.shard_len > 0 && !d.master) return ZS_EINVAL;  // norm-only handle
  if (!zs_args::step_ok(lr, t)) return ZS_EINVAL;
  const bool clip = d.max_norm > 0.0f;
  if (clip && !global_sumsq_dev) return ZS_EINVAL;
  if (clip && !aligned(global_sumsq_dev, 8)) return ZS_EALIGN;
  *use_spill = clip && d.gbar_ws;
  if (*use_spill && !h->spill_valid) return ZS_ESTATE;
  return ZS_OK;
}

// a1 + a2 (apply) + a3 + a4 (+ a5) over one part, after the arguments
// were checked.
// The update's constants at step t with learning rate lr, binary64 from the
// descriptor's binary32 values (the device reads lr, lr*wd, bc1 and bc2
// from a caller's array instead when a launch carries one).
AdamConst make_consts(const zs_desc &d, float lr, int64_t t) {
  AdamConst k;
  const double b1 = d.beta1, b2 = d.beta2;
  k.b1 = b1;
  k.omb1 = 1.0 - b1;
  k.b2 = b2;
  k.omb2 = 1.0 - b2;
  k.bc1 = d.bias_correction ? 1.0 - std::pow(b1, double(t)) : 1.0;
  k.bc2 = d.bias_correction ? 1.0 - std::pow(b2, double(t)) : 1.0;
  k.lr = double(lr);
  k.decay = double(lr) * double(d.weight_decay);
  k.eps = double(d.eps);
  return k;
}

// The step's constants as a launch takes them: fixed (k), or read on the
// device from dyn when dyn is non-null.
struct StepTime {
  AdamConst k;
  const double *dyn;
};

// Whether an update over n_d contribution rows (no spill) takes the wide
// form: from 18 bf16 rows, 32 when it also quantizes, 16 int8 rows (the
// values zero_shard.h documents).  Measured in one process on the same
// buffers, each form against the other: bf16 rows unquantized, the one-chunk
// form 0.5-2.4% faster at 16-17 rows, the wide form 0.5% at 18-20, 3.6% at
// 24, 9% at 32; quantizing, the one-chunk form 6.6-14% faster at 16-24
// rows, the wide form 1% at 32 and 14% at 64; int8 rows, the wide form
// 3.7% faster at 16.
template <class Src>
bool wide_update(const zs_desc &d, bool use_spill) {
  const int from = !kBf16Src<Src>  ? ZS_WIDE_MIN_ROWS_Q8
                   : d.quant_block ? ZS_WIDE_MIN_ROWS_QUANT
                                   : ZS_WIDE_MIN_ROWS;
  return !use_spill && d.n_d >= from;
}

template <class Src>
int launch_step_part(zs_handle *h, const Src &src, const Part &part, const StepTime &when,
                     const double *global_sumsq_dev, bool use_spill) {
  const zs_desc &d = h->d;
  const int64_t n = part.len, off = part.off;
  if (n == 0) return ZS_OK;
  const bool clip = d.max_norm > 0.0f;
  StepArgs<Src> A;
  A.src = use_spill ? src : shifted(src, d.n_d, off);
  A.avg = make_avg(d.n_d);
  A.k = when.k;
  A.dyn = when.dyn;
  A.n = n;
  A.sumsq = clip ? global_sumsq_dev : nullptr;
  A.max_norm = double(d.max_norm);
  A.gbar = use_spill ? d.gbar_ws + off : nullptr;
  A.master = d.master + off;
  A.m = d.m + off;
  A.v = d.v + off;
  A.pout = d.param_out + off;
  A.codes = d.q_codes ? d.q_codes + off : nullptr;
  A.scales = d.q_scales ? d.q_scales + off / (d.quant_block ? d.quant_block : 1) : nullptr;
  const hipStream_t st = part.st;
  const int64_t nvec = (n + kVec - 1) / kVec;
  const bool wide = wide_update<Src>(d, use_spill);
  constexpr int WU = Tune<Src>::wide_unroll;
  const dim3 grid(unsigned(grid_blocks(h, nvec, wide ? WU : 1))), block(kThreads);
#define ZS_LAUNCH_STEP(QL)                                                            \
  do {                                                                                \
    if (wide)                                                                         \
      hipLaunchKernelGGL((step_kernel<QL, WU, Src>), grid, block, 0, st, A);          \
    else                                                                              \
      hipLaunchKernelGGL((step_kernel<QL, 1, Src>), grid, block,                      \
                         QL > 0 && kBf16Src<Src> ? kDenseQLds : 0, st, A);            \
  } while (0)
  switch (d.quant_block) {
    case 0: ZS_LAUNCH_STEP(0); break;
    case 32: ZS_LAUNCH_STEP(4); break;
    case 64: ZS_LAUNCH_STEP(8); break;
    case 128: ZS_LAUNCH_STEP(16); break;
    case 256: ZS_LAUNCH_STEP(32); break;
    case 512: ZS_LAUNCH_STEP(64); break;
    default: return ZS_EINVAL;
  }
#undef ZS_LAUNCH_STEP
  return launched();
}

// The step over one part: the wide update in launches of kWideLaunchLen
// elements, the one-vector update in one.
template <class Src>
int launch_step(zs_handle *h, const Src &src, const Part &part, const StepTime &when,
                const double *global_sumsq_dev, bool use_spill) {
  const bool wide = wide_update<Src>(h->d, use_spill);
  if (!wide || part.len <= kWideLaunchLen)
    return launch_step_part(h, src, part, when, global_sumsq_dev, use_spill);
  for (int64_t o = 0; o < part.len; o += kWideLaunchLen) {
    const int64_t len = part.len - o < kWideLaunchLen ? part.len - o : kWideLaunchLen;
    const Part p{part.off + o, len, part.st, part.partials};
    if (int rc = launch_step_part(h, src, p, when, global_sumsq_dev, use_spill)) return rc;
  }
  return ZS_OK;
}

template <class Src>
int run_step(zs_handle *h, const Src &src, const StepTime &when, const double *global_sumsq_dev,
             bool use_spill) {
  int rc = current_device_ok(h);
  if (rc) return rc;
  h->spill_valid = false;
  return launch_step(h, src, whole(h), when, global_sumsq_dev, use_spill);
}

// ------------------------------------------------------------ bucketed calls

// Fixed-order sum of the per-bucket sums: bucket 0 first.
__global__ void __launch_bounds__(64) bucket_sum_kernel(const double *sums, int64_t nb,
                                                        double *out) {
  if (threadIdx.x != 0) return;
  double s = 0.0;
  for (int64_t j = 0; j < nb; ++j) s += sums[j];
  *out = s;
}

int bucket_args_ok(const zs_handle *h, int64_t bucket_len, int32_t streams) {
  if (bucket_len <= 0 || bucket_len % kBucketAlign != 0) return ZS_EINVAL;
  if (streams < 1 || streams > kMaxBucketStreams) return ZS_EINVAL;
  (void)h;
  return ZS_OK;
}

int64_t bucket_count(const zs_handle *h, int64_t bucket_len) {
  return (h->d.shard_len + bucket_len - 1) / bucket_len;
}

// Worker streams, events and scratch for `streams` workers and `nb`
// buckets of bucket_len elements (created or grown here, before anything
// is launched).
int bucket_setup(zs_handle *h, int32_t streams, int64_t nb, int64_t bucket_len) {
  if (!h->ev_fork && hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess)
    return ZS_EHIP;
  while (h->nworkers < streams) {
    const int w = h->nworkers;
    if (hipStreamCreateWithFlags(&h->workers[w], hipStreamNonBlocking) != hipSuccess)
      return ZS_EHIP;
    if (hipEventCreateWithFlags(&h->ev_join[w], hipEventDisableTiming) != hipSuccess) {
      (void)hipStreamDestroy(h->workers[w]);
      return ZS_EHIP;
    }
    ++h->nworkers;
  }
  const int64_t part_len = norm_partials(bucket_len);
  if (nb > h->bucket_cap || part_len > h->bucket_part_len) {
    // the old arrays may still be in use by queued work
    if (hipStreamSynchronize(static_cast<hipStream_t>(h->d.stream)) != hipSuccess) return ZS_EHIP;
    for (int w = 0; w < h->nworkers; ++w)
      if (hipStreamSynchronize(h->workers[w]) != hipSuccess) return ZS_EHIP;
  }
  if (nb > h->bucket_cap) {
    if (h->bucket_sums) (void)hipFree(h->bucket_sums);
    h->bucket_sums = nullptr;
    h->bucket_cap = 0;
    if (hipMalloc(&h->bucket_sums, nb * sizeof(double)) != hipSuccess) return ZS_ENOMEM;
    h->bucket_cap = nb;
  }
  if (part_len > h->bucket_part_len) {
    if (h->bucket_partials) (void)hipFree(h->bucket_partials);
    h->bucket_partials = nullptr;
    h->bucket_part_len = 0;
    if (hipMalloc(&h->bucket_partials, kMaxBucketStreams * part_len * sizeof(double)) !=
        hipSuccess)
      return ZS_ENOMEM;
    h->bucket_part_len = part_len;
  }
  return ZS_OK;
}

// Workers 0..streams-1 start after everything queued on the handle's stream.
int fork_workers(zs_handle *h, int32_t streams) {
  const hipStream_t st = static_cast<hipStream_t>(h->d.stream);
  if (hipEventRecord(h->ev_fork, st) != hipSuccess) return ZS_EHIP;
  for (int w = 0; w < streams; ++w)
    if (hipStreamWaitEvent(h->workers[w], h->ev_fork, 0) != hipSuccess) return ZS_EHIP;
  return ZS_OK;
}

// The handle's stream continues after everything queued on the workers.
int join_workers(zs_handle *h, int32_t streams) {
  const hipStream_t st = static_cast<hipStream_t>(h->d.stream);
  for (int w = 0; w < streams; ++w) {
    if (hipEventRecord(h->ev_join[w], h->workers[w]) != hipSuccess) return ZS_EHIP;
    if (hipStreamWaitEvent(st, h->ev_join[w], 0) != hipSuccess) return ZS_EHIP;
  }
  return ZS_OK;
}

int wait_ready(hipStream_t st, const void *const *ready, int64_t j) {
  if (!ready || !ready[j]) return ZS_OK;
  hipEvent_t e = static_cast<hipEvent_t>(const_cast<void *>(ready[j]));
  return hipStreamWaitEvent(st, e, 0) == hipSuccess ? ZS_OK : ZS_EHIP;
}

int release_buckets(zs_handle *h) {
  int rc = ZS_OK;
  for (int w = 0; w < h->nworkers; ++w) {
    if (hipStreamSynchronize(h->workers[w]) != hipSuccess) rc = ZS_EHIP;
    if (hipStreamDestroy(h->workers[w]) != hipSuccess) rc = ZS_EHIP;
    if (hipEventDestroy(h->ev_join[w]) != hipSuccess) rc = ZS_EHIP;
  }
  h->nworkers = 0;
  if (h->ev_fork && hipEventDestroy(h->ev_fork) != hipSuccess) rc = ZS_EHIP;
  h->ev_fork = nullptr;
  if (h->bucket_partials && hipFree(h->bucket_partials) != hipSuccess) rc = ZS_EHIP;
  if (h->bucket_sums && hipFree(h->bucket_sums) != hipSuccess) rc = ZS_EHIP;
  h->bucket_partials = h->bucket_sums = nullptr;
  h->bucket_cap = 0;
  h->bucket_part_len = 0;
  return rc;
}

// The bucketed norm pass after the arguments were checked: bucket j on
// worker j mod streams once ready[j] has fired, its sum into bucket_sums[j],
// then the sums in bucket order on the handle's stream.
template <class Src>
int run_gnorm_bucketed(zs_handle *h, const Src &src, int64_t bucket_len, int32_t streams,
                       const void *const *ready, double *sumsq_dev) {
  int rc = current_device_ok(h);
  if (rc) return rc;
  const int64_t n = h->d.shard_len;
  const int64_t nb = bucket_count(h, bucket_len);
  if (nb == 0) return run_gnorm(h, src, sumsq_dev);  // empty shard: S = 0
  if ((rc = bucket_setup(h, streams, nb, bucket_len))) return rc;
  if ((rc = fork_workers(h, streams))) return rc;
  for (int64_t j = 0; j < nb; ++j) {
    const int w = int(j % streams);
    if ((rc = wait_ready(h->workers[w], ready, j))) return rc;
    const int64_t off = j * bucket_len;
    const Part part{off, n - off < bucket_len ? n - off : bucket_len, h->workers[w],
                    h->bucket_partials + int64_t(w) * h->bucket_part_len};
    if ((rc = launch_gnorm(h->d.n_d, h->d.gbar_ws, src, part, h->bucket_sums + j)))
      return rc;
  }
  if ((rc = join_workers(h, streams))) return rc;
  hipLaunchKernelGGL(bucket_sum_kernel, dim3(1), dim3(64), 0,
                     static_cast<hipStream_t>(h->d.stream),
                     static_cast<const double *>(h->bucket_sums), nb, sumsq_dev);
  if ((rc = launched())) return rc;
  h->spill_valid = h->d.gbar_ws != nullptr;
  return ZS_OK;
}

// The bucketed update after the arguments were checked.
template <class Src>
int run_step_bucketed(zs_handle *h, const Src &src, int64_t bucket_len, int32_t streams,
                      const void *const *ready, float lr, int64_t t,
                      const double *global_sumsq_dev, bool use_spill) {
  int rc = current_device_ok(h);
  if (rc) return rc;
  const int64_t n = h->d.shard_len;
  const int64_t nb = bucket_count(h, bucket_len);
  h->spill_valid = false;
  if (nb == 0) return ZS_OK;
  if ((rc = bucket_setup(h, streams, 0, 0))) return rc;
  if ((rc = fork_workers(h, streams))) return rc;
  for (int64_t j = 0; j < nb; ++j) {
    const int w = int(j % streams);
    if ((rc = wait_ready(h->workers[w], ready, j))) return rc;
    const int64_t off = j * bucket_len;
    const Part part{off, n - off < bucket_len ? n - off : bucket_len, h->workers[w], nullptr};
    if ((rc = launch_step(h, src, part, StepTime{make_consts(h->d, lr, t), nullptr},
                          global_sumsq_dev, use_spill)))
      return rc;
  }
  return join_workers(h, streams);
}

}  // namespace

extern "C" {

const char *zero_shard_strerror(int code) {
  switch (code) {
    case ZS_OK: return "ok";
    case ZS_EINVAL: return "invalid argument";
    case ZS_EALIGN: return "pointer not aligned as required";
    case ZS_ENOMEM: return "device scratch allocation failed";
    case ZS_EHIP: return "HIP runtime error or kernel launch failure";
    case ZS_EDEVICE: return "current device is not the gfx950 the handle was made on";
    case ZS_ESTATE: return "call out of order or handle not live";
    case ZS_ETOOBIG: return "shard too long for the allocation-free call's static scratch";
    default: return "unknown zero_shard status";
  }
}

int zero_shard_init(const zs_desc *d, zs_handle **out) {
  if (!d || !out) return ZS_EINVAL;
  *out = nullptr;
  if (!zs_args::geometry_ok(*d) || !zs_args::hyper_ok(*d)) return ZS_EINVAL;
  const int64_t n = d->shard_len;
  if (n > 0) {
    // state and output: all four, or none (a norm-only handle, e.g. for an
    // offloaded update whose state lives in host memory)
    const int given = !!d->master + !!d->m + !!d->v + !!d->param_out;
    if (given != 0 && given != 4) return ZS_EINVAL;
    if (given == 0 && !d->gbar_ws) return ZS_EINVAL;
    if (!aligned(d->master, 16) || !aligned(d->m, 16) || !aligned(d->v, 16) ||
        !aligned(d->param_out, 16))
      return ZS_EALIGN;
    if (d->quant_block > 0) {
      if (!d->q_codes || !d->q_scales) return ZS_EINVAL;
      if (!aligned(d->q_codes, 8) || !aligned(d->q_scales, 4)) return ZS_EALIGN;
    }
    if (d->gbar_ws && !aligned(d->gbar_ws, 16)) return ZS_EALIGN;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ZS_EDEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ZS_EHIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return ZS_EDEVICE;
  // the allocation-free calls' scratch on this device: resolved here, at
  // set-up, so that those calls never have to
  double *static_partials = nullptr;
  if (int rc = scratch_address(&static_partials)) return rc;
  zs_handle *h = new (std::nothrow) zs_handle();
  if (!h) return ZS_ENOMEM;
  h->magic = kMagic;
  h->d = *d;
  h->device = dev;
  h->cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  h->spill_valid = false;
  if (hipMalloc(&h->partials, norm_partials(n) * sizeof(double)) != hipSuccess) {
    delete h;
    return ZS_ENOMEM;
  }
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    g_live.insert(h);
  }
  *out = h;
  return ZS_OK;
}

int zero_shard_gnorm(zs_handle *h, const zs_bf16 *const *contrib, double *sumsq_dev) {
  Bf16Rows src;
  std::memset(&src, 0, sizeof src);
  int rc = gnorm_args_ok(h, sumsq_dev);
  if (rc) return rc;
  if (h->d.shard_len > 0 && (rc = check_rows(h->d.n_d, contrib, &src))) return rc;
  return run_gnorm(h, src, sumsq_dev);
}

int zero_shard_gnorm_q8(zs_handle *h, const int8_t *const *codes, const float *const *scales,
                        int32_t block, double *sumsq_dev) {
  Q8Rows src;
  std::memset(&src, 0, sizeof src);
  int rc = gnorm_args_ok(h, sumsq_dev);
  if (rc) return rc;
  if (quant_lanes(block) < 0) return ZS_EINVAL;
  if (h->d.shard_len > 0 && (rc = check_q8(h, codes, scales, block, &src))) return rc;
  return run_gnorm(h, src, sumsq_dev);
}

int zero_shard_gnorm_noalloc(const zs_desc *d, const zs_bf16 *const *contrib,
                             double *sumsq_dev) {
  if (!d || !sumsq_dev) return ZS_EINVAL;
  if (!zs_args::geometry_ok(*d)) return ZS_EINVAL;
  if (!aligned(sumsq_dev, 8)) return ZS_EALIGN;
  const int64_t n = d->shard_len;
  Bf16Rows src;
  std::memset(&src, 0, sizeof src);
  if (n > 0) {
    if (d->gbar_ws && !aligned(d->gbar_ws, 16)) return ZS_EALIGN;
    if (int rc = check_rows(d->n_d, contrib, &src)) return rc;
  }
  if (norm_blocks<Bf16Rows>(n) > kStaticPartials) return ZS_ETOOBIG;
  int rc = device_is_gfx950();
  if (rc) return rc;
  double *partials = nullptr;
  if ((rc = scratch_address(&partials))) return rc;
  const Part part{0, n, static_cast<hipStream_t>(d->stream), partials};
  return launch_gnorm(d->n_d, d->gbar_ws, src, part, sumsq_dev);
}

int zero_shard_step(zs_handle *h, const zs_bf16 *const *contrib, float lr, int64_t t,
                    const double *global_sumsq_dev) {
  Bf16Rows src;
  std::memset(&src, 0, sizeof src);
  bool spill = false;
  int rc = step_args_ok(h, lr, t, global_sumsq_dev, &spill);
  if (rc) return rc;
  if (h->d.shard_len > 0 && !spill && (rc = check_rows(h->d.n_d, contrib, &src))) return rc;
  return run_step(h, src, StepTime{make_consts(h->d, lr, t), nullptr}, global_sumsq_dev, spill);
}

int zero_shard_step_consts(const zs_desc *d, float lr, int64_t t, double *out) {
  if (!d || !out) return ZS_EINVAL;
  if (!zs_args::hyper_ok(*d) || !zs_args::step_ok(lr, t)) return ZS_EINVAL;
  const AdamConst k = make_consts(*d, lr, t);
  out[0] = k.lr;
  out[1] = k.decay;
  out[2] = k.bc1;
  out[3] = k.bc2;
  return ZS_OK;
}

int zero_shard_step_dev(zs_handle *h, const zs_bf16 *const *contrib, const double *consts_dev,
                        const double *global_sumsq_dev) {
  Bf16Rows src;
  std::memset(&src, 0, sizeof src);
  bool spill = false;
  int rc = step_dev_args_ok(h, consts_dev, global_sumsq_dev, &spill);
  if (rc) return rc;
  if (h->d.shard_len > 0 && !spill && (rc = check_rows(h->d.n_d, contrib, &src))) return rc;
  // b1, b2, eps from the descriptor; lr, lr*wd, bc1, bc2 from consts_dev
  return run_step(h, src, StepTime{make_consts(h->d, 0.0f, 1), consts_dev}, global_sumsq_dev,
                  spill);
}

int zero_shard_step_q8(zs_handle *h, const int8_t *const *codes, const float *const *scales,
                       int32_t block, float lr, int64_t t, const double *global_sumsq_dev) {
  Q8Rows src;
  std::memset(&src, 0, sizeof src);
  bool spill = false;
  int rc = step_args_ok(h, lr, t, global_sumsq_dev, &spill);
  if (rc) return rc;
  if (!spill && quant_lanes(block) < 0) return ZS_EINVAL;
  if (h->d.shard_len > 0 && !spill && (rc = check_q8(h, codes, scales, block, &src))) return rc;
  return run_step(h, src, StepTime{make_consts(h->d, lr, t), nullptr}, global_sumsq_dev, spill);
}

int zero_shard_quant(zs_handle *h, int32_t block) {
  if (!live(h)) return ZS_ESTATE;
  const zs_desc &d = h->d;
  if (quant_lanes(block) < 0) return ZS_EINVAL;
  const int64_t n = d.shard_len;
  if (n > 0) {
    if (!d.param_out || !d.q_codes || !d.q_scales) return ZS_EINVAL;
    if (!aligned(d.q_codes, 8) || !aligned(d.q_scales, 4)) return ZS_EALIGN;
  }
  int rc = current_device_ok(h);
  if (rc) return rc;
  if (n == 0) return ZS_OK;
  QuantArgs A{d.param_out, n, d.q_codes, d.q_scales};
  const hipStream_t st = static_cast<hipStream_t>(d.stream);
  const int64_t nvec = (n + kVec - 1) / kVec;
  const dim3 grid(unsigned(grid_blocks(h, nvec, 1))), blk(kThreads);
  switch (block) {
    case 32: hipLaunchKernelGGL(quant_kernel<4>, grid, blk, 0, st, A); break;
    case 64: hipLaunchKernelGGL(quant_kernel<8>, grid, blk, 0, st, A); break;
    case 128: hipLaunchKernelGGL(quant_kernel<16>, grid, blk, 0, st, A); break;
    case 256: hipLaunchKernelGGL(quant_kernel<32>, grid, blk, 0, st, A); break;
    case 512: hipLaunchKernelGGL(quant_kernel<64>, grid, blk, 0, st, A); break;
    default: return ZS_EINVAL;
  }
  return launched();
}

int zero_shard_dequant(const int8_t *const *codes, const float *const *scales, int32_t n_d,
                       int64_t phi, int32_t block, zs_bf16 *param_out, void *stream) {
  if (n_d < 1 || n_d > ZS_MAX_ND || phi < 0) return ZS_EINVAL;
  const int lanes = quant_lanes(block);
  if (lanes < 0) return ZS_EINVAL;
  if (phi == 0) return ZS_OK;
  if (!codes || !scales || !param_out) return ZS_EINVAL;
  if (!aligned(param_out, 16)) return ZS_EALIGN;
  DequantArgs A;
  std::memset(&A, 0, sizeof A);
  A.per = phi / n_d + (phi % n_d != 0);
  A.phi = phi;
  A.out = param_out;
  while ((1 << A.shift) < lanes) ++A.shift;
  int64_t longest = 0;
  for (int r = 0; r < n_d; ++r) {
    const int64_t len = zero_shard_len(phi, n_d, r);
    if (len == 0) continue;
    if (!codes[r] || !scales[r]) return ZS_EINVAL;
    if (!aligned(codes[r], 8) || !aligned(scales[r], 4)) return ZS_EALIGN;
    A.c[r] = reinterpret_cast<const u32x2 *>(codes[r]);
    A.s[r] = scales[r];
    longest = len > longest ? len : longest;
  }
  int rc = device_is_gfx950();
  if (rc) return rc;
  const int64_t nvec = (longest + kVec - 1) / kVec;
  const int64_t per_block = int64_t(kThreads) * kDqUnroll;
  int64_t gx = (nvec + per_block - 1) / per_block;
  const int64_t cap = kDqBlocks / n_d > 1 ? kDqBlocks / n_d : 1;
  if (gx > cap) gx = cap;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL(dequant_kernel, dim3(unsigned(gx), unsigned(n_d)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), A);
  return launched();
}

int zero_shard_gnorm_bucketed(zs_handle *h, const zs_bf16 *const *contrib, int64_t bucket_len,
                              int32_t streams, const void *const *ready, double *sumsq_dev) {
  Bf16Rows src;
  std::memset(&src, 0, sizeof src);
  int rc = gnorm_args_ok(h, sumsq_dev);
  if (rc) return rc;
  if ((rc = bucket_args_ok(h, bucket_len, streams))) return rc;
  if (h->d.shard_len > 0 && (rc = check_rows(h->d.n_d, contrib, &src))) return rc;
  return run_gnorm_bucketed(h, src, bucket_len, streams, ready, sumsq_dev);
}

int zero_shard_gnorm_bucketed_q8(zs_handle *h, const int8_t *const *codes,
                                 const float *const *scales, int32_t block, int64_t bucket_len,
                                 int32_t streams, const void *const *ready, double *sumsq_dev) {
  Q8Rows src;
  std::memset(&src, 0, sizeof src);
  int rc = gnorm_args_ok(h, sumsq_dev);
  if (rc) return rc;
  if (quant_lanes(block) < 0) return ZS_EINVAL;
  if ((rc = bucket_args_ok(h, bucket_len, streams))) return rc;
  if (h->d.shard_len > 0 && (rc = check_q8(h, codes, scales, block, &src))) return rc;
  return run_gnorm_bucketed(h, src, bucket_len, streams, ready, sumsq_dev);
}

int zero_shard_step_bucketed(zs_handle *h, const zs_bf16 *const *contrib, int64_t bucket_len,
                             int32_t streams, const void *const *ready, float lr, int64_t t,
                             const double *global_sumsq_dev) {
  Bf16Rows src;
  std::memset(&src, 0, sizeof src);
  bool use_spill = false;
  int rc = step_args_ok(h, lr, t, global_sumsq_dev, &use_spill);
  if (rc) return rc;
  if ((rc = bucket_args_ok(h, bucket_len, streams))) return rc;
  if (h->d.shard_len > 0 && !use_spill && (rc = check_rows(h->d.n_d, contrib, &src))) return rc;
  return run_step_bucketed(h, src, bucket_len, streams, ready, lr, t, global_sumsq_dev,
                           use_spill);
}

int zero_shard_step_bucketed_q8(zs_handle *h, const int8_t *const *codes,
                                const float *const *scales, int32_t block, int64_t bucket_len,
                                int32_t streams, const void *const *ready, float lr, int64_t t,
                                const double *global_sumsq_dev) {
  Q8Rows src;
  std::memset(&src, 0, sizeof src);
  bool use_spill = false;
  int rc = step_args_ok(h, lr, t, global_sumsq_dev, &use_spill);
  if (rc) return rc;
  if (quant_lanes(block) < 0) return ZS_EINVAL;
  if ((rc = bucket_args_ok(h, bucket_len, streams))) return rc;
  if (h->d.shard_len > 0 && !use_spill && (rc = check_q8(h, codes, scales, block, &src)))
    return rc;
  return run_step_bucketed(h, src, bucket_len, streams, ready, lr, t, global_sumsq_dev,
                           use_spill);
}

int zero_shard_free(zs_handle *h) {
  if (!h) return ZS_OK;
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    if (!g_live.count(h)) return ZS_ESTATE;
    g_live.erase(h);
  }
  int rc = ZS_OK;
  if (hipStreamSynchronize(static_cast<hipStream_t>(h->d.stream)) != hipSuccess) rc = ZS_EHIP;
  if (release_buckets(h) != ZS_OK) rc = ZS_EHIP;
  if (hipFree(h->partials) != hipSuccess) rc = ZS_EHIP;
  h->magic = 0;
  delete h;
  return rc;
}

}  // extern "C"
