/*
 * zs_gen.h -- seeded, counter-based input generator.
 *
 * One definition, compiled twice: by g++ for the host (gen_host.cpp) and by
 * hipcc for the device (gen_dev.hip).  Both builds produce bit-identical
 * values, so the GPU can fill HBM with a workload while the CPU checker
 * regenerates any window of it on demand.  This file holds none of the
 * optimizer's arithmetic; it only makes numbers.
 *
 * Definition.  A tensor is named by a key (seed, tensor id, step, rank).
 *   h   = mix64(seed ^ tid<<56 ^ step<<32 ^ rank)
 *   w_j = mix64(h + (4 i + j + 1) * 0x9E3779B97F4A7C15),  j = 0..3
 * mix64 is the splitmix64 output finalizer (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).
 * Element i of a standard normal draw is the Irwin-Hall(12) sum of the
 * twelve 16-bit fields of w_0..w_2, centred and scaled:
 *   z = (sum_fields - 12 * 32767.5) * 2^-16      (exact in binary32)
 * which has mean 0, variance 1 and support [-6, 6].  A draw of N(0, sigma)
 * is x = fl32(sigma * z); with outliers on, x = fl32(100 * x) when
 * (w_3 >> 32) mod 100 == 0, i.e. for 1% of the elements.  Int8 gradient
 * codes (quantized contributions) come from the same sum by an integer
 * shift; their per-block scales are |N(0, sigma)| draws of a separate key.  Only integer
 * operations and single IEEE binary32 multiplies are used (no contraction is
 * possible), so host and device agree bit for bit.
 */
#ifndef ZS_GEN_H
#define ZS_GEN_H

#include <stdint.h>

#ifdef __HIPCC__
#define ZSG_FN __host__ __device__ inline
#else
#define ZSG_FN static inline
#endif

#define ZSG_GOLDEN 0x9E3779B97F4A7C15ull

/* tensor ids */
enum { ZSG_MASTER = 0, ZSG_MOM = 1, ZSG_VAR = 2, ZSG_GRAD = 3, ZSG_AUX = 4, ZSG_GRAD_SCALE = 5 };
/* output kinds */
enum { ZSG_KIND_NORMAL = 0, ZSG_KIND_ABS = 1 };

ZSG_FN uint64_t zsg_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

ZSG_FN uint64_t zsg_key(uint64_t seed, uint32_t tid, uint32_t step, uint32_t rank) {
  return zsg_mix64(seed ^ ((uint64_t)tid << 56) ^ ((uint64_t)step << 32) ^ (uint64_t)rank);
}

/* Sum of the four 16-bit fields of w. */
ZSG_FN uint32_t zsg_fields4(uint64_t w) {
  const uint64_t pair = (w & 0x0000FFFF0000FFFFull) + ((w >> 16) & 0x0000FFFF0000FFFFull);
  return (uint32_t)(pair & 0xFFFFFFFFull) + (uint32_t)(pair >> 32);
}

/* Standard-normal-like value for element i of the tensor keyed h. */
ZSG_FN float zsg_stdnormal(uint64_t h, uint64_t i) {
  const uint64_t base = h + (4u * i + 1u) * ZSG_GOLDEN;
  const uint32_t s = zsg_fields4(zsg_mix64(base)) +
                     zsg_fields4(zsg_mix64(base + ZSG_GOLDEN)) +
                     zsg_fields4(zsg_mix64(base + 2u * ZSG_GOLDEN));
  /* 12 * 32767.5 = 393210; s - 393210 fits in 20 bits, exact in binary32 */
  const int32_t c = (int32_t)s - 393210;
  return (float)c * 0x1p-16f;
}

ZSG_FN int zsg_is_outlier(uint64_t h, uint64_t i) {
  const uint64_t w3 = zsg_mix64(h + (4u * i + 4u) * ZSG_GOLDEN);
  return ((uint32_t)(w3 >> 32) % 100u) == 0u;
}

/* x = sigma * z, optionally with 1% x100 outliers; ZSG_KIND_ABS returns |x|. */
ZSG_FN float zsg_value(uint64_t h, uint64_t i, float sigma, int outliers, int kind) {
  float x = sigma * zsg_stdnormal(h, i);
  if (outliers && zsg_is_outlier(h, i)) x = 100.0f * x;
  if (kind == ZSG_KIND_ABS && x < 0.0f) x = -x;
  return x;
}

/* An int8 code for element i: the same twelve-field sum, centred, divided
 * by 2^11 with an arithmetic shift (floor), clamped to [-127, 127]:
 * integers with standard deviation 32 (the shape of block-quantized
 * gradients whose block absmax sits near 4 sigma).  Integer-only. */
ZSG_FN int8_t zsg_code(uint64_t h, uint64_t i) {
  const uint64_t base = h + (4u * i + 1u) * ZSG_GOLDEN;
  const uint32_t s = zsg_fields4(zsg_mix64(base)) +
                     zsg_fields4(zsg_mix64(base + ZSG_GOLDEN)) +
                     zsg_fields4(zsg_mix64(base + 2u * ZSG_GOLDEN));
  int32_t c = ((int32_t)s - 393210) >> 11;
  c = c > 127 ? 127 : (c < -127 ? -127 : c);
  return (int8_t)c;
}

/* Nearest bf16 (ties to even) of a finite binary32, as a bit pattern. */
ZSG_FN uint16_t zsg_to_bf16(float x) {
  union { float f; uint32_t u; } c;
  c.f = x;
  const uint32_t u = c.u;
  const uint32_t round = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + round) >> 16);
}

#endif
