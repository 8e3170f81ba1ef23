/*
 * Exhaustive check of the oracle's binary32 -> bf16 rounding over all 2^32
 * patterns against the definition of round-to-nearest, ties-to-even:
 * of the two bf16 neighbours of x (truncation toward zero, and the next
 * pattern away from zero), take the nearer one measured in binary64, which
 * is exact here; on a tie take the one with an even last bit.  The upper
 * neighbour of the largest finite bf16 is 2^128 (the value infinity stands
 * for when rounding overflows).  NaN must stay NaN with its sign.
 * Prints the number of mismatches and exits non-zero if there are any.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint16_t orc_f32_to_bf16(float x);

static double bf16_value(uint32_t bits16) {
  if ((bits16 & 0x7f80u) == 0x7f80u) return (bits16 & 0x8000u) ? -0x1p128 : 0x1p128;
  uint32_t u = bits16 << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

typedef struct { uint64_t lo, hi, bad; uint32_t first_bad; } job_t;

static void *work(void *arg) {
  job_t *j = (job_t *)arg;
  for (uint64_t w = j->lo; w < j->hi; ++w) {
    const uint32_t u = (uint32_t)w;
    float x;
    memcpy(&x, &u, 4);
    const uint16_t got = orc_f32_to_bf16(x);
    int ok;
    if (isnan(x)) {
      ok = ((got & 0x7f80u) == 0x7f80u) && (got & 0x7fu) && ((got >> 15) == (u >> 31));
    } else {
      const uint32_t a = u >> 16;          /* truncation toward zero */
      const uint32_t b = a + 1u;           /* next pattern away from zero */
      const double xa = bf16_value(a), xb = bf16_value(b), xd = (double)x;
      const double da = fabs(xd - xa), db = fabs(xb - xd);
      uint32_t want;
      if (da < db) want = a;
      else if (db < da) want = b;
      else want = (a & 1u) ? b : a;
      ok = (got == (uint16_t)want);
    }
    if (!ok) {
      if (!j->bad) j->first_bad = u;
      j->bad++;
    }
  }
  return NULL;
}

int main(void) {
  enum { T = 8 };
  pthread_t th[T];
  job_t jobs[T];
  const uint64_t total = 1ull << 32, per = total / T;
  for (int i = 0; i < T; ++i) {
    jobs[i].lo = per * i;
    jobs[i].hi = per * (i + 1);
    jobs[i].bad = 0;
    jobs[i].first_bad = 0;
    pthread_create(&th[i], NULL, work, &jobs[i]);
  }
  uint64_t bad = 0;
  for (int i = 0; i < T; ++i) {
    pthread_join(th[i], NULL);
    if (jobs[i].bad && !bad) printf("first mismatch at 0x%08x\n", jobs[i].first_bad);
    bad += jobs[i].bad;
  }
  printf("mismatches %llu\n", (unsigned long long)bad);
  return bad != 0;
}
