/* Exhaustive check behind the prompt packer's scale computation: for every
 * fp32 value r in [0, 2^17] (the range max - min of an fp16 vector is at
 * most 131008), q1 = fma(fma(-q0, Q, r), c, q0) with q0 = r * c and
 * c = RN(1/Q) equals the IEEE quotient r / Q bit for bit.  Usage:
 * div_by_const Q; prints the number of differing values and exits 0 iff
 * there are none. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float asf(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t asu(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

#define BODY                                                  \
  uint64_t bad = 0;                                           \
  for (uint32_t u = 0; u <= top; u++) {                       \
    const float r = asf(u);                                   \
    volatile float rv = r;                                    \
    const float q = rv / qm;                                  \
    const float q0 = r * c;                                   \
    const float q1 = fmaf(fmaf(-q0, qm, r), c, q0);           \
    bad += asu(q1) != asu(q);                                 \
  }                                                           \
  return bad;

__attribute__((target("fma"))) static uint64_t run_fma(float qm, float c, uint32_t top) { BODY }
static uint64_t run_any(float qm, float c, uint32_t top) { BODY }

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  const float qm = (float)atoi(argv[1]);
  volatile float one = 1.0f;
  const float c = one / qm;
  const uint32_t top = asu(131072.0f);
  const uint64_t bad = __builtin_cpu_supports("fma") ? run_fma(qm, c, top) : run_any(qm, c, top);
  printf("%llu\n", (unsigned long long)bad);
  return bad != 0;
}
