/* Arithmetic identities behind the HIP quantizers' division-free paths,
 * checked on the CPU in IEEE FP32 (round to nearest even, subnormals kept,
 * no contraction; fmaf is the correctly rounded fused multiply-add).
 *
 *   codes <ND>: for ND divisors d spread over [2^-90, 2^100] and every finite
 *     BF16 numerator x with |x| <= d * 2^120, the E2M1 code (nearest-even
 *     ladder, clip to 6, sign kept) of
 *       q = fma(-fma(q0, d, -x), r, q0),  r = RN(1/d), q0 = RN(x r)
 *     equals the code of the IEEE quotient RN(x / d), signed zeros included.
 *   quot <N>: for N random FP32 x in [2^-100, 2^127) and d in [2^-100, 2^100)
 *     with a normal finite quotient, the same q equals RN(x / d).
 *   zeros: q of +0 and -0 keeps the sign for a spread of divisors.
 *
 * Prints the number of checked cases and mismatches; exits 1 on a mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t ubits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static uint32_t e2m1(float v) {
  const float a = fabsf(v);
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return c | ((ubits(v) >> 28) & 8u);
}

/* the residual is formed negated, e = RN(q0 d - x), and q = RN(q0 - e r):
 * -0 then stays -0 (the usual order, RN(q0 + RN(x - q0 d) r), gives +0) */
static float corrected(float x, float d, float r) {
  const float q0 = x * r;
  const float e = fmaf(q0, d, -x);
  return fmaf(-e, r, q0);
}

static uint64_t state = 88172645463325252ull;
static uint64_t next(void) { state ^= state << 13; state ^= state >> 7; state ^= state << 17; return state; }

int main(int argc, char **argv) {
  if (argc != 3) { fprintf(stderr, "usage: %s codes|quot N\n", argv[0]); return 2; }
  const long long n_arg = atoll(argv[2]);
  long long n = 0, bad = 0;
  if (!strcmp(argv[1], "codes")) {
    for (long long i = 0; i < n_arg; ++i) {
      const uint64_t s = next();
      uint32_t m = (uint32_t)((s >> 20) & 0x7FFFFF);
      if (i % 8 == 0) m = 0;
      if (i % 8 == 1) m = 0x7FFFFF;
      float d = bits(((uint32_t)(127 - 90 + s % 190) << 23) | m);
      if (i == 0) d = 0x1p-90f;
      if (i == 1) d = bits(ubits(0x1p100f) - 1);
      const float r = 1.0f / d, lim = d * 0x1p120f;
      for (uint32_t b = 0; b < 65536; ++b) {
        if ((b & 0x7F80) == 0x7F80) continue;  /* Inf, NaN */
        const float x = bits(b << 16);
        if (fabsf(x) > lim) continue;
        ++n;
        if (e2m1(corrected(x, d, r)) != e2m1(x / d)) {
          if (bad < 5) printf("x=%a d=%a\n", x, d);
          ++bad;
        }
      }
    }
  } else if (!strcmp(argv[1], "quot")) {
    for (long long i = 0; i < n_arg; ++i) {
      const float x = bits(((uint32_t)(27 + next() % 227) << 23) | (uint32_t)(next() & 0x7FFFFF));
      const float d = bits(((uint32_t)(27 + next() % 200) << 23) | (uint32_t)(next() & 0x7FFFFF));
      const float ref = x / d;
      if (!isfinite(ref) || ref < 0x1p-126f) continue;
      ++n;
      if (corrected(x, d, 1.0f / d) != ref) {
        if (bad < 5) printf("x=%a d=%a\n", x, d);
        ++bad;
      }
    }
  } else if (!strcmp(argv[1], "zeros")) {
    for (long long i = 0; i < n_arg; ++i) {
      const float d = bits(((uint32_t)(127 - 90 + next() % 190) << 23) | (uint32_t)(next() & 0x7FFFFF));
      for (int sgn = 0; sgn < 2; ++sgn) {
        const float x = sgn ? -0.0f : 0.0f;
        const float q = corrected(x, d, 1.0f / d);
        ++n;
        if (q != 0.0f || signbit(q) != signbit(x)) ++bad;
      }
    }
  } else {
    return 2;
  }
  printf("checked %lld: %lld mismatches\n", n, bad);
  return bad != 0;
}
