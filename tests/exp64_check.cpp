// Host build of the expansion's float64 exp (csrc/exp64.h, shared with the device code):
// prints the table, the worst error over random arguments scaled by the stated bound
// (4 + |d|) * 2^-53, and the special values.  Driven by tests/test_exp64_host.py.
#include <float.h>
#include <math.h>
#include <stdio.h>

#include <random>

#include "exp64.h"

int main() {
  for (int i = 0; i < tv::kExpTab; ++i) printf("tab %d %a\n", i, tv::kExp2Frac64[i]);
  std::mt19937_64 g(20261203);
  std::normal_distribution<float> nd(0.f, 1.f);
  std::uniform_real_distribution<float> sc(-2.f, 4.f);
  double worst = 0.0;
  long n = 0;
  for (int i = 0; i < 2000000; ++i) {
    // float32 logits x <= m over scales 0.01 .. 1e4, d = x - m exact in float64
    const float s = powf(10.f, sc(g));
    const float a = nd(g) * s, b = nd(g) * s;
    const float m = fmaxf(a, b), x = i % 7 == 0 ? m : fminf(a, b);
    const double d = (double)x - (double)m;
    if (d < -708.0) continue;                     // results below the normal range
    const long double ex = expl((long double)d);
    const double got = tv::exp_nonpos(d, tv::kExp2Frac64);
    const double scaled = (double)fabsl(((long double)got - ex) / ex) / ((4.0 - d) * 0x1p-53);
    if (scaled > worst) worst = scaled;
    ++n;
  }
  printf("checked %ld\n", n);
  printf("worst %.6f\n", worst);
  printf("zero %a\n", tv::exp_nonpos(0.0, tv::kExp2Frac64));
  printf("minus_one %a %a\n", tv::exp_nonpos(-1.0, tv::kExp2Frac64), exp(-1.0));
  printf("nan %d\n", (int)isnan(tv::exp_nonpos(NAN, tv::kExp2Frac64)));
  printf("neg_inf %d\n", (int)isnan(tv::exp_nonpos(-INFINITY, tv::kExp2Frac64)));
  printf("huge %a\n", tv::exp_nonpos(-2.0 * (double)FLT_MAX, tv::kExp2Frac64));
  printf("deep %a\n", tv::exp_nonpos(-800.0, tv::kExp2Frac64));
  return 0;
}
