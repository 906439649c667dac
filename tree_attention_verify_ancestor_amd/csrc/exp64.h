// float64 sums of exp(x - m) over float32 logits x <= m, which the draft-tree expansion
// normalises with ("EAGLE" notes, "Well-Calibrated Draft Model": a confidence is a
// softmax of the draft logits).
//
// d = x - m is exact in float64.  With t = fl(d * 64 / ln 2) = n + r, n the nearest
// integer and r = t - n (exact, |r| <= 1/2), exp(d) = 2^floor(n/64) * 2^((n mod 64)/64)
// * 2^(r/64): the middle factor from a table of the 64 values 2^(i/64) rounded to
// nearest, the last from its Taylor polynomial to degree 5 (remainder below 4e-17
// relative).  Each term is within about (4 + |d|) * 2^-53 relative of exp(d): the |d|
// part comes from rounding t and only matters where the term is small.
//
// A NaN d, or d = -inf, gives NaN (r is NaN), never a finite value: a sum that comes
// out NaN flags the row.  Very negative finite d gives 0 (n is clamped at -2^30 for the
// integer conversion; r keeps the unclamped n).
//
// Host and device share this code, so the CPU tests check the device arithmetic.
#pragma once

#include <math.h>

#ifndef TV_HD
#define TV_HD __host__ __device__
#endif

namespace tv {

constexpr int kExpTab = 64;
// 2^(i/64) for i = 0..63, each rounded to the nearest float64
constexpr double kExp2Frac64[kExpTab] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0,
};

constexpr double kExpK = 0x1.71547652b82fep+6;        // 64 / ln 2

// exp(d) for d <= 0; `tab` holds kExp2Frac64 (on the device: a copy in LDS)
TV_HD inline double exp_nonpos(double d, const double* tab) {
  const double t = d * kExpK;
  const double n = rint(t);
  const double r = t - n;                                      // exact
  const int ni = (int)fmax(n, -0x1p30);
  // (ln 2 / 64)^i / i!, i = 5 .. 1
  double p = 0x1.5d87fe78a6731p-40;
  p = fma(p, r, 0x1.3b2ab6fba4e77p-31);
  p = fma(p, r, 0x1.c6b08d704a0c0p-23);
  p = fma(p, r, 0x1.ebfbdff82c58fp-15);
  p = fma(p, r, 0x1.62e42fefa39efp-7);
  p = fma(p, r, 1.0);
  return ldexp(p * tab[ni & (kExpTab - 1)], ni >> 6);
}

}  // namespace tv
