// ssp64.h -- compact binary64 evaluation of sqrtsoftplus(z) = sqrt(ln(1 + e^z)),
// the router scoring function (FLOW = qiita.com/sukimaengineer/items/
// cd76fec76d49a098abed, config table: "sqrtsoftplus").
//
// Used to certify the binary32 rounding of the score, so it only needs a
// relative error far below 2^-40 (the kernel assumes 2^-40); its measured
// error is checked against a binary128 reference by the CPU tests.  Written
// out in plain IEEE operations so that the same source compiles for the host
// (tests) and the device (the router kernel), and so that the kernel stays
// small: a large inlined libm sequence here made the scoring kernel several
// times slower than its memory traffic.
//
//   softplus(z) = max(z, 0) + ln(1 + t),   t = e^-|z| in (0, 1]
//   e^-a:  -a log2(e) = k + f/ln2, |f| <= ln2/2,  e^-a = 2^k e^f, Taylor to f^13
//   ln(1+t) = 2 atanh(u), u = t / (2 + t) in [0, 1/3], series to u^29
#pragma once

#include <math.h>

#ifndef DS4_HD
#if defined(__HIPCC__)
#define DS4_HD __host__ __device__
#else
#define DS4_HD
#endif
#endif

namespace ds4 {

DS4_HD inline double ssp64(float zf) {
  const double z = (double)zf;
  const double a = fabs(z);
  double t = 0.0;
  if (a < 745.0) {
    const double LOG2E = 1.4426950408889634;
    const double LN2_HI = 6.93147180369123816490e-01;  // ln2 split: hi has 21 trailing zero bits
    const double LN2_LO = 1.90821492927058770002e-10;
    const double k = rint(-a * LOG2E);
    const double f = fma(-k, LN2_LO, fma(-k, LN2_HI, -a));
    // e^f, |f| <= 0.347: Horner on the Taylor series up to f^13 / 13!
    double p = 1.0 / 6227020800.0;
    p = fma(p, f, 1.0 / 479001600.0);
    p = fma(p, f, 1.0 / 39916800.0);
    p = fma(p, f, 1.0 / 3628800.0);
    p = fma(p, f, 1.0 / 362880.0);
    p = fma(p, f, 1.0 / 40320.0);
    p = fma(p, f, 1.0 / 5040.0);
    p = fma(p, f, 1.0 / 720.0);
    p = fma(p, f, 1.0 / 120.0);
    p = fma(p, f, 1.0 / 24.0);
    p = fma(p, f, 1.0 / 6.0);
    p = fma(p, f, 0.5);
    p = fma(p, f, 1.0);
    p = fma(p, f, 1.0);
    t = ldexp(p, (int)k);
  }
  // ln(1 + t) = 2 (u + u^3/3 + u^5/5 + ...), u = t / (2 + t)
  const double u = t / (2.0 + t);
  const double u2 = u * u;
  double q = 1.0 / 29.0;
  q = fma(q, u2, 1.0 / 27.0);
  q = fma(q, u2, 1.0 / 25.0);
  q = fma(q, u2, 1.0 / 23.0);
  q = fma(q, u2, 1.0 / 21.0);
  q = fma(q, u2, 1.0 / 19.0);
  q = fma(q, u2, 1.0 / 17.0);
  q = fma(q, u2, 1.0 / 15.0);
  q = fma(q, u2, 1.0 / 13.0);
  q = fma(q, u2, 1.0 / 11.0);
  q = fma(q, u2, 1.0 / 9.0);
  q = fma(q, u2, 1.0 / 7.0);
  q = fma(q, u2, 1.0 / 5.0);
  q = fma(q, u2, 1.0 / 3.0);
  q = fma(q, u2, 1.0);
  const double l1p = 2.0 * u * q;
  const double sp = (z > 0.0 ? z : 0.0) + l1p;
  return sqrt(sp);
}

}  // namespace ds4
