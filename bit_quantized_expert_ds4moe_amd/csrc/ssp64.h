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
// The reduction f = -a - k ln2 uses the Cody-Waite splitting of ln 2 (W. J.
// Cody and W. Waite, "Software Manual for the Elementary Functions", 1980):
// a leading part with trailing zero bits, so that k times it is exact, and a
// correction; the two constants are the split published with Sun's fdlibm.
//
// ssp_dd below evaluates the same function in double-double arithmetic
// (unevaluated sums of two binary64 numbers, about 106 bits) with the
// error-free transformations of Knuth (two-sum) and Dekker (two-product, here
// by a fused multiply-add); it decides the binary32 rounding of the rare
// scores that ssp64 leaves undecided.
#pragma once

#include <math.h>
#include <stdint.h>

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

// ---- double-double --------------------------------------------------------
// A value is hi + lo with |lo| <= ulp(hi)/2.  Every function keeps the order
// of operations as written (no contraction: fused multiply-adds appear only
// where written).
struct DD {
  double hi, lo;
};

DS4_HD inline DD dd_two_sum(double a, double b) {
#pragma clang fp contract(off)
  const double s = a + b;
  const double bb = s - a;
  return DD{s, (a - (s - bb)) + (b - bb)};
}
DS4_HD inline DD dd_quick_two_sum(double a, double b) {  // |a| >= |b|
#pragma clang fp contract(off)
  const double s = a + b;
  return DD{s, b - (s - a)};
}
DS4_HD inline DD dd_two_prod(double a, double b) {
#pragma clang fp contract(off)
  const double p = a * b;
  return DD{p, fma(a, b, -p)};
}
DS4_HD inline DD dd_add(DD a, DD b) {
#pragma clang fp contract(off)
  DD s = dd_two_sum(a.hi, b.hi);
  const DD t = dd_two_sum(a.lo, b.lo);
  s.lo += t.hi;
  s = dd_quick_two_sum(s.hi, s.lo);
  s.lo += t.lo;
  return dd_quick_two_sum(s.hi, s.lo);
}
DS4_HD inline DD dd_neg(DD a) { return DD{-a.hi, -a.lo}; }
DS4_HD inline DD dd_mul(DD a, DD b) {
#pragma clang fp contract(off)
  DD p = dd_two_prod(a.hi, b.hi);
  p.lo += a.hi * b.lo + a.lo * b.hi;
  return dd_quick_two_sum(p.hi, p.lo);
}
// a / d for a binary64 d: two quotient digits and a correction
DS4_HD inline DD dd_div_d(DD a, double d) {
#pragma clang fp contract(off)
  const double q1 = a.hi / d;
  DD r = dd_add(a, dd_neg(dd_two_prod(q1, d)));
  const double q2 = r.hi / d;
  r = dd_add(r, dd_neg(dd_two_prod(q2, d)));
  const double q3 = r.hi / d;
  return dd_add(dd_quick_two_sum(q1, q2), DD{q3, 0.0});
}
// a / b: the same with a double-double divisor
DS4_HD inline DD dd_div(DD a, DD b) {
#pragma clang fp contract(off)
  const double q1 = a.hi / b.hi;
  DD r = dd_add(a, dd_neg(dd_mul(DD{q1, 0.0}, b)));
  const double q2 = r.hi / b.hi;
  r = dd_add(r, dd_neg(dd_mul(DD{q2, 0.0}, b)));
  const double q3 = r.hi / b.hi;
  return dd_add(dd_quick_two_sum(q1, q2), DD{q3, 0.0});
}
// sqrt(a), a >= 0: one Newton correction of the binary64 root
DS4_HD inline DD dd_sqrt(DD a) {
#pragma clang fp contract(off)
  if (!(a.hi > 0.0)) return DD{0.0, 0.0};
  const double x = sqrt(a.hi);
  const DD r = dd_add(a, dd_neg(dd_two_prod(x, x)));
  return dd_quick_two_sum(x, r.hi / (2.0 * x));
}

// sqrtsoftplus(z) in double-double, relative error below 2^-96 (measured
// against decimal arithmetic by the CPU tests; the rounding decision below
// allows 2^-90).  Same reduction as ssp64, with ln 2 as a double-double
// (Sun fdlibm's leading 53 bits and the next 53), Taylor terms of e^f to
// f^24 / 24! and the atanh series to u^71 / 71, each Horner step dividing by
// its integer so that no rounded coefficient enters.
DS4_HD inline DD ssp_dd(float zf) {
#pragma clang fp contract(off)
  const double z = (double)zf;
  const double a = fabs(z);
  DD t{0.0, 0.0};
  if (a < 745.0) {
    const double LOG2E = 1.4426950408889634;
    const DD LN2{0x1.62e42fefa39efp-1, 0x1.abc9e3b39803fp-56};
    const double k = rint(-a * LOG2E);
    const DD kln2 = dd_add(dd_two_prod(k, LN2.hi), dd_two_prod(k, LN2.lo));
    const DD f = dd_add(DD{-a, 0.0}, dd_neg(kln2));
    DD p{1.0, 0.0};
    for (int n = 24; n >= 1; n--) p = dd_add(dd_div_d(dd_mul(p, f), (double)n), DD{1.0, 0.0});
    t = DD{ldexp(p.hi, (int)k), ldexp(p.lo, (int)k)};
  }
  // ln(1 + t) = 2 atanh(u), u = t / (2 + t)
  const DD u = dd_div(t, dd_add(DD{2.0, 0.0}, t));
  const DD u2 = dd_mul(u, u);
  DD q = dd_div_d(DD{1.0, 0.0}, 71.0);
  for (int n = 34; n >= 0; n--) q = dd_add(dd_mul(q, u2), dd_div_d(DD{1.0, 0.0}, (double)(2 * n + 1)));
  const DD l1p = dd_mul(DD{2.0, 0.0}, dd_mul(u, q));
  const DD sp = z > 0.0 ? dd_add(DD{z, 0.0}, l1p) : l1p;
  return dd_sqrt(sp);
}

// The binary32 rounding (nearest, ties to even) of a non-negative value
// v = hi + lo known to within a relative error eps.  ok is false when v lies
// within eps * v of a point halfway between two binary32 values, where the
// rounding cannot be decided.
DS4_HD inline float dd_round_f32(DD v, double eps, bool& ok) {
#pragma clang fp contract(off)
  union {
    float f;
    uint32_t u;
  } c, up, dn;
  c.f = (float)v.hi;
  up.u = c.u + 1u;
  dn.f = c.f;
  if (c.u == 0u) dn.u = 0x80000001u;  // -2^-149: the midpoint below 0 is -2^-150
  else dn.u = c.u - 1u;
  const double m_hi = ((double)c.f + (double)up.f) * 0.5;  // exact: 25 bits
  const double m_lo = ((double)dn.f + (double)c.f) * 0.5;
  const double d_hi = (m_hi - v.hi) - v.lo;  // v below the upper midpoint by this
  const double d_lo = (v.hi - m_lo) + v.lo;  // v above the lower midpoint by this
  float r = c.f;
  double dist = d_hi < d_lo ? d_hi : d_lo;
  if (d_hi < 0.0) {  // v.hi sat on the upper midpoint and v.lo pushed it over
    r = up.f;
    dist = -d_hi;
  } else if (d_lo < 0.0) {
    r = dn.f;
    dist = -d_lo;
  }
  ok = dist > eps * v.hi;
  return r;
}

}  // namespace ds4
