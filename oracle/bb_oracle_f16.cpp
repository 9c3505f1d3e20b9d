/*
 * The CPU oracle in half precision (fp16).  TEST INFRASTRUCTURE ONLY.
 *
 * The band -> bidiagonal reduction of bb_oracle.c, the same body text
 * (bb_oracle_body.h) instantiated a third time with REAL = an emulated
 * IEEE binary16 type, so the steps are those of the fp32 and fp64 oracle
 * (page "Accelerating Bidiagonalization of Banded Matrices through
 * Memory-Aware Bulge-Chasing on GPUs", the FP16 variant of the reduction run
 * in the accuracy study).  The host compiler has no native binary16, so:
 *
 *   - a value is its 16 bits (the memory layout of numpy.float16);
 *   - +, -, *, / and sqrt are evaluated in binary32 (sqrt and division
 *     correctly rounded) and rounded once to binary16, to nearest, ties to
 *     even.  binary32 has 24 >= 2*11 + 2 significand bits, so that double
 *     rounding gives the correctly rounded binary16 result;
 *   - fma(a, b, c) is rounded once: a*b is exact in binary64, a*b + c is
 *     formed exactly as s + e (TwoSum), s is rounded to binary16, and when s
 *     sits exactly halfway between two binary16 numbers the sign of e
 *     decides;
 *   - subnormals are kept; overflow gives infinity.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

namespace {

// binary16 bits -> binary64 (exact)
double h2d(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp(double(m), -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(double(1024 + m), e - 25);
  return s ? -v : v;
}

// binary64 -> binary16, round to nearest, ties to even
uint16_t d2h(double x) {
  const uint16_t sign = signbit(x) ? 0x8000 : 0;
  const double ax = fabs(x);
  if (ax != ax) return uint16_t(sign | 0x7e00);
  if (ax >= 65520.0) return uint16_t(sign | 0x7c00);
  if (ax < 6.103515625e-05) {  // below 2^-14: multiples of 2^-24
    const double q = nearbyint(ldexp(ax, 24));
    return uint16_t(sign | uint16_t(q));  // q = 1024 is the smallest normal
  }
  int E;
  frexp(ax, &E);  // ax in [2^(E-1), 2^E)
  double q = nearbyint(ldexp(ax, 11 - E));
  if (q == 2048.0) {
    q = 1024.0;
    ++E;
  }
  const int be = E - 1 + 15;
  if (be >= 31) return uint16_t(sign | 0x7c00);
  return uint16_t(sign | (be << 10) | (int(q) - 1024));
}

struct H {
  uint16_t bits;
  H() = default;
  H(int x) : bits(d2h(double(x))) {}
  H(double x) : bits(d2h(x)) {}
  static H from_bits(uint16_t b) {
    H h;
    h.bits = b;
    return h;
  }
  double d() const { return h2d(bits); }
};

// binary32 evaluation of a binary16 operation, then one rounding to binary16
H op32(float r) { return H(double(r)); }
[[maybe_unused]] H operator+(H a, H b) { return op32(float(a.d()) + float(b.d())); }
H operator-(H a, H b) { return op32(float(a.d()) - float(b.d())); }
H operator*(H a, H b) { return op32(float(a.d()) * float(b.d())); }
H operator/(H a, H b) { return op32(float(a.d()) / float(b.d())); }
H operator-(H a) { return H::from_bits(uint16_t(a.bits ^ 0x8000)); }
bool operator==(H a, H b) { return a.d() == b.d(); }
bool operator>=(H a, H b) { return a.d() >= b.d(); }

H sqrt16(H a) { return op32(sqrtf(float(a.d()))); }
[[maybe_unused]] H fabs16(H a) { return H::from_bits(uint16_t(a.bits & 0x7fff)); }

// fma rounded once: s + e == a*b + c exactly (TwoSum of the exact product
// and c); ties of s between two binary16 numbers go by the sign of e.
H fma16(H a, H b, H c) {
  const double p = a.d() * b.d();  // 22 significant bits: exact
  const double cc = c.d();
  const double s = p + cc;
  const double bb = s - p;
  const double e = (p - (s - bb)) + (cc - bb);
  H r = H(s);
  if (e != 0 && isfinite(s)) {
    const double rv = r.d();
    if (rv != s) {
      // neighbour of r on the other side of s
      const uint16_t mag = uint16_t(r.bits & 0x7fff);
      const bool away = fabs(s) > fabs(rv);  // s lies beyond r (further from 0)
      const uint16_t omag = away ? uint16_t(mag + 1) : uint16_t(mag - 1);
      const H o = H::from_bits(uint16_t((r.bits & 0x8000) | omag));
      // halfway to an infinity means halfway to 2^16
      const double mid = isinf(rv) ? copysign(65520.0, rv) : 0.5 * (rv + o.d());
      if (s == mid) {  // a tie: the exact value lies on the side of e
        const bool up = e > 0;  // towards +infinity
        const bool o_above = o.d() > rv;
        if (up == o_above) r = o;
      }
    }
    // rv == s: s is a binary16 number and |e| is far below its half-ulp
  }
  return r;
}

}  // namespace

extern "C" {

/* Exposed for the oracle's own pins: one rounding of each operation. */
uint16_t bb_oracle_h16_from_double(double x) { return d2h(x); }
double bb_oracle_h16_to_double(uint16_t h) { return h2d(h); }
uint16_t bb_oracle_h16_fma(uint16_t a, uint16_t b, uint16_t c) {
  return fma16(H::from_bits(a), H::from_bits(b), H::from_bits(c)).bits;
}
uint16_t bb_oracle_h16_div(uint16_t a, uint16_t b) { return (H::from_bits(a) / H::from_bits(b)).bits; }
uint16_t bb_oracle_h16_sqrt(uint16_t a) { return sqrt16(H::from_bits(a)).bits; }

#include "bb_oracle.c"

#define REAL H
#define FMA fma16
#define SQRT sqrt16
#define FABS fabs16
#define SUF(name) name##_f16
#include "bb_oracle_body.h"
#undef REAL
#undef FMA
#undef SQRT
#undef FABS
#undef SUF

}  // extern "C"
