// NF4 levels computed on the host from their definition.
// [QLoRA "Innovation 1: 4-bit NormalFloat (NF4)": levels at quantiles of the
//  standard normal so every bin holds an equal share of a normal weight;
//  the code sketch's table uses the outermost quantile (15 + 1/2)/16.]
//
// Construction: t = Phi^-1(31/32); positive levels Phi^-1(1/2 + j*(15/32)/8)/t
// for j = 1..8, negative levels -Phi^-1(1/2 + j*(15/32)/7)/t for j = 1..7,
// and an exact 0.  Phi^-1 is found by bisection on Phi(x) = erfc(-x/sqrt 2)/2
// in long double, then each level is rounded once to fp32.
#include <cmath>

#include "host_codebook.hpp"

namespace qlin {

namespace {

long double phi(long double x) { return 0.5L * erfcl(-x / sqrtl(2.0L)); }

// Phi^-1(p) for p in (1/2, 1).
long double inv_phi(long double p) {
  long double lo = 0.0L, hi = 16.0L;
  for (int i = 0; i < 256; ++i) {
    const long double mid = 0.5L * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (phi(mid) < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5L * (lo + hi);
}

}  // namespace

void nf4_levels(float out[16]) {
  const long double delta = 31.0L / 32.0L;
  const long double half = delta - 0.5L;
  const long double t = inv_phi(delta);
  out[7] = 0.0f;
  for (int j = 1; j <= 7; ++j)
    out[7 - j] = static_cast<float>(-inv_phi(0.5L + j * half / 7.0L) / t);
  for (int j = 1; j <= 8; ++j)
    out[7 + j] = static_cast<float>(inv_phi(0.5L + j * half / 8.0L) / t);
}

}  // namespace qlin
