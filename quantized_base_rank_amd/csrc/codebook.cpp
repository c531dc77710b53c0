// NormalFloat levels computed on the host from their definition.
// [QLoRA "Innovation 1: 4-bit NormalFloat (NF4)": levels at quantiles of the
//  standard normal so every bin holds an equal share of a normal weight;
//  the code sketch's table uses the outermost quantile (15 + 1/2)/16.
//  LQ-LoRA abstract: the bit-width is chosen per matrix, so the same
//  construction is used for 2 and 3 bits.]
//
// Construction for k bits: delta = 1 - 1/2^(k+1) (the outermost quantile
// (2^k - 1/2)/2^k), t = Phi^-1(delta); positive levels
// Phi^-1(1/2 + j (delta - 1/2)/P)/t for j = 1..P, negative levels
// -Phi^-1(1/2 + j (delta - 1/2)/Q)/t for j = 1..Q, with P = 2^(k-1) and
// Q = 2^(k-1) - 1, and an exact 0.  Phi^-1 is found by bisection on
// Phi(x) = erfc(-x/sqrt 2)/2 in long double, then each level is rounded once
// to fp32.
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

void nf_levels(int bits, float* out) {
  const int P = 1 << (bits - 1), Q = P - 1;
  const long double delta = 1.0L - 1.0L / static_cast<long double>(1 << (bits + 1));
  const long double half = delta - 0.5L;
  const long double t = inv_phi(delta);
  out[Q] = 0.0f;
  for (int j = 1; j <= Q; ++j)
    out[Q - j] = static_cast<float>(-inv_phi(0.5L + j * half / Q) / t);
  for (int j = 1; j <= P; ++j)
    out[Q + j] = static_cast<float>(inv_phi(0.5L + j * half / P) / t);
}

void nf4_levels(float out[16]) { nf_levels(4, out); }

}  // namespace qlin
