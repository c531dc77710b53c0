// Host-side NormalFloat level tables (see codebook.cpp).
#pragma once

namespace qlin {
// 2^bits levels (bits = 2, 3, 4), ascending, into out[0 .. 2^bits - 1]
void nf_levels(int bits, float* out);
void nf4_levels(float out[16]);
}  // namespace qlin
