// Host-side NF4 level table (see codebook.cpp).
#pragma once

namespace qlin {
void nf4_levels(float out[16]);
}  // namespace qlin
