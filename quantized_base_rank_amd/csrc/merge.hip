// QA-LoRA merge: the pooled adapter folded into the INT4 zero points.
// [QA-LoRA abstract, point (ii): after fine-tuning, the adapter merges into
// the quantized weights without loss of accuracy]
//
// With the adapter acting on group sums of x, s (P A^T) B^T adds
// s (B A)[n][g] to every weight of group g in row n, which is exactly a
// shift of that group's additive zero point:
//     zero'[n][g] = RN16( zero[n][g] + s * sum_j B[n][j] A[j][g] ),
// the exact sum rounded once to fp16 (ties to even).
#include "device_common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace qlin {

namespace {

// fp16 neighbours by bit pattern (finite values; -0 and +0 both step to the
// smallest subnormal of the right sign).
__device__ uint32_t f16_next_up(uint32_t b) {
  if (b == 0x8000u) return 0x0001u;
  return (b & 0x8000u) ? b - 1u : b + 1u;
}
__device__ uint32_t f16_next_down(uint32_t b) {
  if (b == 0x0000u) return 0x8001u;
  return (b & 0x8000u) ? b + 1u : b - 1u;
}
__device__ double f16_val(uint32_t b) {
  return static_cast<double>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}
// sign of (hi + lo) - m, with |lo| <= ulp(hi)/2: hi - m is exact when the two
// are within a factor of two, and otherwise far larger than lo
__device__ int dd_cmp(double hi, double lo, double m) {
  const double v = (hi - m) + lo;
  return v > 0.0 ? 1 : (v < 0.0 ? -1 : 0);
}

// One thread per (row n, group g); the threads of a block cover consecutive
// groups of one row, so A[j][g..] is read coalesced and B[n][j] is uniform.
// The sum runs over j in order as a double-double (two-sum for every term):
// each term s * B * A is exact in fp64 (24 + 8 + 8 significant bits), so
// hi + lo is the exact sum unless the terms span more than ~99 bits.  The
// fp16 result is a first candidate from hi, moved across the neighbouring
// rounding boundaries (midpoints of fp16 neighbours, exact in fp64) by the
// sign of the double-double minus the boundary; ties go to the even bits.
__global__ __launch_bounds__(256) void k_qa_merge(const uint16_t* __restrict__ zero,
                                                  const uint16_t* __restrict__ A,
                                                  const uint16_t* __restrict__ B, int64_t G,
                                                  int r, float s, uint16_t* __restrict__ out) {
  const int64_t n = blockIdx.y;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= G) return;
  double hi = static_cast<double>(half_bits_to_f32(zero[n * G + g]));
  double lo = 0.0;
  const double sd = static_cast<double>(s);
  for (int j = 0; j < r; ++j) {
    const double t = sd * static_cast<double>(bf16_to_f32(B[n * r + j])) *
                     static_cast<double>(bf16_to_f32(A[static_cast<int64_t>(j) * G + g]));
    const double sum = hi + t;
    const double bv = sum - hi;
    const double err = (hi - (sum - bv)) + (t - bv);
    hi = sum;
    lo += err;
  }
  {  // renormalise so that |lo| <= ulp(hi) / 2
    const double sum = hi + lo;
    lo = lo - (sum - hi);
    hi = sum;
  }
  uint32_t c = __builtin_bit_cast(uint16_t, static_cast<_Float16>(static_cast<float>(hi)));
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const uint32_t d = f16_next_down(c);
    const int sg = dd_cmp(hi, lo, 0.5 * (f16_val(d) + f16_val(c)));
    if (sg < 0 || (sg == 0 && (c & 1u))) c = d;
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const uint32_t u = f16_next_up(c);
    const int sg = dd_cmp(hi, lo, 0.5 * (f16_val(c) + f16_val(u)));
    if (sg > 0 || (sg == 0 && (c & 1u))) c = u;
  }
  out[n * G + g] = static_cast<uint16_t>(c);
}

}  // namespace

hipError_t launch_qa_merge(const uint16_t* zero, const uint16_t* A, const uint16_t* B, int64_t N,
                           int64_t G, int r, float s, uint16_t* out, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((G + 255) / 256), static_cast<uint32_t>(N));
  hipLaunchKernelGGL(k_qa_merge, grid, dim3(256), 0, stream, zero, A, B, G, r, s, out);
  return hipGetLastError();
}

}  // namespace qlin
