// NormalFloat-k (k = 2, 3, 4 bits) with blocks of 32..256 elements:
// quantizer and decoder.  [LQ-LoRA abstract: bit-width and block size chosen
// per matrix (sub-3-bit averages); QLoRA "Innovation 1: 4-bit NormalFloat
// (NF4)", "Background: what is quantization?" and "Innovation 2: Double
// Quantization" for the levels, the absmax blocks and the 8-bit constants.]
//
// Codes are stored as bit planes: every run of 32 consecutive elements of a
// row fills k little-endian 32-bit words, word p holding bit p of element i
// in its bit i (a row of d_in elements takes d_in * k / 8 bytes).  Block b
// holds elements [b * block, (b + 1) * block) of the row-major weight; with
// double quantization its constant is an int8 code q of a group of 256
// consecutive blocks, reconstructed as RN32(q * s2 / 127).
//
// Every decision that yields an integer is exact: the nearest level of
// w / a counts the level midpoints m (fp64, exact for fp32 levels) with
// w > m * a (exact in fp64: 25 + 24 significant bits); ties go to the lower
// level; an all-zero block takes the zero level.
#include "device_common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace qlin {

namespace {

// One workgroup per group of 256 consecutive blocks; thread t owns block
// 256 g + t (its absmax, then its codes, then the group's 8-bit constants).
template <int BITS>
__global__ __launch_bounds__(256) void k_quant_nf(const float* __restrict__ W, int64_t n_blocks,
                                                  int block, int dq, NfTable tb,
                                                  uint8_t* __restrict__ codes,
                                                  void* __restrict__ absmax_out,
                                                  float* __restrict__ absmax2_out,
                                                  uint32_t* __restrict__ bad_flag) {
  constexpr int NL = 1 << BITS;
  constexpr uint32_t kZero = NL / 2 - 1;
  __shared__ float s_abs[256];
  __shared__ int s_bad[256];
  const int tid = threadIdx.x;
  const int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + tid;
  const bool live = b < n_blocks;
  const float4* src = reinterpret_cast<const float4*>(W + (live ? b : 0) * block);

  float a = 0.0f;
  int bad = 0;
  for (int i = 0; i < block / 4; ++i) {
    const float4 v = src[i];
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    bad |= !(isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w));
  }
  const double ad = static_cast<double>(a);
  double thr[NL - 1];
#pragma unroll
  for (int k = 0; k < NL - 1; ++k) thr[k] = tb.mid[k] * ad;
  uint32_t* dst = reinterpret_cast<uint32_t*>(codes + (live ? b : 0) * block * BITS / 8);
  for (int run = 0; run < block / 32; ++run) {
    uint32_t word[BITS];
#pragma unroll
    for (int p = 0; p < BITS; ++p) word[p] = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = src[run * 8 + i];
      const float w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double wd = static_cast<double>(w4[e]);
        uint32_t idx = 0;
#pragma unroll
        for (int k = 0; k < NL - 1; ++k) idx += (wd > thr[k]) ? 1u : 0u;
        if (a == 0.0f) idx = kZero;
#pragma unroll
        for (int p = 0; p < BITS; ++p) word[p] |= ((idx >> p) & 1u) << (4 * i + e);
      }
    }
    if (live)
#pragma unroll
      for (int p = 0; p < BITS; ++p) dst[run * BITS + p] = word[p];
  }
  if (live && bad) __hip_atomic_fetch_or(bad_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!dq) {
    if (live) static_cast<float*>(absmax_out)[b] = bad ? __builtin_nanf("") : a;
    return;
  }
  s_abs[tid] = live ? a : 0.0f;
  s_bad[tid] = live ? bad : 0;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      s_abs[tid] = fmaxf(s_abs[tid], s_abs[tid + o]);
      s_bad[tid] |= s_bad[tid + o];
    }
    __syncthreads();
  }
  const float s2 = s_abs[0];
  if (live) {
    int8_t q = 0;
    if (s2 > 0.0f) q = static_cast<int8_t>(__builtin_rint((127.0 * ad) / static_cast<double>(s2)));
    static_cast<int8_t*>(absmax_out)[b] = q;
  }
  if (tid == 0) absmax2_out[blockIdx.x] = s_bad[0] ? __builtin_nanf("") : s2;
}

// Decoder (test helper and transcoder source): one thread per run of 32
// elements, W_bf16 = bf16(fl32(c[idx] * a_hat)).
template <int BITS>
__global__ __launch_bounds__(256) void k_dequant_nf(const uint8_t* __restrict__ codes,
                                                    const void* __restrict__ absmax,
                                                    const float* __restrict__ absmax2,
                                                    int64_t n_runs, int block, int dq, NfTable tb,
                                                    uint16_t* __restrict__ out) {
  __shared__ float s_c[16];
  if (threadIdx.x < 16) s_c[threadIdx.x] = tb.c[threadIdx.x];
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= n_runs) return;
  const int64_t blk = t * 32 / block;
  const float scale = dq ? nf4_dq_scale(static_cast<const int8_t*>(absmax)[blk], absmax2[blk >> 8])
                         : static_cast<const float*>(absmax)[blk];
  uint32_t word[BITS];
#pragma unroll
  for (int p = 0; p < BITS; ++p) word[p] = reinterpret_cast<const uint32_t*>(codes)[t * BITS + p];
  u32x4* dst = reinterpret_cast<u32x4*>(out + t * 32);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t pr[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float v[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 8 * q + 2 * h + e;
        uint32_t idx = 0;
#pragma unroll
        for (int p = 0; p < BITS; ++p) idx |= ((word[p] >> i) & 1u) << p;
        v[e] = s_c[idx] * scale;
      }
      pr[h] = pack_bf16x2(v[0], v[1]);
    }
    dst[q] = u32x4{pr[0], pr[1], pr[2], pr[3]};
  }
}

// Transcoder for the layer kernels: one thread per run of 32 elements (one
// group of 32), from bit planes to 4-bit indices in the NF4 packing (byte j
// of each run of 8 holds element j in its low and element j + 4 in its high
// nibble) and the group's fp32 scale split into its low and high 16 bits.
template <int BITS>
__global__ __launch_bounds__(256) void k_transcode_nf(const uint8_t* __restrict__ codes,
                                                      const void* __restrict__ absmax,
                                                      const float* __restrict__ absmax2,
                                                      int64_t n_runs, int block, int dq,
                                                      uint8_t* __restrict__ nib,
                                                      uint16_t* __restrict__ scale_lo,
                                                      uint16_t* __restrict__ scale_hi) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= n_runs) return;
  const int64_t blk = t * 32 / block;
  const float scale = dq ? nf4_dq_scale(static_cast<const int8_t*>(absmax)[blk], absmax2[blk >> 8])
                         : static_cast<const float*>(absmax)[blk];
  uint32_t word[BITS];
#pragma unroll
  for (int p = 0; p < BITS; ++p) word[p] = reinterpret_cast<const uint32_t*>(codes)[t * BITS + p];
  u32x4 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = 8 * q + j;
      uint32_t idx = 0;
#pragma unroll
      for (int p = 0; p < BITS; ++p) idx |= ((word[p] >> i) & 1u) << p;
      w |= idx << (j < 4 ? 8 * j : 8 * (j - 4) + 4);
    }
    out[q] = w;
  }
  reinterpret_cast<u32x4*>(nib)[t] = out;
  const uint32_t bits = __float_as_uint(scale);
  scale_lo[t] = static_cast<uint16_t>(bits & 0xFFFFu);
  scale_hi[t] = static_cast<uint16_t>(bits >> 16);
}

}  // namespace

hipError_t launch_transcode_nf(const uint8_t* codes, const void* absmax, const float* absmax2,
                               int64_t n_el, int bits, int block, int dq, uint8_t* nib,
                               uint16_t* scale_lo, uint16_t* scale_hi, hipStream_t stream) {
  const int64_t runs = n_el / 32;
  const dim3 grid(static_cast<uint32_t>((runs + 255) / 256));
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(k_transcode_nf<2>, grid, dim3(256), 0, stream, codes, absmax, absmax2,
                         runs, block, dq, nib, scale_lo, scale_hi);
      break;
    case 3:
      hipLaunchKernelGGL(k_transcode_nf<3>, grid, dim3(256), 0, stream, codes, absmax, absmax2,
                         runs, block, dq, nib, scale_lo, scale_hi);
      break;
    default:
      hipLaunchKernelGGL(k_transcode_nf<4>, grid, dim3(256), 0, stream, codes, absmax, absmax2,
                         runs, block, dq, nib, scale_lo, scale_hi);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_quant_nf(const float* W, int64_t n_blocks, int bits, int block, int dq,
                           const NfTable& tb, uint8_t* codes, void* absmax, float* absmax2,
                           uint32_t* flag, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((n_blocks + 255) / 256));
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(k_quant_nf<2>, grid, dim3(256), 0, stream, W, n_blocks, block, dq, tb,
                         codes, absmax, absmax2, flag);
      break;
    case 3:
      hipLaunchKernelGGL(k_quant_nf<3>, grid, dim3(256), 0, stream, W, n_blocks, block, dq, tb,
                         codes, absmax, absmax2, flag);
      break;
    default:
      hipLaunchKernelGGL(k_quant_nf<4>, grid, dim3(256), 0, stream, W, n_blocks, block, dq, tb,
                         codes, absmax, absmax2, flag);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_dequant_nf(const uint8_t* codes, const void* absmax, const float* absmax2,
                             int64_t n_el, int bits, int block, int dq, const NfTable& tb,
                             uint16_t* out, hipStream_t stream) {
  const int64_t runs = n_el / 32;
  const dim3 grid(static_cast<uint32_t>((runs + 255) / 256));
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(k_dequant_nf<2>, grid, dim3(256), 0, stream, codes, absmax, absmax2, runs,
                         block, dq, tb, out);
      break;
    case 3:
      hipLaunchKernelGGL(k_dequant_nf<3>, grid, dim3(256), 0, stream, codes, absmax, absmax2, runs,
                         block, dq, tb, out);
      break;
    default:
      hipLaunchKernelGGL(k_dequant_nf<4>, grid, dim3(256), 0, stream, codes, absmax, absmax2, runs,
                         block, dq, tb, out);
      break;
  }
  return hipGetLastError();
}

}  // namespace qlin
