// Quantizers (run once per frozen layer) and the test-only dequantizer.
//
// NF4: [QLoRA "Background: what is quantization?", "Innovation 1: 4-bit
// NormalFloat (NF4)", "Innovation 2: Double Quantization", "The same idea in
// code"].  INT4: [QA-LoRA abstract, group-wise INT4].
//
// Every decision that yields an integer (nearest level, the 8-bit absmax
// code, the INT4 code) is taken with exact or correctly rounded IEEE
// arithmetic, so codes and constants are reproducible bit for bit.
#include <mutex>

#include "device_common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace qlin {

namespace {

// Midpoints of neighbouring levels, as float64 (exact for fp32 levels).
struct Midpoints {
  double m[15];
};

// One workgroup = one group of 256 consecutive blocks of 64 weights.  Each
// wave handles 64 blocks, four at a time: 16 lanes per block, 4 weights per
// lane.
__global__ __launch_bounds__(256) void k_quant_nf4(const float* __restrict__ W, int64_t n_blocks,
                                                   int dq, Midpoints mids,
                                                   uint8_t* __restrict__ codes,
                                                   void* __restrict__ absmax_out,
                                                   float* __restrict__ absmax2_out,
                                                   uint32_t* __restrict__ bad_flag) {
  __shared__ float s_abs[256];
  __shared__ int s_bad[256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int sub = lane >> 4, li = lane & 15;
  const int64_t g = blockIdx.x;
  const int64_t blk0 = g * 256;

  // issue all 16 loads of this wave's 64 blocks before using any of them
  float4 vin[16];
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int64_t b = blk0 + wave * 64 + it * 4 + sub;
    vin[it] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b < n_blocks) vin[it] = reinterpret_cast<const float4*>(W + b * 64)[li];
  }
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int local = wave * 64 + it * 4 + sub;  // block within the group
    const int64_t b = blk0 + local;
    const float4 v = vin[it];
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    int bad = !(isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      a = fmaxf(a, __shfl_xor(a, o, 64));
      bad |= __shfl_xor(bad, o, 64);
    }
    // nearest level of w / a: count midpoints m with w > m * a (exact in fp64)
    const double ad = static_cast<double>(a);
    double thr[15];
#pragma unroll
    for (int k = 0; k < 15; ++k) thr[k] = mids.m[k] * ad;
    const float w4[4] = {v.x, v.y, v.z, v.w};
    uint32_t nib[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double wd = static_cast<double>(w4[e]);
      uint32_t idx = 0;
#pragma unroll
      for (int k = 0; k < 15; ++k) idx += (wd > thr[k]) ? 1u : 0u;
      nib[e] = (a == 0.0f) ? 7u : idx;
    }
    // packed layout: byte j of each run of 8 elements holds element j in
    // its low nibble and element j + 4 in its high nibble; lanes 2i and
    // 2i + 1 hold elements 0..3 and 4..7 of run i
    const uint32_t part = (nib[0] | (nib[1] << 8) | (nib[2] << 16) | (nib[3] << 24)) << ((li & 1) * 4);
    const uint32_t word = part | static_cast<uint32_t>(__shfl_xor(static_cast<int>(part), 1, 64));
    if (b < n_blocks) {
      if ((li & 1) == 0) reinterpret_cast<uint32_t*>(codes + b * 32)[li >> 1] = word;
      if (li == 0) {
        s_abs[local] = a;
        s_bad[local] = bad;
        if (!dq) static_cast<float*>(absmax_out)[b] = bad ? __builtin_nanf("") : a;
        if (bad) __hip_atomic_fetch_or(bad_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else if (li == 0) {
      s_abs[local] = 0.0f;
      s_bad[local] = 0;
    }
  }
  if (!dq) return;
  __syncthreads();
  // second level: s2 = group max; q = round_half_even(127 a / s2) in fp64
  float m = s_abs[tid];
  int bad = s_bad[tid];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    m = fmaxf(m, __shfl_xor(m, o, 64));
    bad |= __shfl_xor(bad, o, 64);
  }
  __shared__ float s_wmax[4];
  __shared__ int s_wbad[4];
  if (lane == 0) {
    s_wmax[wave] = m;
    s_wbad[wave] = bad;
  }
  __syncthreads();
  const float s2 = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
  const int gbad = s_wbad[0] | s_wbad[1] | s_wbad[2] | s_wbad[3];
  const int64_t b = blk0 + tid;
  if (b < n_blocks) {
    int8_t q = 0;
    if (s2 > 0.0f) {
      const double r = (127.0 * static_cast<double>(s_abs[tid])) / static_cast<double>(s2);
      q = static_cast<int8_t>(__builtin_rint(r));
    }
    static_cast<int8_t*>(absmax_out)[b] = q;
  }
  if (tid == 0) absmax2_out[g] = gbad ? __builtin_nanf("") : s2;
}

// fp16 value nearest to (hi - lo) / 15 in exact arithmetic, ties to the even
// significand (hi >= lo, both finite fp32 within the fp16 range).
//
// The difference is formed in fp64 together with its rounding error
// (two-sum), so hi - lo == d + e exactly.  A first candidate comes from the
// fp64 quotient rounded to fp32 and then fp16, which is at most one fp16
// step away from the answer.  The candidate is then checked against the two
// rounding boundaries next to it: a boundary m (the midpoint of neighbouring
// fp16 values) has at most 12 significant bits, so 15 m is exact in fp64,
// and the sign of (d - 15 m) + e is the sign of hi - lo - 15 m: either
// d - 15 m is exact (the two are within a factor of two) or it is far larger
// than e.
__device__ double qs_f16_value(uint32_t bits) {
  return static_cast<double>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}
// -1, 0, +1: the sign of (d + e) - t
__device__ int qs_cmp(double d, double e, double t) {
  const double v = (d - t) + e;
  return v > 0.0 ? 1 : (v < 0.0 ? -1 : 0);
}
__device__ uint16_t int4_scale_bits(float hi, float lo) {
  const double h = static_cast<double>(hi), l = -static_cast<double>(lo);
  const double d = h + l;
  const double bv = d - h;
  const double e = (h - (d - bv)) + (l - bv);
  const _Float16 c0 = static_cast<_Float16>(static_cast<float>(d / 15.0));
  uint32_t c = __builtin_bit_cast(uint16_t, c0);
  if (c != 0) {
    // boundary below the candidate
    const double m = 0.5 * (qs_f16_value(c - 1) + qs_f16_value(c));
    const int s = qs_cmp(d, e, 15.0 * m);
    if (s < 0 || (s == 0 && (c & 1u))) c -= 1;
  }
  {
    // boundary above the candidate (the range of fp16 inputs keeps
    // (hi - lo)/15 far below the largest fp16 value)
    const double m = 0.5 * (qs_f16_value(c) + qs_f16_value(c + 1));
    const int s = qs_cmp(d, e, 15.0 * m);
    if (s > 0 || (s == 0 && (c & 1u))) c += 1;
  }
  return static_cast<uint16_t>(c);
}

// Group-wise asymmetric INT4: 8 lanes per group of 32, 4 weights per lane.
//   zero  = RN16(min),  scale = RN16((max - min) / 15),
//   q     = clamp(round_half_even((w - zero) / scale), 0, 15)  (0 if scale == 0)
// each rounding taken on the exact value.  The code counts the boundaries
// t_k = zero + (k + 1/2) scale (k = 0..14) below w, plus those equal to w
// for odd k (a half-way value goes to the even neighbour); every t_k is exact
// in fp64 (an fp16 value plus an odd multiple of half an fp16 value), so
// each comparison is exact.
__global__ __launch_bounds__(256) void k_quant_int4(const float* __restrict__ W, int64_t n_groups,
                                                    uint8_t* __restrict__ codes,
                                                    uint16_t* __restrict__ scale,
                                                    uint16_t* __restrict__ zero,
                                                    uint32_t* __restrict__ bad_flag) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t grp = t >> 3;
  const int li = threadIdx.x & 7;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (grp < n_groups) v = reinterpret_cast<const float4*>(W + grp * 32)[li];
  float lo = fminf(fminf(v.x, v.y), fminf(v.z, v.w));
  float hi = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
  int bad = 0;
  const float w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) bad |= !(isfinite(w4[e]) && fabsf(w4[e]) <= 65504.0f);
#pragma unroll
  for (int o = 4; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
    bad |= __shfl_xor(bad, o, 64);
  }
  const _Float16 beta_h = static_cast<_Float16>(lo);
  const uint16_t alpha_bits = bad ? static_cast<uint16_t>(0) : int4_scale_bits(hi, lo);
  const double beta = static_cast<double>(beta_h);
  const double alpha = qs_f16_value(alpha_bits);
  uint32_t nib[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double wd = static_cast<double>(w4[e]);
    uint32_t q = 0;
#pragma unroll
    for (int k = 0; k < 15; ++k) {
      const double tk = beta + (static_cast<double>(k) + 0.5) * alpha;
      q += (wd > tk) ? 1u : 0u;
      if (k & 1) q += (wd == tk) ? 1u : 0u;
    }
    nib[e] = alpha_bits == 0 ? 0u : q;
  }
  // the packed layout of the NF4 quantizer: byte j of each run of 8 holds
  // elements j (low nibble) and j + 4 (high nibble)
  const uint32_t part = (nib[0] | (nib[1] << 8) | (nib[2] << 16) | (nib[3] << 24)) << ((li & 1) * 4);
  const uint32_t word = part | static_cast<uint32_t>(__shfl_xor(static_cast<int>(part), 1, 64));
  if (grp < n_groups) {
    if ((li & 1) == 0) reinterpret_cast<uint32_t*>(codes + grp * 16)[li >> 1] = word;
    if (li == 0) {
      scale[grp] = alpha_bits;
      zero[grp] = __builtin_bit_cast(uint16_t, beta_h);
      if (bad) __hip_atomic_fetch_or(bad_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Test-only: W_bf16 through the same lookup-table decode as the fused
// kernels.  One thread per 8 consecutive weights.
template <int FMT>
__global__ __launch_bounds__(256) void k_dequant(WeightView w, uint16_t* __restrict__ out) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = w.N * w.K / 8;
  if (t >= total) return;
  const int64_t e0 = t * 8;
  const int64_t row = e0 / w.K, col = e0 % w.K;
  const Lut16 lut = make_lut<FMT>(w, row, col / FmtTraits<FMT>::kBlock);
  const uint32_t word = reinterpret_cast<const uint32_t*>(w.codes)[t];
  reinterpret_cast<u32x4*>(out)[t] = lut_decode8(lut, word);
}

// Non-finite-input flag of the quantizers: one word in each device's copy of
// this code object.  The quantizer entry points clear it, run the kernel,
// read it back and synchronise, holding quant_flag_lock() throughout.
__device__ uint32_t g_quant_flag;

}  // namespace

std::mutex& quant_flag_lock() {
  static std::mutex m;
  return m;
}

hipError_t quant_flag_ptr(uint32_t** out) {
  // device address of g_quant_flag on the current device, looked up once per
  // device (callers hold quant_flag_lock())
  static uint32_t* cache[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (cache[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_quant_flag));
    if (e != hipSuccess) return e;
    cache[dev] = static_cast<uint32_t*>(p);
  }
  *out = cache[dev];
  return hipSuccess;
}

hipError_t launch_quant_nf4(const float* W, int64_t n_blocks, int dq, const double* mids15,
                            uint8_t* codes, void* absmax, float* absmax2, uint32_t* flag,
                            hipStream_t stream) {
  Midpoints m;
  for (int i = 0; i < 15; ++i) m.m[i] = mids15[i];
  const int64_t groups = (n_blocks + 255) / 256;
  hipLaunchKernelGGL(k_quant_nf4, dim3(static_cast<uint32_t>(groups)), dim3(256), 0, stream, W,
                     n_blocks, dq, m, codes, absmax, absmax2, flag);
  return hipGetLastError();
}

hipError_t launch_quant_int4(const float* W, int64_t n_groups, uint8_t* codes, uint16_t* scale,
                             uint16_t* zero, uint32_t* flag, hipStream_t stream) {
  const int64_t threads = n_groups * 8;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(k_quant_int4, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, W,
                     n_groups, codes, scale, zero, flag);
  return hipGetLastError();
}

hipError_t launch_dequant(const WeightView& w, int fmt, uint16_t* out, hipStream_t stream) {
  const int64_t total = w.N * w.K / 8;
  const int64_t blocks = (total + 255) / 256;
  if (fmt == kFmtNF4)
    hipLaunchKernelGGL(k_dequant<kFmtNF4>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, w, out);
  else if (fmt == kFmtINT4)
    hipLaunchKernelGGL(k_dequant<kFmtINT4>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, w, out);
  else
    hipLaunchKernelGGL(k_dequant<kFmtNFG>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, w, out);
  return hipGetLastError();
}

}  // namespace qlin
