// Device-side building blocks shared by every kernel of the library:
// vector types, bf16 packing, MFMA wrappers, and the per-block 16-entry
// lookup table that turns 4-bit indices into bf16 weights in registers.
//
// Decode rule (both formats): a block/group owns 16 bf16 values
//   NF4 : LUT[i] = bf16(fl32(c[i] * a_hat))        [QLoRA NF4 + double quant]
//   INT4: LUT[i] = bf16(fl32(scale * i + zero))    [QA-LoRA group-wise INT4]
// and an element with index i decodes to LUT[i].  Building the table once per
// (row, block) folds the per-block scale into it, so the per-element work is a
// byte-permute lookup with no multiply.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlin {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Codebook {
  float c[16];
};

// ---------------------------------------------------------------- bf16 bits

// Two fp32 -> packed bf16 pair (round to nearest even): lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

// v_perm_b32: byte i of the result is byte sel.byte[i] of the 8-byte value
// {hi:lo} (selectors 0..3 pick from `lo`, 4..7 from `hi`).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// MFMA wrappers (gfx950 bf16, fp32 accumulate).
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// fp32 -> (hi, lo) bf16 split with hi + lo == v to ~2^-17 relative; used to
// feed fp32 adapter activations through bf16 MFMA without losing precision.
__device__ __forceinline__ void split_bf16(float v, float& hi, float& lo) {
  hi = __uint_as_float(pack_bf16x2(v, 0.0f) << 16);
  lo = v - hi;
}

// -------------------------------------------------------------- lookup table

// 16 bf16 entries held as two byte planes: lo[q] = low bytes of entries
// 4q..4q+3, hi[q] = high bytes of the same entries.
struct Lut16 {
  uint32_t lo[4];
  uint32_t hi[4];
};

// From 8 packed bf16 pairs p[j] = (entry 2j | entry 2j+1 << 16).
__device__ __forceinline__ Lut16 lut_from_pairs(const uint32_t (&p)[8]) {
  Lut16 t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t.lo[q] = perm(p[2 * q + 1], p[2 * q], 0x06040200u);
    t.hi[q] = perm(p[2 * q + 1], p[2 * q], 0x07050301u);
  }
  return t;
}

__device__ __forceinline__ Lut16 lut_nf4(const Codebook& cb, float scale) {
  uint32_t p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = pack_bf16x2(cb.c[2 * j] * scale, cb.c[2 * j + 1] * scale);
  return lut_from_pairs(p);
}

__device__ __forceinline__ Lut16 lut_int4(float scale, float zero) {
  uint32_t p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    p[j] = pack_bf16x2(__builtin_fmaf(scale, static_cast<float>(2 * j), zero),
                       __builtin_fmaf(scale, static_cast<float>(2 * j + 1), zero));
  return lut_from_pairs(p);
}

// Byte-plane lookup of four 4-bit indices held one per byte (low 3 bits in
// `sel`, bit 3 turned into the byte selector offset 4 in `pick`).
__device__ __forceinline__ uint32_t lut_plane4(const uint32_t (&plane)[4], uint32_t sel,
                                               uint32_t pick) {
  const uint32_t a = perm(plane[1], plane[0], sel);  // entries 0..7
  const uint32_t b = perm(plane[3], plane[2], sel);  // entries 8..15
  return perm(b, a, pick);
}

// Decode one dword of 8 packed indices (element e in nibble e) into four
// dwords of bf16 pairs.  Natural order: out[j] = (elem 2j | elem 2j+1 << 16).
__device__ __forceinline__ u32x4 lut_decode8(const Lut16& t, uint32_t w) {
  const uint32_t se = w & 0x07070707u;                              // e0 e2 e4 e6
  const uint32_t so = (w >> 4) & 0x07070707u;                       // e1 e3 e5 e7
  const uint32_t pe = ((w >> 1) & 0x04040404u) | 0x03020100u;       // bit 3 -> +4
  const uint32_t po = ((w >> 5) & 0x04040404u) | 0x03020100u;
  const uint32_t le = lut_plane4(t.lo, se, pe), he = lut_plane4(t.hi, se, pe);
  const uint32_t lo = lut_plane4(t.lo, so, po), ho = lut_plane4(t.hi, so, po);
  const uint32_t x = perm(he, le, 0x05010400u);  // e0 e2
  const uint32_t y = perm(he, le, 0x07030602u);  // e4 e6
  const uint32_t z = perm(ho, lo, 0x05010400u);  // e1 e3
  const uint32_t v = perm(ho, lo, 0x07030602u);  // e5 e7
  u32x4 r;
  r.x = perm(z, x, 0x05040100u);  // e0 e1
  r.y = perm(z, x, 0x07060302u);  // e2 e3
  r.z = perm(v, y, 0x05040100u);  // e4 e5
  r.w = perm(v, y, 0x07060302u);  // e6 e7
  return r;
}

// Same lookup with the elements delivered in the order 0 2 4 6 1 3 5 7
// (four dwords: (e0,e2) (e4,e6) (e1,e3) (e5,e7)).  A matrix product over k is
// unchanged when both operands use one permutation of k, so kernels that can
// permute the other operand once (and reuse it many times) save four permutes
// per eight weights.
__device__ __forceinline__ u32x4 lut_decode8_eo(const Lut16& t, uint32_t w) {
  const uint32_t se = w & 0x07070707u;
  const uint32_t so = (w >> 4) & 0x07070707u;
  const uint32_t pe = ((w >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t po = ((w >> 5) & 0x04040404u) | 0x03020100u;
  const uint32_t le = lut_plane4(t.lo, se, pe), he = lut_plane4(t.hi, se, pe);
  const uint32_t lo = lut_plane4(t.lo, so, po), ho = lut_plane4(t.hi, so, po);
  u32x4 r;
  r.x = perm(he, le, 0x05010400u);
  r.y = perm(he, le, 0x07030602u);
  r.z = perm(ho, lo, 0x05010400u);
  r.w = perm(ho, lo, 0x07030602u);
  return r;
}

// The matching permutation of eight bf16 of the other operand.
__device__ __forceinline__ u32x4 eo_permute(u32x4 d) {
  u32x4 r;
  r.x = perm(d.y, d.x, 0x05040100u);  // x0 x2
  r.y = perm(d.w, d.z, 0x05040100u);  // x4 x6
  r.z = perm(d.y, d.x, 0x07060302u);  // x1 x3
  r.w = perm(d.w, d.z, 0x07060302u);  // x5 x7
  return r;
}

// ------------------------------------------------------- per-block scales

// Double-quantized NF4 block scale: step = fl32(s2 * fl32(1/127)),
// a_hat = fl32(q * step).  [QLoRA "Innovation 2: Double Quantization"]
__device__ __forceinline__ float nf4_dq_scale(int8_t q, float s2) {
  const float step = s2 * (1.0f / 127.0f);
  return static_cast<float>(q) * step;
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Weight decode parameters passed to every fused kernel.
struct WeightView {
  const uint8_t* codes;    // [N][K/2]
  const void* absmax;      // NF4: int8 or float per 64-block
  const float* absmax2;    // NF4 dq: per 256 blocks
  const uint16_t* scale;   // INT4: fp16 per (row, group)
  const uint16_t* zero;
  int64_t N, K;
  int32_t dq;              // NF4: 1 if double-quantized
  Codebook cb;
};

// Scale of NF4 block `b` (flat block index).
__device__ __forceinline__ float nf4_block_scale(const WeightView& w, int64_t b) {
  if (w.dq) {
    const int8_t q = static_cast<const int8_t*>(w.absmax)[b];
    return nf4_dq_scale(q, w.absmax2[b >> 8]);
  }
  return static_cast<const float*>(w.absmax)[b];
}

// Lookup table of one (row, block): NF4 block = 64 elements, INT4 group = 32.
template <int FMT>
__device__ __forceinline__ Lut16 make_lut(const WeightView& w, int64_t row, int64_t blk_in_row);

constexpr int kFmtNF4 = 1;
constexpr int kFmtINT4 = 2;

template <>
__device__ __forceinline__ Lut16 make_lut<kFmtNF4>(const WeightView& w, int64_t row,
                                                  int64_t blk_in_row) {
  const int64_t b = row * (w.K >> 6) + blk_in_row;
  return lut_nf4(w.cb, nf4_block_scale(w, b));
}
template <>
__device__ __forceinline__ Lut16 make_lut<kFmtINT4>(const WeightView& w, int64_t row,
                                                   int64_t grp_in_row) {
  const int64_t g = row * (w.K >> 5) + grp_in_row;
  return lut_int4(half_bits_to_f32(w.scale[g]), half_bits_to_f32(w.zero[g]));
}

// Elements per lookup table for a format.
template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<kFmtNF4> {
  static constexpr int kBlock = 64;
};
template <>
struct FmtTraits<kFmtINT4> {
  static constexpr int kBlock = 32;
};

// ------------------------------------------------------------- misc helpers

__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T warp_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace qlin
