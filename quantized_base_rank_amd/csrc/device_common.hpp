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

// Decode one dword of 8 packed indices into four dwords of bf16 pairs,
// out[j] = (element 2j | element 2j+1 << 16).  Byte b of the dword holds
// element b in its low nibble and element b + 4 in its high nibble, so the
// low nibbles are elements 0..3 and the high nibbles elements 4..7, and one
// byte interleave per output pair puts them in natural order.
// The two byte constants of the selectors are held in vector registers:
// a three-operand instruction on this target takes no literal and at most
// one scalar operand, so with both constants in registers the mask-and-offset
// of each selector is one v_and_or_b32 instead of an and plus an or.  (The
// moves carry no side effects, so the compiler hoists them out of loops.)
__device__ __forceinline__ u32x4 lut_decode8(const Lut16& t, uint32_t w) {
  uint32_t m4, c3210;
  asm("v_mov_b32 %0, 0x04040404" : "=v"(m4));
  asm("v_mov_b32 %0, 0x03020100" : "=v"(c3210));
  const uint32_t sl = w & 0x07070707u;         // e0..e3, low 3 bits
  const uint32_t sh = (w >> 4) & 0x07070707u;  // e4..e7
  const uint32_t pl = ((w >> 1) & m4) | c3210;  // bit 3 -> +4
  const uint32_t ph = ((w >> 5) & m4) | c3210;
  const uint32_t ll = lut_plane4(t.lo, sl, pl), hl = lut_plane4(t.hi, sl, pl);
  const uint32_t lh = lut_plane4(t.lo, sh, ph), hh = lut_plane4(t.hi, sh, ph);
  u32x4 r;
  r.x = perm(hl, ll, 0x05010400u);  // e0 e1
  r.y = perm(hl, ll, 0x07030602u);  // e2 e3
  r.z = perm(hh, lh, 0x05010400u);  // e4 e5
  r.w = perm(hh, lh, 0x07030602u);  // e6 e7
  return r;
}

// ------------------------------------------------------- per-block scales

// Double-quantized NF4 block scale a_hat = RN32(q * s2 / 127): the 8-bit
// grid of a group runs from 0 to its maximum s2 in 127 equal steps, and the
// stored constant is the grid value rounded once to fp32.
// [QLoRA "Innovation 2: Double Quantization"]
// q * s2 is exact in fp64 (7 + 24 significant bits); multiplying it by
// fl64(1/127) stays within 2^-52 relative of the quotient.  A quotient by
// 127 that is not itself an fp32 number lies at least 1/254 of an fp32 ulp
// from every fp32 rounding boundary, so the final fp64 -> fp32 rounding
// yields the correctly rounded quotient (and q = 127 gives s2 exactly).
__device__ __forceinline__ float nf4_dq_scale(int8_t q, float s2) {
  const double p = static_cast<double>(q) * static_cast<double>(s2);
  return static_cast<float>(p * (1.0 / 127.0));
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
// NormalFloat-k weights of any block size, as the layer kernels read them:
// 4-bit level indices in the NF4 packing, the levels in WeightView::cb and
// one fp32 scale per group of 32 elements, its low and high 16 bits held in
// the `scale` and `zero` arrays (the INT4 group layout), so that the loads
// of the INT4 path yield the scale's bits directly.
constexpr int kFmtNFG = 3;

// Lookup table of a group of 32 from its 32-bit group word `sz` (the INT4
// path's scale | zero << 16): INT4 builds bf16(fl32(scale * i + zero)),
// NormalFloat-k builds bf16(fl32(c[i] * scale)) with the word as the fp32
// scale.
template <int FMT>
__device__ __forceinline__ Lut16 lut_group32(const Codebook& cb, uint32_t sz) {
  if constexpr (FMT == kFmtNFG) {
    return lut_nf4(cb, __uint_as_float(sz));
  } else {
    return lut_int4(half_bits_to_f32(static_cast<uint16_t>(sz & 0xFFFFu)),
                    half_bits_to_f32(static_cast<uint16_t>(sz >> 16)));
  }
}

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
template <>
__device__ __forceinline__ Lut16 make_lut<kFmtNFG>(const WeightView& w, int64_t row,
                                                  int64_t grp_in_row) {
  const int64_t g = row * (w.K >> 5) + grp_in_row;
  return lut_group32<kFmtNFG>(w.cb, static_cast<uint32_t>(w.scale[g]) |
                                        (static_cast<uint32_t>(w.zero[g]) << 16));
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
template <>
struct FmtTraits<kFmtNFG> {
  static constexpr int kBlock = 32;
};

// ------------------------------------------------------- transposed LDS read

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16.  Within each group of 16 lanes, lane p supplies the
// LDS address of four consecutive 16-bit elements; lane t = 4a + b receives
// element b of the chunks supplied by lanes a, a + 4, a + 8, a + 12, in that
// order.  So when lane p points at row kbase + p/4, columns c0 + 4(p%4) ..
// +3 of a row-major tile, lane t receives rows kbase .. kbase+3 of column
// c0 + t: four consecutive reduction elements of one operand row, read from a
// tile stored with the reduction index as its row.
__device__ __forceinline__ u32x2 ds_read_tr16(const void* lds_addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds_addr));
  return __builtin_bit_cast(u32x2, v);
}

// MFMA operand (8 consecutive reduction rows kbase..kbase+7 of column c0 + t)
// from a row-major bf16 LDS tile with `stride` bytes per row.  `p` is the
// lane index within its 16-lane group.
__device__ __forceinline__ u32x4 tr16_operand(const uint8_t* tile, int stride, int kbase, int c0,
                                              int p) {
  const uint8_t* a0 = tile + (kbase + (p >> 2)) * stride + (c0 + 4 * (p & 3)) * 2;
  const u32x2 lo = ds_read_tr16(a0);
  const u32x2 hi = ds_read_tr16(a0 + 4 * stride);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// Raw decode parameters of one (row, 64-element block), loaded ahead of use
// so that the loads overlap other work; luts_from_params builds the tables.
// NF4: a = the 8-bit code (meaningful with DQ), b = fp32 bits of the group
// constant s2 (DQ) or of the block absmax (no DQ).
// INT4: a, b = (scale | zero << 16) of the block's two 32-element groups.
struct BlockParams {
  uint32_t a, b;
};

template <int FMT>
__device__ __forceinline__ BlockParams load_block_params(const WeightView& w, int64_t row,
                                                         int64_t blk64, bool valid) {
  BlockParams p{0u, 0u};
  (void)valid;  // indices are clamped by the caller; the loads are unconditional
  if (FMT == kFmtNF4) {
    // Branch-free: both loads are issued for either layout, from addresses
    // that are in bounds for both (byte b of an fp32 absmax array; element
    // b of it, or the group constant), and the result is selected after.
    // A branch here lets the compiler pull the scale arithmetic next to the
    // loads, which then waits for every load issued before them.
    const int64_t b = row * (w.K >> 6) + blk64;
    const float* wide = w.dq ? w.absmax2 + (b >> 8) : static_cast<const float*>(w.absmax) + b;
    const uint32_t q8 =
        static_cast<uint32_t>(static_cast<int32_t>(static_cast<const int8_t*>(w.absmax)[b]));
    // kept raw (no select on the loaded values, which would wait for them):
    // a = the 8-bit code (used with DQ), b = the fp32 group constant (DQ)
    // or the fp32 block absmax (no DQ)
    p.a = q8;
    p.b = __float_as_uint(*wide);
  } else {
    const int64_t g = row * (w.K >> 5) + 2 * blk64;
    p.a = static_cast<uint32_t>(w.scale[g]) | (static_cast<uint32_t>(w.zero[g]) << 16);
    p.b = static_cast<uint32_t>(w.scale[g + 1]) | (static_cast<uint32_t>(w.zero[g + 1]) << 16);
  }
  return p;
}

// NF4 block scale from raw block constants (computed where the table is
// built, not where the constants are loaded).
__device__ __forceinline__ float nf4_params_scale(const WeightView& w, BlockParams p) {
  return w.dq ? nf4_dq_scale(static_cast<int8_t>(p.a), __uint_as_float(p.b)) : __uint_as_float(p.b);
}

// The same scale (zero for an invalid block) formed without branches: both
// forms, then bit selects on the flag and on validity.  Inside a pipelined
// loop a branch here would split the scheduling region and wait for every
// load in flight.
__device__ __forceinline__ float nf4_params_scale_sel(const WeightView& w, BlockParams p, bool valid) {
  const float s2 = __uint_as_float(p.b);
  const float sdq = nf4_dq_scale(static_cast<int8_t>(p.a & 0xFFu), s2);
  const uint32_t dqm = w.dq ? 0xFFFFFFFFu : 0u;
  const uint32_t bits = (__float_as_uint(sdq) & dqm) | (p.b & ~dqm);
  return __uint_as_float(valid ? bits : 0u);
}

// lut[0] decodes elements 0..31 of the block, lut[1] elements 32..63.
template <int FMT>
__device__ __forceinline__ void luts_from_params(const WeightView& w, BlockParams p,
                                                 Lut16 (&lut)[2]) {
  if (FMT == kFmtNF4) {
    lut[0] = lut_nf4(w.cb, nf4_params_scale(w, p));
    lut[1] = lut[0];
  } else {
    lut[0] = lut_group32<FMT>(w.cb, p.a);
    lut[1] = lut_group32<FMT>(w.cb, p.b);
  }
}

// ------------------------------------------- split reductions across workgroups
// Partial sums that another workgroup (possibly on another XCD, with its own
// L2) will read are written through to device-coherent memory (sc0 sc1
// stores) and read back the same way, so publishing them needs only a wait
// for the stores' acknowledgements, not a write-back of the whole L2.

__device__ __forceinline__ void st_sys(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float ld_sys(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_sys4(float* p, f32x4 v) {
  st_sys(p, v[0]);
  st_sys(p + 1, v[1]);
  st_sys(p + 2, v[2]);
  st_sys(p + 3, v[3]);
}
__device__ __forceinline__ f32x4 ld_sys4(const float* p) {
  return f32x4{ld_sys(p), ld_sys(p + 1), ld_sys(p + 2), ld_sys(p + 3)};
}

// Wide (16-byte) write-through stores and coherent loads through a buffer
// resource: buffer_{store,load}_dwordx4 with sc0 sc1.  `off` is a byte offset
// from the (wave-uniform) base; buffers are < 2 GiB.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// A buffer resource over [base, base + bytes) whose fields go through
// readfirstlane, so that it lives in scalar registers even where the compiler
// cannot prove the base wave-uniform (a resource in vector registers turns
// every load into a loop over the lanes).  readfirstlane returns a signed
// int, so each half of the base is taken back to 32 unsigned bits before it
// is widened.
__device__ __forceinline__ rsrc_t uniform_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b))));
  const uint64_t u = (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0,
                                           __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000);
}
__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
constexpr int kCoherent = 1 | 16;  // sc0 | sc1
__device__ __forceinline__ void st_sys16(rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ f32x4 ld_sys16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}
__device__ __forceinline__ f32x2 ld_sys8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherent));
}

// Waits until this workgroup's write-through stores are acknowledged, then
// takes a ticket on `counter` (one per output tile).  Returns the ticket in
// every thread; the workgroup that draws splits - 1 is the last one.
__device__ __forceinline__ uint32_t publish_and_ticket(uint32_t* counter, uint32_t* s_ticket) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    *s_ticket = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *s_ticket;
}

// ------------------------------------------ tile order of the GEMM kernels
// The MFMA kernels run one workgroup per compute unit, so 256 workgroups are
// resident at a time, dealt to the 8 XCDs round-robin (workgroup b on XCD
// b % 8).  xcd_round_order gives each group of 256 consecutive workgroups a
// run of 256 consecutive work items, and within it each XCD a contiguous
// run of 32 (fewer in a last, partial group).  grouped_tile then walks the
// tile grid in blocks of 4 tile rows, column by column, so that the 32
// items of one XCD form a 4 x 8 block of tiles: its workgroups share 4 row
// operands and 8 column operands in that XCD's L2, instead of one row
// operand and 32 column operands.
__device__ __forceinline__ int xcd_round_order(int bid, int n) {
  const int base = bid & ~255;
  const int cnt = n - base < 256 ? n - base : 256;
  const int q = cnt >> 3, rem = cnt & 7, b = bid & 255;
  const int xcd = b & 7, idx = b >> 3;
  return base + (xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx);
}
__device__ __forceinline__ void grouped_tile(int v, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int kGroup = 4;
  const int per = kGroup * tiles_n;
  const int g = v / per, vin = v - g * per;
  const int gm = tiles_m - kGroup * g < kGroup ? tiles_m - kGroup * g : kGroup;
  tm = kGroup * g + vin % gm;
  tn = vin / gm;
}

// ------------------------------------------------------------- misc helpers

__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T warp_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace qlin
