// Fused forward of the adapted 4-bit layer for many tokens:
//     y = x W_bf16^T + (s u) B^T
// [QLoRA "The QLoRA recipe" stage 3 / "The complete QLoRA forward pass": each
// weight block is brought back to bf16 on the fly, multiplied by the input,
// and the adapter correction is added; QA-LoRA abstract for the INT4 groups.]
//
// Tile: 256 tokens x 256 output features per workgroup of 4 waves; wave w
// owns features [64w, 64w+64) for all 256 tokens, so every 4-bit weight is
// decoded exactly once per workgroup, from its codes in LDS into registers
// (byte-permute lookup), and reused by 8 MFMAs.  The 256x128 bf16
// token tile of each K step is streamed into LDS with direct-to-LDS loads
// in two halves, through a ring of four half-stages that keeps every load
// about one and a half K steps ahead (XOR-swizzled 16-byte chunks:
// conflict-free reads); the packed codes follow in two stages.
// The adapter term is 2*ceil(r/16) extra MFMA k-steps on the same
// accumulators, with s*u split into hi + lo bf16 halves.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kTM = 256;
constexpr int kTN = 256;
constexpr int kKS = 128;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw block constants of one K step for a lane's two rows (the scale is
// formed when the table is built, so the loads are consumed a step later).
template <int FMT>
struct StepParams;
template <>
struct StepParams<kFmtNF4> {
  BlockParams bp[2];  // per row: a = the aligned word holding the 8-bit code (DQ), b = fp32 bits of s2 or absmax
  uint32_t sh[2];     // per row: bit position of the code in a
};
template <>
struct StepParams<kFmtINT4> {
  uint32_t s[2], z[2];  // per row: fp16 scales and zeros of the two groups, low group first
};
template <>
struct StepParams<kFmtNFG> : StepParams<kFmtINT4> {};  // the same group words

// Where a lane's block constants live: buffer resources over the constant
// arrays and per-lane offsets, so that a step's loads take only its scalar
// offset (no per-lane address arithmetic, no 64-bit pointers).
template <int FMT>
struct ParamSrc;
template <>
struct ParamSrc<kFmtNF4> {
  rsrc_t r8, rw;     // 8-bit codes (DQ; any bytes otherwise); wide constants
  uint32_t lb[2];    // flat block index of the lane's row at step 0
  uint32_t sh;       // 8 with DQ (group of 256 blocks), else 0
};
template <>
struct ParamSrc<kFmtINT4> {
  rsrc_t rs, rz;
  uint32_t lg[2];    // byte offset of the lane's first group at step 0
};
template <>
struct ParamSrc<kFmtNFG> : ParamSrc<kFmtINT4> {};

template <int FMT>
__device__ __forceinline__ ParamSrc<FMT> param_src(const WeightView& w, const int64_t (&nr)[2], int h);
template <>
__device__ __forceinline__ ParamSrc<kFmtNF4> param_src<kFmtNF4>(const WeightView& w, const int64_t (&nr)[2],
                                                                int h) {
  ParamSrc<kFmtNF4> ps;
  const int64_t nb = w.N * (w.K >> 6);
  ps.r8 = uniform_rsrc(w.absmax, static_cast<uint32_t>(w.dq ? nb : 4 * nb));
  ps.rw = uniform_rsrc(w.dq ? static_cast<const void*>(w.absmax2) : w.absmax,
                       static_cast<uint32_t>(w.dq ? 4 * ((nb + 255) >> 8) : 4 * nb));
#pragma unroll
  for (int r = 0; r < 2; ++r) ps.lb[r] = static_cast<uint32_t>(nr[r] * (w.K >> 6) + h);
  ps.sh = w.dq ? 8u : 0u;
  return ps;
}
template <>
__device__ __forceinline__ ParamSrc<kFmtINT4> param_src<kFmtINT4>(const WeightView& w, const int64_t (&nr)[2],
                                                                  int h) {
  ParamSrc<kFmtINT4> ps;
  const uint32_t bytes = static_cast<uint32_t>(w.N * (w.K >> 5) * 2);
  ps.rs = uniform_rsrc(w.scale, bytes);
  ps.rz = uniform_rsrc(w.zero, bytes);
#pragma unroll
  for (int r = 0; r < 2; ++r) ps.lg[r] = static_cast<uint32_t>((nr[r] * (w.K >> 5) + 2 * h) * 2);
  return ps;
}

template <>
__device__ __forceinline__ ParamSrc<kFmtNFG> param_src<kFmtNFG>(const WeightView& w, const int64_t (&nr)[2],
                                                                int h) {
  ParamSrc<kFmtNFG> ps;
  static_cast<ParamSrc<kFmtINT4>&>(ps) = param_src<kFmtINT4>(w, nr, h);
  return ps;
}

// Block constants of K step ks (blocks 2 ks + h), one load per call: part q
// of 4 is word q % 2 of the lane's row q / 2.  Near the end of K a lane of
// the upper half may read the next row's constants (or zeros past the
// array); such blocks are masked when the table is built.
template <int FMT>
__device__ __forceinline__ void load_params(const ParamSrc<FMT>& ps, int64_t ks, StepParams<FMT>& p, int q);
template <>
__device__ __forceinline__ void load_params<kFmtNF4>(const ParamSrc<kFmtNF4>& ps, int64_t ks,
                                                     StepParams<kFmtNF4>& p, int q) {
  // The 8-bit code comes from the aligned word that holds it (the array
  // length is a multiple of 16 bytes): a byte load whose value is
  // sign-extended where it is used gets merged with that extension and moved
  // down to the use, where the wave would then wait for every load in flight.
  const int r = q >> 1;
  const uint32_t o = ps.lb[r] + static_cast<uint32_t>(2 * ks);
  if ((q & 1) == 0) {
    p.bp[r].a = __builtin_amdgcn_raw_buffer_load_b32(ps.r8, o & ~3u, 0, 0);
    p.sh[r] = (o & 3u) * 8u;
  } else {
    p.bp[r].b = __builtin_amdgcn_raw_buffer_load_b32(ps.rw, (o >> ps.sh) << 2, 0, 0);
  }
}
template <>
__device__ __forceinline__ void load_params<kFmtINT4>(const ParamSrc<kFmtINT4>& ps, int64_t ks,
                                                      StepParams<kFmtINT4>& p, int q) {
  const int g8 = static_cast<int>(8 * ks);  // 4 groups of 2 bytes per step
  const int r = q >> 1;
  if ((q & 1) == 0)
    p.s[r] = __builtin_amdgcn_raw_buffer_load_b32(ps.rs, ps.lg[r], g8, 0);
  else
    p.z[r] = __builtin_amdgcn_raw_buffer_load_b32(ps.rz, ps.lg[r], g8, 0);
}
template <>
__device__ __forceinline__ void load_params<kFmtNFG>(const ParamSrc<kFmtNFG>& ps, int64_t ks,
                                                     StepParams<kFmtNFG>& p, int q) {
  load_params<kFmtINT4>(ps, ks, p, q);
}

template <int FMT>
__device__ __forceinline__ Lut16 step_lut(const WeightView& w, const StepParams<FMT>& p, int r,
                                          int q, bool valid);
template <>
__device__ __forceinline__ Lut16 step_lut<kFmtNF4>(const WeightView& w,
                                                   const StepParams<kFmtNF4>& p, int r, int,
                                                   bool valid) {
  // an invalid block (past K) decodes to zeros through a zero scale
  const BlockParams bp{(p.bp[r].a >> p.sh[r]) & 0xFFu, p.bp[r].b};
  return lut_nf4(w.cb, nf4_params_scale_sel(w, bp, valid));
}
template <int FMT>
__device__ __forceinline__ Lut16 step_lut_group32(const WeightView& w, const StepParams<kFmtINT4>& p,
                                                  int r, int q, bool valid) {
  // scale (low 16 bits) | zero (high 16 bits) of group q
  const uint32_t sz = valid ? perm(p.z[r], p.s[r], q == 0 ? 0x05040100u : 0x07060302u) : 0u;
  return lut_group32<FMT>(w.cb, sz);
}
template <>
__device__ __forceinline__ Lut16 step_lut<kFmtINT4>(const WeightView& w,
                                                    const StepParams<kFmtINT4>& p, int r, int q,
                                                    bool valid) {
  return step_lut_group32<kFmtINT4>(w, p, r, q, valid);
}
template <>
__device__ __forceinline__ Lut16 step_lut<kFmtNFG>(const WeightView& w,
                                                   const StepParams<kFmtNFG>& p, int r, int q,
                                                   bool valid) {
  return step_lut_group32<kFmtNFG>(w, p, r, q, valid);
}

constexpr int kXHalf = kTM * (kKS / 2) * 2;  // token tile of half a K step: 32 KB
constexpr int kCTile = kTN * kKS / 2;        // packed codes of one K step: 16 KB

// Loads in flight per wave between the two barriers of a K step: the group
// issued after the first barrier (token half 0: 8 instructions, codes: 4,
// block constants: 4) and the one after the second (token half 1: 8).
// Every step issues exactly these (past the range they are clamped or
// masked, never skipped), so the waits can count them.
constexpr int kG0Loads = 16;
constexpr int kG1Loads = 8;

// Waits until at most kG0Loads + kG1Loads of this wave's loads are in
// flight and its LDS reads are done, then meets the other waves.  Written as
// one asm block: a fence here would make the compiler wait for every
// direct-to-LDS load in flight, including the ones that are meant to stay in
// flight across the barrier.
__device__ __forceinline__ void stage_barrier() {
  static_assert(kG0Loads + kG1Loads == 24, "the wait below counts 24 loads");
  __asm__ volatile("s_waitcnt vmcnt(24) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A wave-uniform value the compiler may not hoist or fold: each use forms
// what depends on it where it is used.
__device__ __forceinline__ int opaque_sgpr(int v) {
  __asm__ volatile("" : "+s"(v));
  return v;
}

template <int FMT>
__global__ __launch_bounds__(256, 1) void k_fwd_gemm(FwdArgs a) {
  // Four token half-stages and two code stages, each an array of its own so
  // that a read of one is never held for direct-to-LDS loads into another:
  // all 160 KB of LDS.  After the K loop the same memory holds the adapter
  // operands and the output tile.
  __shared__ __attribute__((aligned(16))) uint8_t s_x0[kXHalf];
  __shared__ __attribute__((aligned(16))) uint8_t s_x1[kXHalf];
  __shared__ __attribute__((aligned(16))) uint8_t s_x2[kXHalf];
  __shared__ __attribute__((aligned(16))) uint8_t s_x3[kXHalf];
  __shared__ __attribute__((aligned(16))) uint8_t s_c0[kCTile];
  __shared__ __attribute__((aligned(16))) uint8_t s_c1[kCTile];
  uint32_t* s_ticket = reinterpret_cast<uint32_t*>(s_c0);  // used after the K loop

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t M = a.M, N = a.w.N, K = a.w.K;
  const int tiles_m = static_cast<int>((M + kTM - 1) / kTM);
  const int tiles_n = static_cast<int>((N + kTN - 1) / kTN);
  const int n_work = tiles_m * tiles_n * a.splits;
  const int v = xcd_round_order(static_cast<int>(blockIdx.x), n_work);
  const int sp = v % a.splits;
  const int tmn = v / a.splits;
  int tm, tn;
  grouped_tile(tmn, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * kTM, n0 = static_cast<int64_t>(tn) * kTN;
  const int64_t ksteps = (K + kKS - 1) / kKS;
  const int64_t per = (ksteps + a.splits - 1) / a.splits;
  const int64_t ks0 = sp * per < ksteps ? sp * per : ksteps;
  const int64_t ks1 = ks0 + per < ksteps ? ks0 + per : ksteps;

  int64_t nr[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int64_t n = n0 + wave * 64 + r * 32 + l32;
    nr[r] = n < N ? n : N - 1;
  }
  f32x16 acc[2][8];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int ms = 0; ms < 8; ++ms) acc[r][ms] = f32x16{};

  // Token half-stage of part p of a K step: [256 m][8 pieces of 16 B], piece
  // c holding the step's columns 64 (c / 4) + 32 p + 8 (c % 4) .. +7, so that
  // sub-step 4 p + f reads piece f + 4 h in lane half h (each lane half
  // walks its own 64-column block).  Pieces sit at c ^ ((m / 2) % 8): 16
  // consecutive rows read one piece from 16 distinct bank groups.  Loaded by
  // direct-to-LDS loads through a buffer resource over this tile's rows of
  // x: instruction i of wave w fills rows 32 i + 8 w .. +7 (1 KB), the
  // swizzle applied to the source piece.  Rows past M fall outside the
  // resource (their output rows are never stored).  Pieces past K (the upper
  // block of a last step that holds only 64 columns) and every piece of a
  // step past this split's range load zeros (offset bit 31 set), so no
  // value of another token or step reaches the accumulators.
  const int64_t rows_here = M - m0 < kTM ? M - m0 : kTM;
  const rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.x + m0 * K), 0, static_cast<int>(rows_here * K * 2), 0x00020000);
  const int xpc = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);  // source piece of this lane
  const uint32_t xvoff = static_cast<uint32_t>((8 * wave + (lane >> 3)) * K * 2 + 128 * (xpc >> 2) +
                                               16 * (xpc & 3));
  const uint32_t xvoff_tail = xvoff | (xpc >= 4 ? 0x80000000u : 0u);  // the last step's lane offset
  // a step past the range loads through an empty resource
  const rsrc_t xr_none = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, 0, 0x00020000);
  // (step indices are wave-uniform: taken into scalar registers, so that the
  // range tests are scalar and pick between prepared offsets)
  const int ks1_s = __builtin_amdgcn_readfirstlane(static_cast<int>(ks1));
  const int ks_tail_s = __builtin_amdgcn_readfirstlane(static_cast<int>((K % kKS) != 0 ? ksteps - 1 : -1));
  // LDS offset of this wave's slot in a stage.  Made opaque at each use, so
  // that the destination of every load is formed where the load is issued
  // (scalar adds) instead of being computed once per destination and held
  // for the whole loop, which runs the scalar registers out.
  const int wslot = wave * 1024;
  auto load_xhalf = [&](int64_t ks64, int part, uint8_t* dst, int i0, int n) {
    const int ks = __builtin_amdgcn_readfirstlane(static_cast<int>(ks64));
    const int kc = ks < ks1_s ? ks : ks1_s - 1;
    const uint32_t kb2 = static_cast<uint32_t>(kc * kKS * 2 + 64 * part);
    const rsrc_t rr = ks < ks1_s ? xr : xr_none;
    const uint32_t voff = ks == ks_tail_s ? xvoff_tail : xvoff;
#pragma unroll
    for (int i = i0; i < i0 + n; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rr, (lds_ptr_t)(dst + i * 4096 + opaque_sgpr(wslot)), 16, voff,
          static_cast<int>(static_cast<uint32_t>(i * 32 * K * 2) + kb2), 0, 0);
  };
  // Packed codes of a K step: 256 rows x 64 B in a code stage.  A load
  // instruction covers 16 rows (4 lanes x 16 B each); the four 16-byte
  // pieces of a row are XOR-swizzled by (row / 4) % 4 so that the 16-byte
  // reads of 16 consecutive rows hit distinct banks.  Rows past N fall
  // outside the resource (their outputs are never stored); a step past the
  // range re-reads the last one (its tables are zero).
  const int64_t nrows_here = N - n0 < kTN ? N - n0 : kTN;
  const rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.w.codes + n0 * (K >> 1)), 0, static_cast<int>(nrows_here * (K >> 1)),
      0x00020000);
  const int cpiece = (lane & 3) ^ ((lane >> 4) & 3);
  const uint32_t cvoff = static_cast<uint32_t>((wave * 16 + (lane >> 2)) * (K >> 1) + cpiece * 16);
  auto load_codes = [&](int64_t ks, uint8_t* dst, int i0, int n) {
    const int64_t kc = ks < ks1 ? ks : ks1 - 1;
    const uint32_t kb = static_cast<uint32_t>(kc * (kKS / 2));
#pragma unroll
    for (int i = i0; i < i0 + n; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          cr, (lds_ptr_t)(dst + i * 4096 + opaque_sgpr(wslot)), 16, cvoff,
          static_cast<int>(static_cast<uint32_t>(i * 64 * (K >> 1)) + kb), 0, 0);
  };
  // this lane's 16 code words of a step: rows wave*64 + r*32 + l32, half h
  auto read_codes = [&](const uint8_t* src, u32x4 (&c)[2][2]) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = wave * 64 + r * 32 + l32;
      const int sw = (row >> 2) & 3;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        c[r][q] = *reinterpret_cast<const u32x4*>(src + row * 64 + (((2 * h + q) ^ sw) << 4));
    }
  };
  const ParamSrc<FMT> psrc = param_src<FMT>(a.w, nr, h);
  auto load_step_params = [&](int64_t ks, StepParams<FMT>& p, int r) {
    load_params<FMT>(psrc, ks < ks1 ? ks : ks1 - 1, p, r);
  };
  // the load groups of step ks (see kG0Loads), whole or in quarters: G0
  // quarter q = 2 token pieces, 1 code piece and the constants of row q / 2
  // (a word or the scale, q even; the other word, q odd); G1 quarter q = 2
  // token pieces
  auto issue_g0 = [&](int64_t ks, uint8_t* xdst, uint8_t* cdst, StepParams<FMT>& p, int q) {
    load_xhalf(ks, 0, xdst, 2 * q, 2);
    load_codes(ks, cdst, q, 1);
    load_step_params(ks, p, q);
  };
  auto issue_g1 = [&](int64_t ks, uint8_t* xdst, int q) { load_xhalf(ks, 1, xdst, 2 * q, 2); };

  constexpr int NL = FMT == kFmtNF4 ? 1 : 2;
  Lut16 lut[2][NL];
  auto build_luts = [&](const StepParams<FMT>& p, bool valid) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int q = 0; q < NL; ++q) lut[r][q] = step_lut<FMT>(a.w, p, r, q, valid);
  };
  auto decode_w = [&](const u32x4 (&c)[2][2], int tt, u32x4 (&wf)[2]) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
      wf[r] = lut_decode8(lut[r][NL == 1 ? 0 : (tt >> 2)], c[r][tt >> 2][tt & 3]);
  };
  // token fragments of sub-step f (0..7) from that part's half-stage: row
  // 32 ms + l32, piece (f % 4) + 4 h; the row swizzle (l32 / 2) % 8 does not
  // depend on ms
  const int xsw = (l32 >> 1) & 7;
  auto read_x = [&](const uint8_t* xb, int f, u32x4 (&xf)[8]) {
    const uint32_t o = static_cast<uint32_t>(l32 * 128 + ((((f & 3) + 4 * h) ^ xsw) << 4));
#pragma unroll
    for (int ms = 0; ms < 8; ++ms) xf[ms] = *reinterpret_cast<const u32x4*>(xb + o + ms * 4096);
  };
  auto step_valid = [&](int64_t ks64) {
    const int ks = __builtin_amdgcn_readfirstlane(static_cast<int>(ks64));
    return ks < ks1_s && ks * kKS + h * 64 < static_cast<int>(K);
  };

  // Pipeline.  The K steps run in pairs: step 2j + SI of the range uses
  // token half-stages (s_x0, s_x1) or (s_x2, s_x3) and code stage s_c0 or
  // s_c1 by SI, and block-constant register set P[SI] holds the constants of
  // step ks + 2 from its load to its use.  Sub-step f reads its fragments
  // (and decodes its weights) during sub-step f - 1.  Two barriers per step:
  //   after sub-step 2: part 0 of this step is read by every wave (its
  //     half-stage is free), and this step's part 1 has landed;
  //   after sub-step 6: part 1 is read (free), and part 0, codes and
  //     constants of the next step have landed.
  // Each freed stage is refilled with step ks + 2, and the refills are spread
  // evenly over the step, one load every four or eight MFMAs: the load path
  // of a compute unit takes a 1 KB direct-to-LDS load only every few tens of
  // cycles, and a wave that issues faster than that stalls, matrix cores
  // included.  G0 of step ks + 2 goes out a quarter at a time in sub-steps
  // 3-6 of step ks, G1 in sub-step 7 and sub-steps 0-2 of the next step, so
  // every load has 8 to 11 sub-steps to land.
  const int64_t nsteps = ks1 - ks0;
  const int64_t npairs = (nsteps + 1) >> 1;
  // The prologue issues the groups of the first two steps in this order, up
  // to the first quarter of G1 of the second step (the loop issues the rest
  // in its first three sub-steps), then waits for the first group.
  // Scheduling barriers keep the constants' loads inside their groups, as
  // the waits assume.
  StepParams<FMT> P[2];
#pragma unroll
  for (int q = 0; q < 4; ++q) issue_g0(ks0, s_x0, s_c0, P[0], q);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 4; ++q) issue_g1(ks0, s_x1, q);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 4; ++q) issue_g0(ks0 + 1, s_x2, s_c1, P[1], q);
  __builtin_amdgcn_sched_barrier(0);
  issue_g1(ks0 + 1, s_x3, 0);
  __builtin_amdgcn_sched_barrier(0);
  static_assert(kG1Loads + kG0Loads + kG1Loads / 4 == 26, "prologue wait");
  __asm__ volatile("s_waitcnt vmcnt(26)\n\ts_barrier" ::: "memory");
  build_luts(P[0], step_valid(ks0));

  // Two-stage register pipeline over the eight k16 sub-steps of a K step:
  // while the 16 MFMAs of sub-step tt run, the weight words of tt + 1 are
  // decoded and its token fragments read from LDS.
  u32x4 cw[2][2], wf[2][2], xf[2][8];
  read_codes(s_c0, cw);
  read_x(s_x0, 0, xf[0]);
  decode_w(cw, 0, wf[0]);
  // The loop body has no branches: a branch splits the scheduling region,
  // and the MFMA / decode / load interleave is lost.
  auto step = [&](int64_t ks, auto si_c) __attribute__((always_inline)) {
    constexpr int SI = decltype(si_c)::value;
    uint8_t* const xa = SI == 0 ? s_x0 : s_x2;  // this step, part 0
    uint8_t* const xb = SI == 0 ? s_x1 : s_x3;  // this step, part 1
    uint8_t* const xn = SI == 0 ? s_x2 : s_x0;  // next step, part 0
    uint8_t* const cc = SI == 0 ? s_c0 : s_c1;  // this step's codes (refilled with step ks + 2)
    uint8_t* const cn = SI == 0 ? s_c1 : s_c0;  // next step's codes
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int cur = tt & 1, nxt = cur ^ 1;
      if (tt < 7) {
        decode_w(cw, tt + 1, wf[nxt]);
        read_x(tt + 1 < 4 ? xa : xb, tt + 1, xf[nxt]);
      } else {
        // the next step's tables, codes, first token fragments and first
        // decode (past the range: zero tables)
        build_luts(P[SI ^ 1], step_valid(ks + 1));
        read_codes(cn, cw);
        read_x(xn, 0, xf[nxt]);
        decode_w(cw, 0, wf[nxt]);
      }
      // refills: G1 of step ks + 1 (quarters 1-3, into the previous step's
      // part-1 stage), G0 of step ks + 2, the first quarter of its G1
      if (tt < 3) issue_g1(ks + 1, SI == 0 ? s_x3 : s_x1, tt + 1);
      if (tt >= 3 && tt < 7) issue_g0(ks + 2, xa, cc, P[SI], tt - 3);
      if (tt == 7) issue_g1(ks + 2, xb, 0);
#pragma unroll
      for (int ms = 0; ms < 8; ++ms) {
        acc[0][ms] = mfma32(wf[cur][0], xf[cur][ms], acc[0][ms]);
        acc[1][ms] = mfma32(wf[cur][1], xf[cur][ms], acc[1][ms]);
      }
      // issue order: the LDS reads of the next sub-step first (8 token
      // fragments; in sub-step 7 also the 4 code reads), then per MFMA 3 VALU
      // of the next decode (7 in sub-step 7: the tables as well), and a
      // refill load after every fourth (sub-steps 3-6) or eighth MFMA
      constexpr int kVmemEvery[8] = {8, 8, 8, 4, 4, 4, 4, 8};
      if (tt < 7)
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      else
        __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i % kVmemEvery[tt] == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        if (tt < 7)
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (tt == 2 || tt == 6) stage_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int64_t pi = 0; pi < npairs; ++pi) {
    step(ks0 + 2 * pi, std::integral_constant<int, 0>{});
    step(ks0 + 2 * pi + 1, std::integral_constant<int, 1>{});
  }
  // the loads of the two steps past the range land, and every wave is past
  // its last reads, before the memory is reused
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // adapter term: acc += B[n][j] * (s u[m][j]) over j, in k16 steps, with
  // s u split into hi + lo bf16 halves (two MFMAs per step).  s u of the
  // tile's 256 tokens (as the two halves) and B of its 256 features are
  // staged in LDS 48 adapter columns at a time (rows padded by 16 B against
  // bank conflicts; each operand fills one 28 KB half-stage), every load of a
  // chunk in flight at once.  Indices are clamped and values masked (no
  // divergent branches around loads).
  if (sp == 0 && a.u != nullptr && a.r > 0) {
    const int rr = a.r;
    constexpr int kJC = 48;          // adapter columns per staged chunk
    constexpr int rp = kJC + 8;      // staged row length (elements)
    constexpr int q4 = kJC / 4;      // 4-element pieces of a staged row
    static_assert(kTM * rp * 2 <= kXHalf, "a staged operand fits a half-stage");
    uint16_t* s_uh = reinterpret_cast<uint16_t*>(s_x0);  // [256 m][rp]
    uint16_t* s_ul = reinterpret_cast<uint16_t*>(s_x1);  // [256 m][rp]
    uint16_t* s_b = reinterpret_cast<uint16_t*>(s_x2);   // [256 n][rp]
    constexpr int kUPer = kTM * q4 / 256;                 // 12 pieces of each kind per thread
    for (int jc = 0; jc < rr; jc += kJC) {
      f32x4 uv[kUPer];
      u32x2 bv[kUPer];
#pragma unroll
      for (int q = 0; q < kUPer; ++q) {
        const int it = q * 256 + tid;
        const int row = it / q4, j = jc + (it - row * q4) * 4;
        int64_t mg = m0 + row, ng = n0 + row;
        mg = mg < M ? mg : M - 1;
        ng = ng < N ? ng : N - 1;
        const float* urow = a.u + mg * rr;
        const uint16_t* brow = a.B + ng * rr;
        if ((rr & 3) == 0) {
          const int jj = j < rr ? j : rr - 4;
          uv[q] = *reinterpret_cast<const f32x4*>(urow + jj);
          bv[q] = *reinterpret_cast<const u32x2*>(brow + jj);
        } else {
          uint32_t e4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jj = j + e < rr ? j + e : rr - 1;
            uv[q][e] = urow[jj];
            e4[e] = brow[jj];
          }
          bv[q] = u32x2{e4[0] | (e4[1] << 16), e4[2] | (e4[3] << 16)};
        }
      }
      if (jc > 0) __syncthreads();  // the previous chunk's operands are consumed
#pragma unroll
      for (int q = 0; q < kUPer; ++q) {
        const int it = q * 256 + tid;
        const int row = it / q4, jl = (it - row * q4) * 4, j = jc + jl;
        float hv[4], lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(j + e < rr ? a.s * uv[q][e] : 0.0f, hv[e], lv[e]);
        *reinterpret_cast<u32x2*>(s_uh + row * rp + jl) = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
        *reinterpret_cast<u32x2*>(s_ul + row * rp + jl) = u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])};
        const uint32_t k0 = (j < rr ? 0x0000FFFFu : 0u) | (j + 1 < rr ? 0xFFFF0000u : 0u);
        const uint32_t k1 = (j + 2 < rr ? 0x0000FFFFu : 0u) | (j + 3 < rr ? 0xFFFF0000u : 0u);
        *reinterpret_cast<u32x2*>(s_b + row * rp + jl) = u32x2{bv[q].x & k0, bv[q].y & k1};
      }
      __syncthreads();
      const int jt_n = (rr - jc < kJC ? rr - jc + 15 : kJC) / 16;
      for (int jt = 0; jt < jt_n; ++jt) {
        const int j0 = jt * 16 + h * 8;
        u32x4 bf[2];
#pragma unroll
        for (int r = 0; r < 2; ++r)
          bf[r] = *reinterpret_cast<const u32x4*>(s_b + (wave * 64 + r * 32 + l32) * rp + j0);
#pragma unroll
        for (int ms = 0; ms < 8; ++ms) {
          const int ml = ms * 32 + l32;
          const u32x4 uh = *reinterpret_cast<const u32x4*>(s_uh + ml * rp + j0);
          const u32x4 ul = *reinterpret_cast<const u32x4*>(s_ul + ml * rp + j0);
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            acc[r][ms] = mfma32(bf[r], uh, acc[r][ms]);
            acc[r][ms] = mfma32(bf[r], ul, acc[r][ms]);
          }
        }
      }
    }
    __syncthreads();  // the staged operands are read before s_x is reused
  }

  if (a.splits > 1) {
    // publish this split's partial tile as 16-byte pieces (four consecutive
    // accumulator values of a lane); the tile's last workgroup adds the
    // splits in fixed order
    const rsrc_t pr = make_rsrc(a.partial);
    auto poff = [&](int s2, int r, int ms, int v4) {
      return static_cast<uint32_t>((((static_cast<int64_t>(tmn) * a.splits + s2) * (kTM * kTN)) +
                                    ((r * 8 + ms) * 4 + v4) * 1024 + tid * 4) * 4);
    };
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int ms = 0; ms < 8; ++ms)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          st_sys16(pr, poff(sp, r, ms, v4),
                   f32x4{acc[r][ms][4 * v4], acc[r][ms][4 * v4 + 1], acc[r][ms][4 * v4 + 2], acc[r][ms][4 * v4 + 3]});
    if (publish_and_ticket(a.counters + tmn, s_ticket) != static_cast<uint32_t>(a.splits - 1))
      return;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int ms = 0; ms < 8; ++ms) {
        f32x4 sum[4] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                        f32x4{0.f, 0.f, 0.f, 0.f}};
        for (int s2 = 0; s2 < a.splits; ++s2) {
          f32x4 v[4];
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) v[v4] = ld_sys16(pr, poff(s2, r, ms, v4));
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) sum[v4] += v[v4];
        }
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[r][ms][4 * v4 + e] = sum[v4][e];
      }
    if (tid == 0) a.counters[tmn] = 0u;
  }

  // store: lane holds D[n = 8i + 4h + t][m = l32] of each 32x32 tile, i.e.
  // 8 bytes of 32 different output rows per instruction.  The bf16 tile goes
  // through LDS instead ([256 m][512 B], rows 64 q .. 64 q + 63 in half-stage
  // q, 16-byte pieces at column piece XOR the row's low 5 bits), and leaves
  // as whole 16-byte pieces of rows, 32 consecutive threads per 512-byte row.
  __syncthreads();  // every wave is done with the LDS (adapter operands, ticket)
  uint8_t* const s_y[4] = {s_x0, s_x1, s_x2, s_x3};
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int ms = 0; ms < 8; ++ms) {
      const int row = (ms & 1) * 32 + l32;  // within half-stage ms / 2
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p16 = wave * 8 + r * 4 + i;  // 16-byte piece of the row (columns 8 p16 ..)
        u32x2 o;
        o.x = pack_bf16x2(acc[r][ms][4 * i + 0], acc[r][ms][4 * i + 1]);
        o.y = pack_bf16x2(acc[r][ms][4 * i + 2], acc[r][ms][4 * i + 3]);
        *reinterpret_cast<u32x2*>(s_y[ms >> 1] + row * 512 + ((p16 ^ (row & 31)) << 4) + h * 8) = o;
      }
    }
  __syncthreads();
#pragma unroll
  for (int hs = 0; hs < 4; ++hs)
#pragma unroll 4
    for (int q = 0; q < 8; ++q) {
      const int piece = q * 256 + tid, row = piece >> 5, p16 = piece & 31;  // row within the half-stage
      const int64_t m = m0 + hs * 64 + row, n = n0 + p16 * 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(s_y[hs] + row * 512 + ((p16 ^ (row & 31)) << 4));
      if (m < M && n < N) *reinterpret_cast<u32x4*>(a.y + m * N + n) = v;
    }
}

}  // namespace

int fwd_gemm_tiles(int64_t M, int64_t N) {
  return static_cast<int>(((M + kTM - 1) / kTM) * ((N + kTN - 1) / kTN));
}
int64_t fwd_gemm_partial_floats(int64_t M, int64_t N, int splits) {
  return splits > 1 ? static_cast<int64_t>(fwd_gemm_tiles(M, N)) * splits * kTM * kTN : 0;
}

hipError_t launch_fwd_gemm(const FwdArgs& a, int fmt, hipStream_t stream) {
  const int grid = fwd_gemm_tiles(a.M, a.w.N) * a.splits;
  if (fmt == kFmtNF4)
    hipLaunchKernelGGL(k_fwd_gemm<kFmtNF4>, dim3(grid), dim3(256), 0, stream, a);
  else if (fmt == kFmtINT4)
    hipLaunchKernelGGL(k_fwd_gemm<kFmtINT4>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_fwd_gemm<kFmtNFG>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
