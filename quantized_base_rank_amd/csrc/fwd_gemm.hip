// Fused forward of the adapted 4-bit layer for many tokens:
//     y = x W_bf16^T + (s u) B^T
// [QLoRA "The QLoRA recipe" stage 3 / "The complete QLoRA forward pass": each
// weight block is brought back to bf16 on the fly, multiplied by the input,
// and the adapter correction is added; QA-LoRA abstract for the INT4 groups.]
//
// Tile: 256 tokens x 256 output features per workgroup of 4 waves; wave w
// owns features [64w, 64w+64) for all 256 tokens, so every 4-bit weight is
// decoded exactly once per workgroup, straight from HBM into registers
// (byte-permute lookup, no LDS), and reused by 8 MFMAs.  The 256x128 bf16
// token tile of each K step is streamed into LDS with direct-to-LDS loads
// (double buffered, XOR-swizzled 16-byte chunks: conflict-free reads).
// The adapter term is 2*ceil(r/16) extra MFMA k-steps on the same
// accumulators, with s*u split into hi + lo bf16 halves.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kTM = 256;
constexpr int kTN = 256;
constexpr int kKS = 128;
constexpr int kXTile = kTM * kKS * 2;  // bytes

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Token tile in LDS: 256 B per row (128 k), 16-byte chunks XOR-swizzled by
// the row's low four bits so that 16 consecutive rows (the lanes of one
// LDS cycle) read 16 distinct bank groups.
__device__ __forceinline__ uint32_t xoff(int row, int chunk) {
  return static_cast<uint32_t>(row * 256 + ((chunk ^ (row & 15)) << 4));
}

// Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
// contiguous run of tiles (tile order: token tile major) so that the
// workgroups resident on one XCD share their token rows in its L2.
__device__ __forceinline__ int remap_xcd(int bid, int n) {
  const int q = n >> 3, rem = n & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// Raw block constants of one K step for a lane's two rows (the scale is
// formed when the table is built, so the loads are consumed a step later).
template <int FMT>
struct StepParams;
template <>
struct StepParams<kFmtNF4> {
  BlockParams bp[2];  // per row: a = the 8-bit code (DQ), b = fp32 bits of s2 or absmax
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

// Block constants of K step ks (blocks 2 ks + h).  Near the end of K a lane
// of the upper half may read the next row's constants (or zeros past the
// array); such blocks are masked when the table is built.
template <int FMT>
__device__ __forceinline__ void load_params(const ParamSrc<FMT>& ps, int64_t ks, StepParams<FMT>& p);
template <>
__device__ __forceinline__ void load_params<kFmtNF4>(const ParamSrc<kFmtNF4>& ps, int64_t ks,
                                                     StepParams<kFmtNF4>& p) {
  const uint32_t b2 = static_cast<uint32_t>(2 * ks);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    p.bp[r].a = __builtin_amdgcn_raw_buffer_load_b8(ps.r8, ps.lb[r], static_cast<int>(b2), 0);
    p.bp[r].b = __builtin_amdgcn_raw_buffer_load_b32(ps.rw, ((ps.lb[r] + b2) >> ps.sh) << 2, 0, 0);
  }
}
template <>
__device__ __forceinline__ void load_params<kFmtINT4>(const ParamSrc<kFmtINT4>& ps, int64_t ks,
                                                      StepParams<kFmtINT4>& p) {
  const int g8 = static_cast<int>(8 * ks);  // 4 groups of 2 bytes per step
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    p.s[r] = __builtin_amdgcn_raw_buffer_load_b32(ps.rs, ps.lg[r], g8, 0);
    p.z[r] = __builtin_amdgcn_raw_buffer_load_b32(ps.rz, ps.lg[r], g8, 0);
  }
}

template <>
__device__ __forceinline__ void load_params<kFmtNFG>(const ParamSrc<kFmtNFG>& ps, int64_t ks,
                                                     StepParams<kFmtNFG>& p) {
  load_params<kFmtINT4>(ps, ks, p);
}

template <int FMT>
__device__ __forceinline__ Lut16 step_lut(const WeightView& w, const StepParams<FMT>& p, int r,
                                          int q, bool valid);
template <>
__device__ __forceinline__ Lut16 step_lut<kFmtNF4>(const WeightView& w,
                                                   const StepParams<kFmtNF4>& p, int r, int,
                                                   bool valid) {
  // an invalid block (past K) decodes to zeros through a zero scale
  return lut_nf4(w.cb, nf4_params_scale_sel(w, p.bp[r], valid));
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

constexpr int kCTile = kTN * kKS / 2;  // packed codes of one K step: 16 KB

template <int FMT>
__global__ __launch_bounds__(256, 1) void k_fwd_gemm(FwdArgs a) {
  // two stages of [token tile 64 KB | packed codes 16 KB] = all 160 KB of LDS
  __shared__ __attribute__((aligned(16))) uint8_t s_x[2][kXTile + kCTile];
  uint32_t* s_ticket = reinterpret_cast<uint32_t*>(&s_x[0][0]);  // used after the K loop

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t M = a.M, N = a.w.N, K = a.w.K;
  const int tiles_m = static_cast<int>((M + kTM - 1) / kTM);
  const int tiles_n = static_cast<int>((N + kTN - 1) / kTN);
  const int n_work = tiles_m * tiles_n * a.splits;
  const int t = remap_xcd(static_cast<int>(blockIdx.x), n_work);
  const int sp = t % a.splits;
  const int tmn = t / a.splits;
  const int tm = tmn / tiles_n, tn = tmn % tiles_n;
  const int64_t m0 = static_cast<int64_t>(tm) * kTM, n0 = static_cast<int64_t>(tn) * kTN;
  const int64_t ksteps = (K + kKS - 1) / kKS;
  const int64_t per = (ksteps + a.splits - 1) / a.splits;
  const int64_t ks0 = sp * per;
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

  // Token tile source: a buffer resource over this tile's rows of x, so a
  // load is one instruction with a fixed per-lane offset and a scalar
  // per-step offset.  Rows past M fall outside the resource (their output
  // rows are never stored).  When the last K step holds only 64 columns
  // (K % 128 == 64), its upper eight 16-byte pieces of a row would be the
  // next token's first columns: their offsets are moved past the resource
  // (bit 31), so they load zeros and a non-finite value in one token never
  // reaches another token's output through the zero weights there.
  const int64_t rows_here = M - m0 < kTM ? M - m0 : kTM;
  const rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.x + m0 * K), 0, static_cast<int>(rows_here * K * 2), 0x00020000);
  const int lrow = wave * 4 + (lane >> 4);  // row within each group of 16
  const int xpiece = (lane & 15) ^ lrow;    // 16-byte piece of the step's 128 columns
  const uint32_t xvoff = static_cast<uint32_t>(lrow * K * 2 + (xpiece << 4));
  const uint32_t xtail_oob = xpiece >= 8 ? 0x80000000u : 0u;
  const int64_t ks_tail = (K % kKS) != 0 ? ksteps - 1 : -1;
  auto load_x = [&](int64_t ks, int buf) {
    const uint32_t kb2 = static_cast<uint32_t>(ks * kKS * 2);
    const uint32_t voff = xvoff | (xtail_oob & (ks == ks_tail ? 0xFFFFFFFFu : 0u));
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (lds_ptr_t)(&s_x[buf][(i * 4 + wave) * 1024]), 16, voff,
          static_cast<int>(static_cast<uint32_t>(i * 16 * K * 2) + kb2), 0, 0);
  };
  // Packed codes of a K step: 256 rows x 64 B into LDS next to the token
  // tile.  A load instruction covers 16 rows (4 lanes x 16 B each); the four
  // 16-byte pieces of a row are XOR-swizzled by (row / 4) % 4 so that the
  // 16-byte reads of 16 consecutive rows hit distinct banks.  Rows past N
  // fall outside the resource (their outputs are never stored).
  const int64_t nrows_here = N - n0 < kTN ? N - n0 : kTN;
  const rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.w.codes + n0 * (K >> 1)), 0, static_cast<int>(nrows_here * (K >> 1)),
      0x00020000);
  const int cpiece = (lane & 3) ^ ((lane >> 4) & 3);
  const uint32_t cvoff = static_cast<uint32_t>((wave * 16 + (lane >> 2)) * (K >> 1) + cpiece * 16);
  auto load_codes = [&](int64_t ks, int buf) {
    const uint32_t kb = static_cast<uint32_t>(ks * (kKS / 2));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          cr, (lds_ptr_t)(&s_x[buf][kXTile + (i * 4 + wave) * 1024]), 16, cvoff,
          static_cast<int>(static_cast<uint32_t>(i * 64 * (K >> 1)) + kb), 0, 0);
  };
  // this lane's 16 code words of a step: rows wave*64 + r*32 + l32, half h
  auto read_codes = [&](int buf, u32x4 (&c)[2][2]) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = wave * 64 + r * 32 + l32;
      const int sw = (row >> 2) & 3;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        c[r][q] = *reinterpret_cast<const u32x4*>(&s_x[buf][kXTile + row * 64 + (((2 * h + q) ^ sw) << 4)]);
    }
  };
  const ParamSrc<FMT> psrc = param_src<FMT>(a.w, nr, h);
  auto load_step_params = [&](int64_t ks, StepParams<FMT>& p) { load_params<FMT>(psrc, ks, p); };

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
  auto read_x = [&](const uint8_t* xb, int tt, u32x4 (&xf)[8]) {
#pragma unroll
    for (int ms = 0; ms < 8; ++ms)
      xf[ms] = *reinterpret_cast<const u32x4*>(xb + xoff(ms * 32 + l32, 8 * h + tt));
  };
  auto step_valid = [&](int64_t ks) { return ks * kKS + h * 64 < K; };

  // Tiles and codes run one K step ahead, block constants two.  The stage
  // barrier sits after sub-step 6: by then every wave has read its last
  // token fragments of the step, and the next step's data has landed, so
  // sub-step 7 overlaps its MFMAs with the next step's tables, code reads
  // and first decode (no bubble at the top of a step).
  StepParams<FMT> pc, pn, p2;
  load_x(ks0, 0);
  load_codes(ks0, 0);
  load_step_params(ks0, pc);
  if (ks0 + 1 < ks1) load_step_params(ks0 + 1, pn);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  build_luts(pc, step_valid(ks0));

  // Two-stage register pipeline over the eight k16 sub-steps of a K step:
  // while the 16 MFMAs of sub-step tt run, the weight words of tt + 1 are
  // decoded and its token fragments read from LDS.
  u32x4 cw[2][2], wf[2][2], xf[2][8];
  read_codes(0, cw);
  read_x(s_x[0], 0, xf[0]);
  decode_w(cw, 0, wf[0]);
  // The loop body has no branches (a branch splits the scheduling region and
  // the MFMA / decode interleave is lost), so it is instantiated once per
  // wave with that wave's load slot fixed, and the loads of a missing next
  // step are clamped to re-read the current one into the idle stage.
  auto k_loop = [&](auto wave_c) __attribute__((always_inline)) {
  constexpr int W = decltype(wave_c)::value;
  for (int64_t ks = ks0; ks < ks1; ++ks) {
    const int buf = static_cast<int>((ks - ks0) & 1);
    const int64_t kn = ks + 1 < ks1 ? ks + 1 : ks;
    const int64_t kp = ks + 2 < ks1 ? ks + 2 : ks1 - 1;
    const uint8_t* xb = s_x[buf];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int cur = tt & 1, nxt = cur ^ 1;
      if (tt < 7) {
        decode_w(cw, tt + 1, wf[nxt]);
        read_x(xb, tt + 1, xf[nxt]);
      } else {
        // the next step's tables, codes, first token fragments and first
        // decode (on the last step: harmless reads of the idle stage)
        build_luts(pn, step_valid(ks + 1));
        read_codes(buf ^ 1, cw);
        read_x(s_x[buf ^ 1], 0, xf[nxt]);
        decode_w(cw, 0, wf[nxt]);
      }
#pragma unroll
      for (int ms = 0; ms < 8; ++ms) {
        acc[0][ms] = mfma32(wf[cur][0], xf[cur][ms], acc[0][ms]);
        acc[1][ms] = mfma32(wf[cur][1], xf[cur][ms], acc[1][ms]);
      }
      if (tt < 7) {
        // issue order: the 8 LDS reads of the next sub-step first, then
        // {1 MFMA, 3 VALU of the next decode} x 16
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      } else {
        // the next step's 4 code reads and 8 token-fragment reads first,
        // then {1 MFMA, 7 VALU of its tables and first decode} x 16
        __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // Next step's loads, one wave at a time: a wave blocks while the load
      // path takes its 1 KB load instructions, so the waves take turns
      // (wave w after sub-step w) and the other three keep issuing MFMAs.
      // The target stage was last read before the previous step's barrier.
      if (tt == W) {
        load_x(kn, buf ^ 1);
        load_codes(kn, buf ^ 1);
        load_step_params(kp, p2);
      }
      if (tt == 6) {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    pc = pn;
    pn = p2;
  }
  };
  switch (wave) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    default: k_loop(std::integral_constant<int, 3>{}); break;
  }

  // adapter term: acc += B[n][j] * (s u[m][j]) over j, in k16 steps, with
  // s u split into hi + lo bf16 halves (two MFMAs per step).  s u of the
  // tile's 256 tokens (as the two halves) and B of its 256 features are
  // staged in LDS 64 adapter columns at a time (rows padded by 16 B against
  // bank conflicts), every load of a chunk in flight at once.  Indices are
  // clamped and values masked (no divergent branches around loads).
  if (sp == 0 && a.u != nullptr && a.r > 0) {
    const int rr = a.r;
    constexpr int kJC = 64;          // adapter columns per staged chunk
    constexpr int rp = kJC + 8;      // staged row length (elements)
    constexpr int q4 = kJC / 4;      // 4-element pieces of a staged row
    uint16_t* s_uh = reinterpret_cast<uint16_t*>(&s_x[0][0]);  // [256 m][rp]
    uint16_t* s_ul = s_uh + kTM * rp;                           // [256 m][rp]
    uint16_t* s_b = s_ul + kTM * rp;                            // [256 n][rp], 110.6 KB in all
    constexpr int kUPer = kTM * q4 / 256;                       // 16 pieces of each kind per thread
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
  // through LDS instead ([256 m][512 B], 16-byte pieces at column piece XOR
  // the row's low 5 bits), and leaves as whole 16-byte pieces of rows, 32
  // consecutive threads per 512-byte row.
  __syncthreads();  // every wave is done with the LDS (adapter operands, ticket)
  uint8_t* const s_y = &s_x[0][0];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int ms = 0; ms < 8; ++ms) {
      const int row = ms * 32 + l32;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p16 = wave * 8 + r * 4 + i;  // 16-byte piece of the row (columns 8 p16 ..)
        u32x2 o;
        o.x = pack_bf16x2(acc[r][ms][4 * i + 0], acc[r][ms][4 * i + 1]);
        o.y = pack_bf16x2(acc[r][ms][4 * i + 2], acc[r][ms][4 * i + 3]);
        *reinterpret_cast<u32x2*>(s_y + row * 512 + ((p16 ^ (row & 31)) << 4) + h * 8) = o;
      }
    }
  __syncthreads();
#pragma unroll 8
  for (int q = 0; q < 32; ++q) {
    const int piece = q * 256 + tid, row = piece >> 5, p16 = piece & 31;
    const int64_t m = m0 + row, n = n0 + p16 * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(s_y + row * 512 + ((p16 ^ (row & 31)) << 4));
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
