// Input gradient of the adapted 4-bit layer for many tokens:
//     dX = dY W_bf16 + du A            (QA-LoRA: A repeated over each group)
// [QLoRA "The QLoRA recipe" stage 3: gradients flow back through the frozen,
//  dequantized weight; W itself receives no gradient.]
//
// The reduction runs over the output features n, i.e. across rows of the
// packed weight.  Tile: 256 columns of dX x 256 tokens per workgroup of 4
// waves, one per SIMD.  In each 64-row step wave w decodes the weights of
// columns [64 w, 64 w + 64) (one NF4 block, two INT4 groups): every lane
// one weight row (one table per lane), written row-major into the wave's
// LDS slab.  The products are arranged 2 x 2: wave 2 wk + wm computes
// columns [128 wk, 128 wk + 128) for tokens [128 wm, 128 wm + 128) from its
// own slab and its neighbour's, the transposing LDS read turning 8
// consecutive rows of one column into an MFMA operand.  The next step's
// weights are decoded while the current step's MFMAs run (a two-stage
// register pipeline over the four 16-row sub-steps).  dY streams through a
// ring of four half-step stages and the packed codes (whole rows, shared by
// the four waves) through two stages, by direct-to-LDS loads spread over
// the step; two barriers per step wait with counted vmcnt.  Each LDS stage
// is an array of its own, so that the compiler can tell that reads of one
// stage do not depend on loads still landing in another.
// The adapter term du A is 2*ceil(r/16) extra MFMA k-steps (du split hi +
// lo), read from A^T [K][r].
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kTK = 256;                  // dX columns per tile
constexpr int kTMx = 256;                 // tokens per tile
constexpr int kNS = 64;                   // reduction rows per step
constexpr int kWReg = kNS * 64 * 2;       // one wave's decoded slab: 64 rows x 64 columns, 8 KB
constexpr int kWStage = 4 * kWReg;        // 32 KB
constexpr int kDyHalf = kTMx * (kNS / 2) * 2;  // dY of half a step: 16 KB
constexpr int kCStage = kNS * kTK / 2;    // packed codes of a step: 8 KB

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Decoded slab row n: 128 B, 16-byte piece c (columns 8c .. 8c+7) at
// position (c + 2 n + n / 4) mod 8.  Measured with the LDS bank-conflict
// counter, this placement is conflict-free both for the 16-byte row writes
// (64 lanes, one row each) and for the transposing operand reads; an XOR of
// the row bits, conflict-free for the reads, made every write wait 8 cycles.
__device__ __forceinline__ int wpos(int c, int n) { return (c + 2 * n + (n >> 2)) & 7; }

// dY half-stage [m][32 bf16] (the rows n of two sub-steps): rows of 64 B,
// 16-byte piece c at c ^ ((m / 4) % 4), so that 16 consecutive rows read one
// piece from 16 distinct bank groups.
__device__ __forceinline__ int dsw(int m) { return (m >> 2) & 3; }

// Loads in flight per wave between two barriers: one K step's loads (dY: 8
// instructions, codes: 2, decode constants: 2).  Every step issues exactly
// these (past the range they are clamped or masked, never skipped), so the
// waits can count them.
constexpr int kStepLoads = 12;

// Waits until at most one step's loads of this wave are in flight and its
// LDS accesses are done, then meets the other waves.  One asm block: a fence
// here would make the compiler wait for every direct-to-LDS load in flight.
__device__ __forceinline__ void stage_barrier() {
  static_assert(kStepLoads == 12, "the wait below counts 12 loads");
  __asm__ volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Raw decode constants of one lane's row segment (64 columns).
template <int FMT>
struct RowParams;
template <>
struct RowParams<kFmtNF4> {
  BlockParams bp;  // a = the aligned word holding the 8-bit code (DQ)
  uint32_t sh;     // bit position of the code in a
};
template <>
struct RowParams<kFmtINT4> {
  uint32_t s, z;  // fp16 scales and zeros of the two groups, low group first
};
template <>
struct RowParams<kFmtNFG> : RowParams<kFmtINT4> {};  // the same group words

template <int FMT>
__global__ __launch_bounds__(256, 1) void k_dx_gemm(DxArgs a) {
  // decoded-weight stages (2 x 32 KB), dY half-stages (4 x 16 KB) and code
  // stages (2 x 8 KB), each an array of its own so that a read of one is
  // never held for direct-to-LDS loads into another; after the loop the same
  // memory holds the adapter operands and the output tile
  __shared__ __attribute__((aligned(16))) uint8_t s_w0[kWStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_w1[kWStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_dy0[kDyHalf];
  __shared__ __attribute__((aligned(16))) uint8_t s_dy1[kDyHalf];
  __shared__ __attribute__((aligned(16))) uint8_t s_dy2[kDyHalf];
  __shared__ __attribute__((aligned(16))) uint8_t s_dy3[kDyHalf];
  __shared__ __attribute__((aligned(16))) uint8_t s_c0[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_c1[kCStage];
  uint8_t* const s_w[2] = {s_w0, s_w1};
  uint8_t* const s_c[2] = {s_c0, s_c1};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5, l16 = lane & 15;
  const int64_t M = a.M, N = a.w.N, K = a.w.K;
  const int tiles_m = static_cast<int>((M + kTMx - 1) / kTMx);
  const int tiles_k = static_cast<int>((K + kTK - 1) / kTK);
  // tiles in 4 x 8 blocks per XCD (4 token tiles sharing their dY rows, 8
  // column tiles sharing their packed weight columns)
  int tm, tk;
  grouped_tile(xcd_round_order(static_cast<int>(blockIdx.x), tiles_m * tiles_k), tiles_m, tiles_k, tm, tk);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tk = __builtin_amdgcn_readfirstlane(tk);
  const int64_t m0 = static_cast<int64_t>(tm) * kTMx, k0 = static_cast<int64_t>(tk) * kTK;
  // whole pairs of steps (a step past the last one meets weight rows past N,
  // which decode to zero)
  const int64_t nsteps = (N + kNS - 1) / kNS;
  const int64_t npairs = (nsteps + 1) >> 1;

  // this wave's 64 columns (clamped into the matrix; masked when past K)
  const int64_t kw = k0 + wave * 64;
  const bool kvalid = kw < K;
  const int64_t kwc = kvalid ? kw : k0;

  // products: wave w = 2 wk + wm owns dX columns [128 wk, 128 wk + 128) of
  // the tile (4 column tiles of 32) for tokens [128 wm, 128 wm + 128) (4
  // token tiles of 32); it decodes the weights of columns [64 w, 64 w + 64)
  // (its slab), half of what it and its neighbour (w ^ 1) read.
  const int wk = wave >> 1, wm = wave & 1;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // dY half-stage (part p of step st: the step's rows n 32 p .. 32 p + 31)
  // by direct-to-LDS loads: instruction i of wave w fills tokens
  // 64 i + 16 w .. +15 (1 KB), the swizzle applied to the source piece.
  // Rows past M fall outside the resource (their outputs are never stored).
  // Pieces past N in the last step (they would be the next token's first
  // values) and every piece of a step past the last one load zeros (offset
  // bit 31 set), so that a non-finite dY value never reaches another
  // token's dX through the zero weights there.
  const int64_t dy_rows = M - m0 < kTMx ? M - m0 : kTMx;
  const rsrc_t dyr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.dy + m0 * N), 0, static_cast<int>(dy_rows * N * 2), 0x00020000);
  const int dpiece = (lane & 3) ^ ((lane >> 4) & 3);  // source piece of this lane
  const uint32_t dyvoff = static_cast<uint32_t>((wave * 16 + (lane >> 2)) * N * 2 + (dpiece << 4));
  const int n_tail = static_cast<int>(N % kNS);  // valid rows of the last step (0: all)
  // lane offsets of the last step's two parts (pieces past N out of range)
  uint32_t dyvoff_tail[2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
    dyvoff_tail[p] = dyvoff | ((n_tail != 0 && 32 * p + 8 * dpiece >= n_tail) ? 0x80000000u : 0u);
  // a step past the last one loads through an empty resource
  const rsrc_t dyr_none = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.dy), 0, 0, 0x00020000);
  // (step indices are wave-uniform: read into scalar registers, so that the
  // range tests below are scalar and pick between prepared offsets)
  const int nsteps_s = __builtin_amdgcn_readfirstlane(static_cast<int>(nsteps));
  auto load_dyh = [&](int64_t st64, int part, uint8_t* dst, int i0, int n) {
    const int st = __builtin_amdgcn_readfirstlane(static_cast<int>(st64));
    const int stc = st < nsteps_s ? st : nsteps_s - 1;
    const uint32_t nb = static_cast<uint32_t>(stc * kNS * 2 + 64 * part);
    const rsrc_t rr = st < nsteps_s ? dyr : dyr_none;
    const uint32_t voff = st == nsteps_s - 1 ? dyvoff_tail[part] : dyvoff;
#pragma unroll
    for (int i = i0; i < i0 + n; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rr, (lds_ptr_t)(dst + (i * 4 + wave) * 1024), 16, voff,
          static_cast<int>(static_cast<uint32_t>(i * 64 * N * 2) + nb), 0, 0);
  };

  // Packed codes of a step (64 rows x the tile's 128 bytes) by direct-to-LDS
  // loads, each instruction 8 whole rows (wave w: rows 16 w .. 16 w + 15),
  // 16-byte chunk c of row r at c ^ ((r / 2) % 8).  Rows past N fall outside
  // the resource; columns past K meet masked tables.
  const rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.w.codes), 0,
                                                      static_cast<int>(N * (K >> 1)), 0x00020000);
  uint32_t cvoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int crow = wave * 16 + 8 * i + (lane >> 3);
    cvoff[i] = static_cast<uint32_t>(crow * (K >> 1) + (k0 >> 1) + (((lane & 7) ^ ((crow >> 1) & 7)) << 4));
  }
  auto dma_codes = [&](int64_t st64, int stage, int i0, int n) {
    const int st = __builtin_amdgcn_readfirstlane(static_cast<int>(st64));
    const int64_t stc = st < nsteps_s ? st : nsteps_s - 1;
#pragma unroll
    for (int i = i0; i < i0 + n; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          cr, (lds_ptr_t)(s_c[stage] + (2 * wave + i) * 1024), 16, cvoff[i],
          static_cast<int>(static_cast<uint32_t>(stc * kNS * (K >> 1))), 0, 0);
  };
  // this lane's row segment (row `lane`, the wave's 32 bytes) of a stage
  u32x4 cw[2];
  auto read_codes = [&](int stage) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
      cw[q] = *reinterpret_cast<const u32x4*>(s_c[stage] + lane * 128 + (((2 * wave + q) ^ ((lane >> 1) & 7)) << 4));
  };
  // decode constants of row st*64 + lane, columns [kwc, kwc + 64), by buffer
  // loads with a per-lane offset fixed for the kernel and a scalar step
  // offset (rows past N read zeros; their tables are masked anyway)
  const int64_t nblk = N * (K >> 6);
  rsrc_t pr0, pr1;
  uint32_t plane;
  if constexpr (FMT == kFmtNF4) {
    pr0 = uniform_rsrc(a.w.absmax, static_cast<uint32_t>(a.w.dq ? nblk : 4 * nblk));
    pr1 = uniform_rsrc(a.w.dq ? static_cast<const void*>(a.w.absmax2) : a.w.absmax,
                       static_cast<uint32_t>(a.w.dq ? 4 * ((nblk + 255) >> 8) : 4 * nblk));
    plane = static_cast<uint32_t>(lane * (K >> 6) + (kwc >> 6));
  } else {
    pr0 = uniform_rsrc(a.w.scale, static_cast<uint32_t>(4 * nblk));
    pr1 = uniform_rsrc(a.w.zero, static_cast<uint32_t>(4 * nblk));
    plane = static_cast<uint32_t>((lane * (K >> 5) + (kwc >> 5)) * 2);
  }
  const uint32_t pshift = a.w.dq ? 8u : 0u;
  // (the 8-bit code comes from the aligned word that holds it: a byte load
  // sign-extended at its use gets merged with the extension and sunk to the
  // use, where the wave would wait for every load in flight)
  auto load_params = [&](int64_t st, RowParams<FMT>& rc) {
    if constexpr (FMT == kFmtNF4) {
      const uint32_t o = plane + static_cast<uint32_t>(st * kNS * (K >> 6));
      rc.bp.a = __builtin_amdgcn_raw_buffer_load_b32(pr0, o & ~3u, 0, 0);
      rc.sh = (o & 3u) * 8u;
      rc.bp.b = __builtin_amdgcn_raw_buffer_load_b32(pr1, (o >> pshift) << 2, 0, 0);
    } else {
      const int so = static_cast<int>(st * kNS * (K >> 5) * 2);
      rc.s = __builtin_amdgcn_raw_buffer_load_b32(pr0, plane, so, 0);
      rc.z = __builtin_amdgcn_raw_buffer_load_b32(pr1, plane, so, 0);
    }
  };
  // Tables of a step's row, two sets (by step parity), each built in two
  // parts so that the work spreads over two sub-steps: NF4 entries 0..7 then
  // 8..15 of the block's table, INT4 the tables of the two groups.  An
  // invalid row or column range gets zeros.
  constexpr int NL = FMT == kFmtNF4 ? 1 : 2;
  Lut16 lut[2][NL];
  float lscale[2];
  // Columns past K need no mask: a weight column feeds only its own dX
  // column, and those past K are never stored.  NF4 rows past N read zero
  // constants (their offsets lie past the constant arrays) and so get
  // all-zero tables; INT4 tables of such rows are masked.
  auto build_lut_part = [&](int set, const RowParams<FMT>& rc, int64_t st, int part) {
    const bool valid = FMT == kFmtNF4 || st * kNS + lane < N;
    if constexpr (FMT == kFmtNF4) {
      if (part == 0) lscale[set] = nf4_params_scale_sel(a.w, BlockParams{(rc.bp.a >> rc.sh) & 0xFFu, rc.bp.b}, valid);
      const float sc = lscale[set];
      uint32_t pr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pr[j] = pack_bf16x2(a.w.cb.c[8 * part + 2 * j] * sc, a.w.cb.c[8 * part + 2 * j + 1] * sc);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        lut[set][0].lo[2 * part + q] = perm(pr[2 * q + 1], pr[2 * q], 0x06040200u);
        lut[set][0].hi[2 * part + q] = perm(pr[2 * q + 1], pr[2 * q], 0x07050301u);
      }
    } else {
      const uint32_t sz = valid ? perm(rc.z, rc.s, part == 0 ? 0x05040100u : 0x07060302u) : 0u;
      lut[set][part] = lut_group32<FMT>(a.w.cb, sz);
    }
  };
  // decoded word q (columns 8q .. 8q+7) of this lane's row into a slab stage
  const int wrow = wave * kWReg + lane * 128;
  auto decode_word = [&](int set, int q, int stage) {
    const u32x4 d = lut_decode8(lut[set][NL == 1 ? 0 : (q >> 2)], cw[q >> 2][q & 3]);
    *reinterpret_cast<u32x4*>(s_w[stage] + wrow + (wpos(q, lane) << 4)) = d;
  };

  // MFMA operands of sub-step nn (rows 16 nn .. 16 nn + 15 of the step).
  // A = W^T: column tile i lies in slab 2 wk + i / 2; lane p of each 16-lane
  // group points at row 8 h + p / 4 (+ 4), columns 32 (i % 2) + (l32 & 16)
  // + 4 (p % 4) .. +3 of that slab; the transposing read hands lane t column
  // 32 (i % 2) + (l32 & 16) + t.  B = dY^T: token 128 wm + 32 j + l32,
  // reduction chunk 2 nn + h.  Row terms of nn, the slab and j are immediate
  // offsets (the piece placement repeats every 32 rows, so the A offsets
  // come in two sets, for even and odd nn).  Slabs are written by other
  // waves: the stage barrier after sub-step 2 orders a step's decode (sub-
  // steps 0-2 of the step before) before its first reads (sub-step 3).
  uint32_t aofs[2][2][2];
#pragma unroll
  for (int pn = 0; pn < 2; ++pn)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int r = 8 * h + (l16 >> 2) + 4 * x;
        const int col = 32 * i + (l32 & 16) + 4 * (l16 & 3);
        aofs[pn][i][x] =
            static_cast<uint32_t>(2 * wk * kWReg + r * 128 + (wpos(col >> 3, r + 16 * pn) << 4) + ((col >> 2) & 1) * 8);
      }
  // B operand rows: token 32 j + l32, the lane half's 8 rows n of sub-step
  // 2 q + sub in half-stage q, at piece 2 sub + h
  uint32_t bofs[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
    bofs[sub] = static_cast<uint32_t>((128 * wm + l32) * 64 + (((2 * sub + h) ^ dsw(l32)) << 4));
  auto read_a = [&](int stage, int nn, int i) {
    const uint8_t* wa = s_w[stage] + nn * 16 * 128 + (i >> 1) * kWReg;
    const u32x2 lo = ds_read_tr16(wa + aofs[nn & 1][i & 1][0]);
    const u32x2 hi = ds_read_tr16(wa + aofs[nn & 1][i & 1][1]);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  };
  auto read_b = [&](const uint8_t* dyh, int sub, u32x4 (&bf)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const u32x4*>(dyh + j * 32 * 64 + bofs[sub]);
  };
  // dY half-stages of step parity ri: part 0 in s_dy0 / s_dy2, part 1 in
  // s_dy1 / s_dy3
  auto dyh_of = [&](int ri, int part) -> uint8_t* {
    return ri == 0 ? (part == 0 ? s_dy0 : s_dy1) : (part == 0 ? s_dy2 : s_dy3);
  };

  // Pipeline.  One step st (ri = st & 1: weight stage, dY half-stages, table
  // and constant set of step st + 2) runs the products of st while step
  // st + 1 is decoded from the code registers into the other weight stage
  // (three, three and two words in sub-steps 0, 1, 2) and the tables of step
  // st + 2 are built (sub-steps 2 and 3).  Sub-step nn reads the operands of
  // nn + 1 (in sub-step 3: the first column tile and dY of st + 1, and this
  // lane's codes of st + 2; the second column tile at the top of st + 1).
  // Two barriers per step:
  //   after sub-step 0: dY part 0 of st is read by every wave (free), and
  //     part 1 of st has landed;
  //   after sub-step 2: part 1 of st is read (free), and part 0 of st + 1
  //     and the codes of st + 2 have landed; every wave has read its codes
  //     of st + 1 (that code stage is free).
  // Refills, spread over the step (a burst of direct-to-LDS loads stalls the
  // issuing wave, matrix cores included): sub-step 0: the last half of dY
  // part 1 of st + 1; 1 and 2: dY part 0 of st + 2 and the codes of st + 3;
  // 3: the constants of st + 3 and the first half of dY part 1 of st + 2.
  // Every load has 4-5 sub-steps to land.
  //
  // Prologue: dY of step 0, codes of steps 0 and 1 and the constants of
  // steps 0 and 1 land; step 0 is decoded and the tables of step 1 built;
  // then the loads that the loop expects in flight go out in its order.
  RowParams<FMT> rc[2];
  load_dyh(0, 0, s_dy0, 0, 4);
  load_dyh(0, 1, s_dy1, 0, 4);
  dma_codes(0, 0, 0, 2);
  dma_codes(1, 1, 0, 2);
  load_params(0, rc[0]);
  load_params(1, rc[1]);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  read_codes(0);
  build_lut_part(0, rc[0], 0, 0);
  build_lut_part(0, rc[0], 0, 1);
#pragma unroll
  for (int q = 0; q < 8; ++q) decode_word(0, q, 0);
  build_lut_part(1, rc[1], 1, 0);
  build_lut_part(1, rc[1], 1, 1);
  read_codes(1);
  __syncthreads();  // every wave has read its step-0 codes
  __builtin_amdgcn_sched_barrier(0);
  load_dyh(1, 0, s_dy2, 0, 2);
  dma_codes(2, 0, 0, 1);
  __builtin_amdgcn_sched_barrier(0);
  load_dyh(1, 0, s_dy2, 2, 2);
  dma_codes(2, 0, 1, 1);
  __builtin_amdgcn_sched_barrier(0);
  load_params(2, rc[0]);
  load_dyh(1, 1, s_dy3, 0, 2);
  __builtin_amdgcn_sched_barrier(0);

  u32x4 af[2][4], bf[2][4];
  af[0][0] = read_a(0, 0, 0);
  af[0][1] = read_a(0, 0, 1);
  read_b(s_dy0, 0, bf[0]);
  // The loop body has no branches: a branch splits the scheduling region,
  // and the MFMA / decode / load interleave is lost.
  auto step = [&](int64_t st, auto ri_c) __attribute__((always_inline)) {
    constexpr int ri = decltype(ri_c)::value;
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int cur = nn & 1, nxt = cur ^ 1;
      if (nn == 0) {
        af[cur][2] = read_a(ri, 0, 2);
        af[cur][3] = read_a(ri, 0, 3);
      }
      if (nn < 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) af[nxt][i] = read_a(ri, nn + 1, i);
        read_b(dyh_of(ri, (nn + 1) >> 1), (nn + 1) & 1, bf[nxt]);
      } else {
        af[nxt][0] = read_a(ri ^ 1, 0, 0);
        af[nxt][1] = read_a(ri ^ 1, 0, 1);
        read_b(dyh_of(ri ^ 1, 0), 0, bf[nxt]);
      }
      // words 0-2, 3-5 and 6-7 of the next step's row in sub-steps 0, 1, 2
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q / 3 == nn) decode_word(ri ^ 1, q, ri ^ 1);
      if (nn == 2) build_lut_part(ri, rc[ri], st + 2, 0);
      if (nn == 3) {
        build_lut_part(ri, rc[ri], st + 2, 1);
        read_codes(ri);
      }
      // refills (see above)
      if (nn == 0) load_dyh(st + 1, 1, dyh_of(ri ^ 1, 1), 2, 2);
      if (nn == 1 || nn == 2) {
        load_dyh(st + 2, 0, dyh_of(ri, 0), 2 * (nn - 1), 2);
        dma_codes(st + 3, ri ^ 1, nn - 1, 1);
      }
      if (nn == 3) {
        // the constants first: their use waits for them and every older load
        load_params(st + 3, rc[ri ^ 1]);
        load_dyh(st + 2, 1, dyh_of(ri, 1), 0, 2);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[cur][i], bf[cur][j], acc[i][j]);
      // issue order: the operand reads of the next sub-step first (the LDS,
      // not the matrix cores, is the tighter resource here), then per MFMA
      // 5 VALU of the decode, and a refill load after every fourth, sixth or
      // eighth MFMA
      constexpr int kVmemEvery[4] = {8, 6, 6, 4};
      // (LDS reads: 8 transposing A reads + 4 B reads; sub-step 0 also
      // reads its own last two column tiles, sub-step 3 only two tiles)
      if (nn == 0)
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      else if (nn < 3)
        __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
      else
        __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (g % kVmemEvery[nn] == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (nn == 0 || nn == 2) stage_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int64_t sp = 0; sp < npairs; ++sp) {
    step(2 * sp, std::integral_constant<int, 0>{});
    step(2 * sp + 1, std::integral_constant<int, 1>{});
  }
  // every load has landed and every wave is past its reads before the
  // memory is reused
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // adapter term du A: D[k][m] += sum_j A^T[k][j] du[m][j], in k16 steps,
  // du split into hi + lo bf16 halves.  du of the tile's 256 tokens (as the
  // two halves, in the weight stages) and A^T of its 256 columns (rows
  // 0-127 and 128-255 in two dY half-stages) are staged in LDS 48 adapter
  // columns at a time (rows padded by 16 B against bank conflicts), every
  // load of a chunk in flight at once.  Indices are clamped and values
  // masked (no divergent branches around loads).
  if (a.du != nullptr && a.At != nullptr && a.r > 0) {
    const int rr = a.r;
    constexpr int kJC = 48;          // adapter columns per staged chunk
    constexpr int rp = kJC + 8;      // staged row length (elements): 28 KB per operand
    constexpr int q4 = kJC / 4;      // 4-element pieces of a staged row
    uint16_t* s_dh = reinterpret_cast<uint16_t*>(s_w0);   // [256 m][rp]
    uint16_t* s_dl = reinterpret_cast<uint16_t*>(s_w1);   // [256 m][rp]
    static_assert(128 * rp * 2 <= kDyHalf, "half of A^T fits a dY half-stage");
    // A^T row k of the tile: [128][rp] in s_dy0 (k < 128) or s_dy1
    auto s_at = [&](int k) { return reinterpret_cast<uint16_t*>(k < 128 ? s_dy0 : s_dy1) + (k & 127) * rp; };
    constexpr int kUPer = kTMx * q4 / 256;                 // 12 pieces of each kind per thread
    for (int jc = 0; jc < rr; jc += kJC) {
      f32x4 dv[kUPer];
      u32x2 av[kUPer];
#pragma unroll
      for (int q = 0; q < kUPer; ++q) {
        const int it = q * 256 + tid;
        const int row = it / q4, j = jc + (it - row * q4) * 4;
        int64_t mg = m0 + row, kg = k0 + row;
        mg = mg < M ? mg : M - 1;
        kg = kg < K ? kg : K - 1;
        const float* drow = a.du + mg * rr;
        const uint16_t* arow = a.At + (kg >> a.pool_shift) * rr;  // pooled: one A^T row per group
        if ((rr & 3) == 0) {
          const int jj = j < rr ? j : rr - 4;
          dv[q] = *reinterpret_cast<const f32x4*>(drow + jj);
          av[q] = *reinterpret_cast<const u32x2*>(arow + jj);
        } else {
          uint32_t e4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jj = j + e < rr ? j + e : rr - 1;
            dv[q][e] = drow[jj];
            e4[e] = arow[jj];
          }
          av[q] = u32x2{e4[0] | (e4[1] << 16), e4[2] | (e4[3] << 16)};
        }
      }
      if (jc > 0) __syncthreads();  // the previous chunk's operands are consumed
#pragma unroll
      for (int q = 0; q < kUPer; ++q) {
        const int it = q * 256 + tid;
        const int row = it / q4, jl = (it - row * q4) * 4, j = jc + jl;
        float hv[4], lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(j + e < rr ? dv[q][e] : 0.0f, hv[e], lv[e]);
        *reinterpret_cast<u32x2*>(s_dh + row * rp + jl) = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
        *reinterpret_cast<u32x2*>(s_dl + row * rp + jl) = u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])};
        const uint32_t k0m = (j < rr ? 0x0000FFFFu : 0u) | (j + 1 < rr ? 0xFFFF0000u : 0u);
        const uint32_t k1m = (j + 2 < rr ? 0x0000FFFFu : 0u) | (j + 3 < rr ? 0xFFFF0000u : 0u);
        *reinterpret_cast<u32x2*>(s_at(row) + jl) = u32x2{av[q].x & k0m, av[q].y & k1m};
      }
      __syncthreads();
      const int jt_n = (rr - jc < kJC ? rr - jc + 15 : kJC) / 16;
      for (int jt = 0; jt < jt_n; ++jt) {
        const int j0 = jt * 16 + h * 8;
        u32x4 at[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          at[i] = *reinterpret_cast<const u32x4*>(s_at(128 * wk + i * 32 + l32) + j0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ml = 128 * wm + j * 32 + l32;
          const u32x4 uh = *reinterpret_cast<const u32x4*>(s_dh + ml * rp + j0);
          const u32x4 ul = *reinterpret_cast<const u32x4*>(s_dl + ml * rp + j0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i][j] = mfma32(at[i], uh, acc[i][j]);
            acc[i][j] = mfma32(at[i], ul, acc[i][j]);
          }
        }
      }
    }
  }

  // store: lane holds D[k = 8q + 4h + t][m = l32] of each 32x32 tile, i.e.
  // 8 bytes of 32 different output rows per instruction.  The bf16 tile goes
  // through LDS instead (512 B per token: tokens 0-63 in s_w0, 64-127 in
  // s_w1, then 32 each in the four dY half-stages; 16-byte pieces at column
  // piece XOR the token's low 5 bits) and leaves as whole 16-byte pieces of
  // rows, 32 consecutive threads per row.
  __syncthreads();  // every wave is done with the LDS (adapter operands)
  // staging row of the first token of a 32-token group (a multiple of 32;
  // wave-uniform in the first loop below, known at compile time in the
  // second)
  auto s_out = [&](int row) -> uint8_t* {
    uint8_t* const b = row < 64 ? s_w0 : row < 128 ? s_w1 : row < 160 ? s_dy0 : row < 192 ? s_dy1 : row < 224 ? s_dy2 : s_dy3;
    return b + (row < 128 ? (row & 63) : (row & 31)) * 512;
  };
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row0 = 128 * wm + 32 * j;  // tokens row0 .. row0 + 31, lane l32 holds row0 + l32
    uint8_t* const so = s_out(row0) + l32 * 512;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p16 = 16 * wk + 4 * i + q;  // 16-byte piece of the row (columns 8 p16 ..)
        u32x2 o;
        o.x = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
        o.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        *reinterpret_cast<u32x2*>(so + ((p16 ^ l32) << 4) + h * 8) = o;
      }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const int piece = q * 256 + tid, row = piece >> 5, p16 = piece & 31;
    const int64_t m = m0 + row, k = k0 + p16 * 8;
    // rows 8 q .. 8 q + 7: one staging array per q
    const u32x4 v = *reinterpret_cast<const u32x4*>(s_out(q * 8) + (row - q * 8) * 512 +
                                                    ((p16 ^ (row & 31)) << 4));
    if (m < M && k < K) *reinterpret_cast<u32x4*>(a.dx + m * K + k) = v;
  }
}

}  // namespace

hipError_t launch_dx_gemm(const DxArgs& a, int fmt, hipStream_t stream) {
  const int grid = static_cast<int>(((a.M + kTMx - 1) / kTMx) * ((a.w.K + kTK - 1) / kTK));
  if (fmt == kFmtNF4)
    hipLaunchKernelGGL(k_dx_gemm<kFmtNF4>, dim3(grid), dim3(256), 0, stream, a);
  else if (fmt == kFmtINT4)
    hipLaunchKernelGGL(k_dx_gemm<kFmtINT4>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_dx_gemm<kFmtNFG>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
