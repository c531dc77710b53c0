// Few-token (M <= 16) kernels for large weights, bound by streaming the
// packed weight from HBM.  [QLoRA "The QLoRA recipe" stage 3: each block is
// decoded to bf16 on the fly; "Background: how LoRA works" for the adapter;
// QA-LoRA abstract for INT4 groups]
//
// k_gemv_fwd_stream:  y = x W_bf16^T + s u B^T  (u given)
//   A workgroup owns 128 output features (8 waves x 16) over a share of K
//   and streams it in chunks of 256 columns.  Every lane owns one 64-column
//   block of one row per chunk (32 bytes of codes, one lookup table), which
//   it decodes into the MFMA operand of that block: in k-step t of a chunk,
//   lane group g supplies columns 64 g + 8 t .. + 7, and the token operand
//   is read in the same column order, so each v_mfma_f32_16x16x32_bf16 sums
//   32 of the chunk's columns.  Codes and block constants run four chunks
//   ahead in registers; the token chunk (16 x 256 bf16, shared by the eight
//   waves) is staged in LDS two chunks ahead.  K shares publish fp32 partial
//   sums (write-through stores) and the last workgroup of a row group
//   (atomic ticket) adds them in fixed share order, adds s u B^T and stores
//   y.  Work per workgroup is a long pipelined loop rather than one shot, so
//   a grid of ~256 workgroups (one per compute unit) streams a weight of any
//   size.
//
// k_u_few:  u = alpha X Y^T for M <= 16 rows of X (u = x A^T, du = s dY B)
//   16 x 16 MFMA tiles over (adapter column, token), K split over
//   workgroups with the same ticketed fixed-order fix-up.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kFsWaves = 8;
constexpr int kFsThreads = 64 * kFsWaves;
constexpr int kFsRows = 16 * kFsWaves;   // output features per workgroup
#ifndef QLIN_FS_CHUNK
#define QLIN_FS_CHUNK 256
#endif
#ifndef QLIN_FS_DEPTH
#define QLIN_FS_DEPTH 3
#endif
#ifndef QLIN_FS_WGS_PER_CU
#define QLIN_FS_WGS_PER_CU 2  // resident workgroups per compute unit (8 waves each)
#endif
constexpr int kFsChunk = QLIN_FS_CHUNK;  // columns per step: 256 or 512
constexpr int kFsDepth = QLIN_FS_DEPTH;  // steps of loads in flight beyond the current one
constexpr int kFsR = kFsDepth + 1;       // ring slots = steps per phase of block constants
constexpr int kFsRun = kFsChunk / 4;     // columns of a lane's run per step (g = 0..3)
constexpr int kFsBlk = kFsRun / 64;      // 64-column blocks per run
constexpr int kFsRowBytes = kFsChunk * 2;
constexpr int kFsXPer = kFsChunk / 256;  // 16-byte token pieces per thread and step (32 threads per token row)
static_assert(kFsChunk == 256 || kFsChunk == 512, "step width: 256 or 512 columns");
// Block constants of a phase: kFsPhBlk 64-column blocks of each of the 128
// rows; thread t fills kFsThBlk consecutive blocks of row t / 4.
constexpr int kFsPhBlk = kFsR * kFsChunk / 64;
constexpr int kFsThBlk = kFsPhBlk / 4;
constexpr int kFsTabStride = kFsRows + 16;  // entries per block (+16: lane groups on other banks)
static_assert(kFsThBlk % 4 == 0, "a thread's blocks span whole dwords of 8-bit constants");

// Steps per K share (the shares fill the resident workgroup slots evenly;
// a share's last phase may be partial).
__host__ __device__ inline int fwd_stream_per(int nchk, int S) { return (nchk + S - 1) / S; }

// Per lane and step: the run of codes of its row (columns kFsRun g ..
// kFsRun (g + 1) - 1 of the step, kFsBlk 64-column blocks of 32 bytes) and
// the token pieces this thread stages.
struct FsSlot {
  u32x4 c[2 * kFsBlk];
  u32x4 x[kFsXPer];
};

// One table entry per (row, 64-column block): NF4 the fp32 block scale,
// INT4 / NormalFloat-k groups the two 32-bit group words (scale | zero << 16
// of groups 2b and 2b + 1).  Zero for blocks outside the share or past K,
// which then decode to zeros.
template <int FMT> struct FsEntry { typedef uint32_t type; };
template <> struct FsEntry<kFmtINT4> { typedef uint2 type; };
template <> struct FsEntry<kFmtNFG> { typedef uint2 type; };

// Raw constants of one thread's kFsThBlk blocks, loaded one phase ahead.
template <int FMT, bool DQ>
struct FsRaw {
  uint32_t v[FMT == kFmtNF4 ? (DQ ? kFsThBlk / 4 + 3 : kFsThBlk) : 2 * kFsThBlk];
};

// FMT: weight format.  DQ (NF4): 8-bit block constants with fp32 group
// constants.  AL: rows of group words start on 16-byte boundaries
// (K % 256 == 0), so a thread's words load four at a time.
template <int FMT, bool DQ, bool AL>
__global__ __launch_bounds__(kFsThreads, 2 * QLIN_FS_WGS_PER_CU) void k_gemv_fwd_stream(FwdStreamArgs a) {
  typedef typename FsEntry<FMT>::type Entry;
  __shared__ __attribute__((aligned(16))) uint8_t s_x[2][16 * kFsRowBytes];  // token steps
  __shared__ Entry s_tab[2][kFsPhBlk][kFsTabStride];                         // block constants
  __shared__ uint32_t s_ticket;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t N = a.w.N, K = a.w.K, M = a.M;
  const int64_t Kb = K >> 6;  // 64-column blocks per row
  const int n_rg = static_cast<int>((N + kFsRows - 1) / kFsRows);
  const int rg = static_cast<int>(blockIdx.x) % n_rg;
  const int ks = static_cast<int>(blockIdx.x) / n_rg;
  const int S = a.splits;
  const int nchk = static_cast<int>((K + kFsChunk - 1) / kFsChunk);
  const int per = fwd_stream_per(nchk, S);
  const int c0 = ks * per;
  const int c1 = c0 + per < nchk ? c0 + per : nchk;
  const int64_t n0 = static_cast<int64_t>(rg) * kFsRows;
  const int64_t rows_left = N - n0;  // >= 1
  const int row = wave * 16 + l16;   // this lane's row in the group

  // codes of the group's rows: rows past N and columns past the last row
  // read as zeros (buffer range check); a lane's run past K reads the next
  // row's codes, which meet zero tables
  const uint32_t cbytes = static_cast<uint32_t>(
      rows_left * (K >> 1) < 0xFFFFFFFFll ? rows_left * (K >> 1) : 0xFFFFFFFFll);
  const rsrc_t rc = uniform_rsrc(a.w.codes + n0 * (K >> 1), cbytes);
  const uint32_t voff_c = static_cast<uint32_t>(row * (K >> 1)) + static_cast<uint32_t>(g * (kFsRun / 2));

  // token staging: thread t moves kFsXPer consecutive pieces of token row
  // t >> 5 (rows past M repeat the last token, columns past K the last valid
  // piece; both meet discarded outputs or zero weights)
  const int xrow = tid >> 5, xp0 = (tid & 31) * kFsXPer;
  const int64_t xrc = xrow < M ? xrow : M - 1;
  const rsrc_t rx = uniform_rsrc(a.x, static_cast<uint32_t>(M * K * 2));
  // steps past the share reload its last step (no extra HBM traffic)
  const int clast = c1 > c0 ? c1 - 1 : nchk - 1;
  auto clampc = [&](int c) { return c < clast ? c : clast; };
  // Token offsets: a lane part fixed for the kernel and a chunk part in the
  // scalar operand; the last chunk clamps its columns into the row through
  // a lane part of its own.
  const int64_t klast = static_cast<int64_t>(nchk - 1) * kFsChunk;
  uint32_t xoff[kFsXPer], xoff_last[kFsXPer];
#pragma unroll
  for (int i = 0; i < kFsXPer; ++i) {
    const int64_t rel = (xp0 + i) * 8;
    const int64_t rel_last = klast + rel < K ? rel : K - 8 - klast;
    xoff[i] = static_cast<uint32_t>((xrc * K + rel) * 2);
    xoff_last[i] = static_cast<uint32_t>((xrc * K + rel_last) * 2);
  }
  auto load_slot = [&](int c, FsSlot& sl) {
    const int cc = __builtin_amdgcn_readfirstlane(clampc(c));
    const int cso = static_cast<int>(static_cast<uint32_t>(cc) * static_cast<uint32_t>(kFsChunk / 2));
#pragma unroll
    for (int j = 0; j < 2 * kFsBlk; ++j)
      sl.c[j] = __builtin_amdgcn_raw_buffer_load_b128(rc, voff_c + 16 * j, cso, 0);
    const int xso = static_cast<int>(static_cast<uint32_t>(cc) * static_cast<uint32_t>(kFsChunk * 2));
#pragma unroll
    for (int i = 0; i < kFsXPer; ++i)
      sl.x[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, cc == nchk - 1 ? xoff_last[i] : xoff[i], xso, 0);
  };
  auto store_x = [&](int buf, const FsSlot& sl) {
#pragma unroll
    for (int i = 0; i < kFsXPer; ++i)
      *reinterpret_cast<u32x4*>(&s_x[buf][xrow * kFsRowBytes + (((xp0 + i) ^ xrow) << 4)]) = sl.x[i];
  };

  // block constants: thread t fills blocks gb0 .. gb0 + kFsThBlk - 1 (in the
  // row) of the phase for row frow of the group (clamped into the weight);
  // resources start at the group's first row, so offsets stay 32-bit
  const int frow = tid >> 2, fq = tid & 3;
  const int64_t frl = n0 + frow < N ? frow : rows_left - 1;
  auto first_blk = [&](int cb) { return static_cast<int64_t>(cb) * (kFsChunk / 64) + fq * kFsThBlk; };
  auto cap32 = [](int64_t v) { return static_cast<uint32_t>(v < 0xFFFFFFFFll ? v : 0xFFFFFFFFll); };
  auto load_raw = [&](int cb, FsRaw<FMT, DQ>& r) {
    const int64_t gb0 = first_blk(cb);
    const int64_t gbc = gb0 < Kb ? gb0 : 0;  // past the row: any in-row block (masked)
    if constexpr (FMT == kFmtNF4 && DQ) {
      // the aligned dwords holding the 8-bit constants (zeros past the
      // array), then the group constants of the first and the last block
      const rsrc_t ra = uniform_rsrc(static_cast<const int8_t*>(a.w.absmax) + n0 * Kb, cap32(rows_left * Kb));
      const uint32_t a0 = static_cast<uint32_t>(frl * Kb + gbc) & ~3u;
#pragma unroll
      for (int i = 0; i <= kFsThBlk / 4; ++i)
        r.v[i] = __builtin_amdgcn_raw_buffer_load_b32(ra, a0 + 4 * i, 0, 0);
      const int64_t bf = (n0 + frl) * Kb + gbc;
      const int64_t bl = (n0 + frl) * Kb + (gbc + kFsThBlk - 1 < Kb ? gbc + kFsThBlk - 1 : Kb - 1);
      r.v[kFsThBlk / 4 + 1] = __float_as_uint(a.w.absmax2[bf >> 8]);
      r.v[kFsThBlk / 4 + 2] = __float_as_uint(a.w.absmax2[bl >> 8]);
    } else if constexpr (FMT == kFmtNF4) {
      const float* am = static_cast<const float*>(a.w.absmax) + (n0 + frl) * Kb;
#pragma unroll
      for (int i = 0; i < kFsThBlk; ++i) r.v[i] = __float_as_uint(am[gbc + i < Kb ? gbc + i : Kb - 1]);
    } else {
      // 32-bit words holding the fp16 scales (zeros) of groups 2 i, 2 i + 1
      // of the thread's blocks; past the array they read as zeros
      const int64_t G = K >> 5;
      const rsrc_t rs = uniform_rsrc(a.w.scale + n0 * G, cap32(rows_left * G * 2));
      const rsrc_t rz = uniform_rsrc(a.w.zero + n0 * G, cap32(rows_left * G * 2));
      const uint32_t off = static_cast<uint32_t>((frl * G + 2 * gbc) * 2);
      if constexpr (AL) {
#pragma unroll
        for (int i = 0; i < kFsThBlk / 4; ++i) {
          const u32x4 sv = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, 0, 0);
          const u32x4 zv = __builtin_amdgcn_raw_buffer_load_b128(rz, off + 16 * i, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r.v[4 * i + e] = sv[e];
            r.v[kFsThBlk + 4 * i + e] = zv[e];
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kFsThBlk; ++i) {
          r.v[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * i, 0, 0);
          r.v[kFsThBlk + i] = __builtin_amdgcn_raw_buffer_load_b32(rz, off + 4 * i, 0, 0);
        }
      }
    }
  };
  auto write_tab = [&](int cb, const FsRaw<FMT, DQ>& r, int buf) {
    const int64_t gb0 = first_blk(cb);
    [[maybe_unused]] uint32_t q4[kFsThBlk / 4];
    [[maybe_unused]] int64_t bf = 0;
    if constexpr (FMT == kFmtNF4 && DQ) {
      const int64_t gbc = gb0 < Kb ? gb0 : 0;
      const uint32_t sh = static_cast<uint32_t>(frl * Kb + gbc) & 3u;  // first byte in r.v[0]
#pragma unroll
      for (int k = 0; k < kFsThBlk / 4; ++k) q4[k] = __builtin_amdgcn_alignbyte(r.v[k + 1], r.v[k], sh);
      bf = (n0 + frl) * Kb + gbc;
    }
#pragma unroll
    for (int i = 0; i < kFsThBlk; ++i) {
      // the block's step lies in the share and the block in the row
      const bool ok = cb + (fq * kFsThBlk + i) / (kFsChunk / 64) < c1 && gb0 + i < Kb;
      Entry e;
      if constexpr (FMT == kFmtNF4 && DQ) {
        const int8_t q = static_cast<int8_t>((q4[i >> 2] >> (8 * (i & 3))) & 0xFFu);
        const bool first = ((bf + i) >> 8) == (bf >> 8);
        const float s2 = __uint_as_float(first ? r.v[kFsThBlk / 4 + 1] : r.v[kFsThBlk / 4 + 2]);
        e = ok ? __float_as_uint(nf4_dq_scale(q, s2)) : 0u;
      } else if constexpr (FMT == kFmtNF4) {
        e = ok ? r.v[i] : 0u;
      } else {
        // group words of the block's two groups: low / high halves of scale
        // dword i and zero dword i
        const uint32_t sv = r.v[i], zv = r.v[kFsThBlk + i];
        e.x = ok ? perm(zv, sv, 0x05040100u) : 0u;
        e.y = ok ? perm(zv, sv, 0x07060302u) : 0u;
      }
      s_tab[buf][fq * kFsThBlk + i][frow] = e;
    }
  };

  // Ring of kFsR steps: all loads of a step are issued together, so waiting
  // for the token pieces of step c + 1 (stored at the end of step c) waits
  // only for loads issued kFsDepth steps ago.  The loop body has no branches
  // (a branch join makes the compiler wait for every load in flight): steps
  // past the share decode through zero tables.  The block constants of the
  // next phase load at the start of a phase and enter the other table at its
  // end.
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  FsSlot ring[kFsR];
  {
    FsRaw<FMT, DQ> raw;
    load_raw(c0, raw);
#pragma unroll
    for (int d = 0; d < kFsR; ++d) load_slot(c0 + d, ring[d]);
    write_tab(c0, raw, 0);
  }
  store_x(c0 & 1, ring[0]);
  __syncthreads();

  int tb = 0;
  for (int cb = c0; cb < c1; cb += kFsR, tb ^= 1) {
    FsRaw<FMT, DQ> raw;
    load_raw(cb + kFsR, raw);
#pragma unroll
    for (int d = 0; d < kFsR; ++d) {
      const int c = cb + d;
      const uint8_t* xs = s_x[c & 1];
      // steps past the share (the last phase's tail) skip the arithmetic;
      // the branch is uniform and holds no loads, so waits are unaffected
      if (c < c1) {
#pragma unroll
      for (int j = 0; j < kFsBlk; ++j) {
        const Entry e = s_tab[tb][d * (kFsChunk / 64) + g * kFsBlk + j][row];
        Lut16 lut[2];
        if constexpr (FMT == kFmtNF4) {
          lut[0] = lut_nf4(a.w.cb, __uint_as_float(e));
          lut[1] = lut[0];
        } else {
          lut[0] = lut_group32<FMT>(a.w.cb, e.x);
          lut[1] = lut_group32<FMT>(a.w.cb, e.y);
        }
        // k-step t of block j: columns kFsRun g + 64 j + 8 t .. + 7 of the step
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const u32x4 wf = lut_decode8(lut[t >> 2], ring[d].c[2 * j + (t >> 2)][t & 3]);
          const int q = (kFsRun / 8) * g + 8 * j + t;
          const u32x4 xf = *reinterpret_cast<const u32x4*>(xs + l16 * kFsRowBytes + ((q ^ l16) << 4));
          acc = mfma16(wf, xf, acc);
        }
      }
      }
      // the next step's tokens into the other buffer (last read before the
      // previous barrier), then this slot refills with step c + kFsR
      const int dn = (d + 1) % kFsR;  // (a constant once the loop is unrolled)
      store_x((c + 1) & 1, ring[dn]);
      if (d == kFsR - 1) write_tab(cb + kFsR, raw, tb ^ 1);
      load_slot(c + kFsR, ring[d]);
      __builtin_amdgcn_sched_barrier(0);  // keep the refill here, ahead of later steps' work
      __syncthreads();
    }
  }

  // lane (l16, g) holds y[m = l16][n = n0 + 16 wave + 4 g + v]; lanes of
  // tokens past M hold no output and move no partial sums
  f32x4 sum = acc;
  const bool live = l16 < M;
  if (S > 1) {
    const rsrc_t pr_ = make_rsrc(a.partial);
    const uint32_t mine = static_cast<uint32_t>(((static_cast<int64_t>(ks) * n_rg + rg) * kFsThreads + tid) * 16);
    if (live) st_sys16(pr_, mine, acc);
    if (__builtin_amdgcn_readfirstlane(publish_and_ticket(a.counters + rg, &s_ticket)) !=
        static_cast<uint32_t>(S - 1))
      return;
    if (live) {
    f32x4 part[8];
#pragma unroll
    for (int sp = 0; sp < 8; ++sp) {
      const int spc = sp < S ? sp : S - 1;
      part[sp] = ld_sys16(pr_, static_cast<uint32_t>(((static_cast<int64_t>(spc) * n_rg + rg) * kFsThreads + tid) * 16));
    }
    sum = part[0];
#pragma unroll
    for (int sp = 1; sp < 8; ++sp)
      if (sp < S) sum += part[sp];
    for (int sp0 = 8; sp0 < S; sp0 += 8) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int spc = sp0 + q < S ? sp0 + q : S - 1;
        part[q] = ld_sys16(pr_, static_cast<uint32_t>(((static_cast<int64_t>(spc) * n_rg + rg) * kFsThreads + tid) * 16));
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (sp0 + q < S) sum += part[q];
    }
    }
    if (tid == 0) a.counters[rg] = 0u;
  }

  // adapter term s u B^T as MFMAs over the adapter columns, in the layout of
  // the sums: A operand B[n][j .. j+7] (lane row n = n0 + 16 wave + l16), token
  // operand s u[m][j .. j+7] split into bf16 hi + lo halves (fp32 accuracy)
  const int r = a.r;
  if (a.adapter) {
    const int64_t nb = n0 + wave * 16 + l16;
    const uint16_t* brow = a.B + (nb < N ? nb : N - 1) * r;
    const float* urow = a.u + static_cast<int64_t>(l16 < M ? l16 : M - 1) * r;
    for (int j0 = 0; j0 < r; j0 += 32) {
      uint32_t bw[4], hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 8 * g + 2 * e;
        const uint32_t b0 = j < r ? brow[j] : 0u, b1 = j + 1 < r ? brow[j + 1] : 0u;
        bw[e] = b0 | (b1 << 16);
        float h0, l0, h1, l1;
        split_bf16(j < r ? a.s * urow[j] : 0.0f, h0, l0);
        split_bf16(j + 1 < r ? a.s * urow[j + 1] : 0.0f, h1, l1);
        hw[e] = pack_bf16x2(h0, h1);
        lw[e] = pack_bf16x2(l0, l1);
      }
      const u32x4 bop = {bw[0], bw[1], bw[2], bw[3]};
      sum = mfma16(bop, u32x4{hw[0], hw[1], hw[2], hw[3]}, sum);
      sum = mfma16(bop, u32x4{lw[0], lw[1], lw[2], lw[3]}, sum);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t nn = n0 + wave * 16 + 4 * g + v;
    if (l16 < M && nn < N) a.y[l16 * N + nn] = f32_to_bf16(sum[v]);
  }
}

constexpr int kUfThreads = 256;

__global__ __launch_bounds__(kUfThreads) void k_u_few(UFewArgs a) {
  __shared__ f32x4 s_red[4][64];
  __shared__ uint32_t s_ticket;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int jtiles = (a.J + 15) / 16;
  const int jt = static_cast<int>(blockIdx.x) % jtiles;
  const int sp = static_cast<int>(blockIdx.x) / jtiles;
  const int S = a.splits;
  const int64_t nst = a.K / 32;  // K % 32 == 0
  const int64_t per = (nst + S - 1) / S;
  const int64_t st0 = sp * per;
  const int64_t st1 = st0 + per < nst ? st0 + per : nst;
  const int j = jt * 16 + l16;
  const uint16_t* yrow = a.Y + static_cast<int64_t>(j < a.J ? j : a.J - 1) * a.ldy;
  const uint16_t* xrow = a.X + static_cast<int64_t>(l16 < a.M ? l16 : a.M - 1) * a.ldx;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // wave w takes steps st0 + w, st0 + w + 4, ...; eight steps in flight
  for (int64_t s0 = st0 + wave; s0 < st1; s0 += 32) {
    u32x4 ya[8], xb[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t st = s0 + 4 * q;
      const int64_t k = (st < st1 ? st : s0) * 32 + 8 * g;
      ya[q] = *reinterpret_cast<const u32x4*>(yrow + k);
      xb[q] = *reinterpret_cast<const u32x4*>(xrow + k);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (s0 + 4 * q < st1) acc = mfma16(ya[q], xb[q], acc);
  }
  // lane (l16, g) holds u[m = l16][j = 16 jt + 4 g + v]; the four waves in order
  s_red[wave][lane] = acc;
  __syncthreads();
  f32x4 sum = s_red[0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) sum += s_red[w][lane];
  if (S > 1) {
    const rsrc_t pr = make_rsrc(a.partial);
    if (wave == 0) st_sys16(pr, static_cast<uint32_t>(((sp * jtiles + jt) * 64 + lane) * 16), sum);
    if (__builtin_amdgcn_readfirstlane(publish_and_ticket(a.counters + jt, &s_ticket)) !=
        static_cast<uint32_t>(S - 1))
      return;
    // wave w adds the shares q = w, w + 4, ... in order; then the four
    // waves' sums in wave order
    f32x4 ws = {0.f, 0.f, 0.f, 0.f};
    for (int q0 = wave; q0 < S; q0 += 32) {
      f32x4 part[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int qs = q0 + 4 * q;
        const int qc = qs < S ? qs : wave;
        part[q] = ld_sys16(pr, static_cast<uint32_t>(((qc * jtiles + jt) * 64 + lane) * 16));
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q0 + 4 * q < S) ws += part[q];
    }
    __syncthreads();
    s_red[wave][lane] = ws;
    __syncthreads();
    sum = s_red[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) sum += s_red[w][lane];
    if (tid == 0) a.counters[jt] = 0u;
  }
  if (wave != 0) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int jj = jt * 16 + 4 * g + v;
    if (l16 < a.M && jj < a.J) a.C[l16 * a.ldc + jj] = a.alpha * sum[v];
  }
}

}  // namespace

int fwd_stream_row_groups(int64_t N) { return static_cast<int>((N + kFsRows - 1) / kFsRows); }
int fwd_stream_splits(int64_t N, int64_t K) {
  const int64_t nchk = (K + kFsChunk - 1) / kFsChunk;
  const int64_t rg = fwd_stream_row_groups(N);
  // no more workgroups than the compute units hold at once, so that every
  // share runs in the first (and only) round
  int64_t s = 256 * QLIN_FS_WGS_PER_CU / rg;
  if (s > nchk) s = nchk;
  return static_cast<int>(s < 1 ? 1 : s);
}
int64_t fwd_stream_partial_floats(int64_t N, int64_t K) {
  const int S = fwd_stream_splits(N, K);
  return S > 1 ? static_cast<int64_t>(S) * fwd_stream_row_groups(N) * kFsThreads * 4 : 0;
}

hipError_t launch_gemv_fwd_stream(const FwdStreamArgs& a, int fmt, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(fwd_stream_row_groups(a.w.N) * a.splits)), block(kFsThreads);
  const bool al = a.w.K % 256 == 0;
  if (fmt == kFmtNF4) {
    if (a.w.dq)
      hipLaunchKernelGGL((k_gemv_fwd_stream<kFmtNF4, true, false>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_fwd_stream<kFmtNF4, false, false>), grid, block, 0, stream, a);
  } else if (fmt == kFmtINT4) {
    if (al)
      hipLaunchKernelGGL((k_gemv_fwd_stream<kFmtINT4, false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_fwd_stream<kFmtINT4, false, false>), grid, block, 0, stream, a);
  } else {
    if (al)
      hipLaunchKernelGGL((k_gemv_fwd_stream<kFmtNFG, false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_fwd_stream<kFmtNFG, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

int u_few_tiles(int J) { return (J + 15) / 16; }
int u_few_splits(int J, int64_t K) {
  (void)J;
  // each wave's k-steps (one in four of a share's) in one round of eight
  // loads, and the fix-up's shares (eight per wave) in one round as well
  const int64_t nst = K / 32;
  int64_t s = (nst + 31) / 32;
  if (s > 32) s = 32;
  return static_cast<int>(s < 1 ? 1 : s);
}
int64_t u_few_partial_floats(int J, int64_t K) {
  const int S = u_few_splits(J, K);
  return S > 1 ? static_cast<int64_t>(S) * u_few_tiles(J) * 256 : 0;
}

hipError_t launch_u_few(const UFewArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_u_few, dim3(static_cast<uint32_t>(u_few_tiles(a.J) * a.splits)),
                     dim3(kUfThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
