// Few-token (M <= 16) backward, bound by streaming the packed 4-bit weight
// from HBM rather than by MFMA.
// [QLoRA "The QLoRA recipe": gradients flow through the dequantized weights
//  into the adapter only; QA-LoRA abstract for INT4 groups and the pooled
//  adapter.]
//
//   dX = dY W_bf16 + expand(du A),  du = s dY B,  dA = du^T P,  dB = s dY^T u
//
// The reduction runs over N, across rows of the packed weight, so it is
// split; a workgroup owns 128 columns of dX and 512 rows.  Rows are decoded
// 128 at a time into LDS in natural [n][k] layout and the transposed LDS
// read turns 8 consecutive rows of one column into an MFMA operand.  Every
// workgroup also forms du over its rows and dB for a share of them.
//
// Split reductions publish fp32 partial sums with write-through stores; the
// last workgroup of a column tile (atomic ticket) adds them in fixed split
// order.  Results are bit-identical from run to run and no workgroup waits
// for another.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

// ======================================================================
// backward
// ======================================================================
constexpr int kGdCols = 128;
constexpr int kGdRowsChunk = 128;
constexpr int kGdRowsSplit = 512;
constexpr int kGdChunks = kGdRowsSplit / kGdRowsChunk;
constexpr int kGdWStride = kGdCols * 2 + 32;  // 288 B: rows land 8 banks apart
constexpr int kGdPre = 8;                     // split partials prefetched per thread

// Raw decode constants of a 32-column piece of one row: NF4 -> its 64-block,
// INT4 -> its group (a = scale | zero << 16).
template <int FMT>
__device__ __forceinline__ BlockParams load_piece_params(const WeightView& w, int64_t row,
                                                         int64_t col32) {
  if (FMT == kFmtNF4) return load_block_params<kFmtNF4>(w, row, col32 >> 1, true);
  const int64_t gi = row * (w.K >> 5) + col32;
  BlockParams p;
  p.a = static_cast<uint32_t>(w.scale[gi]) | (static_cast<uint32_t>(w.zero[gi]) << 16);
  p.b = 0u;
  return p;
}
// Table of a piece; a masked piece (ok false) gets all-zero constants, so
// that it decodes to zeros (NF4: a zero scale; INT4: zero scale and offset).
template <int FMT>
__device__ __forceinline__ Lut16 piece_lut(const WeightView& w, BlockParams p, bool ok) {
  p.a = ok ? p.a : 0u;
  p.b = ok ? p.b : 0u;
  if (FMT == kFmtNF4) return lut_nf4(w.cb, nf4_params_scale(w, p));
  return lut_int4(half_bits_to_f32(static_cast<uint16_t>(p.a & 0xFFFFu)),
                  half_bits_to_f32(static_cast<uint16_t>(p.a >> 16)));
}

// Bijection of workgroup ids: XCD x = id % 8 receives the x-th contiguous
// run of linear indices.
__device__ __forceinline__ int gd_xcd_order(int bid, int n) {
  const int q = n >> 3, rem = n & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_dx(GemvDxArgs a) {
  // LDS: two decoded-weight buffers 2 x 36 KB | dY slice 16 KB | B slice 16 KB |
  // wave partials 4 KB | u 8 KB.  The fix-up reuses the first 48 KB.
  constexpr int kWBuf = kGdRowsChunk * kGdWStride;        // 36864
  constexpr int kOffDy = 2 * kWBuf;
  constexpr int kOffB = kOffDy + 16 * kGdRowsSplit * 2;
  constexpr int kOffF = kOffB + kGdRowsSplit * 16 * 2;
  constexpr int kOffU = kOffF + 4096;
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kOffU + 16 * 128 * 4];
  __shared__ uint32_t s_ticket;
  uint16_t* s_dy = reinterpret_cast<uint16_t*>(s_lds + kOffDy);   // [16][512]
  uint8_t* s_b = s_lds + kOffB;                                   // [512][16] bf16, 32 B rows
  float* s_f = reinterpret_cast<float*>(s_lds + kOffF);           // [4][16][16]
  float* s_u = reinterpret_cast<float*>(s_lds + kOffU);           // [16][r]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t N = a.w.N, K = a.w.K, M = a.M;
  const int r = a.r;
  const int tiles = static_cast<int>((K + kGdCols - 1) / kGdCols);
  // Workgroups are dealt to the 8 XCDs round-robin.  Give each XCD a
  // contiguous run of (split, tile) pairs so that neighbouring column tiles,
  // which read the two halves of the same 128-byte lines of packed codes,
  // run on one XCD and the second read hits its L2.
  const int lin = gd_xcd_order(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int tile = lin % tiles;
  const int split = lin / tiles;
  const int64_t kc0 = static_cast<int64_t>(tile) * kGdCols;
  const int64_t nb0 = static_cast<int64_t>(split) * kGdRowsSplit;
  const int64_t nlen = N - nb0 < kGdRowsSplit ? N - nb0 : kGdRowsSplit;
  const bool do_dx = a.dx != nullptr;
  const int jsub = (r + 15) >> 4;
  // this workgroup's share of the split's dB rows
  const int db_rows = (kGdRowsSplit + tiles - 1) / tiles;
  const int db0 = tile * db_rows;

  // Every load below is unconditional, from a clamped address; masks are
  // applied when the values are staged.  (A select on a loaded value next to
  // its load makes the wave wait for that load and all earlier ones.)
  // (1) dY slice: 16 x 512 bf16 = 1024 pieces of 16 B
  u32x4 dyr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = i * 256 + tid;
    const int m = ch >> 6, q = ch & 63;
    const int64_t mc = m < M ? m : M - 1;
    const int qc = q * 8 < nlen ? q : 0;
    dyr[i] = *reinterpret_cast<const u32x4*>(a.dy + mc * N + nb0 + qc * 8);
  }
  // (2) B slice, adapter columns js*16 .. js*16+15: 512 rows x 32 B
  auto load_b = [&](int js, u32x4 (&br)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = i * 256 + tid;
      const int nn = ch >> 1, jh = ch & 1;
      const int j0 = js * 16 + jh * 8;
      const int64_t nnc = nn < nlen ? nn : nlen - 1;
      const uint16_t* br16 = a.B + (nb0 + nnc) * r;
      if ((r & 7) == 0) {
        const int j0c = j0 + 8 <= r ? j0 : r - 8;
        br[i] = *reinterpret_cast<const u32x4*>(br16 + j0c);
      } else {
        uint32_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = br16[j0 + e < r ? j0 + e : r - 1];
        br[i] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                      v[6] | (v[7] << 16)};
      }
    }
  };
  auto store_b = [&](int js, const u32x4 (&bv)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = i * 256 + tid;
      const int nn = ch >> 1, jh = ch & 1;
      const int j0 = js * 16 + jh * 8;
      u32x4 v = bv[i];
      if (nn >= nlen) v = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t keep = (j0 + e < r ? 0x0000FFFFu : 0u) | (j0 + e + 1 < r ? 0xFFFF0000u : 0u);
        v[e >> 1] &= keep;
      }
      *reinterpret_cast<u32x4*>(s_b + (ch >> 1) * 32 + (ch & 1) * 16) = v;
    }
  };
  u32x4 br[4];
  load_b(0, br);
  // (3) u for dB
  float ur[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = i * 256 + tid;
    const int64_t last = M * r - 1;
    ur[i] = a.u[idx < last ? idx : last];
  }
  // (4) weight codes and constants of all chunks, issued after the adapter
  //     operands so that those complete first.  Thread (prow, pp) owns a 32-column piece of
  //     rows c*128 + q*64 + prow; four threads cover a row's 64 B, so each
  //     load instruction reads 16 row segments of 64 B.
  const int prow = tid >> 2, pp = tid & 3;
  const int64_t pcol = kc0 + pp * 32;
  const bool pcol_ok = pcol < K;
  const int64_t pcolc = pcol_ok ? pcol : kc0;
  u32x4 cw[kGdChunks][2];
  BlockParams bp[kGdChunks][2];
#pragma unroll
  for (int c = 0; c < kGdChunks; ++c)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t nl = c * kGdRowsChunk + q * 64 + prow;
      const int64_t nrow = nb0 + (nl < nlen ? nl : nlen - 1);
      cw[c][q] = *reinterpret_cast<const u32x4*>(a.w.codes + nrow * (K >> 1) + (pcolc >> 1));
      bp[c][q] = load_piece_params<FMT>(a.w, nrow, pcolc >> 5);
    }

  // (5) the x tile and (narrow adapters) the A tile of this column tile, for
  //     the fix-up that the tile's last workgroup runs; issued now so that
  //     their latency is hidden (8 KB per workgroup, shared through L2 by
  //     the tile's splits)
  const int fm = tid >> 4;
  const int fcl = (tid & 15) * 8;
  const int64_t fkx = kc0 + fcl < K ? kc0 + fcl : K - 8;
  const bool narrow = r <= 16 && a.pool == 1;  // one load of each kind per thread
  const u32x4 xv = *reinterpret_cast<const u32x4*>(a.x + (fm < M ? fm : M - 1) * K + fkx);
  u32x4 av = u32x4{0u, 0u, 0u, 0u};
  if (narrow)
    av = *reinterpret_cast<const u32x4*>(a.A + static_cast<int64_t>(fm < r ? fm : r - 1) * K + fkx);

  // keep the staging below from being scheduled between the loads above
  __builtin_amdgcn_sched_barrier(0);

  // (6) stage dY, the first B slice and u (masked here)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = i * 256 + tid;
    const int m = ch >> 6, q = ch & 63;
    const bool ok = m < M && q * 8 < nlen;
    *reinterpret_cast<u32x4*>(&s_dy[m * kGdRowsSplit + q * 8]) = ok ? dyr[i] : u32x4{0, 0, 0, 0};
  }
  store_b(0, br);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = i * 256 + tid;
    if (idx < 16 * r) s_u[idx] = idx / r < M ? ur[i] : 0.0f;
  }
  __syncthreads();

  // (7) adapter partial du_p[m][j] = sum_{n in split} dY[m][n] B[n][j]
  float* du_part = a.du_part + (static_cast<int64_t>(tile) * a.splits + split) * (16 * r);
  for (int js = 0; js < jsub; ++js) {
    if (js > 0) {
      u32x4 bn[4];
      load_b(js, bn);
      __syncthreads();
      store_b(js, bn);
      __syncthreads();
    }
    f32x4 accd = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int nbase = (wave * 4 + st) * 32;
      const u32x4 da = *reinterpret_cast<const u32x4*>(&s_dy[l16 * kGdRowsSplit + nbase + g * 8]);
      const u32x4 bb = tr16_operand(s_b, 32, nbase + g * 8, 0, l16);
      accd = mfma16(da, bb, accd);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) s_f[(wave * 16 + 4 * g + v) * 16 + l16] = accd[v];
    __syncthreads();
    {
      const int m = tid >> 4, jl = tid & 15;
      const int j = js * 16 + jl;
      if (j < r)
        st_sys(du_part + m * r + j, ((s_f[(0 * 16 + m) * 16 + jl] + s_f[(1 * 16 + m) * 16 + jl]) +
                                     s_f[(2 * 16 + m) * 16 + jl]) + s_f[(3 * 16 + m) * 16 + jl]);
    }
  }

  // (8) dB[n][j] = s sum_m dY[m][n] u[m][j], rows [db0, db0 + db_rows) of the split
  for (int idx = tid; idx < db_rows * r; idx += 256) {
    const int nn = db0 + idx / r, j = idx % r;
    if (nn >= nlen) break;
    // all 32 operands are read before any is used (one LDS round trip)
    float dv[16], uv[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      dv[m] = bf16_to_f32(s_dy[m * kGdRowsSplit + nn]);
      uv[m] = s_u[m * r + j];
    }
    __builtin_amdgcn_sched_barrier(0);
    float t = 0.0f;
#pragma unroll
    for (int m = 0; m < 16; ++m) t += dv[m] * uv[m];
    a.dB[(nb0 + nn) * r + j] = f32_to_bf16(a.s * t);
  }

  // (9) weight product dX_p[m][k] = sum_{n in split} dY[m][n] W[n][k]; chunk
  //     c + 1 is decoded into the other buffer while chunk c feeds the MFMAs
  f32x4 acc[2];
  acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nchunks = static_cast<int>((nlen + kGdRowsChunk - 1) / kGdRowsChunk);
  // Rows 2 apart start 16 banks apart: the store order alternates by row
  // pair (store s writes 16-byte piece s ^ sw) so that the 16 lanes of a
  // store hit distinct banks.  The pieces are swapped in registers with
  // fixed indices, never by a run-time index into a register vector.
  const uint32_t sw = (static_cast<uint32_t>(prow) >> 1) & 1u;
  // All eight lookups are done before the first store: a store reads its
  // data registers only when the LDS takes it, so a lookup that reuses them
  // right after would wait for the store.
  auto decode = [&](const u32x4 (&cwc)[2], const BlockParams (&bpc)[2], int c, uint8_t* wbuf) {
    u32x4 d[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = q * 64 + prow;
      const bool ok = do_dx && c * kGdRowsChunk + row < nlen && pcol_ok;
      const Lut16 lut = piece_lut<FMT>(a.w, bpc[q], ok);
      const u32x4 cv = cwc[q];
      d[q][0] = lut_decode8(lut, sw ? cv.y : cv.x);
      d[q][1] = lut_decode8(lut, sw ? cv.x : cv.y);
      d[q][2] = lut_decode8(lut, sw ? cv.w : cv.z);
      d[q][3] = lut_decode8(lut, sw ? cv.z : cv.w);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint8_t* dst = wbuf + (q * 64 + prow) * kGdWStride + pp * 64;
      uint8_t* de = dst + (sw << 4);         // pieces 0, 2 (sw 0) or 1, 3 (sw 1)
      uint8_t* dd = dst + ((sw ^ 1u) << 4);  // the other two
      *reinterpret_cast<u32x4*>(de) = d[q][0];
      *reinterpret_cast<u32x4*>(dd) = d[q][1];
      *reinterpret_cast<u32x4*>(de + 32) = d[q][2];
      *reinterpret_cast<u32x4*>(dd + 32) = d[q][3];
    }
  };
  if (do_dx) {
    decode(cw[0], bp[0], 0, s_lds);
    __syncthreads();
    // The chunk loop stays rolled.  A workgroup runs it once, so its
    // instructions are fetched cold and code size costs about as much as
    // the arithmetic; the rolled body is fetched once and then hits the
    // instruction cache.  The codes of later chunks move down one slot per
    // iteration so that every register index stays fixed.
#pragma unroll 1
    for (int c = 0; c < nchunks; ++c) {
      const uint8_t* wb = s_lds + (c & 1) * kWBuf;
      if (c + 1 < nchunks) decode(cw[1], bp[1], c + 1, s_lds + ((c + 1) & 1) * kWBuf);
      // D[k][m] += sum_n W[n][k] dY[m][n]; wave w owns columns [32w, 32w+32)
#pragma unroll
      for (int ns = 0; ns < kGdRowsChunk / 32; ++ns) {
        const int nbase = ns * 32 + g * 8;
        const u32x4 bfr =
            *reinterpret_cast<const u32x4*>(&s_dy[l16 * kGdRowsSplit + c * kGdRowsChunk + nbase]);
#pragma unroll
        for (int ksub = 0; ksub < 2; ++ksub) {
          const u32x4 af = tr16_operand(wb, kGdWStride, nbase, wave * 32 + ksub * 16, l16);
          acc[ksub] = mfma16(af, bfr, acc[ksub]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 1; j + 1 < kGdChunks; ++j) {
        cw[j][0] = cw[j + 1][0];
        cw[j][1] = cw[j + 1][1];
        bp[j][0] = bp[j + 1][0];
        bp[j][1] = bp[j + 1][1];
      }
    }
    // D[16 k][16 m]: lane holds D[4g + v][l16]
    const rsrc_t pr = make_rsrc(a.partial);
#pragma unroll
    for (int ksub = 0; ksub < 2; ++ksub) {
      const int64_t k = kc0 + wave * 32 + ksub * 16 + 4 * g;
      if (k < K)
        st_sys16(pr, static_cast<uint32_t>(((static_cast<int64_t>(split) * 16 + l16) * K + k) * 4),
                 acc[ksub]);
    }
  }

  if (publish_and_ticket(a.counters + tile, &s_ticket) != static_cast<uint32_t>(a.splits - 1))
    return;

  // ---- fix-up of this column tile (the last workgroup of the tile)
  const int S = a.splits;
  const int ps = a.pool_shift;
  const int ncol = K - kc0 < kGdCols ? static_cast<int>(K - kc0) : kGdCols;
  const int ngrp = ncol >> ps;
  const int64_t Ka = K >> ps;
  const int acols = a.pool == 1 ? ncol : ngrp;
  const int64_t ac0 = kc0 >> ps;
  float* s_du = reinterpret_cast<float*>(s_lds);                 // [r][16]   8 KB max
  float* s_px = reinterpret_cast<float*>(s_lds + 8192);          // [16][128] 8 KB
  uint16_t* s_a = reinterpret_cast<uint16_t*>(s_lds + 16384);    // [r][128] 32 KB max
  const int m = fm;
  const int cl = fcl;
  const int64_t kx = fkx;

  // issue every load before using any: split partials of dX and du.  Thread
  // t reads du element (m = t % 16, j = t / 16), so that du lands in LDS
  // transposed, [j][m].
  f32x4 pd[kGdPre][2];
  const rsrc_t pr = make_rsrc(a.partial);
#pragma unroll
  for (int sp = 0; sp < kGdPre; ++sp) {
    const int spc = sp < S ? sp : S - 1;
    const uint32_t off = static_cast<uint32_t>(((static_cast<int64_t>(spc) * 16 + m) * K + kx) * 4);
    pd[sp][0] = ld_sys16(pr, off);
    pd[sp][1] = ld_sys16(pr, off + 16);
  }
  const float* dub = a.du_part + static_cast<int64_t>(tile) * S * (16 * r);
  auto du_src = [&](int idx) { return (idx & 15) * r + (idx >> 4 < r ? idx >> 4 : r - 1); };
  float dv[kGdPre];
  {
    const int src = du_src(tid);
#pragma unroll
    for (int sp = 0; sp < kGdPre; ++sp) dv[sp] = ld_sys(dub + (sp < S ? sp : S - 1) * (16 * r) + src);
  }

  // stage du (all splits), x (as fp32) and A
  {
    float v = 0.0f;
#pragma unroll
    for (int sp = 0; sp < kGdPre; ++sp)
      if (sp < S) v += dv[sp];
    for (int sp = kGdPre; sp < S; ++sp) v += ld_sys(dub + sp * (16 * r) + du_src(tid));
    if (tid < 16 * r) s_du[tid] = a.s * v;
    for (int idx = tid + 256; idx < 16 * r; idx += 256) {
      float w = 0.0f;
      for (int sp = 0; sp < S; ++sp) w += ld_sys(dub + sp * (16 * r) + du_src(idx));
      s_du[idx] = a.s * w;
    }
  }
  {
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = m < M && cl + e < ncol;
      s_px[m * kGdCols + cl + e] = ok ? bf16_to_f32(static_cast<uint16_t>(xw[e >> 1] >> (16 * (e & 1)))) : 0.0f;
    }
  }
  if (narrow) {
    if (m < r) *reinterpret_cast<u32x4*>(&s_a[m * kGdCols + cl]) = av;
  } else {
    for (int idx = tid; idx < r * acols; idx += 256) {
      const int j = idx / acols, c = idx % acols;
      s_a[j * kGdCols + c] = a.A[static_cast<int64_t>(j) * Ka + ac0 + c];
    }
  }
  __syncthreads();
  if (a.pool > 1) {
    // group sums of x in place: P[m][gg] into s_px[m][gg]
    float pv = 0.0f;
    const int mm = tid >> 4, gg = tid & 15;
    if (gg < ngrp)
      for (int e = 0; e < a.pool; ++e) pv += s_px[mm * kGdCols + gg * a.pool + e];
    __syncthreads();
    if (gg < ngrp) s_px[mm * kGdCols + gg] = pv;
    __syncthreads();
  }
  // dA[j][c] = sum_m du[m][j] P[m][c]: thread (c = t % 128) holds column c of
  // P and forms rows j = t / 128, + 2, ... of dA
  {
    const int c = tid & (kGdCols - 1);
    if (c < acols) {
      float pc[16];
#pragma unroll
      for (int mm = 0; mm < 16; ++mm) pc[mm] = s_px[mm * kGdCols + c];
#pragma unroll 4
      for (int j = tid >> 7; j < r; j += 2) {
        const f32x4* dj = reinterpret_cast<const f32x4*>(s_du + j * 16);
        float t = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 d = dj[q];
#pragma unroll
          for (int e = 0; e < 4; ++e) t += d[e] * pc[4 * q + e];
        }
        a.dA[static_cast<int64_t>(j) * Ka + ac0 + c] = f32_to_bf16(t);
      }
    }
  }
  if (do_dx && m < M && kc0 + cl < K) {
    float sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = 0.0f;
#pragma unroll
    for (int sp = 0; sp < kGdPre; ++sp)
      if (sp < S)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[e] += pd[sp][0][e];
          sum[4 + e] += pd[sp][1][e];
        }
    for (int sp = kGdPre; sp < S; ++sp) {
      const uint32_t off = static_cast<uint32_t>(((static_cast<int64_t>(sp) * 16 + m) * K + kx) * 4);
      const f32x4 v0 = ld_sys16(pr, off);
      const f32x4 v1 = ld_sys16(pr, off + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sum[e] += v0[e];
        sum[4 + e] += v1[e];
      }
    }
    // adapter term du A (pooled: each group's value repeated over its columns)
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = 0.0f;
    if (a.pool == 1) {
#pragma unroll 4
      for (int j = 0; j < r; ++j) {
        const float d = s_du[j * 16 + m];
        const u32x4 av8 = *reinterpret_cast<const u32x4*>(&s_a[j * kGdCols + cl]);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          t[e] += d * bf16_lo(av8[e >> 1]);
          t[e + 1] += d * bf16_hi(av8[e >> 1]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = (cl + e) >> ps;
        float te = 0.0f;
        for (int j = 0; j < r; ++j) te += s_du[j * 16 + m] * bf16_to_f32(s_a[j * kGdCols + c]);
        t[e] = te;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] += t[e];
    u32x4 o;
    o.x = pack_bf16x2(sum[0], sum[1]);
    o.y = pack_bf16x2(sum[2], sum[3]);
    o.z = pack_bf16x2(sum[4], sum[5]);
    o.w = pack_bf16x2(sum[6], sum[7]);
    *reinterpret_cast<u32x4*>(a.dx + m * K + kc0 + cl) = o;
  }
  if (tid == 0) a.counters[tile] = 0u;
}

}  // namespace

int gemv_dx_splits(int64_t N) { return static_cast<int>((N + kGdRowsSplit - 1) / kGdRowsSplit); }
int gemv_dx_tiles(int64_t K) { return static_cast<int>((K + kGdCols - 1) / kGdCols); }
int64_t gemv_dx_partial_floats(int64_t N, int64_t K) { return gemv_dx_splits(N) * 16 * K; }
int64_t gemv_dx_dupart_floats(int64_t N, int64_t K, int r) {
  return static_cast<int64_t>(gemv_dx_tiles(K)) * gemv_dx_splits(N) * 16 * r;
}

hipError_t launch_gemv_dx(const GemvDxArgs& a, int fmt, hipStream_t stream) {
  const int grid = gemv_dx_tiles(a.w.K) * a.splits;
  if (fmt == kFmtNF4)
    hipLaunchKernelGGL(k_gemv_dx<kFmtNF4>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_gemv_dx<kFmtINT4>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
