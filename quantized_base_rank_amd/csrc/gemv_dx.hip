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
constexpr int kGdCodeChunk = kGdRowsChunk * 64;  // packed codes of a chunk in LDS: 8 KB
constexpr int kGdWStride = 64 * 2 + 16;          // wave tile row: 64 bf16 + 16 B pad (144 B)
constexpr int kGdWTile = 64 * kGdWStride;        // one wave tile: 64 rows, 9 KB
constexpr int kGdPre = 8;                        // split partials prefetched per thread


// Raw decode constants of a 32-column piece of one row: NF4 -> its 64-block,
// INT4 -> its group (a = scale | zero << 16).
// Tables of one 64-column block; a masked block (ok false) gets all-zero
// constants, so that it decodes to zeros (NF4: a zero scale; INT4: zero
// scale and offset).
template <int FMT>
__device__ __forceinline__ void block_luts(const WeightView& w, BlockParams p, bool ok,
                                           Lut16 (&lut)[2]) {
  p.a = ok ? p.a : 0u;
  p.b = ok ? p.b : 0u;
  luts_from_params<FMT>(w, p, lut);
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
  // LDS: wave tiles 4 x 2 x 9 KB | dY slice 16 KB | B slice 16 KB | wave
  // partials 4 KB | u 8 KB, and the packed codes 4 x 8 KB.  The fix-up
  // reuses the first 48 KB.
  constexpr int kOffW = 0;
  constexpr int kOffDy = kOffW + 4 * 2 * kGdWTile;
  constexpr int kOffB = kOffDy + 16 * kGdRowsSplit * 2;
  constexpr int kOffF = kOffB + kGdRowsSplit * 16 * 2;
  constexpr int kOffU = kOffF + 4096;
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kOffU + 16 * 128 * 4];
  __shared__ __attribute__((aligned(16))) uint8_t s_code[kGdChunks * kGdCodeChunk];
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
  // (4) packed codes of all chunks, issued after the adapter operands so
  //     that those complete first.  For chunk c and row half q, lane L of
  //     wave w loads a 16-byte piece of row q*64 + 16w + L/4 of the chunk:
  //     four lanes cover a row's 64 bytes, so every load instruction reads
  //     whole row segments.  They go to LDS (s_code[c][row][64 B]) just
  //     before the weight product, which reads them in another pattern.
  const int hcol = wave & 1;   // this wave's 64 columns of the tile
  const int vrow = wave >> 1;  // and 64 rows of each chunk
  u32x4 cw[kGdChunks][2];
#pragma unroll
  for (int c = 0; c < kGdChunks; ++c)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int rl = q * 64 + 16 * wave + (lane >> 2);
      const int64_t nl = c * kGdRowsChunk + rl;
      const int64_t nrow = nb0 + (nl < nlen ? nl : nlen - 1);
      int64_t bc = (kc0 >> 1) + (lane & 3) * 16;
      bc = bc + 16 <= (K >> 1) ? bc : (K >> 1) - 16;
      cw[c][q] = *reinterpret_cast<const u32x4*>(a.w.codes + nrow * (K >> 1) + bc);
    }
  // decode constants of this lane's row of each chunk, in its 64-column block
  const bool blk_ok = kc0 + 64 * hcol < K;
  const int64_t blk = (kc0 >> 6) + (blk_ok ? hcol : 0);
  BlockParams bp[kGdChunks];
#pragma unroll
  for (int c = 0; c < kGdChunks; ++c) {
    const int64_t nl = c * kGdRowsChunk + vrow * 64 + lane;
    bp[c] = load_block_params<FMT>(a.w, nb0 + (nl < nlen ? nl : nlen - 1), blk, true);
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

  // (9) weight product dX_p[m][k] = sum_{n in split} dY[m][n] W[n][k].
  //     Wave (hcol, vrow) owns columns 64 hcol .. +63 of the tile and rows
  //     64 vrow .. +63 of each chunk: every lane decodes one row of 64 into the
  //     wave's own LDS tile, and the transposed LDS read turns 8 consecutive
  //     rows of one column into an MFMA operand.  No other wave reads the
  //     tile, so the chunk loop has no barrier; it is software pipelined
  //     (the operands of chunk c are read before chunk c + 1 is decoded into
  //     the other tile) and kept rolled, with the next chunk's constants
  //     moving down one slot per iteration so that register indices stay
  //     fixed.
  f32x4 acc[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nchunks = static_cast<int>((nlen + kGdRowsChunk - 1) / kGdRowsChunk);
  uint8_t* wtile = s_lds + kOffW + wave * 2 * kGdWTile;
  const int rloc = vrow * 64 + lane;  // this lane's row within a chunk
  const int csw = (rloc >> 1) & 3;    // rotation of its code pieces
  auto read_codes = [&](int c, u32x4& c0, u32x4& c1) {
    const uint8_t* crow = s_code + c * kGdCodeChunk + rloc * 64;
    c0 = *reinterpret_cast<const u32x4*>(crow + (((2 * hcol) ^ csw) << 4));
    c1 = *reinterpret_cast<const u32x4*>(crow + (((2 * hcol + 1) ^ csw) << 4));
  };
  auto decode = [&](int c, BlockParams p, const u32x4& c0, const u32x4& c1, uint8_t* dst_tile) {
    const bool ok = do_dx && c * kGdRowsChunk + rloc < nlen && blk_ok;
    Lut16 lut[2];
    block_luts<FMT>(a.w, p, ok, lut);
    u32x4 d[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      d[e] = lut_decode8(lut[0], c0[e]);
      d[4 + e] = lut_decode8(lut[1], c1[e]);
    }
    uint8_t* dst = dst_tile + lane * kGdWStride;
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4*>(dst + e * 16) = d[e];
  };
  if (do_dx) {
    // stage the codes; the 16-byte pieces of a row are stored rotated by
    // bits 1..2 of the row, so that the decode's reads (one piece of each of
    // 64 consecutive rows) spread over all banks
#pragma unroll
    for (int c = 0; c < kGdChunks; ++c)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int rl = q * 64 + 16 * wave + (lane >> 2);
        const int slot = (lane & 3) ^ ((rl >> 1) & 3);
        *reinterpret_cast<u32x4*>(s_code + c * kGdCodeChunk + rl * 64 + slot * 16) = cw[c][q];
      }
    __syncthreads();
    {
      u32x4 c0, c1;
      read_codes(0, c0, c1);
      decode(0, bp[0], c0, c1, wtile);
    }
#pragma unroll 1
    for (int c = 0; c < nchunks; ++c) {
      const uint8_t* wt = wtile + (c & 1) * kGdWTile;
      // the next chunk's codes first (LDS returns in order), then the
      // operands of chunk c: dY (B operand) and the transposed weights
      u32x4 nc0, nc1;
      read_codes(c + 1 < nchunks ? c + 1 : c, nc0, nc1);
      u32x4 bfr[2], af[2][4];
#pragma unroll
      for (int ns = 0; ns < 2; ++ns) {
        bfr[ns] = *reinterpret_cast<const u32x4*>(
            &s_dy[l16 * kGdRowsSplit + c * kGdRowsChunk + vrow * 64 + ns * 32 + g * 8]);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) af[ns][kt] = tr16_operand(wt, kGdWStride, ns * 32 + g * 8, kt * 16, l16);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (c + 1 < nchunks) decode(c + 1, bp[1], nc0, nc1, wtile + ((c + 1) & 1) * kGdWTile);
#pragma unroll
      for (int ns = 0; ns < 2; ++ns)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc[kt] = mfma16(af[ns][kt], bfr[ns], acc[kt]);
#pragma unroll
      for (int j = 1; j + 1 < kGdChunks; ++j) bp[j] = bp[j + 1];
    }
    // add the two row halves (waves 2, 3 hand theirs to waves 0, 1 through
    // the B slice, unused since du) and publish.  D[16 k][16 m]: lane
    // holds D[4g + v][l16].
    float* s_comb = reinterpret_cast<float*>(s_b);  // [2][64][4][4]
    if (vrow == 1)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        *reinterpret_cast<f32x4*>(s_comb + ((hcol * 64 + lane) * 4 + kt) * 4) = acc[kt];
    __syncthreads();
    if (vrow == 0) {
      const rsrc_t pr = make_rsrc(a.partial);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(s_comb + ((hcol * 64 + lane) * 4 + kt) * 4);
        const f32x4 v = acc[kt] + o;
        const int64_t k = kc0 + hcol * 64 + kt * 16 + 4 * g;
        if (k < K)
          st_sys16(pr, static_cast<uint32_t>(((static_cast<int64_t>(split) * 16 + l16) * K + k) * 4), v);
      }
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
