// Few-token (M <= 16) backward, bound by streaming the packed 4-bit weight
// from HBM rather than by MFMA.
// [QLoRA "The QLoRA recipe": gradients flow through the dequantized weights
//  into the adapter only; QA-LoRA abstract for INT4 groups and the pooled
//  adapter.]
//
//   dX = dY W_bf16 + expand(du A),  du = s dY B,  dA = du^T P,  dB = s dY^T u
//
// The reduction runs over N, across rows of the packed weight, so it is
// split: a workgroup owns 128 columns of dX and 512 rows of W.  Each of its
// 16 waves owns 32 of the rows: every lane decodes one 64-column block of
// one row into the wave's own LDS tile, and the transposed LDS read turns 8
// consecutive rows of one column into an MFMA operand.  The same dY operand
// also forms the wave's share of du = dY B, with B read transposed straight
// from memory.  No wave reads another's tile, so there is no barrier until
// the 16 waves' partial sums are added through LDS in fixed order.
//
// Split reductions publish fp32 partial sums with write-through stores; the
// last workgroup of a column tile (atomic ticket) adds them in fixed split
// order and forms dA and the adapter term of dX.  Every workgroup forms dB
// for a share of its split's rows after the ticket, which hides the load
// latency of the tile's fix-up.  Results are bit-identical from run to run
// and no workgroup waits for another.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kGdCols = 128;                          // dX columns per workgroup
constexpr int kGdRowsSplit = 512;                     // rows of W per split
constexpr int kGdWaves = 16;
constexpr int kGdThreads = 64 * kGdWaves;
constexpr int kGdWaveRows = kGdRowsSplit / kGdWaves;  // 32 rows per wave
constexpr int kGdStride = kGdCols * 2 + 32;           // decoded row in LDS: 288 B
constexpr int kGdRegion = kGdWaveRows * kGdStride;    // one wave's LDS: 9 KB
constexpr int kGdPre = 8;                             // splits read per round trip

// Bijection of workgroup ids: XCD x = id % 8 receives the x-th contiguous
// run of linear indices, so that neighbouring column tiles, which read the
// two halves of the same 128-byte lines of packed codes, share an L2.
__device__ __forceinline__ int gd_xcd_order(int bid, int n) {
  const int q = n >> 3, rem = n & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// B transposed: lane (j = l16, g) gets B[rows g*8 .. +7][j] as bf16 pairs;
// columns j >= r and masked row groups read in-bounds elements and are
// zeroed by the caller's masks.
__device__ __forceinline__ void load_bt(const uint16_t* B, int r, int64_t nb0, int row0, int nlen,
                                        int j, uint32_t (&v)[8]) {
  const int jc = j < r ? j : r - 1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int rr = row0 + e < nlen ? row0 + e : nlen - 1;
    v[e] = B[(nb0 + rr) * r + jc];
  }
}
__device__ __forceinline__ u32x4 pack_bt(const uint32_t (&v)[8], bool ok) {
  const u32x4 p = {v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
  return ok ? p : u32x4{0u, 0u, 0u, 0u};
}

template <int FMT>
__global__ __launch_bounds__(kGdThreads) void k_gemv_dx(GemvDxArgs a) {
  // one 9 KB region per wave: staged codes, then the decoded tile
  // [32 rows][128 columns], then the wave's partial sums; after the ticket
  // the whole array holds the dB operands and the fix-up's tiles
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kGdWaves * kGdRegion];
  __shared__ uint16_t s_dbdy[16 * 128];  // dB operands: dY[m][128 rows of the share]
  __shared__ float s_dbu[16 * 128];      // and u[m][j]
  __shared__ uint32_t s_ticket;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform)
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t N = a.w.N, K = a.w.K, M = a.M;
  const int r = a.r;
  const int S = a.splits;
  const int tiles = static_cast<int>((K + kGdCols - 1) / kGdCols);
  const int lin = gd_xcd_order(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int tile = lin % tiles;
  const int split = lin / tiles;
  const int64_t kc0 = static_cast<int64_t>(tile) * kGdCols;
  const int64_t nb0 = static_cast<int64_t>(split) * kGdRowsSplit;
  const int nlen = static_cast<int>(N - nb0 < kGdRowsSplit ? N - nb0 : kGdRowsSplit);
  const bool do_dx = a.dx != nullptr;
  const int jsub = (r + 15) >> 4;
  const int wr0 = wave * kGdWaveRows;  // this wave's first row within the split
  uint8_t* region = s_lds + wave * kGdRegion;

  // (0) operands of dB = s dY^T u for this workgroup's share of the split's
  //     rows (a multiple of 16; the first 128 of them): L2 hits, issued
  //     first and used after the ticket, while the tile's last workgroup
  //     waits for the split partials
  const int db_rows = ((kGdRowsSplit + tiles - 1) / tiles + 15) & ~15;
  const int db0 = tile * db_rows;
  const int dbn = nlen - db0 < db_rows ? nlen - db0 : db_rows;  // <= 0: none
  const int dbc = dbn < 128 ? dbn : 128;
  const int dbm = (tid >> 4) & 15, dbq = tid & 15;
  const bool dbok = tid < 256 && dbm < M && dbq * 8 < dbc;
  const u32x4 dbv = *reinterpret_cast<const u32x4*>(
      a.dy + static_cast<int64_t>(dbok ? dbm : 0) * N + nb0 + (dbok ? db0 + dbq * 8 : 0));
  const int64_t mr = M * r;
  const float u0 = a.u[2 * tid < mr ? 2 * tid : mr - 1];
  const float u1 = a.u[2 * tid + 1 < mr ? 2 * tid + 1 : mr - 1];

  // Every load of the main part is unconditional, from a clamped address;
  // masks are applied where the values are used.
  // (1) dY operand: lane (m = l16, g) holds dY[m][rows g*8 .. +7] of the wave
  //     (d_out % 16 == 0, so a group of 8 rows is wholly valid or masked)
  const int ygrp = wr0 + g * 8;
  const bool yok = ygrp < nlen;
  const u32x4 dy_raw = *reinterpret_cast<const u32x4*>(
      a.dy + static_cast<int64_t>(l16 < M ? l16 : M - 1) * N + nb0 + (yok ? ygrp : 0));
  // (2) B transposed for du columns 0..15
  uint32_t bt_raw[8];
  load_bt(a.B, r, nb0, ygrp, nlen, l16, bt_raw);
  // (3) packed codes of the wave's 32 rows (64 B each), read as whole row
  //     segments: load j, lane L -> row 16 j + L/4, 16-byte piece L%4
  u32x4 craw[2];
  {
    int64_t cb = (kc0 >> 1) + (lane & 3) * 16;
    cb = cb + 16 <= (K >> 1) ? cb : (K >> 1) - 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int rl = wr0 + 16 * j + (lane >> 2);
      rl = rl < nlen ? rl : nlen - 1;
      craw[j] = *reinterpret_cast<const u32x4*>(a.w.codes + (nb0 + rl) * (K >> 1) + cb);
    }
  }
  // (4) decode constants: lane (rr, hh) decodes row rr of the wave, columns
  //     64 hh .. +63 of the tile
  const int rr = lane & 31, hh = lane >> 5;
  const bool blk_ok = kc0 + 64 * hh < K;
  const int rrow = wr0 + rr < nlen ? wr0 + rr : nlen - 1;
  const BlockParams bp =
      load_block_params<FMT>(a.w, nb0 + rrow, (kc0 >> 6) + (blk_ok ? hh : 0), true);
  const bool dec_ok = do_dx && wr0 + rr < nlen && blk_ok;
  // keep every load above ahead of the first use (the scheduler would
  // otherwise sink the block constants below the code staging, a second
  // round trip to HBM)
  __builtin_amdgcn_sched_barrier(0);

  // (5) du columns 0..15 over the wave's rows: D[j][m] = sum_n B[n][j] dY[m][n]
  const u32x4 dyf = yok ? dy_raw : u32x4{0u, 0u, 0u, 0u};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const f32x4 accd = mfma16(pack_bt(bt_raw, l16 < r), dyf, zero4);

  // (6) stage the codes (row rl's piece p at slot p ^ ((rl >> 2) & 3)) and
  //     read back this lane's two pieces; all within the wave's region
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rl = 16 * j + (lane >> 2);
    const int slot = (lane & 3) ^ ((rl >> 2) & 3);
    *reinterpret_cast<u32x4*>(region + rl * 64 + slot * 16) = craw[j];
  }
  const int sw = (rr >> 2) & 3;
  const u32x4 c0 = *reinterpret_cast<const u32x4*>(region + rr * 64 + (((2 * hh) ^ sw) << 4));
  const u32x4 c1 = *reinterpret_cast<const u32x4*>(region + rr * 64 + (((2 * hh + 1) ^ sw) << 4));

  // (7) decode into the wave's tile and form D[k][m] = sum_n W[n][k] dY[m][n]
  //     over its 32 rows for the tile's 8 groups of 16 columns; the partial
  //     sums then overwrite the tile (lane order, 16 B per lane and group)
  if (do_dx) {
    Lut16 lut[2];
    BlockParams p = bp;
    p.a = dec_ok ? p.a : 0u;
    p.b = dec_ok ? p.b : 0u;
    luts_from_params<FMT>(a.w, p, lut);
    uint8_t* dst = region + rr * kGdStride + hh * 128;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<u32x4*>(dst + e * 16) = lut_decode8(lut[0], c0[e]);
      *reinterpret_cast<u32x4*>(dst + 64 + e * 16) = lut_decode8(lut[1], c1[e]);
    }
    f32x4 acc[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
      acc[kt] = mfma16(tr16_operand(region, kGdStride, g * 8, kt * 16, l16), dyf, zero4);
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) *reinterpret_cast<f32x4*>(region + (kt * 64 + lane) * 16) = acc[kt];
  }
  *reinterpret_cast<f32x4*>(region + 8192 + lane * 16) = accd;
  __syncthreads();

  // (8) add the 16 waves in fixed order and publish this split's partials.
  //     Each wave's region holds its D[k][m] in lane order: group kt, lane
  //     (m, g) -> D[kt*16 + 4g .. +3][m] (16 B), then du D[4g + v][m].
  //     Threads read in the same order (conflict-free): 0..511 -> one 16 B
  //     group of dX_p, 512..767 -> one element of du_p.
  const rsrc_t pr = make_rsrc(a.partial);
  float* du_part = a.du_part + (static_cast<int64_t>(tile) * S + split) * (16 * r);
  if (tid < 512) {
    f32x4 v = zero4;
#pragma unroll
    for (int w = 0; w < kGdWaves; ++w) v += *reinterpret_cast<const f32x4*>(s_lds + w * kGdRegion + tid * 16);
    const int kt = tid >> 6, ln = tid & 63;
    const int m = ln & 15;
    const int64_t k = kc0 + kt * 16 + 4 * (ln >> 4);
    if (do_dx && k < K)
      st_sys16(pr, static_cast<uint32_t>(((static_cast<int64_t>(split) * 16 + m) * K + k) * 4), v);
  } else if (tid < 768) {
    const int idx = tid - 512;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kGdWaves; ++w) v += *reinterpret_cast<const float*>(s_lds + w * kGdRegion + 8192 + idx * 4);
    const int m = (idx >> 2) & 15, j = 4 * (idx >> 6) + (idx & 3);
    if (j < r) st_sys(du_part + m * r + j, v);
  }
  // wider adapters: du columns 16 js .. +15, one round each
  for (int js = 1; js < jsub; ++js) {
    uint32_t b[8];
    load_bt(a.B, r, nb0, ygrp, nlen, js * 16 + l16, b);
    const f32x4 ad = mfma16(pack_bt(b, js * 16 + l16 < r), dyf, zero4);
    __syncthreads();
    *reinterpret_cast<f32x4*>(region + 8192 + lane * 16) = ad;
    __syncthreads();
    if (tid < 256) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kGdWaves; ++w) v += *reinterpret_cast<const float*>(s_lds + w * kGdRegion + 8192 + tid * 4);
      const int m = (tid >> 2) & 15, j = js * 16 + 4 * (tid >> 6) + (tid & 3);
      if (j < r) st_sys(du_part + m * r + j, v);
    }
  }

  // (10) the fix-up's x and (narrow) A tiles, loaded by every workgroup
  //      before the ticket as well (L2 hits, hidden by its wait); only the
  //      tile's last workgroup uses them
  const int ps = a.pool_shift;
  const int ncol = K - kc0 < kGdCols ? static_cast<int>(K - kc0) : kGdCols;
  const int ngrp = ncol >> ps;
  const int64_t Ka = K >> ps;
  const int acols = a.pool == 1 ? ncol : ngrp;
  const int64_t ac0 = kc0 >> ps;
  const bool narrow = r <= 16 && a.pool == 1;
  const int fm = (tid >> 4) & 15, fcl = (tid & 15) * 8;
  const int64_t fkx = kc0 + fcl < K ? kc0 + fcl : K - 8;
  u32x4 xv = {0u, 0u, 0u, 0u}, av = {0u, 0u, 0u, 0u};
  if (wave < 4) {
    xv = *reinterpret_cast<const u32x4*>(a.x + static_cast<int64_t>(fm < M ? fm : M - 1) * K + fkx);
    // (a wide or pooled A is staged element-wise below; the pointer stays in
    // bounds either way)
    const uint16_t* ap = narrow ? a.A + static_cast<int64_t>(fm < r ? fm : r - 1) * K + fkx : a.x + fkx;
    av = *reinterpret_cast<const u32x4*>(ap);
  }

  // (uniform: every thread reads the same ticket)
  const bool last = __builtin_amdgcn_readfirstlane(publish_and_ticket(a.counters + tile, &s_ticket)) ==
                    static_cast<uint32_t>(S - 1);

  // ---- after the ticket the LDS holds:
  float* s_du = reinterpret_cast<float*>(s_lds);                  // [r][16]    8 KB max
  float* s_px = reinterpret_cast<float*>(s_lds + 8192);           // [16][128]  8 KB
  uint16_t* s_a = reinterpret_cast<uint16_t*>(s_lds + 16384);     // [r][128]  32 KB max
  float* s_dup = reinterpret_cast<float*>(s_lds + 73728);        // [S][16 r]  du partials, 32 KB max

  // thread roles in the last workgroup: threads 0..255 stage the x and A
  // tile pieces (fm, fcl); wave w < 8 owns dX columns 16 w .. +15, lane
  // (m = l16, g) the four elements dX[m][16 w + 4 g .. +3] (the layout of
  // the published partials and of the fp32 MFMA's output); waves 8..15
  // fetch the du partials as 16-byte pieces (all splits, when they fit in
  // LDS) for a fixed-order sum after a barrier, and then form dA
  const int dm = l16, dkq = 16 * (wave & 7) + 4 * g;
  const int64_t dk = kc0 + dkq < K ? kc0 + dkq : K - 4;
  const float* dub = a.du_part + static_cast<int64_t>(tile) * S * (16 * r);
  auto pd_off = [&](int sp) {
    return static_cast<uint32_t>(((static_cast<int64_t>(sp < S ? sp : S - 1) * 16 + dm) * K + dk) * 4);
  };
  const int dup_pieces = S * 4 * r;                   // 16-byte pieces of all du partials
  const bool dup_lds = dup_pieces * 16 <= 32768;      // they fit in s_dup
  constexpr int kDuPer = 4;                           // pieces per fetching thread, unrolled
  const int du_t = tid - 512;
  f32x4 pd[kGdPre];
  f32x4 dq[kDuPer];
  if (last) {
    // every load issued before any is used
    if (wave < 8) {
#pragma unroll
      for (int sp = 0; sp < kGdPre; ++sp) pd[sp] = ld_sys16(pr, pd_off(sp));
    } else {
      const rsrc_t dr = make_rsrc(dub);
#pragma unroll
      for (int q = 0; q < kDuPer; ++q) {
        const int pc = du_t + q * 512 < dup_pieces ? du_t + q * 512 : dup_pieces - 1;
        dq[q] = ld_sys16(dr, static_cast<uint32_t>(pc * 16));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // (11) dB: stage the operands (and the fix-up's tiles), then the first
  //      128 rows of the share, then any further rows (few column tiles only)
  if (tid < 256) *reinterpret_cast<u32x4*>(&s_dbdy[dbm * 128 + dbq * 8]) = dbok ? dbv : u32x4{0u, 0u, 0u, 0u};
  if (2 * tid < 16 * r) {
    s_dbu[2 * tid] = 2 * tid < mr ? u0 : 0.0f;
    if (2 * tid + 1 < 16 * r) s_dbu[2 * tid + 1] = 2 * tid + 1 < mr ? u1 : 0.0f;
  }
  if (last && tid < 256) {
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = fm < M && fcl + e < ncol;
      s_px[fm * kGdCols + fcl + e] = ok ? bf16_to_f32(static_cast<uint16_t>(xw[e >> 1] >> (16 * (e & 1)))) : 0.0f;
    }
    if (narrow && fm < r) *reinterpret_cast<u32x4*>(&s_a[fm * kGdCols + fcl]) = av;
  }
  if (last && !narrow) {
    for (int idx = tid; idx < r * acols; idx += kGdThreads) {
      const int j = idx / acols, c = idx % acols;
      s_a[j * kGdCols + c] = a.A[static_cast<int64_t>(j) * Ka + ac0 + c];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < dbc * r; idx += kGdThreads) {
    const int nn = idx / r, j = idx % r;
    float dyv[16], uv[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      dyv[m] = bf16_to_f32(s_dbdy[m * 128 + nn]);
      uv[m] = s_dbu[m * r + j];
    }
    float t = 0.0f;
#pragma unroll
    for (int m = 0; m < 16; ++m) t += dyv[m] * uv[m];
    a.dB[(nb0 + db0 + nn) * r + j] = f32_to_bf16(a.s * t);
  }
  for (int cb = 128; cb < dbn; cb += 128) {
    const int cn = dbn - cb < 128 ? dbn - cb : 128;
    const bool ok = tid < 256 && dbm < M && dbq * 8 < cn;
    const u32x4 v = *reinterpret_cast<const u32x4*>(
        a.dy + static_cast<int64_t>(ok ? dbm : 0) * N + nb0 + (ok ? db0 + cb + dbq * 8 : 0));
    __syncthreads();
    if (tid < 256) *reinterpret_cast<u32x4*>(&s_dbdy[dbm * 128 + dbq * 8]) = ok ? v : u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    for (int idx = tid; idx < cn * r; idx += kGdThreads) {
      const int nn = idx / r, j = idx % r;
      float t = 0.0f;
      for (int m = 0; m < 16; ++m) t += bf16_to_f32(s_dbdy[m * 128 + nn]) * s_dbu[m * r + j];
      a.dB[(nb0 + db0 + cb + nn) * r + j] = f32_to_bf16(a.s * t);
    }
  }
  if (!last) return;

  // ---- fix-up of this column tile
  // (12) du = s sum over splits (fixed order), stored transposed [j][m]
  if (dup_lds) {
    if (wave >= 8) {
#pragma unroll
      for (int q = 0; q < kDuPer; ++q)
        if (du_t + q * 512 < dup_pieces) *reinterpret_cast<f32x4*>(s_dup + (du_t + q * 512) * 4) = dq[q];
      const rsrc_t dr = make_rsrc(dub);
      for (int pc = du_t + kDuPer * 512; pc < dup_pieces; pc += 512)
        *reinterpret_cast<f32x4*>(s_dup + pc * 4) = ld_sys16(dr, static_cast<uint32_t>(pc * 16));
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * r; idx += kGdThreads) {
      const int f = (idx & 15) * r + (idx >> 4);  // element (m, j) of a [m][r] partial
      float v = 0.0f;
#pragma unroll 8
      for (int sp = 0; sp < S; ++sp) v += s_dup[sp * 16 * r + f];
      s_du[idx] = a.s * v;
    }
  } else {
    for (int idx = tid; idx < 16 * r; idx += kGdThreads) {
      const int f = (idx & 15) * r + (idx >> 4);
      float v = 0.0f;
      for (int sp = 0; sp < S; ++sp) v += ld_sys(dub + sp * (16 * r) + f);
      s_du[idx] = a.s * v;
    }
  }
  __syncthreads();
  if (a.pool > 1) {
    // group sums of x in place: P[m][gg] into s_px[m][gg]
    float pv = 0.0f;
    const int mm = (tid >> 4) & 15, gg = tid & 15;
    if (tid < 256 && gg < ngrp)
      for (int e = 0; e < a.pool; ++e) pv += s_px[mm * kGdCols + gg * a.pool + e];
    __syncthreads();
    if (tid < 256 && gg < ngrp) s_px[mm * kGdCols + gg] = pv;
    __syncthreads();
  }
  if (wave >= 8) {
    // (13) dA[j][c] = sum_m du[m][j] P[m][c], fp32 MFMA over m (4 per step):
    //      wave 8 + ct owns columns 16 ct .. +15, every 16-row group of j
    const int ct = wave - 8;
    if (ct * 16 < acols) {
      const int c = ct * 16 + l16;
      for (int jt = 0; jt * 16 < r; ++jt) {
        const int ja = jt * 16 + l16;  // A operand row (j) of this lane
        f32x4 d = zero4;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float av_ = ja < r ? s_du[ja * 16 + 4 * st + g] : 0.0f;
          const float bv_ = s_px[(4 * st + g) * kGdCols + c];
          d = __builtin_amdgcn_mfma_f32_16x16x4f32(av_, bv_, d, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = jt * 16 + 4 * g + v;
          if (j < r && c < acols) a.dA[static_cast<int64_t>(j) * Ka + ac0 + c] = f32_to_bf16(d[v]);
        }
      }
    }
  } else if (do_dx) {
    // (14) dX[m][k .. k+3] = sum over splits (fixed order) + du A, the
    //      adapter term as D[k][m] = sum_j A[j][k] du[m][j] (fp32 MFMA over j)
    f32x4 sum = pd[0];
#pragma unroll
    for (int sp = 1; sp < kGdPre; ++sp)
      if (sp < S) sum += pd[sp];
    for (int sp0 = kGdPre; sp0 < S; sp0 += kGdPre) {
      f32x4 t[kGdPre];
#pragma unroll
      for (int q = 0; q < kGdPre; ++q) t[q] = ld_sys16(pr, pd_off(sp0 + q));
#pragma unroll
      for (int q = 0; q < kGdPre; ++q)
        if (sp0 + q < S) sum += t[q];
    }
    const int kcol = 16 * (wave & 7) + l16;  // A operand row (k) of this lane
    const int acol = a.pool == 1 ? kcol : kcol >> ps;
    f32x4 d = zero4;
    for (int j0 = 0; j0 < r; j0 += 4) {
      const int j = j0 + g;
      const float av_ = j < r ? bf16_to_f32(s_a[j * kGdCols + acol]) : 0.0f;
      const float bv_ = j < r ? s_du[j * 16 + l16] : 0.0f;
      d = __builtin_amdgcn_mfma_f32_16x16x4f32(av_, bv_, d, 0, 0, 0);
    }
    if (dm < M && kc0 + dkq < K) {
      u32x2 o;
      o.x = pack_bf16x2(sum[0] + d[0], sum[1] + d[1]);
      o.y = pack_bf16x2(sum[2] + d[2], sum[3] + d[3]);
      *reinterpret_cast<u32x2*>(a.dx + dm * K + kc0 + dkq) = o;
    }
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
    hipLaunchKernelGGL(k_gemv_dx<kFmtNF4>, dim3(grid), dim3(kGdThreads), 0, stream, a);
  else if (fmt == kFmtINT4)
    hipLaunchKernelGGL(k_gemv_dx<kFmtINT4>, dim3(grid), dim3(kGdThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(k_gemv_dx<kFmtNFG>, dim3(grid), dim3(kGdThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
