// Few-token (M <= 16) forward and backward, where the layer is bound by
// streaming the packed 4-bit weight from HBM rather than by MFMA.
// [QLoRA "The QLoRA recipe" stage 3: decode each block to bf16 on the fly;
//  "Background: how LoRA works" for the adapter; QA-LoRA abstract for INT4
//  groups and the pooled adapter.]
//
//   forward   y = x W_bf16^T + s u B^T,  u = P A^T
//   backward  dX = dY W_bf16 + expand(du A),  du = s dY B,
//             dA = du^T P,  dB = s dY^T u
//
// Forward: a workgroup owns 16 output features over a share of K of at most
// 4096 (the whole K for K <= 4096, so no cross-workgroup reduction at all).
// Its 8 waves (two per SIMD) take interleaved 256-wide K chunks, at most two
// each; every lane decodes one 64-element block of one row per chunk and
// loads the matching token and adapter fragments straight into MFMA operand
// registers, all chunks' loads issued before the first is used.  The plain
// adapter's u = x A^T (r <= 16) is formed from the same token fragments.
// Waves combine through LDS in fixed order.
//
// Backward: the reduction runs over N, across rows of the packed weight, so
// it is split; a workgroup owns 128 columns of dX and 512 rows.  Rows are
// decoded 128 at a time into LDS in natural [n][k] layout and the transposed
// LDS read turns 8 consecutive rows of one column into an MFMA operand.
// Every workgroup also forms du over its rows and dB for a share of them.
//
// Split reductions publish fp32 partial sums with write-through stores; the
// last workgroup of an output tile (atomic ticket) adds them in fixed split
// order.  Results are bit-identical from run to run and no workgroup waits
// for another.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

// ======================================================================
// forward
// ======================================================================
constexpr int kGfRows = 16;
constexpr int kGfChunk = 256;
constexpr int kGfKShare = 4096;  // K per workgroup at most (bounds activation re-reads)
constexpr int kGfWaves = 8;
constexpr int kGfPerWave = kGfKShare / kGfChunk / kGfWaves;  // chunks per wave (2)

struct FwdChunk {
  u32x4 cw[2];
  BlockParams bp;
  u32x4 xf[8];
  u32x4 af[8];
};

template <int FMT, bool FUSE_U>
__global__ __launch_bounds__(512) void k_gemv_fwd(GemvFwdArgs a) {
  __shared__ float s_y[kGfWaves][256];
  __shared__ float s_u[kGfWaves][256];
  __shared__ float s_fu[16 * 128];       // final u [16][r]
  __shared__ uint16_t s_b[16 * 128];     // B rows of this tile [16][r]
  __shared__ uint32_t s_ticket;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t N = a.w.N, K = a.w.K, M = a.M;
  const int r = a.r;
  const int S = a.splits;
  const int tiles = static_cast<int>((N + kGfRows - 1) / kGfRows);
  const int tile = static_cast<int>(blockIdx.x) % tiles;
  const int split = static_cast<int>(blockIdx.x) / tiles;
  const int64_t kr0 = static_cast<int64_t>(split) * a.kshare;
  const int64_t krlen = K - kr0 < a.kshare ? K - kr0 : a.kshare;
  const int nch = static_cast<int>((krlen + kGfChunk - 1) / kGfChunk);
  const int64_t n0 = static_cast<int64_t>(tile) * kGfRows;

  // adapter operands of the epilogue, issued first (small, L2-resident)
  uint32_t breg[8];
  float ureg[8];
  if (a.adapter) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = i * 512 + tid;
      const int nn = idx / r;
      const int64_t n = n0 + (nn < 16 ? nn : 15);
      breg[i] = a.B[(n < N ? n : N - 1) * r + idx % r];
      if (!FUSE_U) {
        const int64_t last = M * r - 1;
        ureg[i] = a.u_in[idx < last ? idx : last];
      }
    }
  }

  const int64_t rowc = n0 + l16 < N ? n0 + l16 : N - 1;
  const uint8_t* crow = a.w.codes + rowc * (K >> 1);
  const uint16_t* xrow = a.x + (l16 < M ? l16 : M - 1) * K;
  const uint16_t* arow = a.A + static_cast<int64_t>(l16 < r ? l16 : r - 1) * K;

  // one 256-wide chunk: this lane's row, block g; loads are unconditional
  // (clamped), invalid blocks are masked at use
  auto load = [&](int c, FwdChunk& d, bool& valid) {
    const int64_t kl = static_cast<int64_t>(c) * kGfChunk + g * 64;
    valid = kl < krlen;
    const int64_t kb = kr0 + (valid ? kl : 0);
#pragma unroll
    for (int t = 0; t < 8; ++t) d.xf[t] = *reinterpret_cast<const u32x4*>(xrow + kb + t * 8);
    if (FUSE_U) {
#pragma unroll
      for (int t = 0; t < 8; ++t) d.af[t] = *reinterpret_cast<const u32x4*>(arow + kb + t * 8);
    }
    d.cw[0] = *reinterpret_cast<const u32x4*>(crow + (kb >> 1));
    d.cw[1] = *reinterpret_cast<const u32x4*>(crow + (kb >> 1) + 16);
    d.bp = load_block_params<FMT>(a.w, rowc, kb >> 6, true);
  };

  f32x4 accy = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 accu = f32x4{0.f, 0.f, 0.f, 0.f};
  FwdChunk ch[kGfPerWave];
  bool vch[kGfPerWave];
#pragma unroll
  for (int i = 0; i < kGfPerWave; ++i) {
    const int c = wave + i * kGfWaves;
    load(c < nch ? c : nch - 1, ch[i], vch[i]);
    vch[i] = vch[i] && c < nch;
  }
#pragma unroll
  for (int i = 0; i < kGfPerWave; ++i) {
    Lut16 lut[2];
    luts_from_params<FMT>(a.w, ch[i].bp, lut);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x4 wf = lut_decode8(lut[t >> 2], ch[i].cw[t >> 2][t & 3]);
      accy = mfma16(vch[i] ? wf : u32x4{0, 0, 0, 0}, ch[i].xf[t], accy);
      if (FUSE_U) accu = mfma16(ch[i].xf[t], vch[i] ? ch[i].af[t] : u32x4{0, 0, 0, 0}, accu);
    }
  }

  // combine the waves: lane (l16, g) holds D[4g + v][l16]
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    s_y[wave][lane * 4 + v] = accy[v];
    if (FUSE_U) s_u[wave][lane * 4 + v] = accu[v];
  }
  if (a.adapter) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = i * 512 + tid;
      if (idx < 16 * r) {
        s_b[idx] = static_cast<uint16_t>(breg[i]);
        if (!FUSE_U) s_fu[idx] = ureg[i];
      }
    }
  }
  __syncthreads();
  // threads 0..255 -> y element (n = tid >> 4, m = tid & 15) and u element
  // (m = tid >> 4, j = tid & 15); the waves are added in fixed order
  const int e8 = tid & 255;
  const int en = e8 >> 4, em = e8 & 15;
  const int ysrc = ((en >> 2) * 16 + em) * 4 + (en & 3);
  float ysum = 0.0f;
#pragma unroll
  for (int w = 0; w < kGfWaves; ++w) ysum += s_y[w][ysrc];
  const int um = e8 >> 4, uj = e8 & 15;
  const int usrc = ((um >> 2) * 16 + uj) * 4 + (um & 3);
  float usum = 0.0f;
  if (FUSE_U)
#pragma unroll
    for (int w = 0; w < kGfWaves; ++w) usum += s_u[w][usrc];
  const bool owner = tid < 256;  // threads that finish one element each

  if (S > 1) {
    // publish this split's partial sums; the tile's last workgroup adds them
    float* part = a.partial + (static_cast<int64_t>(split) * tiles + tile) * 512;
    if (owner) {
      st_sys(part + e8, ysum);
      if (FUSE_U) st_sys(part + 256 + e8, usum);
    }
    if (publish_and_ticket(a.counters + tile, &s_ticket) != static_cast<uint32_t>(S - 1)) return;
    float yv[8], uv[8];
#pragma unroll
    for (int sp = 0; sp < 8; ++sp) {
      const float* ps = a.partial + (static_cast<int64_t>(sp < S ? sp : S - 1) * tiles + tile) * 512;
      yv[sp] = ld_sys(ps + e8);
      uv[sp] = FUSE_U ? ld_sys(ps + 256 + e8) : 0.0f;
    }
    ysum = 0.0f;
    usum = 0.0f;
#pragma unroll
    for (int sp = 0; sp < 8; ++sp)
      if (sp < S) {
        ysum += yv[sp];
        usum += uv[sp];
      }
    for (int sp = 8; sp < S; ++sp) {
      const float* ps = a.partial + (static_cast<int64_t>(sp) * tiles + tile) * 512;
      ysum += ld_sys(ps + e8);
      if (FUSE_U) usum += ld_sys(ps + 256 + e8);
    }
    if (tid == 0) a.counters[tile] = 0u;
  }
  if (FUSE_U) {
    if (owner && uj < r) {
      s_fu[um * r + uj] = usum;
      if (tile == 0 && a.u_out != nullptr && um < M) a.u_out[um * r + uj] = usum;
    }
    __syncthreads();
  }
  if (owner && em < M && n0 + en < N) {
    float yv = ysum;
    if (a.adapter) {
      float t = 0.0f;
      for (int j = 0; j < r; ++j) t += s_fu[em * r + j] * bf16_to_f32(s_b[en * r + j]);
      yv += a.s * t;
    }
    a.y[em * N + n0 + en] = f32_to_bf16(yv);
  }
}

// ======================================================================
// backward
// ======================================================================
constexpr int kGdCols = 128;
constexpr int kGdRowsChunk = 128;
constexpr int kGdRowsSplit = 512;
constexpr int kGdChunks = kGdRowsSplit / kGdRowsChunk;
constexpr int kGdWStride = kGdCols * 2 + 32;  // 288 B: rows land 8 banks apart

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
  const int tile = static_cast<int>(blockIdx.x) % tiles;
  const int split = static_cast<int>(blockIdx.x) / tiles;
  const int64_t kc0 = static_cast<int64_t>(tile) * kGdCols;
  const int64_t nb0 = static_cast<int64_t>(split) * kGdRowsSplit;
  const int64_t nlen = N - nb0 < kGdRowsSplit ? N - nb0 : kGdRowsSplit;
  const bool do_dx = a.dx != nullptr;
  const int jsub = (r + 15) >> 4;
  // this workgroup's share of the split's dB rows
  const int db_rows = (kGdRowsSplit + tiles - 1) / tiles;
  const int db0 = tile * db_rows;

  // (1) dY slice: 16 x 512 bf16 = 1024 chunks of 16 B
  u32x4 dyr[4];
  bool dym[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = i * 256 + tid;
    const int m = ch >> 6, q = ch & 63;
    dym[i] = m < M && q * 8 < nlen;
    const int64_t mc = m < M ? m : M - 1;
    const int qc = q * 8 < nlen ? q : 0;
    dyr[i] = *reinterpret_cast<const u32x4*>(a.dy + mc * N + nb0 + qc * 8);
  }
  // (2) B slice, first 16 adapter columns: 512 rows x 32 B
  auto load_b = [&](int js, u32x4 (&br)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = i * 256 + tid;
      const int nn = ch >> 1, jh = ch & 1;
      const int j0 = js * 16 + jh * 8;
      uint32_t v[4] = {0u, 0u, 0u, 0u};
      const int64_t nnc = nn < nlen ? nn : nlen - 1;
      const uint16_t* br16 = a.B + (nb0 + nnc) * r;
      if ((r & 7) == 0) {
        const int j0c = j0 + 8 <= r ? j0 : 0;
        const u32x4 d = *reinterpret_cast<const u32x4*>(br16 + j0c);
        if (nn < nlen && j0 + 8 <= r) {
          v[0] = d.x; v[1] = d.y; v[2] = d.z; v[3] = d.w;
        }
      } else if (nn < nlen) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (j0 + e < r) v[e >> 1] |= static_cast<uint32_t>(br16[j0 + e]) << (16 * (e & 1));
      }
      br[i] = u32x4{v[0], v[1], v[2], v[3]};
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
    const float v = a.u[idx < last ? idx : last];
    ur[i] = (idx < 16 * r && idx / r < M) ? v : 0.0f;
  }
  // (4) weight codes and constants for all chunks (issued last: the loads
  //     above complete first): row (tid >> 1), block (tid & 1)
  const int drow = tid >> 1, dblk = tid & 1;
  const int64_t kb = kc0 + dblk * 64;
  u32x4 cw[kGdChunks][2];
  BlockParams bp[kGdChunks];
  bool ok[kGdChunks];
#pragma unroll
  for (int c = 0; c < kGdChunks; ++c) {
    const int64_t nl = c * kGdRowsChunk + drow;
    ok[c] = do_dx && nl < nlen && kb < K;
    const int64_t nrow = nb0 + (nl < nlen ? nl : nlen - 1);
    const int64_t kbc = kb < K ? kb : K - 64;
    const uint8_t* p = a.w.codes + nrow * (K >> 1) + (kbc >> 1);
    cw[c][0] = *reinterpret_cast<const u32x4*>(p);
    cw[c][1] = *reinterpret_cast<const u32x4*>(p + 16);
    bp[c] = load_block_params<FMT>(a.w, nrow, kbc >> 6, true);
  }

  // (5) stage dY, the first B slice and u
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = i * 256 + tid;
    *reinterpret_cast<u32x4*>(&s_dy[(ch >> 6) * kGdRowsSplit + (ch & 63) * 8]) =
        dym[i] ? dyr[i] : u32x4{0, 0, 0, 0};
  }
  auto store_b = [&](const u32x4 (&bv)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = i * 256 + tid;
      *reinterpret_cast<u32x4*>(s_b + (ch >> 1) * 32 + (ch & 1) * 16) = bv[i];
    }
  };
  store_b(br);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i * 256 + tid < 16 * r) s_u[i * 256 + tid] = ur[i];
  __syncthreads();

  // (6) adapter partial du_p[m][j] = sum_{n in split} dY[m][n] B[n][j]
  float* du_part = a.du_part + (static_cast<int64_t>(tile) * a.splits + split) * (16 * r);
  for (int js = 0; js < jsub; ++js) {
    if (js > 0) {
      u32x4 bn[4];
      load_b(js, bn);
      __syncthreads();
      store_b(bn);
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

  // (7) dB[n][j] = s sum_m dY[m][n] u[m][j], rows [db0, db0 + db_rows) of the split
  for (int idx = tid; idx < db_rows * r; idx += 256) {
    const int nn = db0 + idx / r, j = idx % r;
    if (nn >= nlen) break;
    float t = 0.0f;
#pragma unroll
    for (int m = 0; m < 16; ++m) t += bf16_to_f32(s_dy[m * kGdRowsSplit + nn]) * s_u[m * r + j];
    a.dB[(nb0 + nn) * r + j] = f32_to_bf16(a.s * t);
  }

  // (8) weight product dX_p[m][k] = sum_{n in split} dY[m][n] W[n][k]; chunk
  //     c + 1 is decoded into the other buffer while chunk c feeds the MFMAs
  f32x4 acc[2];
  acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nchunks = static_cast<int>((nlen + kGdRowsChunk - 1) / kGdRowsChunk);
  auto decode = [&](int c, uint8_t* wbuf) {
    Lut16 lut[2];
    luts_from_params<FMT>(a.w, bp[c], lut);
    const uint32_t words[8] = {cw[c][0].x, cw[c][0].y, cw[c][0].z, cw[c][0].w,
                               cw[c][1].x, cw[c][1].y, cw[c][1].z, cw[c][1].w};
    uint8_t* wrow = wbuf + drow * kGdWStride + dblk * 128;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const u32x4 d = ok[c] ? lut_decode8(lut[tt >> 2], words[tt]) : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(wrow + tt * 16) = d;
    }
  };
  if (do_dx) {
    decode(0, s_lds);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kGdChunks; ++c) {
      if (c >= nchunks) break;
      const uint8_t* wb = s_lds + (c & 1) * kWBuf;
      if (c + 1 < nchunks) decode(c + 1, s_lds + ((c + 1) & 1) * kWBuf);
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

  // ---- fix-up of this column tile
  const int S = a.splits;
  const int ps = a.pool_shift;
  const int ncol = K - kc0 < kGdCols ? static_cast<int>(K - kc0) : kGdCols;
  const int ngrp = ncol >> ps;
  const int64_t Ka = K >> ps;
  const int acols = a.pool == 1 ? ncol : ngrp;
  const int64_t ac0 = kc0 >> ps;
  float* s_du = reinterpret_cast<float*>(s_lds);                 // [16][r]   8 KB max
  float* s_px = reinterpret_cast<float*>(s_lds + 8192);          // [16][128] 8 KB
  uint16_t* s_a = reinterpret_cast<uint16_t*>(s_lds + 16384);    // [r][128] 32 KB max
  // issue loads: partial dX, du partials, x tile, A tile
  const int m = tid >> 4;
  const int cl = (tid & 15) * 8;
  const int64_t kx = kc0 + cl < K ? kc0 + cl : K - 8;
  constexpr int kPre = 8;  // split partials prefetched per thread
  f32x4 pd[kPre][2];
  const rsrc_t pr = make_rsrc(a.partial);
  if (do_dx) {
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp) {
      const int spc = sp < S ? sp : S - 1;
      const uint32_t off = static_cast<uint32_t>(((static_cast<int64_t>(spc) * 16 + m) * K + kx) * 4);
      pd[sp][0] = ld_sys16(pr, off);
      pd[sp][1] = ld_sys16(pr, off + 16);
    }
  }
  const float* dub = a.du_part + static_cast<int64_t>(tile) * S * (16 * r);
  for (int idx = tid; idx < 16 * r; idx += 256) {
    float dv[kPre];
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp) dv[sp] = ld_sys(dub + (sp < S ? sp : S - 1) * (16 * r) + idx);
    float v = 0.0f;
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp)
      if (sp < S) v += dv[sp];
    for (int sp = kPre; sp < S; ++sp) v += ld_sys(dub + sp * (16 * r) + idx);
    s_du[idx] = a.s * v;
  }
  {
    const int c = tid & 127, m0 = tid >> 7;
    for (int mm = m0; mm < 16; mm += 2)
      s_px[mm * kGdCols + c] = (mm < M && c < ncol) ? bf16_to_f32(a.x[mm * K + kc0 + c]) : 0.0f;
  }
  for (int idx = tid; idx < r * acols; idx += 256) {
    const int j = idx / acols, c = idx % acols;
    s_a[j * kGdCols + c] = a.A[static_cast<int64_t>(j) * Ka + ac0 + c];
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
  // dA[j][c] = sum_m du[m][j] P[m][c]
  for (int idx = tid; idx < r * acols; idx += 256) {
    const int j = idx / acols, c = idx % acols;
    float t = 0.0f;
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) t += s_du[mm * r + j] * s_px[mm * kGdCols + c];
    a.dA[static_cast<int64_t>(j) * Ka + ac0 + c] = f32_to_bf16(t);
  }
  if (do_dx && m < M && kc0 + cl < K) {
    float sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = 0.0f;
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp)
      if (sp < S)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[e] += pd[sp][0][e];
          sum[4 + e] += pd[sp][1][e];
        }
    for (int sp = kPre; sp < S; ++sp) {
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
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = a.pool == 1 ? cl + e : ((cl + e) >> ps);
      float t = 0.0f;
      for (int j = 0; j < r; ++j) t += s_du[m * r + j] * bf16_to_f32(s_a[j * kGdCols + c]);
      sum[e] += t;
    }
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

int gemv_fwd_tiles(int64_t N) { return static_cast<int>((N + kGfRows - 1) / kGfRows); }
int gemv_fwd_splits(int64_t K) { return static_cast<int>((K + kGfKShare - 1) / kGfKShare); }
int64_t gemv_fwd_kshare(int64_t K) {
  const int64_t per = (K + gemv_fwd_splits(K) - 1) / gemv_fwd_splits(K);
  return (per + kGfChunk - 1) / kGfChunk * kGfChunk;
}
int64_t gemv_fwd_partial_floats(int64_t N, int64_t K) {
  const int S = gemv_fwd_splits(K);
  return S > 1 ? static_cast<int64_t>(S) * gemv_fwd_tiles(N) * 512 : 0;
}

hipError_t launch_gemv_fwd(const GemvFwdArgs& a, int fmt, hipStream_t stream) {
  const int grid = gemv_fwd_tiles(a.w.N) * a.splits;
  const dim3 block(64 * kGfWaves);
  if (fmt == kFmtNF4) {
    if (a.fuse_u)
      hipLaunchKernelGGL((k_gemv_fwd<kFmtNF4, true>), dim3(grid), block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_fwd<kFmtNF4, false>), dim3(grid), block, 0, stream, a);
  } else {
    if (a.fuse_u)
      hipLaunchKernelGGL((k_gemv_fwd<kFmtINT4, true>), dim3(grid), block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_fwd<kFmtINT4, false>), dim3(grid), block, 0, stream, a);
  }
  return hipGetLastError();
}

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
