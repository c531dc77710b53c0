// Input gradient of the adapted 4-bit layer for many tokens:
//     dX = dY W_bf16 + du A            (QA-LoRA: + du A repeated per group)
// [QLoRA "The QLoRA recipe" stage 3: gradients flow back through the frozen,
//  dequantized weight; W itself receives no gradient.]
//
// The reduction runs over the output features n, i.e. across rows of the
// packed weight.  Each 64 x 256 weight slab of a step is decoded in its
// natural row orientation (wave w: columns [32 w, 32 w + 32) of the tile,
// lane l: row l, one table per lane) and written to LDS row-major; the
// transposing LDS read turns 8 consecutive rows of one column into an MFMA
// operand.
//
// Tile: 256 columns of dX x 256 tokens per workgroup, 8 waves (two per SIMD)
// each owning 128 columns x 64 tokens.  The two waves that share a SIMD work
// in opposite order within a step (products then the next step's decode, or
// the reverse), so that one wave's lookups overlap the other's products.
// The next step's dY tile (buffer loads into registers) and the codes two
// steps ahead load during the step; the dY tile goes to LDS at its end.  Both
// LDS stages are double buffered, one barrier per step.  The adapter term
// du A is 2*ceil(r/16) extra MFMA k-steps (du split hi + lo), read from A^T
// [K][r].
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kTK = 256;                  // dX columns per tile
constexpr int kTMx = 256;                 // tokens per tile
constexpr int kNS = 64;                   // reduction rows per step
constexpr int kWRow = kTK * 2;            // one W row of the tile in LDS: 512 B
constexpr int kWStage = kNS * kWRow;      // 32 KB
constexpr int kDyStage = kTMx * kNS * 2;  // 32 KB

// dY tile [m][64 bf16]: rows of 128 B, 16-byte chunks XOR-swizzled by row
__device__ __forceinline__ uint32_t off64(int row, int chunk) {
  return static_cast<uint32_t>(row * 128 + ((chunk ^ (row & 7)) << 4));
}

// Position of the 16-byte piece c (columns 8c .. 8c+7) of W row r.  The
// row term spreads the 16 consecutive rows that one write instruction covers
// over 16 positions; the column term puts the two column halves read by one
// transposing read (pieces 4j, 4j+1 and 4j+2, 4j+3) in different 128-byte
// halves.
__device__ __forceinline__ int wpos(int c, int r) {
  return c ^ (((c >> 1) & 1) << 3) ^ (((r & 7) << 1) | ((r >> 3) & 1));
}

__device__ __forceinline__ int remap_xcd(int bid, int n) {
  const int q = n >> 3, rem = n & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// Codes and raw decode constants of one lane's 32-column piece of a step.
template <int FMT>
struct StepCodes;
template <>
struct StepCodes<kFmtNF4> {
  u32x4 cw;
  BlockParams bp;
  bool valid;
};
template <>
struct StepCodes<kFmtINT4> {
  u32x4 cw;
  uint32_t sz;  // scale | zero << 16 of the piece's group
  bool valid;
};

template <int FMT>
__global__ __launch_bounds__(512, 1) void k_dx_gemm(DxArgs a) {
  // [W stage 0 | W stage 1 | dY stage 0 | dY stage 1], 128 KB; after the
  // loop the same memory holds the adapter operands
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[2 * kWStage + 2 * kDyStage];
  uint8_t (*const s_w)[kWStage] = reinterpret_cast<uint8_t (*)[kWStage]>(s_lds);            // [n][k] bf16, pieces at wpos
  uint8_t (*const s_dy)[kDyStage] = reinterpret_cast<uint8_t (*)[kDyStage]>(s_lds + 2 * kWStage);  // [m][n] bf16

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5, l16 = lane & 15;
  const int wk = wave & 1, wm = (wave >> 1) & 3;  // products: columns wk*128.., tokens wm*64..
  const bool mfma_first = wave < 4;              // waves w and w + 4 share a SIMD
  const int64_t M = a.M, N = a.w.N, K = a.w.K;
  const int tiles_m = static_cast<int>((M + kTMx - 1) / kTMx);
  const int tiles_k = static_cast<int>((K + kTK - 1) / kTK);
  const int t = remap_xcd(static_cast<int>(blockIdx.x), tiles_m * tiles_k);
  // (uniform; said so, so that the buffer resource below stays scalar)
  const int tm = __builtin_amdgcn_readfirstlane(t / tiles_k);
  const int tk = __builtin_amdgcn_readfirstlane(t % tiles_k);
  const int64_t m0 = static_cast<int64_t>(tm) * kTMx, k0 = static_cast<int64_t>(tk) * kTK;
  const int64_t nsteps = (N + kNS - 1) / kNS;

  // decode assignment: row `lane` of each step, columns [32 wave, +32)
  const int64_t kcol = k0 + wave * 32;
  const bool kvalid = kcol < K;
  const int64_t kcc = kvalid ? kcol : k0;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // dY tile of a step (256 tokens x 64 rows of dY^T) through registers from a
  // buffer resource over the tile's tokens: instruction i of lane L, wave w
  // holds 16 bytes of token row 64 i + 8 w + L / 8, chunk (L % 8) XOR the row,
  // and writes them where a whole-line direct-to-LDS load would put them.
  // Rows past M read as zero (their outputs are never stored); a chunk past
  // N reads the row's last 8 columns (those weight rows decode to zero).
  const int64_t dy_rows = M - m0 < kTMx ? M - m0 : kTMx;
  const rsrc_t dyr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.dy + m0 * N), 0, static_cast<int>(dy_rows * N * 2), 0x00020000);
  const int dy_lrow = wave * 8 + (lane >> 3);
  const int dy_c = (lane & 7) ^ (dy_lrow & 7);
  u32x4 dyv[4];
  auto load_dy = [&](int64_t st) {
    int64_t n = st * kNS + dy_c * 8;
    n = n < N ? n : N - 8;  // also clamps a step past the last
    const uint32_t voff = static_cast<uint32_t>((dy_lrow * N + n) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dyv[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(dyr, voff, static_cast<int>(i * 64 * N * 2), 0));
  };
  auto store_dy = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&s_dy[buf][(i * 8 + wave) * 1024 + lane * 16]) = dyv[i];
  };

  auto load_codes = [&](int64_t st, StepCodes<FMT>& sc) {
    const int64_t n = st * kNS + lane;
    sc.valid = kvalid && n < N;
    // unconditional loads from clamped addresses; invalid rows decode to zero
    const int64_t nc = n < N ? n : N - 1;
    sc.cw = *reinterpret_cast<const u32x4*>(a.w.codes + nc * (K >> 1) + (kcc >> 1));
    if constexpr (FMT == kFmtNF4) {
      sc.bp = load_block_params<kFmtNF4>(a.w, nc, kcc >> 6, true);
    } else {
      const int64_t gi = nc * (K >> 5) + (kcc >> 5);
      sc.sz = static_cast<uint32_t>(a.w.scale[gi]) | (static_cast<uint32_t>(a.w.zero[gi]) << 16);
    }
  };
  // one table per lane (an invalid row gets all-zero constants), 4 lookups
  // of 8, 16-byte writes to the lane's row
  auto decode = [&](const StepCodes<FMT>& sc, uint8_t* wt) {
    Lut16 lut;
    if constexpr (FMT == kFmtNF4) {
      BlockParams bp = sc.bp;
      bp.a = sc.valid ? bp.a : 0u;
      bp.b = sc.valid ? bp.b : 0u;
      lut = lut_nf4(a.w.cb, nf4_params_scale(a.w, bp));
    } else {
      const uint32_t sz = sc.valid ? sc.sz : 0u;
      lut = lut_int4(half_bits_to_f32(static_cast<uint16_t>(sz & 0xFFFFu)),
                     half_bits_to_f32(static_cast<uint16_t>(sz >> 16)));
    }
    u32x4 d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = lut_decode8(lut, sc.cw[q]);
    uint8_t* row = wt + lane * kWRow;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(row + (wpos(4 * wave + q, lane) << 4)) = d[q];
  };

  // MFMA operand: rows nb .. nb+7 of column col0 + (lane % 16) of a W tile,
  // two transposing reads of 4 rows.  Within a step, rows nb = 16 nn + 8 h +
  // (lane % 16) / 4 (+ 4) keep their row bits 0..3 for every nn, so the
  // positions depend on nn only through an immediate offset of nn * 16 rows:
  // the byte offsets for nn = 0 are formed once.
  uint32_t wofs[2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = wk * 128 + i * 32 + (l32 & 16) + 4 * (l16 & 3);
      const int c = col >> 3, half8 = ((col >> 2) & 1) * 8;
      const int r = 8 * h + (l16 >> 2) + 4 * x;
      wofs[x][i] = static_cast<uint32_t>(r * kWRow + (wpos(c, r) << 4) + half8);
    }
  // D[k][m] += sum_n W^T[k][n] dY^T[n][m] over a step: lane (l32, h) of the
  // A operand holds 8 rows of column k, of the B operand 8 rows of token m
  const int dyx = h ^ (l32 & 7);  // chunk 2 nn + h of row ... + l32 sits at (2 nn) ^ dyx
  // The operands of sub-step nn + 1 are read before the products of nn, so
  // that their LDS latency overlaps those products.
  auto read_ops = [&](const uint8_t* wt, const uint8_t* db, int nn, u32x4 (&af)[4], u32x4 (&bf)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x2 lo = ds_read_tr16(wt + nn * 16 * kWRow + wofs[0][i]);
      const u32x2 hi = ds_read_tr16(wt + nn * 16 * kWRow + wofs[1][i]);
      af[i] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bf[j] = *reinterpret_cast<const u32x4*>(db + (wm * 64 + j * 32 + l32) * 128 + (((2 * nn) ^ dyx) << 4));
  };
  auto products = [&](int buf) {
    const uint8_t* wt = s_w[buf];
    const uint8_t* db = s_dy[buf];
    u32x4 af[2][4], bf[2][2];
    read_ops(wt, db, 0, af[0], bf[0]);
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int cur = nn & 1;
      if (nn + 1 < 4) read_ops(wt, db, nn + 1, af[cur ^ 1], bf[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[cur][i], bf[cur][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  StepCodes<FMT> sc_next, sc_after;
  load_dy(0);
  load_codes(0, sc_next);
  store_dy(0);
  decode(sc_next, s_w[0]);
  if (nsteps > 1) load_codes(1, sc_next);
  __syncthreads();

  for (int64_t st = 0; st < nsteps; ++st) {
    const int buf = static_cast<int>(st & 1);
    const bool more = st + 1 < nsteps;
    // unconditional (clamped) loads: with a fixed number of loads per step
    // the compiler waits for exactly the older ones it needs
    load_dy(st + 1);
    load_codes(st + 2, sc_after);
    // one copy of the products; the decode sits before them in waves 4..7
    // and after them in waves 0..3 (a scalar branch either way)
    if (more && !mfma_first) decode(sc_next, s_w[buf ^ 1]);
    products(buf);
    if (more && mfma_first) decode(sc_next, s_w[buf ^ 1]);
    if (more) store_dy(buf ^ 1);
    sc_next = sc_after;
    __syncthreads();
  }

  // adapter term du A: D[k][m] += sum_j A^T[k][j] du[m][j], in k16 steps,
  // du split into hi + lo bf16 halves.  du of the tile's 256 tokens (as the
  // two halves) and A^T of its 256 columns are staged in LDS 64 adapter
  // columns at a time (rows padded by 16 B against bank conflicts), every
  // load of a chunk in flight at once.  Indices are clamped and values
  // masked (no divergent branches around loads).
  if (a.du != nullptr && a.At != nullptr && a.r > 0) {
    const int rr = a.r;
    constexpr int kJC = 64;          // adapter columns per staged chunk
    constexpr int rp = kJC + 8;      // staged row length (elements)
    constexpr int q4 = kJC / 4;      // 4-element pieces of a staged row
    uint16_t* s_dh = reinterpret_cast<uint16_t*>(s_lds);  // [256 m][rp]
    uint16_t* s_dl = s_dh + kTMx * rp;                     // [256 m][rp]
    uint16_t* s_at = s_dl + kTMx * rp;                     // [256 k][rp], 110.6 KB in all
    constexpr int kUPer = kTMx * q4 / 512;                 // 8 pieces of each kind per thread
    for (int jc = 0; jc < rr; jc += kJC) {
      f32x4 dv[kUPer];
      u32x2 av[kUPer];
#pragma unroll
      for (int q = 0; q < kUPer; ++q) {
        const int it = q * 512 + tid;
        const int row = it / q4, j = jc + (it - row * q4) * 4;
        int64_t mg = m0 + row, kg = k0 + row;
        mg = mg < M ? mg : M - 1;
        kg = kg < K ? kg : K - 1;
        const float* drow = a.du + mg * rr;
        const uint16_t* arow = a.At + kg * rr;
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
      __syncthreads();  // the loop's (or the previous chunk's) operands are consumed
#pragma unroll
      for (int q = 0; q < kUPer; ++q) {
        const int it = q * 512 + tid;
        const int row = it / q4, jl = (it - row * q4) * 4, j = jc + jl;
        float hv[4], lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(j + e < rr ? dv[q][e] : 0.0f, hv[e], lv[e]);
        *reinterpret_cast<u32x2*>(s_dh + row * rp + jl) = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
        *reinterpret_cast<u32x2*>(s_dl + row * rp + jl) = u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])};
        const uint32_t k0m = (j < rr ? 0x0000FFFFu : 0u) | (j + 1 < rr ? 0xFFFF0000u : 0u);
        const uint32_t k1m = (j + 2 < rr ? 0x0000FFFFu : 0u) | (j + 3 < rr ? 0xFFFF0000u : 0u);
        *reinterpret_cast<u32x2*>(s_at + row * rp + jl) = u32x2{av[q].x & k0m, av[q].y & k1m};
      }
      __syncthreads();
      const int jt_n = (rr - jc < kJC ? rr - jc + 15 : kJC) / 16;
      for (int jt = 0; jt < jt_n; ++jt) {
        const int j0 = jt * 16 + h * 8;
        u32x4 af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = *reinterpret_cast<const u32x4*>(s_at + (wk * 128 + i * 32 + l32) * rp + j0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int ml = wm * 64 + j * 32 + l32;
          const u32x4 uh = *reinterpret_cast<const u32x4*>(s_dh + ml * rp + j0);
          const u32x4 ul = *reinterpret_cast<const u32x4*>(s_dl + ml * rp + j0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i][j] = mfma32(af[i], uh, acc[i][j]);
            acc[i][j] = mfma32(af[i], ul, acc[i][j]);
          }
        }
      }
    }
  }

  // store: lane holds D[k = 8q + 4h + t][m = l32] of each 32x32 tile
  const int64_t G = a.Gq != nullptr ? (K >> a.pool_shift) : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t m = m0 + wm * 64 + j * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t k = k0 + wk * 128 + i * 32 + 8 * q + 4 * h;
        if (k >= K) continue;
        float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
        float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (a.Gq != nullptr) {
          const float* gr = a.Gq + m * G;
          v0 += gr[(k + 0) >> a.pool_shift];
          v1 += gr[(k + 1) >> a.pool_shift];
          v2 += gr[(k + 2) >> a.pool_shift];
          v3 += gr[(k + 3) >> a.pool_shift];
        }
        u32x2 o;
        o.x = pack_bf16x2(v0, v1);
        o.y = pack_bf16x2(v2, v3);
        *reinterpret_cast<u32x2*>(a.dx + m * K + k) = o;
      }
    }
}

}  // namespace

hipError_t launch_dx_gemm(const DxArgs& a, int fmt, hipStream_t stream) {
  const int grid = static_cast<int>(((a.M + kTMx - 1) / kTMx) * ((a.w.K + kTK - 1) / kTK));
  if (fmt == kFmtNF4)
    hipLaunchKernelGGL(k_dx_gemm<kFmtNF4>, dim3(grid), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(k_dx_gemm<kFmtINT4>, dim3(grid), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
