// Input gradient of the adapted 4-bit layer for many tokens:
//     dX = dY W_bf16 + du A            (QA-LoRA: + du A repeated per group)
// [QLoRA "The QLoRA recipe" stage 3: gradients flow back through the frozen,
//  dequantized weight; W itself receives no gradient.]
//
// The reduction runs over the output features n, i.e. across rows of the
// packed weight, while every row decodes with its own per-block table.  So
// each 64 x 256 weight slab is decoded cooperatively in its natural row
// orientation (every thread: two rows x 32 columns, one table per row) and
// written to LDS transposed as bf16 pairs [k][n, n+1]; the waves then read
// 8 consecutive n of one column as one 16-byte MFMA operand.
//
// Tile: 256 columns of dX x 256 tokens per workgroup, 4 waves as 2 x 2 of
// 128 x 128.  The next step's dY tile and codes are loaded into registers
// while the current step's products run and are written to LDS after them;
// both LDS stages are double buffered.  The adapter term du A is 2*ceil(r/16) extra
// MFMA k-steps (du split hi + lo), read from A^T [K][r].
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kTK = 256;    // dX columns per tile
constexpr int kTMx = 256;   // tokens per tile
constexpr int kNS = 64;     // reduction rows per step
constexpr int kStage = kTK * kNS * 2;  // 32 KB per operand per stage

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// [row][64 bf16] rows of 128 B, 16-byte chunks XOR-swizzled by row
__device__ __forceinline__ uint32_t off64(int row, int chunk) {
  return static_cast<uint32_t>(row * 128 + ((chunk ^ (row & 7)) << 4));
}

__device__ __forceinline__ int remap_xcd(int bid, int n) {
  const int q = n >> 3, rem = n & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

template <int FMT>
struct DxParams;
template <>
struct DxParams<kFmtNF4> {
  BlockParams bp[2];  // raw: the scale is formed when the table is built
};
template <>
struct DxParams<kFmtINT4> {
  uint32_t sz[2];
};

template <int FMT>
__global__ __launch_bounds__(256, 1) void k_dx_gemm(DxArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_w[2][kStage];   // [k][n] bf16
  __shared__ __attribute__((aligned(16))) uint8_t s_dy[2][kStage];  // [m][n] bf16

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int wk = wave & 1, wm = wave >> 1;
  const int64_t M = a.M, N = a.w.N, K = a.w.K;
  const int tiles_m = static_cast<int>((M + kTMx - 1) / kTMx);
  const int tiles_k = static_cast<int>((K + kTK - 1) / kTK);
  const int t = remap_xcd(static_cast<int>(blockIdx.x), tiles_m * tiles_k);
  // (uniform; said so, so that the buffer resource below stays scalar)
  const int tm = __builtin_amdgcn_readfirstlane(t / tiles_k);
  const int tk = __builtin_amdgcn_readfirstlane(t % tiles_k);
  const int64_t m0 = static_cast<int64_t>(tm) * kTMx, k0 = static_cast<int64_t>(tk) * kTK;
  const int64_t nsteps = (N + kNS - 1) / kNS;

  // decode assignment: rows 2p, 2p+1 of the step, columns [32 kq, 32 kq + 32)
  const int p = tid & 31, kq = tid >> 5;
  const int64_t kcol = k0 + kq * 32;
  const bool kvalid = kcol < K;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // dY tile of a step (256 tokens x 64 rows of dY^T) through registers:
  // lane L of wave w, instruction i holds 16 bytes of token row
  // (4i + w) * 8 + L / 8, chunk (L % 8) XOR-swizzled by the row, and writes
  // them where a whole-line direct-to-LDS load would have put them.  (After
  // a direct-to-LDS load the compiler holds every later LDS read until the
  // load lands, which would expose the next step's load latency.)
  // The rows go through a buffer resource over the tile's tokens: one 32-bit
  // offset per lane and a scalar offset per instruction (rows past M read as
  // zero; their outputs are never stored).  A chunk past N reads the row's
  // last 8 columns (those weight rows are masked to zero).
  const int64_t dy_rows = M - m0 < kTMx ? M - m0 : kTMx;
  const rsrc_t dyr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.dy + m0 * N), 0, static_cast<int>(dy_rows * N * 2), 0x00020000);
  const int dy_lrow = wave * 8 + (lane >> 3);   // row in instruction 0; + 32 per instruction
  const int dy_c = (lane & 7) ^ (dy_lrow & 7);  // this lane's chunk (32 rows keep row & 7)
  u32x4 dyv[8];
  auto load_dy = [&](int64_t st) {
    int64_t n = st * kNS + dy_c * 8;
    n = n < N ? n : N - 8;
    const uint32_t voff = static_cast<uint32_t>((dy_lrow * N + n) * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dyv[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(dyr, voff, static_cast<int>(i * 32 * N * 2), 0));
  };
  auto store_dy = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(&s_dy[buf][(i * 4 + wave) * 1024 + lane * 16]) = dyv[i];
  };

  u32x4 cw[2];
  DxParams<FMT> prm;
  bool rvalid[2];
  auto load_codes = [&](int64_t st) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int64_t n = st * kNS + 2 * p + r;
      rvalid[r] = kvalid && n < N;
      // unconditional loads from clamped addresses; invalid rows are masked at decode
      const int64_t nc = n < N ? n : N - 1;
      const int64_t kc = kvalid ? kcol : 0;
      cw[r] = *reinterpret_cast<const u32x4*>(a.w.codes + nc * (K >> 1) + (kc >> 1));
      if constexpr (FMT == kFmtNF4) {
        prm.bp[r] = load_block_params<kFmtNF4>(a.w, nc, kc >> 6, true);
      } else {
        const int64_t gi = nc * (K >> 5) + (kc >> 5);
        prm.sz[r] = static_cast<uint32_t>(a.w.scale[gi]) | (static_cast<uint32_t>(a.w.zero[gi]) << 16);
      }
    }
  };

  auto decode_store = [&](int buf) {
    Lut16 lut[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if constexpr (FMT == kFmtNF4)
        lut[r] = lut_nf4(a.w.cb, nf4_params_scale(a.w, prm.bp[r]));
      else
        lut[r] = lut_int4(half_bits_to_f32(static_cast<uint16_t>(prm.sz[r] & 0xFFFFu)),
                          half_bits_to_f32(static_cast<uint16_t>(prm.sz[r] >> 16)));
    }
    uint8_t* wb = s_w[buf];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 d0 = lut_decode8(lut[0], cw[0][q]);
      u32x4 d1 = lut_decode8(lut[1], cw[1][q]);
      if (!rvalid[0]) d0 = u32x4{0, 0, 0, 0};
      if (!rvalid[1]) d1 = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // columns kq*32 + 8q + 2e and +1: pairs (row 2p, row 2p+1)
        const uint32_t lo = perm(d1[e], d0[e], 0x05040100u);
        const uint32_t hi = perm(d1[e], d0[e], 0x07060302u);
        const int kr = kq * 32 + 8 * q + 2 * e;
        const int chunk = p >> 2, within = (p & 3) * 4;
        *reinterpret_cast<uint32_t*>(wb + off64(kr, chunk) + within) = lo;
        *reinterpret_cast<uint32_t*>(wb + off64(kr + 1, chunk) + within) = hi;
      }
    }
  };

  load_dy(0);
  load_codes(0);
  store_dy(0);
  decode_store(0);
  __syncthreads();

  for (int64_t st = 0; st < nsteps; ++st) {
    const int buf = static_cast<int>(st & 1);
    const bool more = st + 1 < nsteps;
    if (more) {
      load_dy(st + 1);
      load_codes(st + 1);
    }
    const uint8_t* wb = s_w[buf];
    const uint8_t* db = s_dy[buf];
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int chunk = 2 * nn + h;
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(wb + off64(wk * 128 + i * 32 + l32, chunk));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(db + off64(wm * 128 + j * 32 + l32, chunk));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) {
      store_dy(buf ^ 1);
      decode_store(buf ^ 1);
    }
    __syncthreads();
  }

  // adapter term du A: D[k][m] += sum_j A^T[k][j] du[m][j]
  if (a.du != nullptr && a.At != nullptr && a.r > 0) {
    const int rr = a.r;
    const int jsteps = (rr + 15) / 16;
    for (int jt = 0; jt < jsteps; ++jt) {
      const int j0 = jt * 16 + h * 8;
      u32x4 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t k = k0 + wk * 128 + i * 32 + l32;
        k = k < K ? k : K - 1;
        const uint16_t* ar = a.At + k * rr;
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ja = j0 + 2 * e, jb = ja + 1;
          const uint32_t lo = ar[ja < rr ? ja : rr - 1];
          const uint32_t hi = ar[jb < rr ? jb : rr - 1];
          v[e] = (ja < rr ? lo : 0u) | ((jb < rr ? hi : 0u) << 16);
        }
        af[i] = u32x4{v[0], v[1], v[2], v[3]};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int64_t m = m0 + wm * 128 + j * 32 + l32;
        m = m < M ? m : M - 1;
        const float* dr = a.du + m * rr;
        float hv[8], lv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jj = j0 + e;
          const float dv = dr[jj < rr ? jj : rr - 1];
          split_bf16(jj < rr ? dv : 0.0f, hv[e], lv[e]);
        }
        u32x4 uh, ul;
        uh.x = pack_bf16x2(hv[0], hv[1]); uh.y = pack_bf16x2(hv[2], hv[3]);
        uh.z = pack_bf16x2(hv[4], hv[5]); uh.w = pack_bf16x2(hv[6], hv[7]);
        ul.x = pack_bf16x2(lv[0], lv[1]); ul.y = pack_bf16x2(lv[2], lv[3]);
        ul.z = pack_bf16x2(lv[4], lv[5]); ul.w = pack_bf16x2(lv[6], lv[7]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i][j] = mfma32(af[i], uh, acc[i][j]);
          acc[i][j] = mfma32(af[i], ul, acc[i][j]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // store: lane holds D[k = 8q + 4h + t][m = l32] of each 32x32 tile
  const int64_t G = a.Gq != nullptr ? (K >> a.pool_shift) : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t m = m0 + wm * 128 + j * 32 + l32;
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
    hipLaunchKernelGGL(k_dx_gemm<kFmtNF4>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_dx_gemm<kFmtINT4>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
