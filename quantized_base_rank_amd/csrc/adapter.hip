// Low-rank adapter products.  [QLoRA "Background: how LoRA works" and the
// code sketch: u = x A^T, then B u; backward into A and B only.  QA-LoRA
// abstract: the adapter of the group-wise variant sees pooled inputs.]
//
//   NT  C[m][j] = alpha * sum_k X[m][k] * Y[j][k]        u = x A^T, du = s dY B
//
// The product reduces over a long dimension with a narrow (rank-r) output,
// so the reduction is split across workgroups; partial sums are written to
// the workspace and the last workgroup of each output tile (atomic ticket)
// adds them in fixed split order, which keeps results bit-identical run to
// run.  (The transposed products dB and dA are in adapter_tn.hip.)
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

// ---------------------------------------------------------------- NT skinny
// Workgroup: 4 waves, 64 rows of X, all J (<= 32 JT) columns, a slice of K
// in 128-column chunks.  A chunk of X (64 rows x 256 B) and of Y (32 JT rows
// x 256 B) is read as whole 128-byte lines into registers two chunks ahead
// (the loop is unrolled by two so that the two register sets stay fixed)
// and written to LDS (double buffered, 16-byte pieces XOR-swizzled by row)
// one chunk ahead; wave (mh, jh) forms rows 32 mh .. +31 x column tiles
// jh, jh + 2 (32 columns each), so no cross-wave sum is needed.  Pieces past
// K or past M / J are zero.
constexpr int kNtRowsPerWg = 64;
constexpr int kNtChunk = 128;
constexpr int kNtTileFloats = 128 * kNtRowsPerWg;  // one tile's partial, [j][m]

__device__ __forceinline__ uint32_t nt_off(int row, int piece) {
  return static_cast<uint32_t>(row * 256 + ((piece ^ (row & 15)) << 4));
}

template <int JT>
__global__ __launch_bounds__(256) void k_nt_skinny(NtArgs a) {
  constexpr int kYP = JT * 2;  // Y pieces per thread and chunk (32 JT rows x 16 pieces / 256)
  __shared__ __attribute__((aligned(16))) uint8_t s_x[2][kNtRowsPerWg * 256];
  __shared__ __attribute__((aligned(16))) uint8_t s_y[2][JT * 32 * 256];
  __shared__ uint32_t s_ticket;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int mh = wave & 1, jh = wave >> 1;
  const int m_tiles = static_cast<int>((a.M + kNtRowsPerWg - 1) / kNtRowsPerWg);
  const int tile = static_cast<int>(blockIdx.x) % m_tiles;
  const int split = static_cast<int>(blockIdx.x) / m_tiles;
  const int64_t m0 = static_cast<int64_t>(tile) * kNtRowsPerWg;
  const int64_t nchunks = (a.K + kNtChunk - 1) / kNtChunk;
  const int64_t per = (nchunks + a.splits - 1) / a.splits;
  const int64_t c0 = split * per;
  const int64_t c1 = c0 + per < nchunks ? c0 + per : nchunks;

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  // piece i of this thread: X row (tid + 256 i) / 16 (i < 4), Y row (i < kYP)
  u32x4 xr[2][4], yr[2][kYP];
  auto load = [&](int64_t c, u32x4 (&xv)[4], u32x4 (&yv)[kYP]) {
    const int64_t cc = c < nchunks ? c : nchunks - 1;  // a chunk past the last re-reads it
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i, row = p >> 4;
      const int64_t k = cc * kNtChunk + (p & 15) * 8;
      const int64_t m = m0 + row < a.M ? m0 + row : a.M - 1;
      xv[i] = *reinterpret_cast<const u32x4*>(a.X + m * a.ldx + (k < a.K ? k : 0));
    }
#pragma unroll
    for (int i = 0; i < kYP; ++i) {
      const int q = tid + 256 * i, row = q >> 4;
      const int64_t k = cc * kNtChunk + (q & 15) * 8;
      const int jr = row < a.J ? row : a.J - 1;
      yv[i] = *reinterpret_cast<const u32x4*>(a.Y + static_cast<int64_t>(jr) * a.ldy + (k < a.K ? k : 0));
    }
  };
  auto store = [&](int64_t c, int buf, const u32x4 (&xv)[4], const u32x4 (&yv)[kYP]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i, row = p >> 4;
      const bool ok = m0 + row < a.M && c * kNtChunk + (p & 15) * 8 < a.K;
      *reinterpret_cast<u32x4*>(&s_x[buf][nt_off(row, p & 15)]) = ok ? xv[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kYP; ++i) {
      const int q = tid + 256 * i, row = q >> 4;
      const bool ok = row < a.J && c * kNtChunk + (q & 15) * 8 < a.K;
      *reinterpret_cast<u32x4*>(&s_y[buf][nt_off(row, q & 15)]) = ok ? yv[i] : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kNtChunk / 16; ++kk) {
      const u32x4 xf = *reinterpret_cast<const u32x4*>(&s_x[buf][nt_off(mh * 32 + l32, 2 * kk + h)]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int jt = jh + 2 * t;
        if (jt < JT) {
          const u32x4 yf = *reinterpret_cast<const u32x4*>(&s_y[buf][nt_off(jt * 32 + l32, 2 * kk + h)]);
          acc[t] = mfma32(xf, yf, acc[t]);
        }
      }
    }
  };

  // chunk c sits in LDS stage (c - c0) & 1 and, before that, in register set
  // (c - c0) & 1; the loads of chunk c + 2 are issued while chunk c is used
  if (c0 < c1) {
    load(c0, xr[0], yr[0]);
    load(c0 + 1, xr[1], yr[1]);
    store(c0, 0, xr[0], yr[0]);
    __syncthreads();
  }
  for (int64_t c = c0; c < c1; c += 2) {
    // even chunk c: registers 0 are free (chunk c is in LDS stage 0)
    load(c + 2, xr[0], yr[0]);
    compute(0);
    if (c + 1 < c1) store(c + 1, 1, xr[1], yr[1]);
    __syncthreads();
    if (c + 1 >= c1) break;
    // odd chunk c + 1: registers 1 are free
    load(c + 3, xr[1], yr[1]);
    compute(1);
    if (c + 2 < c1) store(c + 2, 0, xr[0], yr[0]);
    __syncthreads();
  }

  // lane holds D[m = 32 mh + 8i + 4h + v][j = 32 jt + l32] at acc[t][4i + v]:
  // partial sums of a tile are kept [j][m], four consecutive m per 16 bytes
  const rsrc_t pr = make_rsrc(a.partial);
  auto poff = [&](int sp, int t, int i) {
    return static_cast<uint32_t>(((static_cast<int64_t>(tile) * a.splits + sp) * kNtTileFloats +
                                  ((jh + 2 * t) * 32 + l32) * kNtRowsPerWg + mh * 32 + 8 * i + 4 * h) * 4);
  };
  // only column tiles below JT carry partial sums (a wave whose tiles are
  // all past JT, e.g. jh = 1 when JT = 1, publishes and reads nothing)
  if (a.splits > 1) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (jh + 2 * t < JT)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          st_sys16(pr, poff(split, t, i), f32x4{acc[t][4 * i], acc[t][4 * i + 1], acc[t][4 * i + 2], acc[t][4 * i + 3]});
    if (__builtin_amdgcn_readfirstlane(publish_and_ticket(a.counters + tile, &s_ticket)) !=
        static_cast<uint32_t>(a.splits - 1))
      return;
    f32x4 sum[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sum[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < a.splits; sp0 += 4) {
      f32x4 v[4][2][4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (jh + 2 * t < JT)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[q][t][i] = ld_sys16(pr, poff(sp0 + q < a.splits ? sp0 + q : a.splits - 1, t, i));
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (sp0 + q < a.splits)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            if (jh + 2 * t < JT)
#pragma unroll
              for (int i = 0; i < 4; ++i) sum[t][i] += v[q][t][i];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][4 * i + v] = sum[t][i][v];
    if (tid == 0) a.counters[tile] = 0u;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = (jh + 2 * t) * 32 + l32;
    if (j >= a.J) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + mh * 32 + 8 * i + 4 * h + v;
        if (m < a.M) a.C[m * a.ldc + j] = a.alpha * acc[t][4 * i + v];
      }
  }
}

// ----------------------------------------------------------- transpose bf16
__global__ __launch_bounds__(256) void k_transpose16(const uint16_t* __restrict__ in, int64_t rows,
                                                     int64_t cols, uint16_t* __restrict__ out) {
  __shared__ uint16_t tile[32][33];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 32, c0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 8 rows per pass
  for (int i = ty; i < 32; i += 8) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? in[r * cols + c] : static_cast<uint16_t>(0);
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) out[c * rows + r] = tile[tx][i];
  }
}

}  // namespace

hipError_t launch_nt_skinny(const NtArgs& a, hipStream_t stream) {
  const int m_tiles = static_cast<int>((a.M + kNtRowsPerWg - 1) / kNtRowsPerWg);
  const dim3 grid(static_cast<uint32_t>(m_tiles * a.splits));
  switch ((a.J + 31) / 32) {
    case 1: hipLaunchKernelGGL(k_nt_skinny<1>, grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(k_nt_skinny<2>, grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(k_nt_skinny<3>, grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(k_nt_skinny<4>, grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

int nt_tiles(int64_t M) { return static_cast<int>((M + kNtRowsPerWg - 1) / kNtRowsPerWg); }
int64_t nt_partial_floats(int64_t M, int splits) {
  return splits > 1 ? static_cast<int64_t>(nt_tiles(M)) * splits * kNtTileFloats : 0;
}

hipError_t launch_transpose16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                              hipStream_t stream) {
  dim3 grid(static_cast<uint32_t>((cols + 31) / 32), static_cast<uint32_t>((rows + 31) / 32));
  hipLaunchKernelGGL(k_transpose16, grid, dim3(256), 0, stream, in, rows, cols, out);
  return hipGetLastError();
}

}  // namespace qlin
