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
// Workgroup: 4 waves, one 32-row tile of X, all J (<= 128) columns, a slice
// of K.  Each wave takes every 4th k16 step of the slice; the waves' sums are
// combined through LDS in wave order.
constexpr int kNtRowsPerWg = 32;

__global__ __launch_bounds__(256) void k_nt_skinny(NtArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int m_tiles = static_cast<int>((a.M + kNtRowsPerWg - 1) / kNtRowsPerWg);
  const int tile = blockIdx.x % m_tiles;
  const int split = blockIdx.x / m_tiles;
  const int64_t m0 = static_cast<int64_t>(tile) * kNtRowsPerWg;
  const int64_t k_steps = a.K / 16;  // K % 16 == 0
  const int64_t per = (k_steps + a.splits - 1) / a.splits;
  const int64_t s_begin = split * per;
  const int64_t s_end = s_begin + per < k_steps ? s_begin + per : k_steps;
  const int jsub = (a.J + 31) / 32;  // 1..4

  f32x16 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x16{};

  const int64_t mrow = m0 + l32 < a.M ? m0 + l32 : a.M - 1;
  const uint16_t* xrow = a.X + mrow * a.ldx;
  // each wave keeps kNtU k16 steps of loads in flight
  constexpr int kNtU = 4;
  for (int64_t st0 = s_begin + wave * kNtU; st0 < s_end; st0 += 4 * kNtU) {
    u32x4 xa[kNtU], yb[kNtU][4];
#pragma unroll
    for (int u = 0; u < kNtU; ++u) {
      const int64_t st = st0 + u < s_end ? st0 + u : s_end - 1;
      const int64_t k = st * 16 + h * 8;
      xa[u] = *reinterpret_cast<const u32x4*>(xrow + k);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = q * 32 + l32;
        const int jc = j < a.J ? j : a.J - 1;
        yb[u][q] = u32x4{0, 0, 0, 0};
        if (q < jsub) {  // uniform
          const u32x4 d = *reinterpret_cast<const u32x4*>(a.Y + static_cast<int64_t>(jc) * a.ldy + k);
          if (j < a.J) yb[u][q] = d;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kNtU; ++u) {
      if (st0 + u < s_end) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < jsub) acc[q] = mfma32(xa[u], yb[u][q], acc[q]);
      }
    }
  }

  // combine the four waves: D tile [32 m][32 j] per q; lane holds
  // D[8i + 4h + t][l32] at acc[q][4i + t]
  __shared__ float s_red[4][4][16][64];  // [wave][q][elem][lane] 64 KB
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) s_red[wave][q][e][lane] = acc[q][e];
  __syncthreads();
  // thread tid handles (q = wave, lane) -> sum over the 4 waves in order
  float sum[16];
  {
    const int q = wave;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      sum[e] = ((s_red[0][q][e][lane] + s_red[1][q][e][lane]) + s_red[2][q][e][lane]) +
               s_red[3][q][e][lane];
  }
  const int q = wave;
  float* part = a.partial + (static_cast<int64_t>(tile) * a.splits + split) * (4 * 16 * 64);
  if (a.splits > 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) st_sys(part + (q * 16 + e) * 64 + lane, sum[e]);
    __shared__ uint32_t s_ticket;
    if (publish_and_ticket(a.counters + tile, &s_ticket) != static_cast<uint32_t>(a.splits - 1))
      return;
    const float* base = a.partial + static_cast<int64_t>(tile) * a.splits * (4 * 16 * 64);
#pragma unroll
    for (int e = 0; e < 16; ++e) sum[e] = 0.0f;
    for (int sp = 0; sp < a.splits; ++sp) {
      float v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        v[e] = ld_sys(base + sp * (4 * 16 * 64) + (q * 16 + e) * 64 + lane);
#pragma unroll
      for (int e = 0; e < 16; ++e) sum[e] += v[e];
    }
    if (tid == 0) a.counters[tile] = 0u;
  }
  if (q >= jsub) return;
  const int j = q * 32 + l32;
  if (j >= a.J) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t m = m0 + 8 * i + 4 * h + t;
      if (m < a.M) a.C[m * a.ldc + j] = a.alpha * sum[4 * i + t];
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
  hipLaunchKernelGGL(k_nt_skinny, dim3(m_tiles * a.splits), dim3(256), 0, stream, a);
  return hipGetLastError();
}

int nt_tiles(int64_t M) { return static_cast<int>((M + kNtRowsPerWg - 1) / kNtRowsPerWg); }
int64_t nt_partial_floats(int64_t M, int splits) {
  return splits > 1 ? static_cast<int64_t>(nt_tiles(M)) * splits * (4 * 16 * 64) : 0;
}

hipError_t launch_transpose16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                              hipStream_t stream) {
  dim3 grid(static_cast<uint32_t>((cols + 31) / 32), static_cast<uint32_t>((rows + 31) / 32));
  hipLaunchKernelGGL(k_transpose16, grid, dim3(256), 0, stream, in, rows, cols, out);
  return hipGetLastError();
}

}  // namespace qlin
