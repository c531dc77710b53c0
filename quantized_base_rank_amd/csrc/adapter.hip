// Low-rank adapter products.  [QLoRA "Background: how LoRA works" and the
// code sketch: u = x A^T, then B u; backward into A and B only.  QA-LoRA
// abstract: the adapter of the group-wise variant sees pooled inputs.]
//
//   NT  C[m][j] = alpha * sum_k X[m][k] * Y[j][k]        u = x A^T, du = s dY B
//   TN  C[p][j] = alpha * sum_m X[m][p] * Z[m][j]        dB = s dY^T u, dA = du^T x
//
// Both reduce over a long dimension with a narrow (rank-r) output, so the
// reduction is split across workgroups; partial sums are written to the
// workspace and the last workgroup of each output tile (atomic ticket) adds
// them in fixed split order, which keeps results bit-identical run to run.
// fp32 operands (u, du) enter bf16 MFMA as hi + lo pairs.
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

// ---------------------------------------------------------------- TN skinny
// Workgroup: a 64-column tile of X (p), all J (<= 128) columns of Z, a slice
// of rows m.  Per 32-row step both tiles are staged transposed in LDS (m
// innermost), Z as hi and lo bf16 halves.  Wave w owns p-sub (w & 1) and the
// j-subs of parity (w >> 1).
constexpr int kTnP = 64;
constexpr int kTnM = 32;

__global__ __launch_bounds__(256) void k_tn_skinny(TnArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int p_tiles = static_cast<int>((a.P + kTnP - 1) / kTnP);
  const int tile = blockIdx.x % p_tiles;
  const int split = blockIdx.x / p_tiles;
  const int64_t p0 = static_cast<int64_t>(tile) * kTnP;
  const int64_t m_steps = (a.M + kTnM - 1) / kTnM;
  const int64_t per = (m_steps + a.splits - 1) / a.splits;
  const int64_t s_begin = split * per;
  const int64_t s_end = s_begin + per < m_steps ? s_begin + per : m_steps;
  const int jsub = (a.J + 31) / 32;

  // [p][m] bf16, row = 32 m = 64 B, padded to 80 B to spread banks
  constexpr int kRow = 40;  // in uint16 units
  __shared__ uint16_t s_x[kTnP * kRow];
  __shared__ uint16_t s_zh[128 * kRow];
  __shared__ uint16_t s_zl[128 * kRow];

  f32x16 acc[2];
  acc[0] = f32x16{};
  acc[1] = f32x16{};
  const int psub = wave & 1;
  const int jpar = wave >> 1;

  for (int64_t st = s_begin; st < s_end; ++st) {
    const int64_t mb = st * kTnM;
    // stage X[mb..mb+31][p0..p0+63]: 32 rows x 8 chunks of 8 -> 256 chunks
    {
      const int mm = tid & 31, pc = tid >> 5;  // pc 0..7
      const int64_t m = mb + mm;
      const int64_t p = p0 + pc * 8;
      uint16_t v[8];
      if (m < a.M && p + 8 <= a.P) {
        const u32x4 d = *reinterpret_cast<const u32x4*>(a.X + m * a.ldx + p);
        v[0] = d.x & 0xFFFF; v[1] = d.x >> 16; v[2] = d.y & 0xFFFF; v[3] = d.y >> 16;
        v[4] = d.z & 0xFFFF; v[5] = d.z >> 16; v[6] = d.w & 0xFFFF; v[7] = d.w >> 16;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = (m < a.M && p + e < a.P) ? a.X[m * a.ldx + p + e] : static_cast<uint16_t>(0);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s_x[(pc * 8 + e) * kRow + mm] = v[e];
    }
    // stage Z[mb..mb+31][0..J-1] fp32 -> hi/lo bf16, transposed
    for (int idx = tid; idx < kTnM * 128; idx += 256) {
      const int mm = idx & 31, j = idx >> 5;
      const int64_t m = mb + mm;
      float z = 0.0f;
      if (m < a.M && j < a.J) z = a.Z[m * a.ldz + j];
      float hi, lo;
      split_bf16(z, hi, lo);
      s_zh[j * kRow + mm] = static_cast<uint16_t>(__float_as_uint(hi) >> 16);
      s_zl[j * kRow + mm] = f32_to_bf16(lo);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int mo = kk * 16 + h * 8;
      const u32x4 xa = *reinterpret_cast<const u32x4*>(&s_x[(psub * 32 + l32) * kRow + mo]);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = jpar + 2 * qq;
        if (q < jsub) {
          const u32x4 zh = *reinterpret_cast<const u32x4*>(&s_zh[(q * 32 + l32) * kRow + mo]);
          const u32x4 zl = *reinterpret_cast<const u32x4*>(&s_zl[(q * 32 + l32) * kRow + mo]);
          acc[qq] = mfma32(xa, zh, acc[qq]);
          acc[qq] = mfma32(xa, zl, acc[qq]);
        }
      }
    }
    __syncthreads();
  }

  // partial layout: [tile][split][wave][qq][16][64]
  constexpr int kPart = 4 * 2 * 16 * 64;
  float sum[2][16];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum[qq][e] = acc[qq][e];
  if (a.splits > 1) {
    float* part = a.partial + (static_cast<int64_t>(tile) * a.splits + split) * kPart;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int e = 0; e < 16; ++e) st_sys(part + ((wave * 2 + qq) * 16 + e) * 64 + lane, sum[qq][e]);
    __shared__ uint32_t s_ticket;
    if (publish_and_ticket(a.counters + tile, &s_ticket) != static_cast<uint32_t>(a.splits - 1))
      return;
    const float* base = a.partial + static_cast<int64_t>(tile) * a.splits * kPart;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum[qq][e] = 0.0f;
    for (int sp = 0; sp < a.splits; ++sp) {
      float v[2][16];
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          v[qq][e] = ld_sys(base + sp * kPart + ((wave * 2 + qq) * 16 + e) * 64 + lane);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum[qq][e] += v[qq][e];
    }
    if (tid == 0) a.counters[tile] = 0u;
  }
  // D[p][j]: lane holds D[8i + 4h + t][l32]
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int q = jpar + 2 * qq;
    if (q >= jsub) continue;
    const int j = q * 32 + l32;
    if (j >= a.J) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t p = p0 + psub * 32 + 8 * i + 4 * h + t;
        if (p >= a.P) continue;
        const uint16_t v = f32_to_bf16(a.alpha * sum[qq][4 * i + t]);
        if (a.out_transposed)
          a.C[static_cast<int64_t>(j) * a.ldc + p] = v;
        else
          a.C[p * a.ldc + j] = v;
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

// ------------------------------------------------------ QA-LoRA (pooled) ops
// P[m][g] = sum of x[m][32g .. 32g+31] (fp32); u[m][j] = sum_g P[m][g] A[j][g].
// One workgroup per token row; the pooled row stays in LDS.
__global__ __launch_bounds__(256) void k_qa_pool_u(QaArgs a) {
  extern __shared__ float s_p[];  // [G]
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* xr = a.x + m * a.K;
  for (int64_t g = tid; g < a.G; g += 256) {
    const uint16_t* xs = xr + g * a.pool;
    float acc = 0.0f;
    for (int i = 0; i < a.pool; ++i) acc += bf16_to_f32(xs[i]);
    s_p[g] = acc;
    if (a.P_out) a.P_out[m * a.G + g] = acc;
  }
  __syncthreads();
  if (!a.u_out) return;
  const int wave = tid >> 6, lane = tid & 63;
  for (int j = wave; j < a.r; j += 4) {
    const uint16_t* ar = a.A + static_cast<int64_t>(j) * a.G;
    float acc = 0.0f;
    for (int64_t g = lane; g < a.G; g += 64) acc += s_p[g] * bf16_to_f32(ar[g]);
    acc = warp_sum(acc);
    if (lane == 0) a.u_out[m * a.r + j] = acc;
  }
}

// Gq[m][g] = sum_j du[m][j] A[j][g]  (the pooled adapter's input gradient
// before it is repeated over the group).
__global__ __launch_bounds__(256) void k_qa_grad_in(QaArgs a) {
  const int64_t m = blockIdx.y;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (g >= a.G) return;
  const float* dur = a.du + m * a.r;
  float acc = 0.0f;
  for (int j = 0; j < a.r; ++j) acc += dur[j] * bf16_to_f32(a.A[static_cast<int64_t>(j) * a.G + g]);
  a.Gq_out[m * a.G + g] = acc;
}

// dA[j][g] = sum_m du[m][j] P[m][g], fixed summation order over m.
__global__ __launch_bounds__(256) void k_qa_dA(QaArgs a) {
  const int j = blockIdx.y;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (g >= a.G) return;
  float acc = 0.0f;
  for (int64_t m = 0; m < a.M; ++m) acc += a.du[m * a.r + j] * a.P_in[m * a.G + g];
  a.dA_out[static_cast<int64_t>(j) * a.G + g] = f32_to_bf16(acc);
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

hipError_t launch_tn_skinny(const TnArgs& a, hipStream_t stream) {
  const int p_tiles = static_cast<int>((a.P + kTnP - 1) / kTnP);
  hipLaunchKernelGGL(k_tn_skinny, dim3(p_tiles * a.splits), dim3(256), 0, stream, a);
  return hipGetLastError();
}

int tn_tiles(int64_t P) { return static_cast<int>((P + kTnP - 1) / kTnP); }
int64_t tn_partial_floats(int64_t P, int splits) {
  return splits > 1 ? static_cast<int64_t>(tn_tiles(P)) * splits * (4 * 2 * 16 * 64) : 0;
}

hipError_t launch_transpose16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                              hipStream_t stream) {
  dim3 grid(static_cast<uint32_t>((cols + 31) / 32), static_cast<uint32_t>((rows + 31) / 32));
  hipLaunchKernelGGL(k_transpose16, grid, dim3(256), 0, stream, in, rows, cols, out);
  return hipGetLastError();
}

hipError_t launch_qa_pool_u(const QaArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_qa_pool_u, dim3(static_cast<uint32_t>(a.M)), dim3(256),
                     static_cast<uint32_t>(a.G * sizeof(float)), stream, a);
  return hipGetLastError();
}

hipError_t launch_qa_grad_in(const QaArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<uint32_t>((a.G + 255) / 256), static_cast<uint32_t>(a.M));
  hipLaunchKernelGGL(k_qa_grad_in, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_qa_dA(const QaArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<uint32_t>((a.G + 255) / 256), static_cast<uint32_t>(a.r));
  hipLaunchKernelGGL(k_qa_dA, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
