// Pooled-adapter products of the group-wise INT4 variant.  [QA-LoRA
// abstract: the adapter of the group-wise variant sees the input summed over
// each quantization group, so its rank-r products run on G = K / 32 pooled
// features.]
//
//   P[m][g]  = sum_{i < 32} x[m][32 g + i]     u[m][j]  = sum_g P[m][g] A[j][g]
//   dA[j][g] = sum_m du[m][j] P[m][g]
//
// (The input gradient du A, repeated over each group, is added by the large-M
// input-gradient GEMM from A^T with one row per group.)
//
// The pool is the INT4 group (32), the only pooled case.  Every sum is taken
// in a fixed order, so results are bit-identical from run to run.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kQaPool = 32;
constexpr int kQaTokMax = 8;  // tokens per workgroup (pooling, input gradient)
constexpr int kQaDaTile = 64;  // dA tile: 64 adapter rows x 64 groups
constexpr int kQaDaBlk = 32;   // tokens staged per step of a dA partial
constexpr int kQaMaxRank = 128;

// P and u for a block of tokens (1024 threads).  A pass loads 8 16-byte
// pieces per thread, flattened over (token, piece) so that every load of
// the pass is in flight at once (two passes cover 8 tokens of K = 11008);
// each thread adds its pieces' 8 elements in order and the four
// neighbouring lanes that hold one group add their sums pairwise in lane
// order.  u then takes the block's P from LDS into fp32 MFMAs (below).
constexpr int kQaThreads = 1024;
constexpr int kQaPer = 8;  // loads per thread and pass
__global__ __launch_bounds__(kQaThreads) void k_qa_pool_u(QaArgs a) {
  extern __shared__ float s_p[];  // [tok][G]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tok = a.tok;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * tok;
  const int64_t G = a.G, K = a.K;
  const int npiece = static_cast<int>(K / 8);  // 16-byte pieces per token row (a multiple of 4)
  const int total = tok * npiece;
  // LDS after the P block: the slices' partial u tiles, then A (staged)
  const int jt = (a.r + 15) >> 4, nsl = 16 / jt, rp = jt * 16;
  float* s_red = s_p + tok * G;  // [nsl][tok][rp]
  uint16_t* s_A = reinterpret_cast<uint16_t*>(s_red + nsl * tok * rp);
  // the first pieces of A are loaded before the pooling passes, so that
  // their latency overlaps them (indices clamped: no branch around loads)
  constexpr int kAPre = 4;
  const int64_t n16 = a.stage_a ? static_cast<int64_t>(a.r) * G / 8 : 0;
  u32x4 apre[kAPre];
  if (n16 > 0) {
#pragma unroll
    for (int i = 0; i < kAPre; ++i) {
      const int64_t idx = i * kQaThreads + tid;
      apre[i] = reinterpret_cast<const u32x4*>(a.A)[idx < n16 ? idx : n16 - 1];
    }
  }
  for (int p0 = 0; p0 < total; p0 += kQaThreads * kQaPer) {
    u32x4 w[kQaPer];
    int tk[kQaPer], pc[kQaPer];
#pragma unroll
    for (int i = 0; i < kQaPer; ++i) {
      const int pf = p0 + i * kQaThreads + tid;
      const int pcl = pf < total ? pf : total - 1;
      tk[i] = pcl / npiece;
      pc[i] = pcl - tk[i] * npiece;
      const int64_t m = m0 + tk[i];
      w[i] = *reinterpret_cast<const u32x4*>(a.x + (m < a.M ? m : a.M - 1) * K + static_cast<int64_t>(pc[i]) * 8);
    }
#pragma unroll
    for (int i = 0; i < kQaPer; ++i) {
      float v = bf16_lo(w[i].x);
      v += bf16_hi(w[i].x);
      v += bf16_lo(w[i].y);
      v += bf16_hi(w[i].y);
      v += bf16_lo(w[i].z);
      v += bf16_hi(w[i].z);
      v += bf16_lo(w[i].w);
      v += bf16_hi(w[i].w);
      // (lane 4q + 0 + lane 4q + 1) + (lane 4q + 2 + lane 4q + 3), the same
      // value in all four lanes
      const float v1 = __shfl_xor(v, 1, 64);
      const float q1 = (lane & 1) ? v1 + v : v + v1;
      const float q2 = __shfl_xor(q1, 2, 64);
      const float q = (lane & 2) ? q2 + q1 : q1 + q2;
      const int pf = p0 + i * kQaThreads + tid;
      const int64_t m = m0 + tk[i];
      if ((lane & 3) == 0 && pf < total) {
        const int64_t g = pc[i] >> 2;
        s_p[tk[i] * G + g] = q;
        if (a.P_out != nullptr && m < a.M) a.P_out[m * G + g] = q;
      }
    }
  }
  if (a.u_out == nullptr) return;
  // u of the block's tokens with fp32 MFMAs (16 x 16 x 4): row i = token,
  // column = adapter row j, reduction over the groups.  The 16 waves split
  // into ceil(r/16) column tiles times 16 / ceil(r/16) slices of the group
  // range; each slice's partial tile goes to LDS and the slices are added
  // in slice order.  In step e of a 16-group block, lane quarter q takes
  // group 16 b + 4 e + q (token rows past the block and columns past r are
  // zero operands).  A goes to LDS first when it fits.
  if (n16 > 0) {
#pragma unroll
    for (int i = 0; i < kAPre; ++i) {
      const int64_t idx = i * kQaThreads + tid;
      if (idx < n16) reinterpret_cast<u32x4*>(s_A)[idx] = apre[i];
    }
    for (int64_t i = kAPre * kQaThreads + tid; i < n16; i += kQaThreads)
      reinterpret_cast<u32x4*>(s_A)[i] = reinterpret_cast<const u32x4*>(a.A)[i];
  }
  __syncthreads();
  const int sl = wave / jt, j = (wave % jt) * 16 + (lane & 15);
  if (sl < nsl) {
    const int t = lane & 15, q = lane >> 4;
    const bool tv = t < tok, jv = j < a.r;
    const float* prow = s_p + (tv ? t : 0) * G;
    const int64_t aro = static_cast<int64_t>(jv ? j : 0) * G;
    const int nblk = static_cast<int>((G + 15) >> 4);
    const int b0 = sl * nblk / nsl, b1 = (sl + 1) * nblk / nsl;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int b = b0; b < b1; ++b) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t g = b * 16 + 4 * e + q;
        const bool gv = g < G;
        const int64_t gc = gv ? g : G - 1;
        const float pv = prow[gc];
        const uint16_t ab = a.stage_a ? s_A[aro + gc] : a.A[aro + gc];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tv && gv ? pv : 0.0f, jv && gv ? bf16_to_f32(ab) : 0.0f,
                                                   acc, 0, 0, 0);
      }
    }
    // lane holds rows 4 q + v of column j
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tt = 4 * q + v;
      if (tt < tok && jv) s_red[(sl * tok + tt) * rp + j] = acc[v];
    }
  }
  __syncthreads();
  for (int i = tid; i < tok * a.r; i += kQaThreads) {
    const int tt = i / a.r, jj = i - tt * a.r;
    float sum = s_red[tt * rp + jj];
    for (int k = 1; k < nsl; ++k) sum += s_red[(k * tok + tt) * rp + jj];
    if (m0 + tt < a.M) a.u_out[(m0 + tt) * a.r + jj] = sum;
  }
}

// P alone (the backward pass, which has u): the same sums as above, the
// token rows taken as one flat run of 16-byte pieces (four to a group), 8
// pieces of each thread in flight.
constexpr int kQaPoolPer = 8;
__global__ __launch_bounds__(256) void k_qa_pool(const uint16_t* __restrict__ x, float* __restrict__ P,
                                                 int64_t total) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (256 * kQaPoolPer);
  u32x4 w[kQaPoolPer];
#pragma unroll
  for (int i = 0; i < kQaPoolPer; ++i) {
    const int64_t pf = base + i * 256 + tid;
    w[i] = *reinterpret_cast<const u32x4*>(x + (pf < total ? pf : total - 1) * 8);
  }
#pragma unroll
  for (int i = 0; i < kQaPoolPer; ++i) {
    float v = bf16_lo(w[i].x);
    v += bf16_hi(w[i].x);
    v += bf16_lo(w[i].y);
    v += bf16_hi(w[i].y);
    v += bf16_lo(w[i].z);
    v += bf16_hi(w[i].z);
    v += bf16_lo(w[i].w);
    v += bf16_hi(w[i].w);
    const float v1 = __shfl_xor(v, 1, 64);
    const float q1 = (lane & 1) ? v1 + v : v + v1;
    const float q2 = __shfl_xor(q1, 2, 64);
    const float q = (lane & 2) ? q2 + q1 : q1 + q2;
    const int64_t pf = base + i * 256 + tid;
    if ((lane & 3) == 0 && pf < total) P[pf >> 2] = q;
  }
}

// Partial dA over one slice of tokens: workgroup (group tile, adapter-row
// tile, slice) adds du[m][j] P[m][g] over the slice's tokens in increasing m
// into part[slice][j][g].  The operands of 32 tokens at a time are staged
// in LDS; each thread owns a 4 x 4 block of the 64 x 64 tile.
__global__ __launch_bounds__(256) void k_qa_dA_part(QaArgs a) {
  __shared__ __attribute__((aligned(16))) float s_du[kQaDaBlk][kQaDaTile];
  __shared__ __attribute__((aligned(16))) float s_pp[kQaDaBlk][kQaDaTile];
  const int tid = threadIdx.x;
  const int64_t G = a.G;
  const int r = a.r;
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * kQaDaTile;
  const int j0 = static_cast<int>(blockIdx.y) * kQaDaTile;
  const int slice = static_cast<int>(blockIdx.z);
  const int64_t per = (a.M + a.splits - 1) / a.splits;
  const int64_t mb0 = slice * per;
  const int64_t mb1 = mb0 + per < a.M ? mb0 + per : a.M;
  const int tj = tid >> 4, tg = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[i][k] = 0.0f;
  for (int64_t mb = mb0; mb < mb1; mb += kQaDaBlk) {
#pragma unroll
    for (int e = 0; e < (kQaDaBlk * kQaDaTile) / 256; ++e) {
      const int idx = e * 256 + tid;
      const int mm = idx / kQaDaTile, cc = idx % kQaDaTile;
      const int64_t m = mb + mm;
      const bool mok = m < mb1;
      s_du[mm][cc] = mok && j0 + cc < r ? a.du[m * r + j0 + cc] : 0.0f;
      s_pp[mm][cc] = mok && g0 + cc < G ? a.P_in[m * G + g0 + cc] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int mm = 0; mm < kQaDaBlk; ++mm) {
      const f32x4 d = *reinterpret_cast<const f32x4*>(&s_du[mm][tj * 4]);
      const f32x4 p = *reinterpret_cast<const f32x4*>(&s_pp[mm][tg * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] += d[i] * p[k];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = j0 + tj * 4 + i;
    if (j >= r) continue;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t g = g0 + tg * 4 + k;
      if (g < G) a.part[(static_cast<int64_t>(slice) * r + j) * G + g] = acc[i][k];
    }
  }
}

// dA[j][g] = the slices' partial sums, added in a fixed order: four
// neighbouring lanes each add a quarter of the slices in slice order (loads
// issued eight at a time), then the quarters are added pairwise in lane
// order.
__global__ __launch_bounds__(256) void k_qa_dA_sum(QaArgs a) {
  const int64_t n = static_cast<int64_t>(a.r) * a.G;
  const int lane = threadIdx.x & 63, qq = threadIdx.x & 3;
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 2;
  const int64_t e = e0 < n ? e0 : n - 1;
  const int per = (a.splits + 3) / 4;
  const int s0 = qq * per;
  const int s1 = s0 + per < a.splits ? s0 + per : a.splits;
  float v = 0.0f;
  for (int sp = s0; sp < s1; sp += 8) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = sp + i < s1 ? a.part[(sp + i) * n + e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (sp + i < s1) v += t[i];
  }
  const float v1 = __shfl_xor(v, 1, 64);
  const float p = (lane & 1) ? v1 + v : v + v1;
  const float p2 = __shfl_xor(p, 2, 64);
  const float q = (lane & 2) ? p2 + p : p + p2;
  if (qq == 0 && e0 < n) a.dA_out[e0] = f32_to_bf16(q);
}

// Tokens per workgroup of the pooling kernel: the P block of all its tokens
// sits in LDS (at most 64 KB).
int qa_tokens(int64_t G) {
  const int64_t t = 16384 / G;
  return static_cast<int>(t < 1 ? 1 : (t > kQaTokMax ? kQaTokMax : t));
}

}  // namespace

int qa_dA_splits(int64_t M) {
  const int64_t s = (M + kQaDaBlk - 1) / kQaDaBlk;
  return static_cast<int>(s < 1 ? 1 : (s > 64 ? 64 : s));
}
int64_t qa_dA_partial_floats(int64_t M, int32_t r, int64_t G) {
  return static_cast<int64_t>(qa_dA_splits(M)) * r * G;
}

hipError_t launch_qa_pool_u(const QaArgs& in, hipStream_t stream) {
  if (in.pool != kQaPool || in.K % kQaPool != 0) return hipErrorInvalidValue;
  QaArgs a = in;
  if (a.u_out == nullptr) {
    if (a.P_out == nullptr) return hipErrorInvalidValue;
    const int64_t total = a.M * a.K / 8;
    if (total == 0) return hipSuccess;
    const int64_t per = 256 * kQaPoolPer;
    hipLaunchKernelGGL(k_qa_pool, dim3(static_cast<uint32_t>((total + per - 1) / per)), dim3(256), 0, stream,
                       a.x, a.P_out, total);
    return hipGetLastError();
  }
  if (a.r < 1 || a.r > kQaMaxRank) return hipErrorInvalidValue;
  a.tok = qa_tokens(a.G);
  const int jt = (a.r + 15) / 16;
  size_t lds = static_cast<size_t>(a.tok) * a.G * sizeof(float) +
               static_cast<size_t>(16 / jt) * a.tok * jt * 16 * sizeof(float);
  if (lds > 65536) return hipErrorInvalidValue;
  const size_t a_bytes = static_cast<size_t>(a.r) * a.G * sizeof(uint16_t);
  a.stage_a = a.u_out != nullptr && a.G % 8 == 0 && lds + a_bytes <= 65536;
  if (a.stage_a) lds += a_bytes;
  const uint32_t grid = static_cast<uint32_t>((a.M + a.tok - 1) / a.tok);
  hipLaunchKernelGGL(k_qa_pool_u, dim3(grid), dim3(kQaThreads), static_cast<uint32_t>(lds), stream, a);
  return hipGetLastError();
}

hipError_t launch_qa_dA(const QaArgs& in, hipStream_t stream) {
  QaArgs a = in;
  a.splits = qa_dA_splits(a.M);
  dim3 grid(static_cast<uint32_t>((a.G + kQaDaTile - 1) / kQaDaTile),
            static_cast<uint32_t>((a.r + kQaDaTile - 1) / kQaDaTile), static_cast<uint32_t>(a.splits));
  hipLaunchKernelGGL(k_qa_dA_part, grid, dim3(256), 0, stream, a);
  const int64_t n = static_cast<int64_t>(a.r) * a.G;
  hipLaunchKernelGGL(k_qa_dA_sum, dim3(static_cast<uint32_t>((4 * n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
