// Low-rank plus quantized decomposition W ~ Q + L of an fp32 weight, with Q
// an NF4 weight and L = U C of rank r.  [LQ-LoRA abstract: each pretrained
// matrix is decomposed iteratively into a high-precision low-rank component
// and a quantized component]
//
// L starts at zero.  Each iteration quantizes D = W - U C with the NF4
// quantizer, forms the residual R = W - W_bf16(Q) against the weight the
// layer computes with, and replaces (U, C) by the rank-r part of R: subspace
// iteration from a caller-drawn start, orthonormalised by CholeskyQR2 (the
// thin QR with a positive diagonal, which is unique), then C = U^T R.
//
// Everything runs in fp32 on the device: one GEMM kernel on the fp32 matrix
// cores, with strided operands (split over the reduction with a fixed-order
// second pass), serves every product; a one-workgroup kernel factors the r x r Gram matrix in
// fp64, and the orthonormal factor follows by triangular solves (a column of
// the tall matrix per thread).  U is kept transposed (r x N) and C as
// r x K, so that both tall factors are r rows of contiguous data.
#include <algorithm>
#include <cmath>

#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

// ------------------------------------------------------------------ GEMM
// C[m][n] = alpha sum_k A(m, k) B(n, k) + beta Cin[m][n], A(m, k) at
// A[m * sam + k * sak], B(n, k) at B[n * sbn + k * sbk]; each operand has a
// contiguous index (k, or m / n: stride 1), every other stride and the
// contiguous extent are multiples of 4 floats, and the bases are 16-byte
// aligned (the host checks).  On the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32: fp32 products and sums): 64 x 256 output tiles,
// four waves of 64 x 64, 32 k per chunk.  A chunk of each operand is
// staged in LDS in its memory order ([x][k] when k is contiguous, [k][x]
// otherwise; rows padded against bank conflicts) from registers loaded one
// chunk ahead.  MFMA s of a chunk sums k = s (lanes 0-31) and k = 16 + s
// (lanes 32-63), so that a lane reads 16 consecutive k of a [x][k] row.
// Rows, columns and k past the ranges are zero.  With splits > 1, split z
// writes its sum over its share of k to P[z][m][n] and k_lq_reduce
// finishes.
constexpr int kMt = 64, kNt = 128, kKc = 32;

struct GemmArgs {
  const float* A; int64_t sam, sak;
  const float* B; int64_t sbn, sbk;
  float* C; int64_t ldc;
  const float* Cin; int64_t ldci;  // beta term (nullptr: none)
  float alpha, beta;
  int64_t M, N, K;
  int32_t splits;
  float* P;                         // [splits][M][N] when splits > 1
};

// LDS row strides (floats): [x][k] rows of 32 k, [k][x] rows of TX x
constexpr int kXkStride = kKc + 4;
template <int TX>
constexpr int kx_stride() { return TX + 2; }
template <bool KC, int TX>
constexpr int stage_floats() { return KC ? TX * kXkStride : kKc * kx_stride<TX>(); }
constexpr int kOutStride = kNt + 8;  // output staging rows: the two lane halves hit disjoint banks

// One operand's chunk: TX rows x (m or n) from x0, 32 k from kb, limited
// to x < xn and k < k1.  Thread t holds pieces t + 256 i (4 floats each).
template <bool KC, int TX>
struct Chunk {
  static constexpr int kPieces = TX * kKc / 4 / 256;
  f32x4 v[kPieces];
  __device__ __forceinline__ void load(const float* X, int64_t sx, int64_t sk, int64_t x0, int64_t xn, int64_t kb,
                                       int64_t k1, int tid) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int p = tid + 256 * i;
      if constexpr (KC) {  // row x = p / 8, k = 4 (p % 8) .. +3
        const int64_t x = x0 + p / 8, k = kb + 4 * (p % 8);
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        if (x < xn && k < k1) t = *reinterpret_cast<const f32x4*>(X + x * sx + k);
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = k + e < k1 ? t[e] : 0.0f;
        v[i] = t;
      } else {  // k row p / (TX / 4), x = 4 (p % (TX / 4)) .. +3
        const int64_t k = kb + p / (TX / 4), x = x0 + 4 * (p % (TX / 4));
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        if (k < k1 && x < xn) t = *reinterpret_cast<const f32x4*>(X + k * sk + x);
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = x + e < xn ? t[e] : 0.0f;
        v[i] = t;
      }
    }
  }
  __device__ __forceinline__ void store(float* T, int tid) const {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int p = tid + 256 * i;
      float* d = KC ? T + (p / 8) * kXkStride + 4 * (p % 8) : T + (p / (TX / 4)) * kx_stride<TX>() + 4 * (p % (TX / 4));
      if constexpr (KC) {
        *reinterpret_cast<f32x4*>(d) = v[i];
      } else {  // rows of TX + 2 floats: 8-byte aligned pieces
        *reinterpret_cast<f32x2*>(d) = f32x2{v[i][0], v[i][1]};
        *reinterpret_cast<f32x2*>(d + 2) = f32x2{v[i][2], v[i][3]};
      }
    }
  }
};

// The 16 values of a lane for one 32-row fragment (rows xb .. xb + 31 of
// the stage; lane half h covers k = 16 h .. 16 h + 15)
template <bool KC, int TX>
__device__ __forceinline__ void read_frag(const float* T, int xb, int l32, int h, float (&f)[16]) {
  if constexpr (KC) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(T + (xb + l32) * kXkStride + 16 * h + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) f[4 * q + e] = t[e];
    }
  } else {
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) f[s2] = T[(16 * h + s2) * kx_stride<TX>() + xb + l32];
  }
}

// Two workgroups per compute unit (two waves per SIMD): while one waits
// for its loads or at its barrier, the other's products run.  Operands are
// loaded into registers two chunks ahead (two register sets, the chunk loop
// unrolled by two).
template <bool AKC, bool BKC>
__global__ __launch_bounds__(256, 2) void k_lq_mm(GemmArgs a) {
  constexpr int kAS = stage_floats<AKC, kMt>();
  // (the B stages also hold the output tile after the loop)
  constexpr int kBS = stage_floats<BKC, kNt>() > kMt * kOutStride / 2 ? stage_floats<BKC, kNt>() : kMt * kOutStride / 2;
  __shared__ __attribute__((aligned(16))) float s_a[2][kAS];
  __shared__ __attribute__((aligned(16))) float s_b[2][kBS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kMt, n0 = static_cast<int64_t>(blockIdx.x) * kNt;
  const int z = blockIdx.z;
  // whole chunks per split, so that every k-contiguous load is 16-byte aligned
  const int64_t kper = ((a.K + a.splits - 1) / a.splits + kKc - 1) / kKc * kKc;
  const int64_t k0 = z * kper < a.K ? z * kper : a.K;
  const int64_t k1 = k0 + kper < a.K ? k0 + kper : a.K;
  const int64_t nch = (k1 - k0 + kKc - 1) / kKc;

  f32x16 acc[2] = {f32x16{}, f32x16{}};  // rows 32 i .. +31, columns 32 wave .. +31
  Chunk<AKC, kMt> ca[2];
  Chunk<BKC, kNt> cb[2];
  auto load = [&](int64_t c, int set) {
    const int64_t kb = k0 + c * kKc;
    ca[set].load(a.A, AKC ? a.sam : 1, AKC ? 1 : a.sak, m0, a.M, kb, k1, tid);
    cb[set].load(a.B, BKC ? a.sbn : 1, BKC ? 1 : a.sbk, n0, a.N, kb, k1, tid);
  };
  // chunk c: LDS stage c & 1; before that, register set c & 1
  if (nch > 0) load(0, 0);
  if (nch > 1) load(1, 1);
  if (nch > 0) {
    ca[0].store(s_a[0], tid);
    cb[0].store(s_b[0], tid);
  }
  __syncthreads();
  auto chunk = [&](int64_t c, auto set_c) __attribute__((always_inline)) {
    constexpr int S = decltype(set_c)::value;  // c & 1
    if (c + 2 < nch) load(c + 2, S);           // set S held chunk c, already in LDS
    float fa[2][16], fb[16];
#pragma unroll
    for (int i = 0; i < 2; ++i) read_frag<AKC, kMt>(s_a[S], 32 * i, l32, h, fa[i]);
    read_frag<BKC, kNt>(s_b[S], 32 * wave, l32, h, fb);
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2)
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][s2], fb[s2], acc[i], 0, 0, 0);
    if (c + 1 < nch) {
      ca[S ^ 1].store(s_a[S ^ 1], tid);
      cb[S ^ 1].store(s_b[S ^ 1], tid);
    }
    __syncthreads();
  };
  for (int64_t c = 0; c < nch; c += 2) {
    chunk(c, std::integral_constant<int, 0>{});
    if (c + 1 < nch) chunk(c + 1, std::integral_constant<int, 1>{});
  }

  // output: the tile goes through LDS ([64 m][kOutStride], in the B stages)
  // and leaves as 16-byte pieces of rows (32 threads per 128-float row)
  float* const s_o = &s_b[0][0];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      s_o[(32 * i + 8 * (v >> 2) + 4 * h + (v & 3)) * kOutStride + 32 * wave + l32] = acc[i][v];
  __syncthreads();
  const int c4 = 4 * (tid & 31);
  const int64_t n = n0 + c4;
  float* const out = a.splits > 1 ? a.P + static_cast<int64_t>(z) * a.M * a.N : a.C;
  const int64_t ldo = a.splits > 1 ? a.N : a.ldc;
  const bool vec = (ldo & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0 &&
                   (a.splits > 1 || a.Cin == nullptr || ((a.ldci & 3) == 0 && (reinterpret_cast<uintptr_t>(a.Cin) & 15) == 0));
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = q * 8 + (tid >> 5);
    const int64_t m = m0 + row;
    if (m >= a.M || n >= a.N) continue;
    f32x4 y = *reinterpret_cast<const f32x4*>(&s_o[row * kOutStride + c4]);
    if (a.splits == 1) {
      y *= a.alpha;
      if (a.Cin != nullptr) {
        const float* ci = a.Cin + m * a.ldci + n;
        if (vec && n + 3 < a.N) {
          const f32x4 t = *reinterpret_cast<const f32x4*>(ci);
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(a.beta, t[e], y[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < a.N) y[e] = __builtin_fmaf(a.beta, ci[e], y[e]);
        }
      }
    }
    float* o = out + m * ldo + n;
    if (vec && n + 3 < a.N) {
      *reinterpret_cast<f32x4*>(o) = y;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < a.N) o[e] = y[e];
    }
  }
}

// Split sums in split order, then the alpha / beta epilogue.
__global__ __launch_bounds__(256) void k_lq_reduce(GemmArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= a.M * a.N) return;
  const int64_t m = i / a.N, n = i % a.N;
  float s = 0.0f;
  for (int z = 0; z < a.splits; ++z) s += a.P[z * a.M * a.N + i];
  float v = a.alpha * s;
  if (a.Cin != nullptr) v = __builtin_fmaf(a.beta, a.Cin[m * a.ldci + n], v);
  a.C[m * a.ldc + n] = v;
}

// --------------------------------------------------- residual and norms
// R = W - W_bf16(Q) for an NF4 weight (codes [N][K/2], 64-element blocks,
// optional double quantization); thread = 8 elements (one dword of codes).
// The workgroup's sum of squares of R goes to part[block] (fp64).
__global__ __launch_bounds__(256) void k_lq_resid(const float* __restrict__ W, const uint8_t* __restrict__ codes,
                                                   const void* absmax, const float* absmax2, int32_t dq,
                                                   Codebook cb, int64_t n_el, float* __restrict__ R,
                                                   double* part) {
  __shared__ double s_red[256];
  const int tid = threadIdx.x;
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * 256 + tid) * 8;
  double ss = 0.0;
  if (e0 < n_el) {
    const int64_t b = e0 >> 6;
    float scale;
    if (dq) scale = nf4_dq_scale(static_cast<const int8_t*>(absmax)[b], absmax2[b >> 8]);
    else scale = static_cast<const float*>(absmax)[b];
    const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + e0 / 2);
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(W + e0);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(W + e0 + 4);
    float out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // element j: byte j & 3, low nibble for j < 4, high nibble after
      const uint32_t idx = (w >> (8 * (j & 3) + (j < 4 ? 0 : 4))) & 0xFu;
      const float wb = bf16_to_f32(f32_to_bf16(cb.c[idx] * scale));
      const float xv = j < 4 ? x0[j] : x1[j - 4];
      out[j] = xv - wb;
      ss += static_cast<double>(out[j]) * static_cast<double>(out[j]);
    }
    *reinterpret_cast<f32x4*>(R + e0) = f32x4{out[0], out[1], out[2], out[3]};
    *reinterpret_cast<f32x4*>(R + e0 + 4) = f32x4{out[4], out[5], out[6], out[7]};
  }
  s_red[tid] = ss;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) s_red[tid] += s_red[tid + o];
    __syncthreads();
  }
  if (tid == 0) part[blockIdx.x] = s_red[0];
}

// Sum of squares of x[0 .. n) into part[block] (fp64).
__global__ __launch_bounds__(256) void k_lq_sumsq(const float* __restrict__ x, int64_t n, double* part) {
  __shared__ double s_red[256];
  const int tid = threadIdx.x;
  double ss = 0.0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + tid; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    ss += static_cast<double>(x[i]) * static_cast<double>(x[i]);
  s_red[tid] = ss;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) s_red[tid] += s_red[tid + o];
    __syncthreads();
  }
  if (tid == 0) part[blockIdx.x] = s_red[0];
}

// out = sum of part[0 .. n): thread t adds the t-th contiguous slice in
// order, then the 256 slice sums are added in order (one fixed order).
__global__ __launch_bounds__(256) void k_lq_total(const double* part, int64_t n, double* out) {
  __shared__ double s_red[256];
  const int tid = threadIdx.x;
  const int64_t per = (n + 255) / 256;
  const int64_t i0 = tid * per, i1 = i0 + per < n ? i0 + per : n;
  double s = 0.0;
  for (int64_t i = i0; i < i1; ++i) s += part[i];
  s_red[tid] = s;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int i = 0; i < 256; ++i) t += s_red[i];
    *out = t;
  }
}

// err = sqrt(max(0, |R|^2 - |C|^2)) / |W|: with U orthonormal and C = U^T R,
// |R - U C|^2 = |R|^2 - |C|^2.
__global__ void k_lq_err(const double* rr, const double* cc, const double* ww, float* err) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const double d = *rr - *cc;
  const double w = *ww > 0.0 ? std::sqrt(*ww) : 1.0;
  *err = static_cast<float>(std::sqrt(d > 0.0 ? d : 0.0) / w);
}

// ------------------------------------------------------ small factorisation
// G (r x r, fp32, symmetric) = U^T U with U upper triangular and a positive
// diagonal: right-looking fp64 Cholesky, then U^{-1} written out as fp32.  A
// pivot that is not positive (a rank-deficient start) becomes 1 with a zero
// row, which keeps the result finite.
constexpr int kLqMaxR = 128;

// Cholesky factor U (upper triangular, U^T U = G) of the r x r Gram matrix
// and its inverse, in fp64.  Thread (ti, tc) of a 16 x 16 grid keeps the
// elements (ti + 16 p, tc + 16 q) in registers, so each elimination step
// reads only the published pivot row from LDS (double buffered, one barrier
// per step): right-looking on unscaled rows, a[i][c] -= a[j][i] a[j][c] / d_j,
// then row j of U is a[j][.] / sqrt(d_j).  The inverse X = U^{-1} solves
// U X = I from the last row up, the same way: row i of X is the updated
// row i of B (B = I at the start) over u_ii, published, and every row k < i
// of B loses U[k][i] times it (U read from LDS).  The output is
// Uinv[j][i] = (U^{-1})[j][i] in fp32, row stride ldu (zero below the
// diagonal and in the padding), the left operand of X <- U^{-T} X.  A pivot
// that is not positive and finite (a zero or rank-deficient Gram matrix)
// gives a zero row of U with a unit diagonal, so the matching row of X
// passes through unchanged.
// S: register slots per thread along each dimension (r <= 16 S).
// 1 / d for d > 0: the hardware reciprocal refined by two Newton steps
// (within an ulp or two of the quotient; the divide sequence would sit on the
// serial chain of every elimination step).
__device__ __forceinline__ double recip64(double d) {
  double y = __builtin_amdgcn_rcp(d);
  double e = __builtin_fma(-d, y, 1.0);
  y = __builtin_fma(y, e, y);
  e = __builtin_fma(-d, y, 1.0);
  return __builtin_fma(y, e, y);
}

template <int S>
__global__ __launch_bounds__(256) void k_lq_cholinv(const float* __restrict__ G, int r, float* __restrict__ Uinv,
                                                    int ldu) {
  constexpr int kChS = S;
  __shared__ double s_u[kLqMaxR * (kLqMaxR + 1)];  // U, row stride r + 1 (read-only during the inverse)
  __shared__ double s_row[2][kLqMaxR];              // published pivot row / row of X
  __shared__ double s_piv[kLqMaxR];                 // sqrt of each pivot (0: not positive)
  __shared__ double s_rd[kLqMaxR];                  // 1 / u_ii
  const int tid = threadIdx.x;
  const int ti = tid >> 4, tc = tid & 15;
  const int ld = r + 1;
  double a[kChS][kChS];
#pragma unroll
  for (int p = 0; p < kChS; ++p)
#pragma unroll
    for (int q = 0; q < kChS; ++q) {
      const int i = ti + 16 * p, c = tc + 16 * q;
      a[p][q] = (i < r && c < r && c >= i) ? static_cast<double>(G[i * r + c]) : 0.0;
    }
  // publish row 0 (its owners: ti == 0, slot p == 0)
  if (ti == 0) {
#pragma unroll
    for (int q = 0; q < kChS; ++q)
      if (tc + 16 * q < r) s_row[0][tc + 16 * q] = a[0][q];
  }
  __syncthreads();
  for (int j = 0; j < r; ++j) {
    const double* prow = s_row[j & 1];
    const double d = prow[j];
    const double inv = (d > 0.0 && std::isfinite(d)) ? recip64(d) : 0.0;
    // all of the step's LDS reads first, then a branch-free update (a
    // branch around each slot would wait for its own read in turn)
    double rowc[kChS], rowi[kChS];
#pragma unroll
    for (int q = 0; q < kChS; ++q) rowc[q] = prow[tc + 16 * q];
#pragma unroll
    for (int p = 0; p < kChS; ++p) rowi[p] = prow[ti + 16 * p];
#pragma unroll
    for (int p = 0; p < kChS; ++p) {
      const int i = ti + 16 * p;
      const double t = rowi[p] * inv;
#pragma unroll
      for (int q = 0; q < kChS; ++q) {
        const int c = tc + 16 * q;
        const double v = __builtin_fma(-t, rowc[q], a[p][q]);
        a[p][q] = (i > j && c >= i && c < r) ? v : a[p][q];
      }
    }
    // publish row j + 1, now final (rows are updated only by earlier pivots)
    const int jn = j + 1;
    if (jn < r && ti == (jn & 15)) {
#pragma unroll
      for (int p = 0; p < kChS; ++p)
        if (p == (jn >> 4)) {
#pragma unroll
          for (int q = 0; q < kChS; ++q) {
            const int c = tc + 16 * q;
            if (c >= jn && c < r) s_row[jn & 1][c] = a[p][q];
          }
        }
    }
    __syncthreads();
  }
  // pivots, then U = rows over sqrt(pivot) into LDS (zero below the diagonal)
#pragma unroll
  for (int p = 0; p < kChS; ++p)
#pragma unroll
    for (int q = 0; q < kChS; ++q) {
      const int i = ti + 16 * p, c = tc + 16 * q;
      if (i == c && i < r) {
        const double d = a[p][q];
        const double pv = (d > 0.0 && std::isfinite(d)) ? std::sqrt(d) : 0.0;
        s_piv[i] = pv;
        s_rd[i] = pv > 0.0 ? 1.0 / pv : 1.0;
      }
    }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kChS; ++p)
#pragma unroll
    for (int q = 0; q < kChS; ++q) {
      const int i = ti + 16 * p, c = tc + 16 * q;
      if (i < r && c < r) {
        const double pv = s_piv[i];
        s_u[i * ld + c] = c < i ? 0.0 : c == i ? (pv > 0.0 ? pv : 1.0) : (pv > 0.0 ? a[p][q] / pv : 0.0);
      }
    }
  __syncthreads();
  // inverse: B = I in the registers, rows solved from the last one up
#pragma unroll
  for (int p = 0; p < kChS; ++p)
#pragma unroll
    for (int q = 0; q < kChS; ++q) a[p][q] = (ti + 16 * p == tc + 16 * q) ? 1.0 : 0.0;
  auto solve_row = [&](int i) {  // row i of X from row i of B, by its owners; published
    if (ti == (i & 15)) {
      const double rd = s_rd[i];
#pragma unroll
      for (int p = 0; p < kChS; ++p)
        if (p == (i >> 4)) {
#pragma unroll
          for (int q = 0; q < kChS; ++q) {
            const int c = tc + 16 * q;
            if (c < r) {
              a[p][q] = c >= i ? a[p][q] * rd : 0.0;
              s_row[i & 1][c] = a[p][q];
            }
          }
        }
    }
  };
  solve_row(r - 1);
  __syncthreads();
  for (int i = r - 1; i > 0; --i) {
    const double* xrow = s_row[i & 1];
    double xc[kChS], uki[kChS];
#pragma unroll
    for (int q = 0; q < kChS; ++q) xc[q] = xrow[tc + 16 * q];
#pragma unroll
    for (int p = 0; p < kChS; ++p) uki[p] = s_u[(ti + 16 * p) * ld + i];
#pragma unroll
    for (int p = 0; p < kChS; ++p) {
      const int k = ti + 16 * p;
#pragma unroll
      for (int q = 0; q < kChS; ++q) {
        const int c = tc + 16 * q;
        const double v = __builtin_fma(-uki[p], xc[q], a[p][q]);
        a[p][q] = (k < i && c >= i && c < r) ? v : a[p][q];
      }
    }
    solve_row(i - 1);
    __syncthreads();
  }
  // Uinv[i][c] = X[i][c] for c >= i (zero below the diagonal); padding zero
#pragma unroll
  for (int p = 0; p < kChS; ++p)
#pragma unroll
    for (int q = 0; q < kChS; ++q) {
      const int i = ti + 16 * p, c = tc + 16 * q;
      if (i < r && c < r) Uinv[i * ldu + c] = c >= i ? static_cast<float>(a[p][q]) : 0.0f;
    }
  for (int e = tid; e < r * (ldu - r); e += 256) {
    const int i = e / (ldu - r), c = r + e % (ldu - r);
    Uinv[i * ldu + c] = 0.0f;
  }
}

// bf16 outputs: B[n][j] = Ut[j][n]; A[j][k] = C[j][k].
__global__ __launch_bounds__(256) void k_lq_outputs(const float* __restrict__ Ut, const float* __restrict__ Ct,
                                                     int64_t N, int64_t K, int r, uint16_t* __restrict__ B,
                                                     uint16_t* __restrict__ A) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < N * r) {
    const int64_t n = i / r, j = i % r;
    B[i] = f32_to_bf16(Ut[j * N + n]);
  }
  if (i < static_cast<int64_t>(r) * K) A[i] = f32_to_bf16(Ct[i]);
}

}  // namespace

// ------------------------------------------------------------- host side

namespace {

int64_t lq_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + kMt - 1) / kMt) * ((N + kNt - 1) / kNt);
  if (tiles < 1) return 1;  // an empty product (rank 0) is never launched
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t cap = (K + 255) / 256;  // at least 256 of the reduction per split
  if (s > cap) s = cap;
  return s < 1 ? 1 : (s > 256 ? 256 : s);
}

hipError_t gemm(GemmArgs a, float* scratch, hipStream_t st) {
  a.splits = static_cast<int32_t>(lq_splits(a.M, a.N, a.K));
  a.P = scratch;
  const bool akc = a.sak == 1, bkc = a.sbk == 1;
  // each operand needs a contiguous index, 4-float strides, rows whose
  // contiguous extent rounded up to 4 fits their stride (4-float pieces
  // never leave a row's storage) and 16-byte bases
  const int64_t ao = akc ? a.sam : a.sak, bo = bkc ? a.sbn : a.sbk;
  if ((!akc && a.sam != 1) || (!bkc && a.sbn != 1) || (ao & 3) != 0 || (bo & 3) != 0 ||
      ((akc ? a.K : a.M) + 3) / 4 * 4 > ao || ((bkc ? a.K : a.N) + 3) / 4 * 4 > bo ||
      (reinterpret_cast<uintptr_t>(a.A) & 15) != 0 || (reinterpret_cast<uintptr_t>(a.B) & 15) != 0)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>((a.N + kNt - 1) / kNt), static_cast<uint32_t>((a.M + kMt - 1) / kMt),
                  static_cast<uint32_t>(a.splits));
  if (akc && bkc)
    hipLaunchKernelGGL((k_lq_mm<true, true>), grid, dim3(256), 0, st, a);
  else if (akc)
    hipLaunchKernelGGL((k_lq_mm<true, false>), grid, dim3(256), 0, st, a);
  else if (bkc)
    hipLaunchKernelGGL((k_lq_mm<false, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_lq_mm<false, false>), grid, dim3(256), 0, st, a);
  if (a.splits > 1) {
    const int64_t n = a.M * a.N;
    hipLaunchKernelGGL(k_lq_reduce, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

size_t lq_gemm_scratch_floats(int64_t N, int64_t K, int r) {
  // the largest split-sum buffer of any product below
  const int64_t shapes[][3] = {{r, N, K}, {r, K, N}, {r, r, N}, {r, r, K}, {r, N, r}, {r, K, r}, {N, K, r}};
  int64_t best = 0;
  for (const auto& s : shapes) {
    const int64_t sp = lq_splits(s[0], s[1], s[2]);
    if (sp > 1) best = std::max<int64_t>(best, sp * s[0] * s[1]);
  }
  return static_cast<size_t>(best);
}

// X (r x L, fp32) <- the Q factor of its transpose's thin QR (CholeskyQR2:
// twice the Gram matrix, its Cholesky factor U and X <- U^{-T} X, the last
// as a product with the inverted factor; the first pass writes the scratch
// s.T, the second writes X back).
hipError_t lq_orth(float* X, int64_t L, int r, LqScratch s, hipStream_t st) {
  const int ldu = (r + 3) & ~3;
  float* src = X;
  float* dst = s.T;
  for (int pass = 0; pass < 2; ++pass) {
    GemmArgs g{};
    g.A = src; g.sam = L; g.sak = 1; g.B = src; g.sbn = L; g.sbk = 1;
    g.C = s.G; g.ldc = r; g.alpha = 1.0f; g.M = r; g.N = r; g.K = L;
    hipError_t e = gemm(g, s.P, st);
    if (e != hipSuccess) return e;
    if (r <= 64)
      hipLaunchKernelGGL(k_lq_cholinv<4>, dim3(1), dim3(256), 0, st, s.G, r, s.Uinv, ldu);
    else
      hipLaunchKernelGGL(k_lq_cholinv<8>, dim3(1), dim3(256), 0, st, s.G, r, s.Uinv, ldu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GemmArgs t{};
    t.A = s.Uinv; t.sam = 1; t.sak = ldu; t.B = src; t.sbn = 1; t.sbk = L;
    t.C = dst; t.ldc = L; t.alpha = 1.0f; t.M = r; t.N = L; t.K = r;
    if ((e = gemm(t, s.P, st)) != hipSuccess) return e;
    std::swap(src, dst);
  }
  return hipSuccess;
}

// Ut (r x N) <- orth(R V) with V given as Vt (r x K).
hipError_t lq_range(const float* R, const float* Vt, int64_t N, int64_t K, int r, float* Ut, LqScratch s,
                    hipStream_t st) {
  GemmArgs g{};
  g.A = Vt; g.sam = K; g.sak = 1; g.B = R; g.sbn = K; g.sbk = 1;
  g.C = Ut; g.ldc = N; g.alpha = 1.0f; g.M = r; g.N = N; g.K = K;
  hipError_t e = gemm(g, s.P, st);
  if (e != hipSuccess) return e;
  return lq_orth(Ut, N, r, s, st);
}

// Ct (r x K) <- U^T R with U given as Ut (r x N).
hipError_t lq_coords(const float* R, const float* Ut, int64_t N, int64_t K, int r, float* Ct, LqScratch s,
                     hipStream_t st) {
  GemmArgs g{};
  g.A = Ut; g.sam = N; g.sak = 1; g.B = R; g.sbn = 1; g.sbk = K;
  g.C = Ct; g.ldc = K; g.alpha = 1.0f; g.M = r; g.N = K; g.K = N;
  return gemm(g, s.P, st);
}

// D = W - U C  (U as Ut r x N, C as Ct r x K)
hipError_t lq_subtract(const float* W, const float* Ut, const float* Ct, int64_t N, int64_t K, int r, float* D,
                       LqScratch s, hipStream_t st) {
  GemmArgs g{};
  g.A = Ut; g.sam = 1; g.sak = N; g.B = Ct; g.sbn = 1; g.sbk = K;
  g.C = D; g.ldc = K; g.Cin = W; g.ldci = K; g.alpha = -1.0f; g.beta = 1.0f;
  g.M = N; g.N = K; g.K = r;
  return gemm(g, s.P, st);
}

hipError_t lq_resid(const float* W, const WeightView& w, float* R, LqScratch s, hipStream_t st) {
  const int64_t n_el = w.N * w.K;
  const int64_t blocks = (n_el / 8 + 255) / 256;
  hipLaunchKernelGGL(k_lq_resid, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, W, w.codes, w.absmax,
                     w.absmax2, w.dq, w.cb, n_el, R, s.parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lq_total, dim3(1), dim3(256), 0, st, s.parts, blocks, s.sums + 0);
  return hipGetLastError();
}

hipError_t lq_sumsq(const float* x, int64_t n, double* out, LqScratch s, hipStream_t st) {
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(1024, (n + 255) / 256));
  hipLaunchKernelGGL(k_lq_sumsq, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, x, n, s.parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lq_total, dim3(1), dim3(256), 0, st, s.parts, blocks, out);
  return hipGetLastError();
}

hipError_t lq_err(LqScratch s, float* err, hipStream_t st) {
  hipLaunchKernelGGL(k_lq_err, dim3(1), dim3(64), 0, st, s.sums + 0, s.sums + 1, s.sums + 2, err);
  return hipGetLastError();
}

hipError_t lq_outputs(const float* Ut, const float* Ct, int64_t N, int64_t K, int r, uint16_t* B, uint16_t* A,
                      hipStream_t st) {
  const int64_t n = std::max<int64_t>(N * r, static_cast<int64_t>(r) * K);
  hipLaunchKernelGGL(k_lq_outputs, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, st, Ut, Ct, N, K, r,
                     B, A);
  return hipGetLastError();
}

int64_t lq_resid_parts(int64_t n_el) { return std::max<int64_t>((n_el / 8 + 255) / 256, 1024); }

}  // namespace qlin
