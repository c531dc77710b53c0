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
// Everything runs in fp32 on the device: one tiled GEMM kernel with strided
// operands (split over the reduction with a fixed-order second pass) serves
// every product; a one-workgroup kernel factors the r x r Gram matrix in
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
// A[m * sam + k * sak], B(n, k) at B[n * sbn + k * sbk].  64 x 64 tiles,
// 16 k per step, 256 threads of 4 x 4 outputs.  With splits > 1, split z
// writes its sum over its share of k to P[z][m][n] and k_lq_reduce finishes.
constexpr int kGt = 64, kGk = 16;

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

__global__ __launch_bounds__(256) void k_lq_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) float As[kGk][kGt + 4];
  __shared__ __attribute__((aligned(16))) float Bs[kGk][kGt + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kGt, n0 = static_cast<int64_t>(blockIdx.x) * kGt;
  const int z = blockIdx.z;
  const int64_t kper = (a.K + a.splits - 1) / a.splits;
  const int64_t k0 = z * kper, k1 = k0 + kper < a.K ? k0 + kper : a.K;
  float acc[4][4] = {};
  // tile loads: 1024 elements of each operand, four per thread, along
  // whichever index is contiguous in memory
  auto load_tile = [&](const float* X, int64_t sx, int64_t sk, int64_t x0, int64_t xn, int64_t kb,
                       float (&T)[kGk][kGt + 4]) {
    float v[4];
    if (sk == 1) {
      const int xi = tid >> 2, kk = (tid & 3) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t x = x0 + xi, k = kb + kk + e;
        v[e] = (x < xn && k < k1) ? X[x * sx + k] : 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) T[kk + e][xi] = v[e];
    } else {
      const int kk = tid >> 4, xi = (tid & 15) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t x = x0 + xi + e, k = kb + kk;
        v[e] = (x < xn && k < k1) ? X[x * sx + k * sk] : 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) T[kk][xi + e] = v[e];
    }
  };
  for (int64_t kb = k0; kb < k1; kb += kGk) {
    load_tile(a.A, a.sam, a.sak, m0, a.M, kb, As);
    load_tile(a.B, a.sbn, a.sbk, n0, a.N, kb, Bs);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGk; ++kk) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(&As[kk][ty * 4]);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(&Bs[kk][tx * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n >= a.N) continue;
      if (a.splits > 1) {
        a.P[(z * a.M + m) * a.N + n] = acc[i][j];
      } else {
        float v = a.alpha * acc[i][j];
        if (a.Cin != nullptr) v = __builtin_fmaf(a.beta, a.Cin[m * a.ldci + n], v);
        a.C[m * a.ldc + n] = v;
      }
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
// diagonal: right-looking fp64 Cholesky in LDS, U written out as fp32.  A
// pivot that is not positive (a rank-deficient start) becomes 1 with a zero
// row, which keeps the result finite.
constexpr int kLqMaxR = 128;

__global__ __launch_bounds__(256) void k_lq_chol(const float* __restrict__ G, int r, float* __restrict__ U) {
  __shared__ double s_a[kLqMaxR * (kLqMaxR + 1)];  // r x r, row stride r + 1
  __shared__ double s_piv;
  const int tid = threadIdx.x;
  const int ld = r + 1;
  for (int i = tid; i < r * r; i += 256) s_a[(i / r) * ld + i % r] = static_cast<double>(G[i]);
  __syncthreads();
  for (int j = 0; j < r; ++j) {
    if (tid == 0) {
      const double d = s_a[j * ld + j];
      s_piv = (d > 0.0 && std::isfinite(d)) ? std::sqrt(d) : 0.0;
      s_a[j * ld + j] = s_piv > 0.0 ? s_piv : 1.0;
    }
    __syncthreads();
    const double piv = s_piv;
    for (int c = j + 1 + tid; c < r; c += 256) s_a[j * ld + c] = piv > 0.0 ? s_a[j * ld + c] / piv : 0.0;
    __syncthreads();
    // trailing update of the upper triangle: a[i][c] -= u[j][i] u[j][c]
    for (int i = j + 1 + (tid >> 5); i < r; i += 8) {
      const double uji = s_a[j * ld + i];
      for (int c = i + (tid & 31); c < r; c += 32) s_a[i * ld + c] -= uji * s_a[j * ld + c];
    }
    __syncthreads();
  }
  for (int i = tid; i < r * r; i += 256) {
    const int row = i / r, col = i % r;
    U[i] = row <= col ? static_cast<float>(s_a[row * ld + col]) : 0.0f;
  }
}

// X (r x L) <- its thin-QR Q factor given U: column l of X is solved from
// U^T q = x by forward substitution, one column per thread, in an LDS tile.
constexpr int kTrCols = 64;

__global__ __launch_bounds__(kTrCols) void k_lq_trsm(const float* __restrict__ U, int r, int64_t L,
                                                      float* __restrict__ X) {
  __shared__ float s_u[kLqMaxR * kLqMaxR];
  __shared__ float s_x[kLqMaxR][kTrCols];
  const int tid = threadIdx.x;
  const int64_t l = static_cast<int64_t>(blockIdx.x) * kTrCols + tid;
  for (int i = tid; i < r * r; i += kTrCols) s_u[i] = U[i];
  for (int i = 0; i < r; ++i) s_x[i][tid] = l < L ? X[i * L + l] : 0.0f;
  __syncthreads();
  for (int i = 0; i < r; ++i) {
    float v = s_x[i][tid];
    for (int k = 0; k < i; ++k) v = __builtin_fmaf(-s_u[k * r + i], s_x[k][tid], v);
    s_x[i][tid] = v / s_u[i * r + i];
  }
  if (l < L)
    for (int i = 0; i < r; ++i) X[i * L + l] = s_x[i][tid];
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
  const int64_t tiles = ((M + kGt - 1) / kGt) * ((N + kGt - 1) / kGt);
  if (tiles < 1) return 1;  // an empty product (rank 0) is never launched
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t cap = (K + 255) / 256;  // at least 256 of the reduction per split
  if (s > cap) s = cap;
  return s < 1 ? 1 : (s > 256 ? 256 : s);
}

hipError_t gemm(GemmArgs a, float* scratch, hipStream_t st) {
  a.splits = static_cast<int32_t>(lq_splits(a.M, a.N, a.K));
  a.P = scratch;
  const dim3 grid(static_cast<uint32_t>((a.N + kGt - 1) / kGt), static_cast<uint32_t>((a.M + kGt - 1) / kGt),
                  static_cast<uint32_t>(a.splits));
  hipLaunchKernelGGL(k_lq_gemm, grid, dim3(256), 0, st, a);
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
// twice the Gram matrix, its Cholesky factor U, and X <- X U^{-1} as
// triangular solves).
hipError_t lq_orth(float* X, int64_t L, int r, LqScratch s, hipStream_t st) {
  for (int pass = 0; pass < 2; ++pass) {
    GemmArgs g{};
    g.A = X; g.sam = L; g.sak = 1; g.B = X; g.sbn = L; g.sbk = 1;
    g.C = s.G; g.ldc = r; g.alpha = 1.0f; g.M = r; g.N = r; g.K = L;
    hipError_t e = gemm(g, s.P, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_lq_chol, dim3(1), dim3(256), 0, st, s.G, r, s.Uinv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_lq_trsm, dim3(static_cast<uint32_t>((L + kTrCols - 1) / kTrCols)), dim3(kTrCols), 0, st,
                       s.Uinv, r, L, X);
    if ((e = hipGetLastError()) != hipSuccess) return e;
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
