// Host-visible launchers of the library's HIP kernels and their argument
// blocks.  Only the C ABI layer (api.cpp) calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace qlin {

// ---------------------------------------------------------------- quantizers
hipError_t launch_quant_nf4(const float* W, int64_t n_blocks, int dq, const double* mids15,
                            uint8_t* codes, void* absmax, float* absmax2, hipStream_t stream);
hipError_t launch_quant_int4(const float* W, int64_t n_groups, uint8_t* codes, uint16_t* scale,
                             uint16_t* zero, hipStream_t stream);
hipError_t launch_dequant(const WeightView& w, int fmt, uint16_t* out, hipStream_t stream);

// ------------------------------------------------------------ adapter ops
struct NtArgs {  // C[m][j] = alpha * sum_k X[m][k] Y[j][k]
  const uint16_t* X;  int64_t ldx;
  const uint16_t* Y;  int64_t ldy;
  float* C;           int64_t ldc;
  int64_t M, K;       // K % 16 == 0
  int32_t J;          // <= 128
  int32_t splits;
  float alpha;
  float* partial;     // nt_partial_floats(M, splits)
  uint32_t* counters; // nt_tiles(M)
};
hipError_t launch_nt_skinny(const NtArgs& a, hipStream_t stream);
int nt_tiles(int64_t M);
int64_t nt_partial_floats(int64_t M, int splits);

struct Tn2Args {  // C[p][j] (or C[j][p]) = alpha * sum_m X[m][p] Z[m][j], Z as bf16 hi/lo planes
  const uint16_t* X;  int64_t ldx;
  const uint16_t* Zh; const uint16_t* Zl;  // [M][tn2_jp(J)]
  uint16_t* C;        int64_t ldc;
  int64_t M, P;
  int32_t J;          // <= 128
  int32_t splits;     // token shares
  int32_t out_transposed;
  float alpha;
  float* partial;     // tn2_partial_floats(P, J, splits)
  uint32_t* counters; // tn2_tiles(P)
};
int tn2_jp(int J);
int tn2_tiles(int64_t P);
int64_t tn2_partial_floats(int64_t P, int J, int splits);
hipError_t launch_split_hl(const float* Z, int64_t M, int J, int64_t ldz, uint16_t* Zh,
                           uint16_t* Zl, hipStream_t stream);
hipError_t launch_tn2(const Tn2Args& a, hipStream_t stream);

hipError_t launch_transpose16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                              hipStream_t stream);

struct QaArgs {  // pooled-adapter helpers (QA-LoRA)
  const uint16_t* x;  // [M][K]
  const uint16_t* A;  // [r][G]
  const float* du;    // [M][r]
  const float* P_in;  // [M][G]
  float* P_out;       // [M][G]
  float* u_out;       // [M][r]
  uint16_t* dA_out;   // [r][G]
  float* part;        // dA partial sums [splits][r][G]
  int64_t M, K, G;
  int32_t r, pool;
  int32_t splits, tok, stage_a;  // set by the launchers
};
hipError_t launch_qa_pool_u(const QaArgs& a, hipStream_t stream);
int qa_dA_splits(int64_t M);
int64_t qa_dA_partial_floats(int64_t M, int32_t r, int64_t G);
hipError_t launch_qa_dA(const QaArgs& a, hipStream_t stream);

// ------------------------------------------------- fused 4-bit GEMM kernels
// y[M][N] = x W_bf16^T + (s u) B^T, large M (MFMA tiles of 256 x 256).
struct FwdArgs {
  WeightView w;
  const uint16_t* x;   // [M][K]
  int64_t M;
  const uint16_t* B;   // [N][r] adapter
  const float* u;      // [M][r] fp32, or nullptr (no adapter term)
  int32_t r;
  float s;
  uint16_t* y;         // [M][N]
  int32_t splits;      // split of the K loop across workgroups (>= 1)
  float* partial;      // fwd_gemm_partial_floats
  uint32_t* counters;  // fwd_gemm_tiles
};
hipError_t launch_fwd_gemm(const FwdArgs& a, int fmt, hipStream_t stream);
int fwd_gemm_tiles(int64_t M, int64_t N);
int64_t fwd_gemm_partial_floats(int64_t M, int64_t N, int splits);

// dX[M][K] = dY W_bf16 + du A (A repeated over the groups of a pooled adapter), large M.
struct DxArgs {
  WeightView w;
  const uint16_t* dy;  // [M][N]
  int64_t M;
  const uint16_t* At;  // [K >> pool_shift][r] (A transposed) or nullptr
  const float* du;     // [M][r] or nullptr
  int32_t r;
  int32_t pool;        // power of two
  int32_t pool_shift;  // log2(pool)
  uint16_t* dx;        // [M][K]
};
hipError_t launch_dx_gemm(const DxArgs& a, int fmt, hipStream_t stream);

// Few-token (M <= 16) weight-streaming kernels, one launch per pass; the
// adapter terms are folded into the split reductions.
struct GemvFwdArgs {
  WeightView w;
  const uint16_t* x;   // [M][K]
  int64_t M;           // 1..16
  const uint16_t* A;   // [r][K/pool]
  const uint16_t* B;   // [N][r]
  int32_t r;
  float s;
  int32_t adapter;     // 1: add s u B^T
  int32_t fuse_u;      // 1: form u = x A^T here (plain adapter, r <= 16)
  const float* u_in;   // [M][r] when the adapter is on and u is not formed here
  uint16_t* y;         // [M][N]
  float* u_out;        // [M][r] or nullptr (written when fuse_u)
  int32_t splits;      // gemv_fwd_splits(K)
  int64_t kshare;      // gemv_fwd_kshare(K)
  float* partial;      // gemv_fwd_partial_floats (splits > 1)
  uint32_t* counters;  // gemv_fwd_tiles
};
hipError_t launch_gemv_fwd(const GemvFwdArgs& a, int fmt, hipStream_t stream);
int gemv_fwd_splits(int64_t K);
int gemv_fwd_tiles(int64_t N);
int64_t gemv_fwd_kshare(int64_t K);
int64_t gemv_fwd_partial_floats(int64_t N, int64_t K);

struct GemvDxArgs {
  WeightView w;
  const uint16_t* x;   // [M][K]
  const uint16_t* dy;  // [M][N]
  int64_t M;           // 1..16
  const uint16_t* A;   // [r][K/pool]
  const uint16_t* B;   // [N][r]
  const float* u;      // [M][r]
  int32_t r, pool, pool_shift;
  float s;
  uint16_t* dx;        // [M][K] or nullptr
  uint16_t* dA;        // [r][K/pool]
  uint16_t* dB;        // [N][r]
  int32_t splits;      // N split
  float* partial;      // gemv_dx_partial_floats
  float* du_part;      // gemv_dx_dupart_floats
  uint32_t* counters;  // gemv_dx_tiles
};
hipError_t launch_gemv_dx(const GemvDxArgs& a, int fmt, hipStream_t stream);
int gemv_dx_splits(int64_t N);
int gemv_dx_tiles(int64_t K);
int64_t gemv_dx_partial_floats(int64_t N, int64_t K);
int64_t gemv_dx_dupart_floats(int64_t N, int64_t K, int r);

}  // namespace qlin
