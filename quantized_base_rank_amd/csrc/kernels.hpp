// Host-visible launchers of the library's HIP kernels and their argument
// blocks.  Only the C ABI layer (api.cpp) calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "device_common.hpp"

namespace qlin {

constexpr int kMaxDevices = 64;

// ---------------------------------------------------------------- quantizers
// The quantizers report non-finite input through a per-device flag word
// (quant_flag_ptr, on the current device); callers hold quant_flag_lock()
// from clearing the flag until they have read it back.
std::mutex& quant_flag_lock();
hipError_t quant_flag_ptr(uint32_t** out);
hipError_t launch_quant_nf4(const float* W, int64_t n_blocks, int dq, const double* mids15,
                            uint8_t* codes, void* absmax, float* absmax2, uint32_t* flag,
                            hipStream_t stream);
hipError_t launch_quant_int4(const float* W, int64_t n_groups, uint8_t* codes, uint16_t* scale,
                             uint16_t* zero, uint32_t* flag, hipStream_t stream);
hipError_t launch_dequant(const WeightView& w, int fmt, uint16_t* out, hipStream_t stream);

// Gradients of INT4 group scales and zero points: dscale[n][g] =
// sum_{k in g} q[n][k] dW[n][k], dzero[n][g] = sum_{k in g} dW[n][k],
// dW = dY^T x (fp32 outputs [N][K/32])
struct LoqaArgs {
  const uint8_t* codes;   // [N][K/2], the NF4 / INT4 nibble packing
  const uint16_t* x;      // bf16 [M][K]
  const uint16_t* dy;     // bf16 [M][N]
  float* dscale;
  float* dzero;
  int64_t M, N, K;        // K % 64 == 0, N % 16 == 0
};
hipError_t launch_int4_scale_zero_grad(const LoqaArgs& a, hipStream_t stream);

// NormalFloat-k (bits 2..4, blocks 32..256, bit-plane codes)
struct NfTable {
  float c[16];     // levels (2^bits used)
  double mid[15];  // midpoints of neighbouring levels (2^bits - 1 used)
};
hipError_t launch_quant_nf(const float* W, int64_t n_blocks, int bits, int block, int dq,
                           const NfTable& tb, uint8_t* codes, void* absmax, float* absmax2,
                           uint32_t* flag, hipStream_t stream);
hipError_t launch_dequant_nf(const uint8_t* codes, const void* absmax, const float* absmax2,
                             int64_t n_el, int bits, int block, int dq, const NfTable& tb,
                             uint16_t* out, hipStream_t stream);
// bit planes -> 4-bit indices in the NF4 packing + per-32 fp32 scales split
// into low / high 16-bit planes (the kFmtNFG layout read by the layer)
hipError_t launch_transcode_nf(const uint8_t* codes, const void* absmax, const float* absmax2,
                               int64_t n_el, int bits, int block, int dq, uint8_t* nib,
                               uint16_t* scale_lo, uint16_t* scale_hi, hipStream_t stream);
// zero'[n][g] = RN16(zero[n][g] + s sum_j B[n][j] A[j][g]) (QA-LoRA merge)
hipError_t launch_qa_merge(const uint16_t* zero, const uint16_t* A, const uint16_t* B, int64_t N,
                           int64_t G, int r, float s, uint16_t* out, hipStream_t stream);

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

// Few-token forward for large weights (streamed, K split over workgroups):
// y = x W^T + s u B^T with u given
struct FwdStreamArgs {
  WeightView w;
  const uint16_t* x;   // [M][K], M <= 16
  int64_t M;
  const uint16_t* B;   // [N][r]
  const float* u;      // [M][r] (adapter on)
  int32_t r;
  float s;
  int32_t adapter;
  uint16_t* y;         // [M][N]
  int32_t splits;      // fwd_stream_splits(N, K)
  float* partial;      // fwd_stream_partial_floats(N, K)
  uint32_t* counters;  // fwd_stream_row_groups(N)
};
hipError_t launch_gemv_fwd_stream(const FwdStreamArgs& a, int fmt, hipStream_t stream);
int fwd_stream_row_groups(int64_t N);
int fwd_stream_splits(int64_t N, int64_t K);
int64_t fwd_stream_partial_floats(int64_t N, int64_t K);

// dX = dY W_bf16 + expand(du A) for M <= 16 tokens on a large weight
struct DxStreamArgs {
  WeightView w;
  const uint16_t* dy;   // [M][N], M <= 16
  int64_t M;
  const uint16_t* A;    // [r][K >> pool_shift] (adapter on)
  const float* du;      // [M][r] (adapter on)
  int32_t r, pool_shift;
  int32_t adapter;
  uint16_t* dx;         // [M][K]
  const uint16_t* x;    // [M][K] (dA)
  uint16_t* dA;         // [r][K], or nullptr: dA = du^T x formed per panel (unpooled adapter)
  int32_t splits;       // dx_stream_splits(N, K, fmt)
  float* partial;       // dx_stream_partial_floats(N, K, fmt)
  uint32_t* counters;   // dx_stream_panels(K)
};
hipError_t launch_gemv_dx_stream(const DxStreamArgs& a, int fmt, hipStream_t stream);
int dx_stream_panels(int64_t K);
int dx_stream_splits(int64_t N, int64_t K, int fmt);
int64_t dx_stream_partial_floats(int64_t N, int64_t K, int fmt);
bool dx_stream_fits(int64_t N, int64_t K, int fmt);

// du = s dY B (MFMA on bf16 inputs, fp32 sums, fixed order) and
// dB = s dY^T u (fp32) for M <= 16 tokens
struct AdapterFewArgs {
  const uint16_t* dy;   // [M][N]
  int64_t M, N;
  const uint16_t* B;    // [N][r]
  const float* u;       // [M][r]
  int32_t r;
  float s;
  float* du;            // [M][r]
  uint16_t* dB;         // [N][r]
  int32_t shares;       // adapter_few_shares(N)
  float* partial;       // adapter_few_partial_floats(N)
  uint32_t* counters;   // 1
};
hipError_t launch_du_few(const AdapterFewArgs& a, hipStream_t stream);
int adapter_few_shares(int64_t N);
int64_t adapter_few_partial_floats(int64_t N);

// Low-rank plus quantized decomposition (lq.hip): device scratch and steps
struct LqScratch {
  float* G;       // r x r Gram matrix
  float* Uinv;    // r x roundup(r, 4): inverse of the Gram matrix's Cholesky factor
  float* T;       // r x max(N, K): the first CholeskyQR pass's output
  float* P;       // split sums, lq_gemm_scratch_floats
  double* parts;  // lq_resid_parts(N K) per-workgroup sums
  double* sums;   // [0] |R|^2, [1] |C|^2, [2] |W|^2
};
size_t lq_gemm_scratch_floats(int64_t N, int64_t K, int r);
int64_t lq_resid_parts(int64_t n_el);
hipError_t lq_orth(float* X, int64_t L, int r, LqScratch s, hipStream_t st);
hipError_t lq_range(const float* R, const float* Vt, int64_t N, int64_t K, int r, float* Ut, LqScratch s,
                    hipStream_t st);
hipError_t lq_coords(const float* R, const float* Ut, int64_t N, int64_t K, int r, float* Ct, LqScratch s,
                     hipStream_t st);
hipError_t lq_subtract(const float* W, const float* Ut, const float* Ct, int64_t N, int64_t K, int r, float* D,
                       LqScratch s, hipStream_t st);
hipError_t lq_resid(const float* W, const WeightView& w, float* R, LqScratch s, hipStream_t st);
hipError_t lq_sumsq(const float* x, int64_t n, double* out, LqScratch s, hipStream_t st);
hipError_t lq_err(LqScratch s, float* err, hipStream_t st);
hipError_t lq_outputs(const float* Ut, const float* Ct, int64_t N, int64_t K, int r, uint16_t* B, uint16_t* A,
                      hipStream_t st);

// C[m][j] = alpha sum_k X[m][k] Y[j][k] for M <= 16 rows of X, J <= 128
struct UFewArgs {
  const uint16_t* X;  int64_t ldx;
  const uint16_t* Y;  int64_t ldy;
  float* C;           int64_t ldc;
  int64_t M, K;       // M <= 16, K % 32 == 0
  int32_t J;
  int32_t splits;     // u_few_splits(J, K)
  float alpha;
  float* partial;     // u_few_partial_floats(J, K)
  uint32_t* counters; // u_few_tiles(J)
};
hipError_t launch_u_few(const UFewArgs& a, hipStream_t stream);
int u_few_tiles(int J);
int u_few_splits(int J, int64_t K);
int64_t u_few_partial_floats(int J, int64_t K);
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
