// C ABI of the library (declared in include/qlin.h): argument validation,
// workspace planning and kernel dispatch.  Validation happens before any
// HIP call, so every argument error is reported without touching a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "host_codebook.hpp"
#include "kernels.hpp"
#include "qlin.h"

namespace qlin {

namespace {

constexpr int64_t kMaxRank = 128;
constexpr int64_t kSmallM = 16;  // weight-streaming kernels up to this many tokens

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? QLIN_OK : QLIN_E_HIP; }

#define QLIN_TRY(expr)                      \
  do {                                      \
    const hipError_t e_ = (expr);           \
    if (e_ != hipSuccess) return QLIN_E_HIP; \
  } while (0)

// Validate a packed weight descriptor (pointers may be checked for NULL and
// alignment only; the library never dereferences device memory on the host).
int check_weight(const qlin_qweight* w) {
  if (w == nullptr) return QLIN_E_NULL;
  if (w->reserved != 0) return QLIN_E_UNSUPPORTED;
  if (w->d_out < 1 || w->d_in < 1) return QLIN_E_SHAPE;
  if (w->d_out % 16 != 0) return QLIN_E_SHAPE;
  if (w->codes == nullptr) return QLIN_E_NULL;
  if (!aligned16(w->codes)) return QLIN_E_ALIGN;
  if (w->format == QLIN_FMT_NF4) {
    if (w->block != 64) return QLIN_E_UNSUPPORTED;
    if (w->dq_block != 0 && w->dq_block != 256) return QLIN_E_UNSUPPORTED;
    if (w->d_in % 64 != 0) return QLIN_E_SHAPE;
    if (w->absmax == nullptr) return QLIN_E_NULL;
    if (!aligned16(w->absmax)) return QLIN_E_ALIGN;
    if (w->dq_block != 0) {
      if (w->absmax2 == nullptr) return QLIN_E_NULL;
      if (!aligned16(w->absmax2)) return QLIN_E_ALIGN;
    }
    return QLIN_OK;
  }
  if (w->format == QLIN_FMT_INT4_GROUP) {
    if (w->block != 32) return QLIN_E_UNSUPPORTED;
    if (w->dq_block != 0) return QLIN_E_UNSUPPORTED;
    if (w->d_in % 64 != 0) return QLIN_E_SHAPE;
    if (w->scale == nullptr || w->zero == nullptr) return QLIN_E_NULL;
    if (!aligned16(w->scale) || !aligned16(w->zero)) return QLIN_E_ALIGN;
    return QLIN_OK;
  }
  return QLIN_E_UNSUPPORTED;
}

int check_layer(const qlin_qweight* w, int64_t M, int32_t r, float s, int32_t pool) {
  const int st = check_weight(w);
  if (st != QLIN_OK) return st;
  if (M < 1 || M > (int64_t{1} << 31)) return QLIN_E_SHAPE;
  if (r < 1 || r > kMaxRank) return QLIN_E_SHAPE;
  if (!std::isfinite(s)) return QLIN_E_SHAPE;
  if (pool != 1) {
    if (w->format != QLIN_FMT_INT4_GROUP || pool != w->block) return QLIN_E_UNSUPPORTED;
  }
  return QLIN_OK;
}

WeightView make_view(const qlin_qweight* w) {
  WeightView v{};
  v.codes = w->codes;
  v.absmax = w->absmax;
  v.absmax2 = w->absmax2;
  v.scale = w->scale;
  v.zero = w->zero;
  v.N = w->d_out;
  v.K = w->d_in;
  v.dq = w->dq_block != 0 ? 1 : 0;
  nf4_levels(v.cb.c);
  return v;
}

int fmt_of(const qlin_qweight* w) { return w->format == QLIN_FMT_NF4 ? kFmtNF4 : kFmtINT4; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Work split of the reductions and the workspace layout for one layer shape.
struct Plan {
  bool small = false;
  int fwd_splits = 1;
  int nt_splits_u = 1, nt_splits_du = 1;
  int tn2_splits_dB = 1, tn2_splits_dA = 1;
  int gf_splits = 1, gd_splits = 1;
  size_t off_counters = 0, off_u = 0, off_du = 0, off_Bt = 0, off_At = 0, off_P = 0,
         off_z = 0, off_partial = 0, total = 0;
};

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

Plan make_plan(const qlin_qweight* w, int64_t M, int32_t r, int32_t pool) {
  Plan p;
  const int64_t N = w->d_out, K = w->d_in, G = K / pool;
  p.small = M <= kSmallM;
  // skinny products: ~256 workgroups of 64 rows (one per compute unit; at
  // 4096 x 4096 and 4096 x 11008 twice as many ran 7-14 % slower, half as
  // many 28-50 % slower), at least 4 chunks of 128 columns per split
  p.nt_splits_u = static_cast<int>(clamp64(std::min<int64_t>(256 / nt_tiles(M), ceil_div(K, 128) / 4), 1, 64));
  p.nt_splits_du = static_cast<int>(clamp64(std::min<int64_t>(256 / nt_tiles(M), ceil_div(N, 128) / 4), 1, 64));
  // token-share splits of the adapter-gradient reductions: ~320 workgroups,
  // at least 256 tokens per share
  const int64_t max_shares = std::max<int64_t>(1, M / 256);
  p.tn2_splits_dB = static_cast<int>(clamp64(ceil_div(320, tn2_tiles(N)), 1, std::min<int64_t>(max_shares, 64)));
  p.tn2_splits_dA = static_cast<int>(clamp64(ceil_div(320, tn2_tiles(K)), 1, std::min<int64_t>(max_shares, 64)));
  if (!p.small) {
    const int tiles = fwd_gemm_tiles(M, N);
    if (tiles < 192) p.fwd_splits = static_cast<int>(clamp64(ceil_div(256, tiles), 1, std::max<int64_t>(1, ceil_div(K, 128) / 4)));
  }
  p.gf_splits = gemv_fwd_splits(K);
  p.gd_splits = gemv_dx_splits(N);

  int64_t counters = std::max<int64_t>({nt_tiles(M), gemv_fwd_tiles(N),
                                        gemv_dx_tiles(K), int64_t{fwd_gemm_tiles(M, N)},
                                        int64_t{tn2_tiles(N)}, int64_t{tn2_tiles(K)}});
  int64_t partial = std::max<int64_t>({nt_partial_floats(M, p.nt_splits_u),
                                       nt_partial_floats(M, p.nt_splits_du),
                                       tn2_partial_floats(N, r, p.tn2_splits_dB),
                                       tn2_partial_floats(K, r, p.tn2_splits_dA)});
  if (p.small) {
    partial = std::max<int64_t>({partial,
                                 gemv_fwd_partial_floats(N, K),
                                 gemv_dx_partial_floats(N, K) + gemv_dx_dupart_floats(N, K, r)});
  } else {
    partial = std::max<int64_t>(partial, fwd_gemm_partial_floats(M, N, p.fwd_splits));
    if (pool > 1) partial = std::max<int64_t>(partial, qa_dA_partial_floats(M, r, G));
  }
  size_t off = 0;
  p.off_counters = off; off = align256(off + counters * sizeof(uint32_t));
  p.off_u = off;        off = align256(off + static_cast<size_t>(M) * r * sizeof(float));
  p.off_du = off;       off = align256(off + static_cast<size_t>(M) * r * sizeof(float));
  p.off_Bt = off;       off = align256(off + static_cast<size_t>(N) * r * sizeof(uint16_t));
  p.off_At = off;       off = align256(off + static_cast<size_t>(G) * r * sizeof(uint16_t));
  p.off_P = off;        off = align256(off + (pool > 1 ? static_cast<size_t>(M) * G * sizeof(float) : 0));
  p.off_z = off;        off = align256(off + (p.small ? 0 : 4 * static_cast<size_t>(M) * tn2_jp(r) * sizeof(uint16_t)));
  p.off_partial = off;  off = align256(off + static_cast<size_t>(partial) * sizeof(float));
  p.total = off;
  return p;
}

template <typename T>
T* ws_at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

// u = P A^T (P = x, or the group sums of x) into `u` (fp32 [M][r]).
int compute_u(const qlin_qweight* w, const uint16_t* x, int64_t M, const uint16_t* A, int32_t r,
              int32_t pool, float* u, const Plan& p, void* ws, hipStream_t stream) {
  if (pool == 1) {
    NtArgs a{};
    a.X = x; a.ldx = w->d_in;
    a.Y = A; a.ldy = w->d_in;
    a.C = u; a.ldc = r;
    a.M = M; a.K = w->d_in; a.J = r;
    a.splits = p.nt_splits_u;
    a.alpha = 1.0f;
    a.partial = ws_at<float>(ws, p.off_partial);
    a.counters = ws_at<uint32_t>(ws, p.off_counters);
    return hip_status(launch_nt_skinny(a, stream));
  }
  QaArgs q{};
  q.x = x; q.A = A; q.u_out = u; q.P_out = nullptr;
  q.M = M; q.K = w->d_in; q.G = w->d_in / pool; q.r = r; q.pool = pool;
  return hip_status(launch_qa_pool_u(q, stream));
}

}  // namespace

}  // namespace qlin

using namespace qlin;

extern "C" {

const char* qlin_status_string(int status) {
  switch (status) {
    case QLIN_OK: return "ok";
    case QLIN_E_NULL: return "null pointer";
    case QLIN_E_SHAPE: return "invalid shape or size";
    case QLIN_E_ALIGN: return "device pointer not 16-byte aligned";
    case QLIN_E_NONFINITE: return "non-finite or out-of-range input";
    case QLIN_E_UNSUPPORTED: return "unsupported parameter combination";
    case QLIN_E_WORKSPACE: return "workspace missing or too small";
    case QLIN_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int qlin_nf4_codebook(float out[16]) {
  if (out == nullptr) return QLIN_E_NULL;
  nf4_levels(out);
  return QLIN_OK;
}

int qlin_quantize_nf4(const float* W, int64_t d_out, int64_t d_in, int32_t block, int32_t dq_block,
                      uint8_t* codes, void* absmax, float* absmax2, hipStream_t stream) {
  if (W == nullptr || codes == nullptr || absmax == nullptr) return QLIN_E_NULL;
  if (dq_block != 0 && absmax2 == nullptr) return QLIN_E_NULL;
  if (block != 64) return QLIN_E_UNSUPPORTED;
  if (dq_block != 0 && dq_block != 256) return QLIN_E_UNSUPPORTED;
  if (d_out < 1 || d_in < 1 || d_in % 64 != 0) return QLIN_E_SHAPE;
  if (d_out > (int64_t{1} << 40) / d_in) return QLIN_E_SHAPE;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax) ||
      (dq_block != 0 && !aligned16(absmax2)))
    return QLIN_E_ALIGN;
  float cb[16];
  nf4_levels(cb);
  double mids[15];
  for (int i = 0; i < 15; ++i) mids[i] = (static_cast<double>(cb[i]) + static_cast<double>(cb[i + 1])) / 2.0;
  const int64_t n_blocks = d_out * d_in / 64;
  QLIN_TRY(launch_quant_nf4(W, n_blocks, dq_block != 0 ? 1 : 0, mids, codes, absmax, absmax2, stream));
  QLIN_TRY(hipStreamSynchronize(stream));
  // non-finite input is reported through NaN constants
  if (dq_block != 0) {
    std::vector<float> s2(static_cast<size_t>((n_blocks + 255) / 256));
    QLIN_TRY(hipMemcpy(s2.data(), absmax2, s2.size() * sizeof(float), hipMemcpyDeviceToHost));
    for (float v : s2)
      if (std::isnan(v)) return QLIN_E_NONFINITE;
  } else {
    std::vector<float> am(static_cast<size_t>(n_blocks));
    QLIN_TRY(hipMemcpy(am.data(), absmax, am.size() * sizeof(float), hipMemcpyDeviceToHost));
    for (float v : am)
      if (std::isnan(v)) return QLIN_E_NONFINITE;
  }
  return QLIN_OK;
}

int qlin_quantize_int4_group(const float* W, int64_t d_out, int64_t d_in, int32_t group,
                             uint8_t* codes, uint16_t* scale, uint16_t* zero, hipStream_t stream) {
  if (W == nullptr || codes == nullptr || scale == nullptr || zero == nullptr) return QLIN_E_NULL;
  if (group != 32) return QLIN_E_UNSUPPORTED;
  if (d_out < 1 || d_in < 1 || d_in % 32 != 0) return QLIN_E_SHAPE;
  if (d_out > (int64_t{1} << 40) / d_in) return QLIN_E_SHAPE;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(scale) || !aligned16(zero)) return QLIN_E_ALIGN;
  const int64_t n_groups = d_out * d_in / 32;
  QLIN_TRY(launch_quant_int4(W, n_groups, codes, scale, zero, stream));
  QLIN_TRY(hipStreamSynchronize(stream));
  std::vector<uint16_t> sc(static_cast<size_t>(n_groups));
  QLIN_TRY(hipMemcpy(sc.data(), scale, sc.size() * sizeof(uint16_t), hipMemcpyDeviceToHost));
  for (uint16_t v : sc)
    if ((v & 0x7C00u) == 0x7C00u) return QLIN_E_NONFINITE;
  return QLIN_OK;
}

size_t qlin_workspace_bytes(const qlin_qweight* w, int64_t M, int32_t r, int32_t pool) {
  if (check_layer(w, M, r, 0.0f, pool) != QLIN_OK) return 0;
  return make_plan(w, M, r, pool).total;
}

int qlin_fwd(const qlin_qweight* w, const uint16_t* x, int64_t M, const uint16_t* A,
             const uint16_t* B, int32_t r, float s, int32_t pool, uint16_t* y, float* u_out,
             void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_layer(w, M, r, s, pool);
  if (st != QLIN_OK) return st;
  if (x == nullptr || A == nullptr || B == nullptr || y == nullptr) return QLIN_E_NULL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) ||
      (u_out != nullptr && !aligned16(u_out)))
    return QLIN_E_ALIGN;
  const Plan p = make_plan(w, M, r, pool);
  if (workspace == nullptr || ws_bytes < p.total) return QLIN_E_WORKSPACE;
  if (!aligned16(workspace)) return QLIN_E_ALIGN;

  const WeightView v = make_view(w);
  const int fmt = fmt_of(w);
  float* u = u_out != nullptr ? u_out : ws_at<float>(workspace, p.off_u);
  const bool adapter = s != 0.0f;
  // the few-token kernel forms u itself for a plain adapter of rank <= 16
  const bool fuse_u = p.small && pool == 1 && r <= 16;
  if (!fuse_u && (adapter || u_out != nullptr)) {
    st = compute_u(w, x, M, A, r, pool, u, p, workspace, stream);
    if (st != QLIN_OK) return st;
  }
  if (p.small) {
    GemvFwdArgs a{};
    a.w = v; a.x = x; a.M = M; a.A = A; a.B = B; a.r = r; a.s = s;
    a.adapter = adapter ? 1 : 0;
    a.fuse_u = (fuse_u && (adapter || u_out != nullptr)) ? 1 : 0;
    a.u_in = u;
    a.y = y; a.u_out = u_out;
    a.splits = gemv_fwd_splits(w->d_in);
    a.kshare = gemv_fwd_kshare(w->d_in);
    a.partial = ws_at<float>(workspace, p.off_partial);
    a.counters = ws_at<uint32_t>(workspace, p.off_counters);
    return hip_status(launch_gemv_fwd(a, fmt, stream));
  }
  FwdArgs a{};
  a.w = v; a.x = x; a.M = M; a.B = B; a.u = adapter ? u : nullptr; a.r = r; a.s = s; a.y = y;
  a.splits = p.fwd_splits;
  a.partial = ws_at<float>(workspace, p.off_partial);
  a.counters = ws_at<uint32_t>(workspace, p.off_counters);
  return hip_status(launch_fwd_gemm(a, fmt, stream));
}

int qlin_bwd(const qlin_qweight* w, const uint16_t* x, int64_t M, const uint16_t* A,
             const uint16_t* B, int32_t r, float s, int32_t pool, const uint16_t* dy,
             const float* u_saved, uint16_t* dx, uint16_t* dA, uint16_t* dB, void* workspace,
             size_t ws_bytes, hipStream_t stream) {
  int st = check_layer(w, M, r, s, pool);
  if (st != QLIN_OK) return st;
  if (x == nullptr || A == nullptr || B == nullptr || dy == nullptr || dA == nullptr ||
      dB == nullptr)
    return QLIN_E_NULL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(dy) || !aligned16(dA) ||
      !aligned16(dB) || (dx != nullptr && !aligned16(dx)) ||
      (u_saved != nullptr && !aligned16(u_saved)))
    return QLIN_E_ALIGN;
  const Plan p = make_plan(w, M, r, pool);
  if (workspace == nullptr || ws_bytes < p.total) return QLIN_E_WORKSPACE;
  if (!aligned16(workspace)) return QLIN_E_ALIGN;

  const int64_t N = w->d_out, K = w->d_in, G = K / pool;
  const WeightView v = make_view(w);
  const int fmt = fmt_of(w);
  float* partial = ws_at<float>(workspace, p.off_partial);
  uint32_t* counters = ws_at<uint32_t>(workspace, p.off_counters);
  float* du = ws_at<float>(workspace, p.off_du);
  uint16_t* Bt = ws_at<uint16_t>(workspace, p.off_Bt);

  // u (saved by the forward pass, or recomputed)
  const float* u = u_saved;
  if (u == nullptr) {
    float* uw = ws_at<float>(workspace, p.off_u);
    st = compute_u(w, x, M, A, r, pool, uw, p, workspace, stream);
    if (st != QLIN_OK) return st;
    u = uw;
  }
  if (p.small) {
    // one launch: du, dB, dA and dX folded into the weight-streaming kernel
    GemvDxArgs a{};
    a.w = v; a.x = x; a.dy = dy; a.M = M; a.A = A; a.B = B; a.u = u; a.r = r; a.pool = pool;
    a.pool_shift = __builtin_ctz(static_cast<unsigned>(pool)); a.s = s;
    a.dx = dx; a.dA = dA; a.dB = dB; a.splits = p.gd_splits;
    a.partial = partial;
    a.du_part = partial + gemv_dx_partial_floats(N, K);
    a.counters = counters;
    return hip_status(launch_gemv_dx(a, fmt, stream));
  }
  // du = s dY B  (B^T staged so both operands are contiguous along n)
  QLIN_TRY(launch_transpose16(B, N, r, Bt, stream));
  {
    NtArgs a{};
    a.X = dy; a.ldx = N; a.Y = Bt; a.ldy = N; a.C = du; a.ldc = r;
    a.M = M; a.K = N; a.J = r; a.splits = p.nt_splits_du; a.alpha = s;
    a.partial = partial; a.counters = counters;
    QLIN_TRY(launch_nt_skinny(a, stream));
  }
  // dB = s dY^T u  (u as bf16 hi/lo planes)
  const int64_t jp = tn2_jp(r);
  uint16_t* zp = ws_at<uint16_t>(workspace, p.off_z);
  {
    QLIN_TRY(launch_split_hl(u, M, r, r, zp, zp + M * jp, stream));
    Tn2Args a{};
    a.X = dy; a.ldx = N; a.Zh = zp; a.Zl = zp + M * jp; a.C = dB; a.ldc = r;
    a.M = M; a.P = N; a.J = r; a.splits = p.tn2_splits_dB; a.out_transposed = 0; a.alpha = s;
    a.partial = partial; a.counters = counters;
    QLIN_TRY(launch_tn2(a, stream));
  }
  // dA = du^T P
  if (pool == 1) {
    QLIN_TRY(launch_split_hl(du, M, r, r, zp + 2 * M * jp, zp + 3 * M * jp, stream));
    Tn2Args a{};
    a.X = x; a.ldx = K; a.Zh = zp + 2 * M * jp; a.Zl = zp + 3 * M * jp; a.C = dA; a.ldc = K;
    a.M = M; a.P = K; a.J = r; a.splits = p.tn2_splits_dA; a.out_transposed = 1; a.alpha = 1.0f;
    a.partial = partial; a.counters = counters;
    QLIN_TRY(launch_tn2(a, stream));
  } else {
    QaArgs q{};
    q.x = x; q.A = A; q.du = du; q.M = M; q.K = K; q.G = G; q.r = r; q.pool = pool;
    q.P_out = ws_at<float>(workspace, p.off_P);
    QLIN_TRY(launch_qa_pool_u(q, stream));
    q.P_in = q.P_out;
    q.dA_out = dA;
    q.part = partial;
    QLIN_TRY(launch_qa_dA(q, stream));
  }
  if (dx == nullptr) return QLIN_OK;
  // dX = dY W_bf16 + du A; with the pooled adapter A^T has one row per group
  // and column k of dX reads row k >> log2(pool)
  uint16_t* At = ws_at<uint16_t>(workspace, p.off_At);
  QLIN_TRY(launch_transpose16(A, r, G, At, stream));
  DxArgs a{};
  a.w = v; a.dy = dy; a.M = M; a.At = At; a.du = du; a.r = r;
  a.pool = pool; a.pool_shift = __builtin_ctz(static_cast<unsigned>(pool));
  a.dx = dx;
  return hip_status(launch_dx_gemm(a, fmt, stream));
}

int qlin_dequant_bf16(const qlin_qweight* w, uint16_t* W_out, hipStream_t stream) {
  const int st = check_weight(w);
  if (st != QLIN_OK) return st;
  if (W_out == nullptr) return QLIN_E_NULL;
  if (!aligned16(W_out)) return QLIN_E_ALIGN;
  const WeightView v = make_view(w);
  return hip_status(launch_dequant(v, fmt_of(w), W_out, stream));
}

}  // extern "C"
