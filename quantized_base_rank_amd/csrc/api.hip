// C ABI of the library (declared in include/qlin.h): argument validation,
// workspace planning and kernel dispatch.  Validation happens before any
// HIP call, so every argument error is reported without touching a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
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
  if (w->d_out < 1 || w->d_in < 1) return QLIN_E_SHAPE;
  if (w->d_out % 16 != 0) return QLIN_E_SHAPE;
  if (w->codes == nullptr) return QLIN_E_NULL;
  if (!aligned16(w->codes)) return QLIN_E_ALIGN;
  if (w->format == QLIN_FMT_NF4 || w->format == QLIN_FMT_NF) {
    if (w->format == QLIN_FMT_NF4) {
      if (w->bits != 0) return QLIN_E_UNSUPPORTED;
      if (w->block != 64) return QLIN_E_UNSUPPORTED;
    } else {
      if (w->bits < 2 || w->bits > 4) return QLIN_E_UNSUPPORTED;
      if (w->block != 32 && w->block != 64 && w->block != 128 && w->block != 256)
        return QLIN_E_UNSUPPORTED;
      if (w->d_in % w->block != 0) return QLIN_E_SHAPE;
    }
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
    if (w->bits != 0) return QLIN_E_UNSUPPORTED;
    if (w->block != 32) return QLIN_E_UNSUPPORTED;
    if (w->dq_block != 0) return QLIN_E_UNSUPPORTED;
    if (w->d_in % 64 != 0) return QLIN_E_SHAPE;
    if (w->scale == nullptr || w->zero == nullptr) return QLIN_E_NULL;
    if (!aligned16(w->scale) || !aligned16(w->zero)) return QLIN_E_ALIGN;
    return QLIN_OK;
  }
  return QLIN_E_UNSUPPORTED;
}

// r_min = 0 admits the adapter-free layer (forward only).
int check_layer(const qlin_qweight* w, int64_t M, int32_t r, float s, int32_t pool, int32_t r_min = 1) {
  const int st = check_weight(w);
  if (st != QLIN_OK) return st;
  if (M < 1 || M > (int64_t{1} << 31)) return QLIN_E_SHAPE;
  if (r < r_min || r > kMaxRank) return QLIN_E_SHAPE;
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
  if (w->format == QLIN_FMT_NF)
    nf_levels(w->bits, v.cb.c);  // (the rest of the 16 entries stay zero)
  else
    nf4_levels(v.cb.c);
  return v;
}

// The layer kernels' format: NormalFloat-k weights are read through the
// per-call transcoded form (kFmtNFG).
int fmt_of(const qlin_qweight* w) {
  return w->format == QLIN_FMT_NF4 ? kFmtNF4 : (w->format == QLIN_FMT_NF ? kFmtNFG : kFmtINT4);
}

NfTable nf_table(int bits) {
  NfTable t{};
  nf_levels(bits, t.c);
  const int n = 1 << bits;
  for (int i = 0; i + 1 < n; ++i)
    t.mid[i] = (static_cast<double>(t.c[i]) + static_cast<double>(t.c[i + 1])) / 2.0;
  return t;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Ticket counters of the split reductions live in a fixed region at the
// start of every workspace, the same for every layer shape, and nothing else
// is ever written there.  Every completed call leaves its counters at zero,
// so a workspace zero-filled once can be reused by calls of any shape (a
// counter region whose length followed the shape would overlap, for a later
// call of another shape, bytes where an earlier call left u or partial sums).
constexpr size_t kCounterBytes = size_t{64} << 10;
constexpr int64_t kCounterWords = static_cast<int64_t>(kCounterBytes / sizeof(uint32_t));

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Work split of the reductions and the workspace layout for one layer shape.
struct Plan {
  bool small = false;
  bool stream = false;  // few tokens, large weight: the streamed forward
  int fs_splits = 1, uf_splits = 1;
  bool dx_stream = false;  // few tokens, large weight: streamed input gradient
  int ds_splits = 1;
  bool fits = true;  // the shape's ticket counters fit the fixed region
  int fwd_splits = 1;
  int nt_splits_u = 1, nt_splits_du = 1;
  int tn2_splits_dB = 1, tn2_splits_dA = 1;
  int gf_splits = 1, gd_splits = 1;
  size_t off_counters = 0, off_u = 0, off_du = 0, off_Bt = 0, off_At = 0, off_P = 0,
         off_z = 0, off_partial = 0, off_tc = 0, total = 0;
};

// Bytes of the transcoded NormalFloat-k weight (4-bit indices, then the
// low and high 16-bit planes of the per-32 scales); 0 for other formats.
size_t transcode_bytes(const qlin_qweight* w) {
  if (w->format != QLIN_FMT_NF) return 0;
  const size_t n_el = static_cast<size_t>(w->d_out) * static_cast<size_t>(w->d_in);
  return align256(n_el / 2) + 2 * align256(n_el / 32 * sizeof(uint16_t));
}

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
  // few tokens on a weight above 32 M elements: streamed forward (the
  // one-shot kernels are shaped for one round of workgroups at 4096 x 4096)
  p.stream = p.small && N * K > (int64_t{1} << 25);
  p.fs_splits = fwd_stream_splits(N, K);
  p.uf_splits = u_few_splits(r > 0 ? r : 1, K);
  p.dx_stream = p.stream && dx_stream_fits(N, K, fmt_of(w));
  p.ds_splits = dx_stream_splits(N, K, fmt_of(w));

  // counters each kernel takes tickets on (only when it splits a reduction;
  // the few-token backward always does)
  int64_t counters = std::max<int64_t>({p.nt_splits_u > 1 || p.nt_splits_du > 1 ? nt_tiles(M) : 0,
                                        p.tn2_splits_dB > 1 ? tn2_tiles(N) : 0,
                                        p.tn2_splits_dA > 1 ? tn2_tiles(K) : 0});
  if (p.small)
    counters = std::max<int64_t>({counters, p.gf_splits > 1 ? gemv_fwd_tiles(N) : 0, gemv_dx_tiles(K),
                                  p.fs_splits > 1 ? fwd_stream_row_groups(N) : 0,
                                  p.dx_stream && p.ds_splits > 1 ? dx_stream_panels(K) : 0,
                                  p.uf_splits > 1 ? u_few_tiles(r > 0 ? r : 1) : 0});
  else if (p.fwd_splits > 1)
    counters = std::max<int64_t>(counters, fwd_gemm_tiles(M, N));
  p.fits = counters <= kCounterWords;
  int64_t partial = std::max<int64_t>({nt_partial_floats(M, p.nt_splits_u),
                                       nt_partial_floats(M, p.nt_splits_du),
                                       tn2_partial_floats(N, r, p.tn2_splits_dB),
                                       tn2_partial_floats(K, r, p.tn2_splits_dA)});
  if (p.small) {
    partial = std::max<int64_t>({partial,
                                 gemv_fwd_partial_floats(N, K),
                                 gemv_dx_partial_floats(N, K) + gemv_dx_dupart_floats(N, K, r),
                                 p.stream ? fwd_stream_partial_floats(N, K) : 0,
                                 p.dx_stream ? dx_stream_partial_floats(N, K, fmt_of(w)) : 0,
                                 p.dx_stream ? adapter_few_partial_floats(N) : 0,
                                 p.dx_stream && pool > 1 ? qa_dA_partial_floats(M, r, G) : 0,
                                 u_few_partial_floats(r > 0 ? r : 1, K)});
  } else {
    partial = std::max<int64_t>(partial, fwd_gemm_partial_floats(M, N, p.fwd_splits));
    if (pool > 1) partial = std::max<int64_t>(partial, qa_dA_partial_floats(M, r, G));
  }
  size_t off = 0;
  p.off_counters = off; off = kCounterBytes;
  p.off_u = off;        off = align256(off + static_cast<size_t>(M) * r * sizeof(float));
  p.off_du = off;       off = align256(off + static_cast<size_t>(M) * r * sizeof(float));
  p.off_Bt = off;       off = align256(off + static_cast<size_t>(N) * r * sizeof(uint16_t));
  p.off_At = off;       off = align256(off + static_cast<size_t>(G) * r * sizeof(uint16_t));
  p.off_P = off;        off = align256(off + (pool > 1 ? static_cast<size_t>(M) * G * sizeof(float) : 0));
  // (hi/lo planes of u and du for the transposed products; the few-token
  // streamed path uses them only for dA when dX is not wanted)
  p.off_z = off;        off = align256(off + (p.small && !p.dx_stream ? 0 : 4 * static_cast<size_t>(M) * tn2_jp(r) * sizeof(uint16_t)));
  p.off_partial = off;  off = align256(off + static_cast<size_t>(partial) * sizeof(float));
  p.off_tc = off;       off += transcode_bytes(w);
  p.total = off;
  return p;
}

// The weight as the layer kernels read it.  NormalFloat-k weights are first
// transcoded (on `stream`, into `tc`: transcode_bytes(w) bytes) to 4-bit
// indices and per-32 fp32 scales; the levels stay in the view's codebook.
int layer_view(const qlin_qweight* w, uint8_t* tc, hipStream_t stream, WeightView* out) {
  WeightView v = make_view(w);
  if (w->format == QLIN_FMT_NF) {
    const size_t n_el = static_cast<size_t>(w->d_out) * static_cast<size_t>(w->d_in);
    uint8_t* nib = tc;
    uint16_t* lo = reinterpret_cast<uint16_t*>(tc + align256(n_el / 2));
    uint16_t* hi = reinterpret_cast<uint16_t*>(tc + align256(n_el / 2) + align256(n_el / 32 * sizeof(uint16_t)));
    QLIN_TRY(launch_transcode_nf(w->codes, w->absmax, w->absmax2, static_cast<int64_t>(n_el), w->bits,
                                 w->block, w->dq_block != 0 ? 1 : 0, nib, lo, hi, stream));
    v.codes = nib;
    v.scale = lo;
    v.zero = hi;
    v.absmax = nullptr;
    v.absmax2 = nullptr;
    v.dq = 0;
  }
  *out = v;
  return QLIN_OK;
}

// Runs one quantizer launch between clearing and reading back the device's
// non-finite flag, then synchronises `stream`.  The flag is one word per
// device, so quantizer calls of this process take turns on a mutex.
template <typename Launch>
int run_flagged(hipStream_t stream, Launch launch) {
  std::lock_guard<std::mutex> guard(quant_flag_lock());
  uint32_t* flag = nullptr;
  QLIN_TRY(quant_flag_ptr(&flag));
  QLIN_TRY(hipMemsetAsync(flag, 0, sizeof(uint32_t), stream));
  QLIN_TRY(launch(flag));
  uint32_t bad = 0;
  QLIN_TRY(hipMemcpyAsync(&bad, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, stream));
  QLIN_TRY(hipStreamSynchronize(stream));
  return bad != 0 ? QLIN_E_NONFINITE : QLIN_OK;
}

template <typename T>
T* ws_at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

// Profiling aid: qlin_profile_next_launch arms one (kernel name, start,
// stop) triple; the next launch of that kernel records `start` just before
// and `stop` just after itself on its stream, and disarms the hook.
struct ProfileHook {
  std::mutex m;
  bool armed = false;
  char name[64] = {};
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfileHook& profile_hook() {
  static ProfileHook h;
  return h;
}

template <typename Launch>
hipError_t hooked(const char* name, hipStream_t stream, Launch launch) {
  hipEvent_t start = nullptr, stop = nullptr;
  {
    ProfileHook& h = profile_hook();
    std::lock_guard<std::mutex> g(h.m);
    if (h.armed && std::strcmp(h.name, name) == 0) {
      start = h.start;
      stop = h.stop;
      h.armed = false;
    }
  }
  if (start != nullptr) {
    const hipError_t e = hipEventRecord(start, stream);
    if (e != hipSuccess) return e;
  }
  const hipError_t e = launch();
  if (e != hipSuccess || stop == nullptr) return e;
  return hipEventRecord(stop, stream);
}

// u = P A^T (P = x, or the group sums of x) into `u` (fp32 [M][r]).
int compute_u(const qlin_qweight* w, const uint16_t* x, int64_t M, const uint16_t* A, int32_t r,
              int32_t pool, float* u, int splits_u, float* partial, uint32_t* counters,
              hipStream_t stream) {
  if (pool == 1 && M <= kSmallM) {
    UFewArgs a{};
    a.X = x; a.ldx = w->d_in;
    a.Y = A; a.ldy = w->d_in;
    a.C = u; a.ldc = r;
    a.M = M; a.K = w->d_in; a.J = r;
    a.splits = u_few_splits(r, w->d_in);
    a.alpha = 1.0f;
    a.partial = partial;
    a.counters = counters;
    return hip_status(hooked("k_u_few", stream, [&] { return launch_u_few(a, stream); }));
  }
  if (pool == 1) {
    NtArgs a{};
    a.X = x; a.ldx = w->d_in;
    a.Y = A; a.ldy = w->d_in;
    a.C = u; a.ldc = r;
    a.M = M; a.K = w->d_in; a.J = r;
    a.splits = splits_u;
    a.alpha = 1.0f;
    a.partial = partial;
    a.counters = counters;
    return hip_status(hooked("k_nt_skinny", stream, [&] { return launch_nt_skinny(a, stream); }));
  }
  QaArgs q{};
  q.x = x; q.A = A; q.u_out = u; q.P_out = nullptr;
  q.M = M; q.K = w->d_in; q.G = w->d_in / pool; q.r = r; q.pool = pool;
  return hip_status(hooked("k_qa_pool_u", stream, [&] { return launch_qa_pool_u(q, stream); }));
}

// Whether the few-token forward forms u itself (plain adapter of rank <= 16).
bool fwd_fuses_u(const Plan& p, int32_t r, int32_t pool) {
  return p.small && !p.stream && pool == 1 && r <= 16;
}

// The forward pass on explicit buffers: `u_tmp` (fp32 [M][r], used when
// u_out is NULL), `partial` (split partial sums) and `counters` (ticket
// counters, zero on entry and left at zero).
int fwd_core(const qlin_qweight* w, const uint16_t* x, int64_t M, const uint16_t* A,
             const uint16_t* B, int32_t r, float s, int32_t pool, uint16_t* y, float* u_out,
             const Plan& p, float* u_tmp, float* partial, uint32_t* counters, uint8_t* tc,
             hipStream_t stream) {
  WeightView v;
  const int vst = layer_view(w, tc, stream, &v);
  if (vst != QLIN_OK) return vst;
  const int fmt = fmt_of(w);
  float* u = u_out != nullptr ? u_out : u_tmp;
  const bool adapter = r > 0 && s != 0.0f;
  const bool fuse_u = fwd_fuses_u(p, r, pool);
  if (!fuse_u && (adapter || u_out != nullptr)) {
    const int st = compute_u(w, x, M, A, r, pool, u, p.nt_splits_u, partial, counters, stream);
    if (st != QLIN_OK) return st;
  }
  if (p.stream) {
    FwdStreamArgs a{};
    a.w = v; a.x = x; a.M = M; a.B = B; a.u = u; a.r = r; a.s = s;
    a.adapter = adapter ? 1 : 0;
    a.y = y;
    a.splits = p.fs_splits;
    a.partial = partial;
    a.counters = counters;
    return hip_status(hooked("k_gemv_fwd_stream", stream,
                             [&] { return launch_gemv_fwd_stream(a, fmt, stream); }));
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
    a.partial = partial;
    a.counters = counters;
    return hip_status(hooked("k_gemv_fwd", stream, [&] { return launch_gemv_fwd(a, fmt, stream); }));
  }
  FwdArgs a{};
  a.w = v; a.x = x; a.M = M; a.B = B; a.u = adapter ? u : nullptr; a.r = r; a.s = s; a.y = y;
  a.splits = p.fwd_splits;
  a.partial = partial;
  a.counters = counters;
  return hip_status(hooked("k_fwd_gemm", stream, [&] { return launch_fwd_gemm(a, fmt, stream); }));
}

// Argument checks shared by qlin_fwd and qlin_fwd_noalloc.
int check_fwd_args(const qlin_qweight* w, const uint16_t* x, int64_t M, const uint16_t* A,
                   const uint16_t* B, int32_t r, float s, int32_t pool, const uint16_t* y,
                   const float* u_out) {
  const int st = check_layer(w, M, r, s, pool, 0);
  if (st != QLIN_OK) return st;
  if (r == 0) {
    // no adapter: A and B are not read, and there is no u to return
    if (u_out != nullptr) return QLIN_E_SHAPE;
    if (x == nullptr || y == nullptr) return QLIN_E_NULL;
    if (!aligned16(x) || !aligned16(y)) return QLIN_E_ALIGN;
    return QLIN_OK;
  }
  if (x == nullptr || A == nullptr || B == nullptr || y == nullptr) return QLIN_E_NULL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) ||
      (u_out != nullptr && !aligned16(u_out)))
    return QLIN_E_ALIGN;
  return QLIN_OK;
}

// ------------------------------------------------- forward without allocation
// qlin_fwd_noalloc runs qlin_fwd's kernels on a file-scope device array
// instead of a caller workspace.  Layout: [0, 64 KiB) the ticket counters
// (the same fixed region as in a workspace), then u (when not returned) and
// the split partial sums of the forward kernels only.
constexpr size_t kScratchBytes = size_t{64} << 20;  // per device, held until exit
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct FwdScratch {
  size_t off_u = 0, off_partial = 0, off_tc = 0, total = 0;
};

FwdScratch fwd_scratch_layout(const qlin_qweight* w, int64_t M, int32_t r, int32_t pool,
                              const Plan& p) {
  const int64_t N = w->d_out, K = w->d_in;
  int64_t partial = 0;
  if (pool == 1 && !fwd_fuses_u(p, r, pool))
    partial = p.small ? u_few_partial_floats(r > 0 ? r : 1, K) : nt_partial_floats(M, p.nt_splits_u);
  partial = std::max<int64_t>(partial, p.stream ? fwd_stream_partial_floats(N, K)
                                       : (p.small ? gemv_fwd_partial_floats(N, K)
                                                  : fwd_gemm_partial_floats(M, N, p.fwd_splits)));
  FwdScratch f;
  size_t off = kCounterBytes;
  f.off_u = off;       off = align256(off + static_cast<size_t>(M) * (r > 0 ? r : 0) * sizeof(float));
  f.off_partial = off; off = align256(off + static_cast<size_t>(partial) * sizeof(float));
  f.off_tc = off;      off += transcode_bytes(w);
  f.total = off;
  return f;
}

__global__ void k_zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Device address of `scratch` on the current device.  At the first call on
// a device: looks the address up (the host-side name of a __device__ array
// is not a device address) and zeroes the counter region with a kernel on
// `stream`, ahead of that call's own kernels.
int scratch_ptr(hipStream_t stream, uint8_t** out) {
  static std::mutex m;
  static uint8_t* ptr[kMaxDevices] = {};
  std::lock_guard<std::mutex> g(m);
  int dev = 0;
  QLIN_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return QLIN_E_UNSUPPORTED;
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    QLIN_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    constexpr int n = static_cast<int>(kCounterBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(k_zero_words, dim3((n + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), n);
    QLIN_TRY(hipGetLastError());
    ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = ptr[dev];
  return QLIN_OK;
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
  if (d_out < 1 || d_in < 1 || d_in % 64 != 0 || d_out % 16 != 0) return QLIN_E_SHAPE;
  if (d_out > (int64_t{1} << 40) / d_in) return QLIN_E_SHAPE;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax) ||
      (dq_block != 0 && !aligned16(absmax2)))
    return QLIN_E_ALIGN;
  float cb[16];
  nf4_levels(cb);
  double mids[15];
  for (int i = 0; i < 15; ++i) mids[i] = (static_cast<double>(cb[i]) + static_cast<double>(cb[i + 1])) / 2.0;
  const int64_t n_blocks = d_out * d_in / 64;
  return run_flagged(stream, [&](uint32_t* flag) {
    return launch_quant_nf4(W, n_blocks, dq_block != 0 ? 1 : 0, mids, codes, absmax, absmax2,
                            flag, stream);
  });
}

int qlin_nf_codebook(int32_t bits, float* out) {
  if (out == nullptr) return QLIN_E_NULL;
  if (bits < 2 || bits > 4) return QLIN_E_UNSUPPORTED;
  nf_levels(bits, out);
  return QLIN_OK;
}

int qlin_quantize_nf(const float* W, int64_t d_out, int64_t d_in, int32_t bits, int32_t block,
                     int32_t dq_block, uint8_t* codes, void* absmax, float* absmax2,
                     hipStream_t stream) {
  if (W == nullptr || codes == nullptr || absmax == nullptr) return QLIN_E_NULL;
  if (dq_block != 0 && absmax2 == nullptr) return QLIN_E_NULL;
  if (bits < 2 || bits > 4) return QLIN_E_UNSUPPORTED;
  if (block != 32 && block != 64 && block != 128 && block != 256) return QLIN_E_UNSUPPORTED;
  if (dq_block != 0 && dq_block != 256) return QLIN_E_UNSUPPORTED;
  if (d_out < 1 || d_in < 1 || d_in % 64 != 0 || d_in % block != 0 || d_out % 16 != 0)
    return QLIN_E_SHAPE;
  if (d_out > (int64_t{1} << 40) / d_in) return QLIN_E_SHAPE;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax) ||
      (dq_block != 0 && !aligned16(absmax2)))
    return QLIN_E_ALIGN;
  const NfTable tb = nf_table(bits);
  const int64_t n_blocks = d_out * d_in / block;
  return run_flagged(stream, [&](uint32_t* flag) {
    return launch_quant_nf(W, n_blocks, bits, block, dq_block != 0 ? 1 : 0, tb, codes, absmax,
                           absmax2, flag, stream);
  });
}

int qlin_quantize_int4_group(const float* W, int64_t d_out, int64_t d_in, int32_t group,
                             uint8_t* codes, uint16_t* scale, uint16_t* zero, hipStream_t stream) {
  if (W == nullptr || codes == nullptr || scale == nullptr || zero == nullptr) return QLIN_E_NULL;
  if (group != 32) return QLIN_E_UNSUPPORTED;
  // the layer streams INT4 weights 64 columns (two groups) at a time and
  // tiles rows by 16, so the quantizer accepts exactly the shapes it can use
  if (d_out < 1 || d_in < 1 || d_in % 64 != 0 || d_out % 16 != 0) return QLIN_E_SHAPE;
  if (d_out > (int64_t{1} << 40) / d_in) return QLIN_E_SHAPE;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(scale) || !aligned16(zero)) return QLIN_E_ALIGN;
  const int64_t n_groups = d_out * d_in / 32;
  return run_flagged(stream, [&](uint32_t* flag) {
    return launch_quant_int4(W, n_groups, codes, scale, zero, flag, stream);
  });
}

size_t qlin_workspace_bytes(const qlin_qweight* w, int64_t M, int32_t r, int32_t pool) {
  if (check_layer(w, M, r, 0.0f, pool, 0) != QLIN_OK) return 0;
  const Plan p = make_plan(w, M, r, pool);
  return p.fits ? p.total : 0;
}

int qlin_fwd(const qlin_qweight* w, const uint16_t* x, int64_t M, const uint16_t* A,
             const uint16_t* B, int32_t r, float s, int32_t pool, uint16_t* y, float* u_out,
             void* workspace, size_t ws_bytes, hipStream_t stream) {
  const int st = check_fwd_args(w, x, M, A, B, r, s, pool, y, u_out);
  if (st != QLIN_OK) return st;
  const Plan p = make_plan(w, M, r, pool);
  if (!p.fits) return QLIN_E_SHAPE;
  if (workspace == nullptr || ws_bytes < p.total) return QLIN_E_WORKSPACE;
  if (!aligned16(workspace)) return QLIN_E_ALIGN;
  return fwd_core(w, x, M, A, B, r, s, pool, y, u_out, p, ws_at<float>(workspace, p.off_u),
                  ws_at<float>(workspace, p.off_partial), ws_at<uint32_t>(workspace, p.off_counters),
                  ws_at<uint8_t>(workspace, p.off_tc), stream);
}

int qlin_fwd_noalloc(const qlin_qweight* w, const uint16_t* x, int64_t M, const uint16_t* A,
                     const uint16_t* B, int32_t r, float s, int32_t pool, uint16_t* y,
                     float* u_out, hipStream_t stream) {
  const int st = check_fwd_args(w, x, M, A, B, r, s, pool, y, u_out);
  if (st != QLIN_OK) return st;
  const Plan p = make_plan(w, M, r, pool);
  if (!p.fits) return QLIN_E_SHAPE;
  const FwdScratch f = fwd_scratch_layout(w, M, r, pool, p);
  if (f.total > kScratchBytes) return QLIN_E_WORKSPACE;
  uint8_t* base = nullptr;
  const int sst = scratch_ptr(stream, &base);
  if (sst != QLIN_OK) return sst;
  return fwd_core(w, x, M, A, B, r, s, pool, y, u_out, p, reinterpret_cast<float*>(base + f.off_u),
                  reinterpret_cast<float*>(base + f.off_partial), reinterpret_cast<uint32_t*>(base),
                  base + f.off_tc, stream);
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
  if (!p.fits) return QLIN_E_SHAPE;
  if (workspace == nullptr || ws_bytes < p.total) return QLIN_E_WORKSPACE;
  if (!aligned16(workspace)) return QLIN_E_ALIGN;

  const int64_t N = w->d_out, K = w->d_in, G = K / pool;
  WeightView v;
  st = layer_view(w, ws_at<uint8_t>(workspace, p.off_tc), stream, &v);
  if (st != QLIN_OK) return st;
  const int fmt = fmt_of(w);
  float* partial = ws_at<float>(workspace, p.off_partial);
  uint32_t* counters = ws_at<uint32_t>(workspace, p.off_counters);
  float* du = ws_at<float>(workspace, p.off_du);
  uint16_t* Bt = ws_at<uint16_t>(workspace, p.off_Bt);

  // u (saved by the forward pass, or recomputed)
  const float* u = u_saved;
  if (u == nullptr) {
    float* uw = ws_at<float>(workspace, p.off_u);
    st = compute_u(w, x, M, A, r, pool, uw, p.nt_splits_u, partial, counters, stream);
    if (st != QLIN_OK) return st;
    u = uw;
  }
  if (p.small && !p.dx_stream) {
    // one launch: du, dB, dA and dX folded into the weight-streaming kernel
    GemvDxArgs a{};
    a.w = v; a.x = x; a.dy = dy; a.M = M; a.A = A; a.B = B; a.u = u; a.r = r; a.pool = pool;
    a.pool_shift = __builtin_ctz(static_cast<unsigned>(pool)); a.s = s;
    a.dx = dx; a.dA = dA; a.dB = dB; a.splits = p.gd_splits;
    a.partial = partial;
    a.du_part = partial + gemv_dx_partial_floats(N, K);
    a.counters = counters;
    return hip_status(hooked("k_gemv_dx", stream, [&] { return launch_gemv_dx(a, fmt, stream); }));
  }
  const int64_t jp = tn2_jp(r);
  uint16_t* zp = ws_at<uint16_t>(workspace, p.off_z);
  if (p.dx_stream) {
    // few tokens: du = s dY B and dB = s dY^T u in one launch (dA, which
    // needs the finished du, is formed by the streamed input gradient)
    AdapterFewArgs f{};
    f.dy = dy; f.M = M; f.N = N; f.B = B; f.u = u; f.r = r; f.s = s;
    f.du = du; f.dB = dB; f.shares = adapter_few_shares(N);
    f.partial = partial; f.counters = counters;
    QLIN_TRY(hooked("k_du_few", stream, [&] { return launch_du_few(f, stream); }));
  } else {
    // du = s dY B  (B^T staged so both operands are contiguous along n)
    QLIN_TRY(hooked("k_transpose16", stream, [&] { return launch_transpose16(B, N, r, Bt, stream); }));
    {
      NtArgs a{};
      a.X = dy; a.ldx = N; a.Y = Bt; a.ldy = N; a.C = du; a.ldc = r;
      a.M = M; a.K = N; a.J = r; a.splits = p.nt_splits_du; a.alpha = s;
      a.partial = partial; a.counters = counters;
      QLIN_TRY(hooked("k_nt_skinny", stream, [&] { return launch_nt_skinny(a, stream); }));
    }
    // dB = s dY^T u  (u as bf16 hi/lo planes)
    QLIN_TRY(hooked("k_split_hl", stream, [&] { return launch_split_hl(u, M, r, r, zp, zp + M * jp, stream); }));
    Tn2Args a{};
    a.X = dy; a.ldx = N; a.Zh = zp; a.Zl = zp + M * jp; a.C = dB; a.ldc = r;
    a.M = M; a.P = N; a.J = r; a.splits = p.tn2_splits_dB; a.out_transposed = 0; a.alpha = s;
    a.partial = partial; a.counters = counters;
    QLIN_TRY(hooked("k_tn2", stream, [&] { return launch_tn2(a, stream); }));
  }
  // dA = du^T P
  if (pool == 1 && p.dx_stream && dx != nullptr) {
    // formed per column panel by the streamed input gradient below
  } else if (pool == 1) {
    QLIN_TRY(hooked("k_split_hl", stream, [&] { return launch_split_hl(du, M, r, r, zp + 2 * M * jp, zp + 3 * M * jp, stream); }));
    Tn2Args a{};
    a.X = x; a.ldx = K; a.Zh = zp + 2 * M * jp; a.Zl = zp + 3 * M * jp; a.C = dA; a.ldc = K;
    a.M = M; a.P = K; a.J = r; a.splits = p.tn2_splits_dA; a.out_transposed = 1; a.alpha = 1.0f;
    a.partial = partial; a.counters = counters;
    QLIN_TRY(hooked("k_tn2", stream, [&] { return launch_tn2(a, stream); }));
  } else {
    QaArgs q{};
    q.x = x; q.A = A; q.du = du; q.M = M; q.K = K; q.G = G; q.r = r; q.pool = pool;
    q.P_out = ws_at<float>(workspace, p.off_P);
    QLIN_TRY(hooked("k_qa_pool_u", stream, [&] { return launch_qa_pool_u(q, stream); }));
    q.P_in = q.P_out;
    q.dA_out = dA;
    q.part = partial;
    QLIN_TRY(hooked("k_qa_dA", stream, [&] { return launch_qa_dA(q, stream); }));
  }
  if (dx == nullptr) return QLIN_OK;
  if (p.dx_stream) {
    // few tokens on a large weight: dX streamed, du A added in the fix-up
    DxStreamArgs a{};
    a.w = v; a.dy = dy; a.M = M; a.A = A; a.du = du; a.r = r;
    a.pool_shift = __builtin_ctz(static_cast<unsigned>(pool));
    a.adapter = (r > 0 && s != 0.0f) ? 1 : 0;
    a.dx = dx;
    a.x = x;
    a.dA = (r > 0 && pool == 1) ? dA : nullptr;
    a.splits = p.ds_splits;
    a.partial = partial;
    a.counters = counters;
    return hip_status(hooked("k_gemv_dx_stream", stream, [&] { return launch_gemv_dx_stream(a, fmt, stream); }));
  }
  // dX = dY W_bf16 + du A; with the pooled adapter A^T has one row per group
  // and column k of dX reads row k >> log2(pool)
  uint16_t* At = ws_at<uint16_t>(workspace, p.off_At);
  QLIN_TRY(hooked("k_transpose16", stream, [&] { return launch_transpose16(A, r, G, At, stream); }));
  DxArgs a{};
  a.w = v; a.dy = dy; a.M = M; a.At = At; a.du = du; a.r = r;
  a.pool = pool; a.pool_shift = __builtin_ctz(static_cast<unsigned>(pool));
  a.dx = dx;
  return hip_status(hooked("k_dx_gemm", stream, [&] { return launch_dx_gemm(a, fmt, stream); }));
}

int qlin_qa_merge(const qlin_qweight* w, const uint16_t* A, const uint16_t* B, int32_t r, float s,
                  uint16_t* zero_out, hipStream_t stream) {
  const int st = check_weight(w);
  if (st != QLIN_OK) return st;
  if (w->format != QLIN_FMT_INT4_GROUP) return QLIN_E_UNSUPPORTED;
  if (r < 1 || r > kMaxRank) return QLIN_E_SHAPE;
  if (!std::isfinite(s)) return QLIN_E_SHAPE;
  if (A == nullptr || B == nullptr || zero_out == nullptr) return QLIN_E_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(zero_out)) return QLIN_E_ALIGN;
  const int64_t G = w->d_in / w->block;
  return hip_status(launch_qa_merge(w->zero, A, B, w->d_out, G, r, s, zero_out, stream));
}

// ------------------------------------------ low-rank plus quantized (LQ)

namespace {

struct LqLayout {
  size_t off_r = 0, off_ut = 0, off_ct = 0, off_t = 0, off_g = 0, off_uinv = 0, off_p = 0, off_parts = 0,
         off_sums = 0, total = 0;
};

LqLayout lq_layout(int64_t N, int64_t K, int32_t r) {
  LqLayout l;
  size_t off = 0;
  const size_t f = sizeof(float);
  l.off_r = off;     off = align256(off + static_cast<size_t>(N) * K * f);
  l.off_ut = off;    off = align256(off + static_cast<size_t>(r) * N * f);
  l.off_ct = off;    off = align256(off + static_cast<size_t>(r) * K * f);
  l.off_t = off;     off = align256(off + static_cast<size_t>(r) * std::max(N, K) * f);
  l.off_g = off;     off = align256(off + static_cast<size_t>(r) * r * f);
  l.off_uinv = off;  off = align256(off + static_cast<size_t>(r) * ((r + 3) & ~3) * f);
  l.off_p = off;     off = align256(off + lq_gemm_scratch_floats(N, K, r) * f);
  l.off_parts = off; off = align256(off + static_cast<size_t>(lq_resid_parts(N * K)) * sizeof(double));
  l.off_sums = off;  off = align256(off + 4 * sizeof(double));
  l.total = off;
  return l;
}

}  // namespace

size_t qlin_lq_workspace_bytes(int64_t d_out, int64_t d_in, int32_t r) {
  if (d_out < 1 || d_in < 1 || r < 0 || r > kMaxRank) return 0;
  return lq_layout(d_out, d_in, r).total;
}

int qlin_lq_nf4(const float* W, int64_t d_out, int64_t d_in, int32_t r, int32_t iters, int32_t power,
                const float* omega_t, int32_t dq_block, uint8_t* codes, void* absmax, float* absmax2,
                uint16_t* B_out, uint16_t* A_out, float* err_out, void* workspace, size_t ws_bytes,
                hipStream_t stream) {
  if (W == nullptr || codes == nullptr || absmax == nullptr) return QLIN_E_NULL;
  if (dq_block != 0 && absmax2 == nullptr) return QLIN_E_NULL;
  if (dq_block != 0 && dq_block != 256) return QLIN_E_UNSUPPORTED;
  if (d_out < 1 || d_in < 1 || d_in % 64 != 0 || d_out % 16 != 0) return QLIN_E_SHAPE;
  if (d_out > (int64_t{1} << 40) / d_in) return QLIN_E_SHAPE;
  if (r < 0 || r > kMaxRank || r > d_out || r > d_in || iters < 1 || power < 0) return QLIN_E_SHAPE;
  if (r > 0 && (omega_t == nullptr || B_out == nullptr || A_out == nullptr)) return QLIN_E_NULL;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax) || (dq_block != 0 && !aligned16(absmax2)) ||
      (omega_t != nullptr && !aligned16(omega_t)))
    return QLIN_E_ALIGN;
  const LqLayout l = lq_layout(d_out, d_in, r);
  if (workspace == nullptr || ws_bytes < l.total) return QLIN_E_WORKSPACE;
  if (!aligned16(workspace)) return QLIN_E_ALIGN;
  const int64_t N = d_out, K = d_in;
  float* R = ws_at<float>(workspace, l.off_r);
  float* Ut = ws_at<float>(workspace, l.off_ut);
  float* Ct = ws_at<float>(workspace, l.off_ct);
  LqScratch sc{};
  sc.G = ws_at<float>(workspace, l.off_g);
  sc.Uinv = ws_at<float>(workspace, l.off_uinv);
  sc.T = ws_at<float>(workspace, l.off_t);
  sc.P = ws_at<float>(workspace, l.off_p);
  sc.parts = ws_at<double>(workspace, l.off_parts);
  sc.sums = ws_at<double>(workspace, l.off_sums);

  qlin_qweight q{};
  q.format = QLIN_FMT_NF4; q.d_out = N; q.d_in = K; q.block = 64; q.dq_block = dq_block;
  q.codes = codes; q.absmax = absmax; q.absmax2 = dq_block != 0 ? absmax2 : nullptr;
  const WeightView v = make_view(&q);
  float cb[16];
  nf4_levels(cb);
  double mids[15];
  for (int i = 0; i < 15; ++i) mids[i] = (static_cast<double>(cb[i]) + static_cast<double>(cb[i + 1])) / 2.0;
  const int64_t n_blocks = N * K / 64;

  QLIN_TRY(lq_sumsq(W, N * K, sc.sums + 2, sc, stream));
  for (int t = 0; t < iters; ++t) {
    // Q_t = NF4(W - L_{t-1}); L_0 = 0 quantizes W itself
    const float* D = W;
    if (t > 0 && r > 0) {
      QLIN_TRY(lq_subtract(W, Ut, Ct, N, K, r, R, sc, stream));
      D = R;
    }
    const int qs = run_flagged(stream, [&](uint32_t* flag) {
      return launch_quant_nf4(D, n_blocks, dq_block != 0 ? 1 : 0, mids, codes, absmax, absmax2, flag, stream);
    });
    if (qs != QLIN_OK) return qs;
    // R = W - W_bf16(Q_t), |R|^2
    QLIN_TRY(lq_resid(W, v, R, sc, stream));
    if (r > 0) {
      // U = orth(R Omega); power steps V = orth(R^T U), U = orth(R V); C = U^T R
      QLIN_TRY(lq_range(R, omega_t, N, K, r, Ut, sc, stream));
      for (int i = 0; i < power; ++i) {
        QLIN_TRY(lq_coords(R, Ut, N, K, r, Ct, sc, stream));
        QLIN_TRY(lq_orth(Ct, K, r, sc, stream));
        QLIN_TRY(lq_range(R, Ct, N, K, r, Ut, sc, stream));
      }
      QLIN_TRY(lq_coords(R, Ut, N, K, r, Ct, sc, stream));
      QLIN_TRY(lq_sumsq(Ct, static_cast<int64_t>(r) * K, sc.sums + 1, sc, stream));
    } else {
      QLIN_TRY(lq_sumsq(Ct, 0, sc.sums + 1, sc, stream));
    }
    if (err_out != nullptr) QLIN_TRY(lq_err(sc, err_out + t, stream));
  }
  if (r > 0) QLIN_TRY(lq_outputs(Ut, Ct, N, K, r, B_out, A_out, stream));
  return hip_status(hipStreamSynchronize(stream));
}

int qlin_int4_scale_zero_grad(const qlin_qweight* w, const uint16_t* x, int64_t M,
                              const uint16_t* dy, float* dscale, float* dzero,
                              hipStream_t stream) {
  const int st = check_weight(w);
  if (st != QLIN_OK) return st;
  if (w->format != QLIN_FMT_INT4_GROUP) return QLIN_E_UNSUPPORTED;
  if (M < 1 || M > (int64_t{1} << 31)) return QLIN_E_SHAPE;
  if (x == nullptr || dy == nullptr || dscale == nullptr || dzero == nullptr) return QLIN_E_NULL;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dscale) || !aligned16(dzero))
    return QLIN_E_ALIGN;
  LoqaArgs a{};
  a.codes = w->codes; a.x = x; a.dy = dy; a.dscale = dscale; a.dzero = dzero;
  a.M = M; a.N = w->d_out; a.K = w->d_in;
  return hip_status(hooked("k_int4_scale_zero_grad", stream,
                           [&] { return launch_int4_scale_zero_grad(a, stream); }));
}

int qlin_profile_next_launch(const char* kernel, hipEvent_t start, hipEvent_t stop) {
  ProfileHook& h = profile_hook();
  std::lock_guard<std::mutex> g(h.m);
  if (kernel == nullptr) {
    h.armed = false;
    return QLIN_OK;
  }
  if (start == nullptr || stop == nullptr) return QLIN_E_NULL;
  if (std::strlen(kernel) >= sizeof(h.name)) return QLIN_E_SHAPE;
  std::strcpy(h.name, kernel);
  h.start = start;
  h.stop = stop;
  h.armed = true;
  return QLIN_OK;
}

int qlin_dequant_bf16(const qlin_qweight* w, uint16_t* W_out, hipStream_t stream) {
  const int st = check_weight(w);
  if (st != QLIN_OK) return st;
  if (W_out == nullptr) return QLIN_E_NULL;
  if (!aligned16(W_out)) return QLIN_E_ALIGN;
  if (w->format == QLIN_FMT_NF)
    return hip_status(launch_dequant_nf(w->codes, w->absmax, w->absmax2, w->d_out * w->d_in, w->bits,
                                        w->block, w->dq_block != 0 ? 1 : 0, nf_table(w->bits), W_out,
                                        stream));
  const WeightView v = make_view(w);
  return hip_status(launch_dequant(v, fmt_of(w), W_out, stream));
}

}  // extern "C"
