// Weight-streaming kernels for few tokens (M <= 16), where the layer is bound
// by reading the packed 4-bit weight from HBM rather than by MFMA.
// [QLoRA "The QLoRA recipe" stage 3: decode each block to bf16 on the fly;
//  QA-LoRA abstract for INT4 groups.]
//
// Forward  y[m][n]  = sum_k x[m][k] W[n][k] + s sum_j u[m][j] B[n][j]
// Backward dX[m][k] = sum_n dY[m][n] W[n][k] + sum_j du[m][j] A[j][k]
//
// Both split the reduction across workgroups so that ~all of the weight is
// requested at once (the weight stream is a few bandwidth-delay products).
// Every lane decodes one whole 64-element block of a row (one lookup table
// per 64 weights), MFMA 16x16x32 does the token dimension.  Partial sums go
// to the workspace; the last workgroup of each output tile (atomic ticket)
// adds them in fixed order and applies the adapter term, so results are
// bit-identical from run to run.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

// ------------------------------------------------------------------ forward
constexpr int kGfRows = 64;    // output features per workgroup (4 waves x 16)
constexpr int kGfKC = 1024;    // reduction length per workgroup

template <int FMT>
__device__ __forceinline__ void gemv_luts(const WeightView& w, int64_t row, int64_t blk64, bool valid,
                                          Lut16 (&lut)[2]) {
  if (FMT == kFmtNF4) {
    lut[0] = valid ? make_lut<kFmtNF4>(w, row, blk64) : Lut16{};
    lut[1] = lut[0];
  } else {
    lut[0] = valid ? make_lut<kFmtINT4>(w, row, blk64 * 2) : Lut16{};
    lut[1] = valid ? make_lut<kFmtINT4>(w, row, blk64 * 2 + 1) : Lut16{};
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_fwd(GemvFwdArgs a) {
  // x chunk [16 tokens][1024 k] bf16, elements of every 8 permuted 0 2 4 6 1 3 5 7,
  // 16-byte chunks XOR-swizzled by token row.
  __shared__ __attribute__((aligned(16))) uint16_t s_x[16 * kGfKC];
  __shared__ uint32_t s_ticket;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t N = a.w.N, K = a.w.K, M = a.M;
  const int tiles = static_cast<int>((N + kGfRows - 1) / kGfRows);
  const int tile = static_cast<int>(blockIdx.x) % tiles;
  const int split = static_cast<int>(blockIdx.x) / tiles;
  const int64_t k0 = static_cast<int64_t>(split) * kGfKC;
  const int64_t klen = K - k0 < kGfKC ? K - k0 : kGfKC;

  // issue this lane's weight loads first: row, blocks c*256 + g*64 of the chunk
  const int64_t row = static_cast<int64_t>(tile) * kGfRows + wave * 16 + l16;
  const int64_t rowc = row < N ? row : N - 1;
  const uint8_t* crow = a.w.codes + rowc * (K >> 1);
  u32x4 cw[4][2];
  bool valid[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t kk = c * 256 + g * 64;
    valid[c] = kk < klen;
    if (valid[c]) {
      const uint8_t* p = crow + ((k0 + kk) >> 1);
      cw[c][0] = *reinterpret_cast<const u32x4*>(p);
      cw[c][1] = *reinterpret_cast<const u32x4*>(p + 16);
    } else {
      cw[c][0] = cw[c][1] = u32x4{0, 0, 0, 0};
    }
  }

  // stage x
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = i * 256 + tid;
    const int m = ch >> 7, q = ch & 127;
    u32x4 d = u32x4{0, 0, 0, 0};
    if (m < M && q * 8 < klen) d = *reinterpret_cast<const u32x4*>(a.x + m * K + k0 + q * 8);
    *reinterpret_cast<u32x4*>(&s_x[m * kGfKC + ((q ^ (m & 7)) << 3)]) = eo_permute(d);
  }
  __syncthreads();

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    Lut16 lut[2];
    gemv_luts<FMT>(a.w, rowc, (k0 + c * 256 + g * 64) >> 6, valid[c], lut);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const uint32_t word = cw[c][tt >> 2][tt & 3];
      const u32x4 wf = lut_decode8_eo(lut[tt >> 2], word);
      const int q = c * 32 + g * 8 + tt;
      const u32x4 xf = *reinterpret_cast<const u32x4*>(&s_x[l16 * kGfKC + ((q ^ (l16 & 7)) << 3)]);
      acc = mfma16(valid[c] ? wf : u32x4{0, 0, 0, 0}, xf, acc);
    }
  }

  // D[16 rows][16 tokens]: lane holds D[4g + v][l16]
  const int64_t nb = static_cast<int64_t>(tile) * kGfRows + wave * 16 + 4 * g;
  if (nb < N)
    *reinterpret_cast<f32x4*>(a.partial + (static_cast<int64_t>(split) * 16 + l16) * N + nb) = acc;
  __threadfence();
  __syncthreads();
  if (tid == 0) s_ticket = atomicAdd(a.counters + tile, 1u);
  __syncthreads();
  if (s_ticket != static_cast<uint32_t>(a.splits - 1)) return;
  __threadfence();

  // fix-up: 16 tokens x 64 features, 4 features per thread
  const int m = tid >> 4;
  const int64_t n = static_cast<int64_t>(tile) * kGfRows + (tid & 15) * 4;
  if (m < M && n < N) {
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.splits; ++sp)
      sum += __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(a.partial + (static_cast<int64_t>(sp) * 16 + m) * N + n));
    if (a.u != nullptr) {
      const float* ur = a.u + m * a.r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t* br = a.B + (n + e) * a.r;
        float t = 0.0f;
        for (int j = 0; j < a.r; ++j) t += ur[j] * bf16_to_f32(br[j]);
        sum[e] += a.s * t;
      }
    }
    u32x2 o;
    o.x = pack_bf16x2(sum[0], sum[1]);
    o.y = pack_bf16x2(sum[2], sum[3]);
    *reinterpret_cast<u32x2*>(a.y + m * N + n) = o;
  }
  if (tid == 0) a.counters[tile] = 0u;
}

// ----------------------------------------------------------------- backward
// Workgroup: 128 output columns k x a range of rows n (split).  Per chunk of
// 128 rows every thread decodes one 64-block of one row into LDS (natural
// [n][k] layout, swizzled); MFMA A-operands (8 consecutive n of one column)
// are gathered from it with 16-bit reads.
constexpr int kGdCols = 128;
constexpr int kGdRowsChunk = 128;
constexpr int kGdRowsSplit = 512;
constexpr int kGdRowBytes = kGdCols * 2;  // 256 B per row in LDS

__device__ __forceinline__ int gd_off(int n, int k) {
  // 16-byte chunk index of column k, swizzled by n so that a 16-bit gather
  // of rows n..n+7 over 16 columns hits distinct banks
  const int chunk = (k >> 3) ^ (((n >> 3) & 3) << 1);
  return n * kGdRowBytes + chunk * 16 + (k & 7) * 2;
}

template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_dx(GemvDxArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_w[kGdRowsChunk * kGdRowBytes];  // 32 KB
  __shared__ __attribute__((aligned(16))) uint16_t s_dy[16 * kGdRowsSplit];        // 16 KB
  __shared__ uint32_t s_ticket;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t N = a.w.N, K = a.w.K, M = a.M;
  const int tiles = static_cast<int>((K + kGdCols - 1) / kGdCols);
  const int tile = static_cast<int>(blockIdx.x) % tiles;
  const int split = static_cast<int>(blockIdx.x) / tiles;
  const int64_t kc0 = static_cast<int64_t>(tile) * kGdCols;
  const int64_t nb0 = static_cast<int64_t>(split) * kGdRowsSplit;
  const int64_t nlen = N - nb0 < kGdRowsSplit ? N - nb0 : kGdRowsSplit;

  // stage dY[0..15][nb0 .. nb0+nlen) (zeros outside)
  for (int ch = tid; ch < 16 * (kGdRowsSplit / 8); ch += 256) {
    const int m = ch / (kGdRowsSplit / 8), q = ch % (kGdRowsSplit / 8);
    u32x4 d = u32x4{0, 0, 0, 0};
    if (m < M && q * 8 < nlen) d = *reinterpret_cast<const u32x4*>(a.dy + m * N + nb0 + q * 8);
    *reinterpret_cast<u32x4*>(&s_dy[m * kGdRowsSplit + q * 8]) = d;
  }

  f32x4 acc[2];
  acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // decode assignment: thread -> row (tid >> 1) of the chunk, 64-block (tid & 1)
  const int drow = tid >> 1, dblk = tid & 1;
  for (int64_t ch0 = 0; ch0 < nlen; ch0 += kGdRowsChunk) {
    {
      const int64_t n = nb0 + ch0 + drow;
      const bool ok = (ch0 + drow) < nlen && (kc0 + dblk * 64) < K;
      const int64_t nc = n < N ? n : N - 1;
      const int64_t kb = kc0 + dblk * 64;
      u32x4 c0 = u32x4{0, 0, 0, 0}, c1 = u32x4{0, 0, 0, 0};
      Lut16 lut[2];
      if (ok) {
        const uint8_t* p = a.w.codes + nc * (K >> 1) + (kb >> 1);
        c0 = *reinterpret_cast<const u32x4*>(p);
        c1 = *reinterpret_cast<const u32x4*>(p + 16);
      }
      gemv_luts<FMT>(a.w, nc, kb >> 6, ok, lut);
      const uint32_t words[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const u32x4 d = ok ? lut_decode8(lut[tt >> 2], words[tt]) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(&s_w[gd_off(drow, dblk * 64 + tt * 8)]) = d;
      }
    }
    __syncthreads();
    // MFMA: D[k][m] += sum_n W[n][k] dY[m][n]; wave w owns columns [32w, 32w+32)
#pragma unroll
    for (int ns = 0; ns < kGdRowsChunk / 32; ++ns) {
      const int nbase = ns * 32 + g * 8;
      const u32x4 bfr = *reinterpret_cast<const u32x4*>(&s_dy[l16 * kGdRowsSplit + ch0 + nbase]);
#pragma unroll
      for (int ksub = 0; ksub < 2; ++ksub) {
        const int kcol = wave * 32 + ksub * 16 + l16;
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = *reinterpret_cast<const uint16_t*>(&s_w[gd_off(nbase + 2 * e, kcol)]);
          const uint32_t hi = *reinterpret_cast<const uint16_t*>(&s_w[gd_off(nbase + 2 * e + 1, kcol)]);
          v[e] = lo | (hi << 16);
        }
        acc[ksub] = mfma16(u32x4{v[0], v[1], v[2], v[3]}, bfr, acc[ksub]);
      }
    }
    __syncthreads();
  }

  // D[16 k][16 m]: lane holds D[4g + v][l16] -> k = kc0 + 32w + 16 ksub + 4g + v, m = l16
#pragma unroll
  for (int ksub = 0; ksub < 2; ++ksub) {
    const int64_t k = kc0 + wave * 32 + ksub * 16 + 4 * g;
    if (k < K)
      *reinterpret_cast<f32x4*>(a.partial + (static_cast<int64_t>(split) * 16 + l16) * K + k) = acc[ksub];
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_ticket = atomicAdd(a.counters + tile, 1u);
  __syncthreads();
  if (s_ticket != static_cast<uint32_t>(a.splits - 1)) return;
  __threadfence();

  // fix-up: 16 tokens x 128 columns; thread -> token (tid >> 4), 8 columns
  const int m = tid >> 4;
  const int64_t k = kc0 + (tid & 15) * 8;
  if (m < M && k < K) {
    float sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = 0.0f;
    for (int sp = 0; sp < a.splits; ++sp) {
      const float* p = a.partial + (static_cast<int64_t>(sp) * 16 + m) * K + k;
      const f32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
      const f32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sum[e] += v0[e];
        sum[4 + e] += v1[e];
      }
    }
    if (a.du != nullptr) {
      const float* dr = a.du + m * a.r;
      const int64_t ka = K;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (a.pool == 1) {
          float t = 0.0f;
          for (int j = 0; j < a.r; ++j) t += dr[j] * bf16_to_f32(a.A[static_cast<int64_t>(j) * ka + k + e]);
          sum[e] += t;
        }
      }
    }
    if (a.Gq != nullptr) {
      const int64_t G = K >> a.pool_shift;
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] += a.Gq[m * G + ((k + e) >> a.pool_shift)];
    }
    u32x4 o;
    o.x = pack_bf16x2(sum[0], sum[1]);
    o.y = pack_bf16x2(sum[2], sum[3]);
    o.z = pack_bf16x2(sum[4], sum[5]);
    o.w = pack_bf16x2(sum[6], sum[7]);
    *reinterpret_cast<u32x4*>(a.dx + m * K + k) = o;
  }
  if (tid == 0) a.counters[tile] = 0u;
}

}  // namespace

int gemv_fwd_splits(int64_t K) { return static_cast<int>((K + kGfKC - 1) / kGfKC); }
int gemv_fwd_tiles(int64_t N) { return static_cast<int>((N + kGfRows - 1) / kGfRows); }
int64_t gemv_fwd_partial_floats(int64_t N, int64_t K) { return gemv_fwd_splits(K) * 16 * N; }

hipError_t launch_gemv_fwd(const GemvFwdArgs& a, int fmt, hipStream_t stream) {
  const int grid = gemv_fwd_tiles(a.w.N) * a.splits;
  if (fmt == kFmtNF4)
    hipLaunchKernelGGL(k_gemv_fwd<kFmtNF4>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_gemv_fwd<kFmtINT4>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

int gemv_dx_splits(int64_t N) { return static_cast<int>((N + kGdRowsSplit - 1) / kGdRowsSplit); }
int gemv_dx_tiles(int64_t K) { return static_cast<int>((K + kGdCols - 1) / kGdCols); }
int64_t gemv_dx_partial_floats(int64_t N, int64_t K) { return gemv_dx_splits(N) * 16 * K; }

hipError_t launch_gemv_dx(const GemvDxArgs& a, int fmt, hipStream_t stream) {
  const int grid = gemv_dx_tiles(a.w.K) * a.splits;
  if (fmt == kFmtNF4)
    hipLaunchKernelGGL(k_gemv_dx<kFmtNF4>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_gemv_dx<kFmtINT4>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
