// Adapter gradients for few tokens (M <= 16), with fixed summation order.
// ["Background: how LoRA works": y = x W^T + s (x A^T) B^T, so with
// u = x A^T the gradients are du = s dY B, dB = s dY^T u, dA = du^T x]
//
// k_du_few:  du = s dY B and dB = s dY^T u, as two ranges of one grid.
//   du: the reduction runs over the N rows of dY^T and B, split into up to
//   32 shares of 256-row chunks; a workgroup stages a chunk of B in LDS and
//   forms its share with MFMAs on the bf16 inputs (exact products, fp32
//   sums).  Shares publish fp32 partial sums (write-through stores) and the
//   last share's workgroup (atomic ticket) adds them in share order, every
//   thread one element with sixteen shares' loads in flight.
//   dB: a thread forms sixteen adapter columns of one row of dB in fp32
//   FMAs over the tokens in order.
// (dA = du^T x needs the finished du: the streamed input-gradient kernel
// forms it per column panel after its own reduction.)
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kAfThreads = 256;
constexpr int kAfChunk = 256;                 // rows of B staged at a time
constexpr int kAfMaxShares = 32;
constexpr int kAfMaxR = 128;
constexpr int kAfBStride = kAfMaxR * 2 + 16;  // staged B row in bytes (zero-padded)

int du_shares(int64_t N) {
  const int64_t chunks = (N + kAfChunk - 1) / kAfChunk;
  return static_cast<int>(chunks < kAfMaxShares ? chunks : kAfMaxShares);
}

// dB rows for blocks past the du shares: thread (t % 64 -> row n, t / 64 ->
// 16-column group of the adapter) forms sixteen independent fp32 sums over
// the tokens, in token order.  The thread's sixteen dY values load before
// the staging barrier, so that they are in flight with the staging loads.
__device__ __forceinline__ void db_block(const AdapterFewArgs& a, int block, float (*s_t)[kAfMaxR]) {
  const int tid = threadIdx.x;
  const int64_t M = a.M, N = a.N;
  const int r = a.r;
  const int ngrp = (r + 15) / 16;
  const int64_t unit = static_cast<int64_t>(block) * 4 + (tid >> 6);
  const int sub = tid & 63;
  const int jg = static_cast<int>(unit % ngrp);
  const int64_t n = unit / ngrp * 64 + sub;
  const bool ok = unit < (N + 63) / 64 * ngrp && n < N;
  float tv[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) tv[m] = (ok && m < M) ? bf16_to_f32(a.dy[m * N + n]) : 0.0f;
  {
    constexpr int kPer = 16 * kAfMaxR / kAfThreads;
    float v[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = tid + e * kAfThreads, m = i / kAfMaxR, j = i % kAfMaxR;
      v[e] = (m < M && j < r) ? a.u[m * r + j] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = tid + e * kAfThreads;
      s_t[i / kAfMaxR][i % kAfMaxR] = v[e];
    }
  }
  __syncthreads();
  if (!ok) return;
  f32x4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 2
  for (int m = 0; m < 16; ++m) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 uu = *reinterpret_cast<const f32x4*>(&s_t[m][16 * jg + 4 * q]);
      acc[q][0] = __builtin_fmaf(tv[m], uu[0], acc[q][0]);
      acc[q][1] = __builtin_fmaf(tv[m], uu[1], acc[q][1]);
      acc[q][2] = __builtin_fmaf(tv[m], uu[2], acc[q][2]);
      acc[q][3] = __builtin_fmaf(tv[m], uu[3], acc[q][3]);
    }
  }
  uint16_t* dbrow = a.dB + n * r + 16 * jg;
  if (r % 16 == 0) {
    // sixteen columns = 32 bytes of the row, 16-byte aligned
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 8 * h + 2 * e;
        w[e] = static_cast<uint32_t>(f32_to_bf16(a.s * acc[c / 4][c % 4])) |
               (static_cast<uint32_t>(f32_to_bf16(a.s * acc[(c + 1) / 4][(c + 1) % 4])) << 16);
      }
      *reinterpret_cast<u32x4*>(dbrow + 8 * h) = u32x4{w[0], w[1], w[2], w[3]};
    }
  } else {
#pragma unroll
    for (int c = 0; c < 16; ++c)
      if (16 * jg + c < r) dbrow[c] = f32_to_bf16(a.s * acc[c / 4][c % 4]);
  }
}

__global__ __launch_bounds__(kAfThreads) void k_du_few(AdapterFewArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_b[kAfChunk * kAfBStride];  // B rows (bf16)
  __shared__ uint32_t s_ticket;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t M = a.M, N = a.N;
  const int r = a.r;
  const int rp = (r + 15) & ~15;  // adapter columns in whole 16-column tiles
  const int ntile = rp / 16;
  const int S = a.shares;
  if (static_cast<int>(blockIdx.x) >= S) {
    db_block(a, static_cast<int>(blockIdx.x) - S, reinterpret_cast<float (*)[kAfMaxR]>(s_b));
    return;
  }
  const int64_t nchunk = (N + kAfChunk - 1) / kAfChunk;
  const int64_t per = (nchunk + S - 1) / S;
  const int64_t c0 = blockIdx.x * per, c1 = c0 + per < nchunk ? c0 + per : nchunk;

  // lane (l16, g) holds D[m = 4 g + v][j = 16 tile + l16]; wave w takes
  // adapter-column tiles w, w + 4
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const uint16_t* dyrow = a.dy + static_cast<int64_t>(l16 < M ? l16 : M - 1) * N;
  for (int64_t ch = c0; ch < c1; ++ch) {
    const int64_t n0 = ch * kAfChunk;
    const int nrows = static_cast<int>(N - n0 < kAfChunk ? N - n0 : kAfChunk);
    __syncthreads();  // the previous chunk's reads are done
    if (r % 8 == 0) {
      // the chunk's rows are contiguous: 16 bytes per load, a thread's loads
      // all in flight before its LDS stores
      constexpr int kPer = kAfChunk * (kAfMaxR / 8) / kAfThreads;
      const int q8 = rp / 8, per_row = r / 8;
      u32x4 v[kPer];
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int i = tid + e * kAfThreads;
        const int c = i / q8, q = i % q8;
        v[e] = (c < nrows && q < per_row && i < kAfChunk * q8)
                   ? *reinterpret_cast<const u32x4*>(a.B + (n0 + c) * r + 8 * q)
                   : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int i = tid + e * kAfThreads;
        if (i < kAfChunk * q8) *reinterpret_cast<u32x4*>(s_b + (i / q8) * kAfBStride + 16 * (i % q8)) = v[e];
      }
    } else {
      for (int i = tid; i < kAfChunk * rp; i += kAfThreads) {
        const int c = i / rp, j = i % rp;
        reinterpret_cast<uint16_t*>(s_b + c * kAfBStride)[j] = (c < nrows && j < r) ? a.B[(n0 + c) * r + j] : 0u;
      }
    }
    // this lane's dY operands of the chunk (8 rows each, all in or all out)
    u32x4 aop[kAfChunk / 32];
#pragma unroll
    for (int kk = 0; kk < kAfChunk / 32; ++kk) {
      const int c = kk * 32 + 8 * g;
      aop[kk] = c < nrows ? *reinterpret_cast<const u32x4*>(dyrow + n0 + c) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kAfChunk / 32; ++kk) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int tile = wave + 4 * t;
        if (tile < ntile) {
          // rows kk 32 + 8 g .. + 7 of column 16 tile + l16, read transposed
          const uint8_t* p0 = s_b + (kk * 32 + 8 * g + (l16 >> 2)) * kAfBStride + (16 * tile + 4 * (l16 & 3)) * 2;
          const u32x2 lo = ds_read_tr16(p0), hi = ds_read_tr16(p0 + 4 * kAfBStride);
          acc[t] = mfma16(aop[kk], u32x4{lo.x, lo.y, hi.x, hi.y}, acc[t]);
        }
      }
    }
  }
  if (S > 1) {
    const rsrc_t pr = make_rsrc(a.partial);
    // partial of share sh, tile t, lane l at ((sh * 8 + t) * 64 + l) * 16 bytes
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (wave + 4 * t < ntile)
        st_sys16(pr, static_cast<uint32_t>(((static_cast<int64_t>(blockIdx.x) * 8 + wave + 4 * t) * 64 + lane) * 16), acc[t]);
    if (__builtin_amdgcn_readfirstlane(publish_and_ticket(a.counters, &s_ticket)) != static_cast<uint32_t>(S - 1))
      return;
    // thread (tile = wave + 4 t, lane) adds its element over the shares in
    // order, sixteen shares' loads in flight at a time
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
      if (wave + 4 * t < ntile) {
        for (int s0 = 0; s0 < S; s0 += 16) {
          f32x4 part[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int sh = s0 + q < S ? s0 + q : S - 1;
            part[q] = ld_sys16(pr, static_cast<uint32_t>(((static_cast<int64_t>(sh) * 8 + wave + 4 * t) * 64 + lane) * 16));
          }
#pragma unroll
          for (int q = 0; q < 16; ++q)
            if (s0 + q < S) sum += part[q];
        }
      }
      acc[t] = sum;
    }
    if (tid == 0) a.counters[0] = 0u;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = 16 * (wave + 4 * t) + l16;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < M && j < r) a.du[m * r + j] = a.s * acc[t][v];
    }
  }
}

}  // namespace

int adapter_few_shares(int64_t N) { return du_shares(N); }
int64_t adapter_few_partial_floats(int64_t N) {
  const int S = du_shares(N);
  return S > 1 ? static_cast<int64_t>(S) * 8 * 64 * 4 : 0;
}

static int db_few_blocks(int64_t N, int r) { return static_cast<int>(((N + 63) / 64 * ((r + 15) / 16) + 3) / 4); }

hipError_t launch_du_few(const AdapterFewArgs& a, hipStream_t stream) {
  // a.shares workgroups of du, then the dB rows
  hipLaunchKernelGGL(k_du_few, dim3(static_cast<uint32_t>(a.shares + db_few_blocks(a.N, a.r))), dim3(kAfThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace qlin
