// Gradients of the INT4 group scales and zero points (trainable
// quantization parameters).  [LoQA abstract: the scale and the zero point
// of the quantized weight are fine-tuned through a LoRA-compatible operator;
// QA-LoRA abstract for the group-wise INT4 weight]
//
// With W[n][k] = alpha[n][g] q[n][k] + beta[n][g] (g = k / 32) and
// y = x W^T, the gradients of <dY, y> are
//     dalpha[n][g] = sum_{k in g} q[n][k] dW[n][k],
//     dbeta[n][g]  = sum_{k in g} dW[n][k],      dW = dY^T x,
// the bf16 rounding of W passed straight through.  dW is formed tile by
// tile with bf16 MFMAs (a 2 M N K flop contraction over the tokens) and
// reduced to the group sums in registers; it never reaches memory.
//
// A workgroup owns a 128 (n) x 128 (k) tile of dW (four waves of 64 x 64)
// and runs over all tokens in steps of 32: the step's dY[m][n0..] and
// x[m][k0..] slices are staged row-major in LDS, and the transposing LDS
// read turns 8 consecutive tokens of one column into an MFMA operand.  The
// next step's slices are loaded into registers during the current step's
// MFMAs.  Sums run in a fixed order: results are identical from run to run.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kLqT = 128;                // tile edge (n and k)
constexpr int kLqM = 32;                 // tokens per step
constexpr int kLqStride = kLqT * 2 + 16; // staged row: 272 B (bank spread)

__global__ __launch_bounds__(256) void k_int4_scale_zero_grad(LoqaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_dy[kLqM * kLqStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_x[kLqM * kLqStride];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int tiles_k = static_cast<int>((K + kLqT - 1) / kLqT);
  const int tn = static_cast<int>(blockIdx.x) / tiles_k, tk = static_cast<int>(blockIdx.x) % tiles_k;
  const int64_t n0 = static_cast<int64_t>(tn) * kLqT, k0 = static_cast<int64_t>(tk) * kLqT;
  const int wn = (wave >> 1) * 64, wk = (wave & 1) * 64;  // the wave's 64 x 64 block

  // staging: thread t moves 16-byte pieces t and t + 256 of each slice
  // (32 rows x 16 pieces); pieces past M, N or K are zero
  auto load_slice = [&](const uint16_t* src, int64_t ld, int64_t c0, int64_t cmax, int64_t m0,
                        u32x4 (&v)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 256 * i;
      const int row = piece >> 4, col = (piece & 15) * 8;
      const int64_t m = m0 + row, c = c0 + col;
      const bool ok = m < M && c < cmax;
      v[i] = ok ? *reinterpret_cast<const u32x4*>(src + m * ld + c) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_slice = [&](uint8_t* dst, const u32x4 (&v)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 256 * i;
      *reinterpret_cast<u32x4*>(dst + (piece >> 4) * kLqStride + (piece & 15) * 16) = v[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t steps = (M + kLqM - 1) / kLqM;
  u32x4 vd[2], vx[2];
  load_slice(a.dy, N, n0, N, 0, vd);
  load_slice(a.x, K, k0, K, 0, vx);
  for (int64_t st = 0; st < steps; ++st) {
    __syncthreads();  // the previous step's operands are consumed
    store_slice(s_dy, vd);
    store_slice(s_x, vx);
    __syncthreads();
    if (st + 1 < steps) {
      load_slice(a.dy, N, n0, N, (st + 1) * kLqM, vd);
      load_slice(a.x, K, k0, K, (st + 1) * kLqM, vx);
    }
    u32x4 an[4], bk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      an[i] = tr16_operand(s_dy, kLqStride, 8 * g, wn + 16 * i, l16);
      bk[i] = tr16_operand(s_x, kLqStride, 8 * g, wk + 16 * i, l16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(an[i], bk[j], acc[i][j]);
  }

  // epilogue: lane (l16, g) holds dW[n = wn + 16 i + 4 g + v][k = wk + 16 j + l16];
  // group c of the wave's 64 columns is made of column blocks j = 2c, 2c + 1
  const int64_t G = K >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t n = n0 + wn + 16 * i + 4 * g + v;
      const int64_t nc = n < N ? n : N - 1;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float sa = 0.0f, sb = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 2 * c + h;
          int64_t k = k0 + wk + 16 * j + l16;
          k = k < K ? k : K - 1;
          const uint8_t byte = a.codes[nc * (K >> 1) + (k >> 3) * 4 + (k & 3)];
          const float q = static_cast<float>((k & 4) ? (byte >> 4) : (byte & 15));
          const float d = acc[i][j][v];
          sa += q * d;
          sb += d;
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          sa += __shfl_xor(sa, o, 64);
          sb += __shfl_xor(sb, o, 64);
        }
        const int64_t gg = (k0 + wk) / 32 + c;
        if (l16 == 0 && n < N && gg < G) {
          a.dscale[n * G + gg] = sa;
          a.dzero[n * G + gg] = sb;
        }
      }
    }
  }
}

}  // namespace

int64_t loqa_tiles(int64_t N, int64_t K) { return ((N + kLqT - 1) / kLqT) * ((K + kLqT - 1) / kLqT); }

hipError_t launch_int4_scale_zero_grad(const LoqaArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_int4_scale_zero_grad, dim3(static_cast<uint32_t>(loqa_tiles(a.N, a.K))),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
