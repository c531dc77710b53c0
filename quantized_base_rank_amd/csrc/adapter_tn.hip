// Adapter gradients for many tokens, as streaming reductions over the token
// dimension.  [QLoRA "The QLoRA recipe: quantize, then adapt": gradients
// reach the adapter only; "Background: how LoRA works" for the product.]
//
//   C[p][j] = alpha * sum_m X[m][p] Z[m][j]
//     dB = s dY^T u   (X = dY, P = d_out, Z = u,  C = dB [d_out][r])
//     dA = du^T x     (X = x,  P = d_in,  Z = du, C = dA [r][d_in], transposed)
//
// The work is one pass over X (dY or x), which is large; u / du are narrow.
// A workgroup owns 128 columns of X and a share of the tokens.  Each 32-token
// stage of X and of Z is copied to LDS in its natural layout with whole-line
// direct-to-LDS loads into a ring of stages (four for r <= 64, three above),
// issued that many stages less one ahead, so that two workgroups per compute
// unit keep up to 48 KB of X in flight (r <= 64); the transposing LDS read (ds_read_b64_tr_b16)
// turns 8 consecutive tokens of one column into an MFMA operand, so neither
// operand is transposed in memory.  Z enters the bf16 MFMA as two planes,
// hi = bf16(z) and lo = bf16(z - hi), keeping its fp32 precision.  Token
// shares publish fp32 partial sums with write-through stores; the last
// workgroup of a column tile (atomic ticket) adds them in fixed order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// fp32 [M][J] -> bf16 hi and lo planes [M][JP] (columns J..JP-1 zero).
__global__ __launch_bounds__(256) void k_split_hl(const float* __restrict__ Z, int64_t M, int J,
                                                  int64_t ldz, int JP, uint16_t* __restrict__ Zh,
                                                  uint16_t* __restrict__ Zl) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= M * JP) return;
  const int64_t m = t / JP;
  const int j = static_cast<int>(t - m * JP);
  const float z = j < J ? Z[m * ldz + j] : 0.0f;
  float hi, lo;
  split_bf16(z, hi, lo);
  Zh[t] = static_cast<uint16_t>(__float_as_uint(hi) >> 16);
  Zl[t] = f32_to_bf16(lo);
}

constexpr int kTp = 128;  // columns of X per workgroup
constexpr int kTm = 32;   // tokens per stage

// 16-byte chunk swizzle of a staged row: 16 lanes of a transposing read take
// 4 consecutive rows x 2 adjacent chunks; XOR-ing the chunk index with
// 2 * (row % 4) puts those 8 chunks in distinct banks.  Rows 8 apart (the
// other half-wave) flip chunk bit 3 when a row has 16 chunks.
template <int CHUNKS>
__device__ __forceinline__ int tn_swz(int row) {
  return ((row & 3) << 1) ^ (CHUNKS >= 16 ? (((row >> 3) & 1) << 3) : 0);
}

// Byte offset of element (row, col) in a staged tile of CHUNKS 16-byte
// chunks per row.
template <int CHUNKS>
__device__ __forceinline__ int tn_off(int row, int col) {
  const int byte = col * 2;
  return row * CHUNKS * 16 + ((((byte >> 4) ^ tn_swz<CHUNKS>(row))) << 4) + (byte & 15);
}

// MFMA operand from a staged tile: 8 consecutive rows kbase..kbase+7 of
// column c0 + p (p = lane within its 16-lane group).
template <int CHUNKS>
__device__ __forceinline__ u32x4 tn_operand(const uint8_t* tile, int kbase, int c0, int p) {
  const int r0 = kbase + (p >> 2), c = c0 + 4 * (p & 3);
  const u32x2 lo = ds_read_tr16(tile + tn_off<CHUNKS>(r0, c));
  const u32x2 hi = ds_read_tr16(tile + tn_off<CHUNKS>(r0 + 4, c));
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// Workgroups are dealt to the 8 XCDs round-robin: give each XCD a contiguous
// run of (share, tile) pairs so that the workgroups on one XCD read the same
// token share of Z from its L2.
__device__ __forceinline__ int tn_xcd_order(int bid, int n) {
  const int q = n >> 3, rem = n & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

template <int JP>
__global__ __launch_bounds__(256) void k_tn2(Tn2Args a) {
  constexpr int JG = JP / 16;              // 16-wide groups of j
  constexpr int kXC = kTp * 2 / 16;        // 16 chunks per X row
  constexpr int kZC = JP * 2 / 16;         // 8 or 16 chunks per Z row
  constexpr int kXB = kTm * kTp * 2;       // 8 KB
  constexpr int kZB = kTm * JP * 2;        // 4 or 8 KB per plane
  constexpr int kStage = kXB + 2 * kZB;
  constexpr int kRing = JP == 64 ? 4 : 3;  // 64 or 72 KB: two workgroups per compute unit
  // one array per ring slot: a read of one slot then does not wait for the
  // direct-to-LDS loads still landing in the others
  __shared__ __attribute__((aligned(16))) uint8_t s0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t s1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t s2[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t s3[kRing == 4 ? kStage : 16];
  __shared__ uint32_t s_ticket;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int tiles = static_cast<int>((a.P + kTp - 1) / kTp);
  const int lin = tn_xcd_order(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int tile = lin % tiles, split = lin / tiles;
  const int64_t p0 = static_cast<int64_t>(tile) * kTp;
  const int64_t per = (a.M + a.splits - 1) / a.splits;
  const int64_t mb0 = static_cast<int64_t>(split) * per;
  const int64_t mb1 = mb0 + per < a.M ? mb0 + per : a.M;
  const int nstages = mb1 > mb0 ? static_cast<int>((mb1 - mb0 + kTm - 1) / kTm) : 0;

  // Buffer resources over this share's rows: tokens past the share fall
  // outside them and read as zero.  Columns past P in the last tile read the
  // next row's values; their outputs are never stored.
  const int64_t rows = mb1 - mb0;
  const rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.X + mb0 * a.ldx + p0), 0,
      static_cast<int>(rows > 0 ? (rows - 1) * a.ldx * 2 + (a.P - p0) * 2 : 0), 0x00020000);
  const rsrc_t zhr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.Zh + mb0 * JP), 0, static_cast<int>(rows * JP * 2), 0x00020000);
  const rsrc_t zlr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.Zl + mb0 * JP), 0, static_cast<int>(rows * JP * 2), 0x00020000);

  // stage loads: X 8 instructions of 4 rows x 256 B; each Z plane
  // kZB / 1 KB instructions of (1024 / (kZC * 16)) rows; instruction i is
  // issued by wave i % 4, so every wave issues kStageLoads per stage.  A stage
  // past the share starts at its end and reads zeros (outside the resources).
  auto load_stage = [&](int st, uint8_t* sb) {
    const uint32_t m_rel = static_cast<uint32_t>((st < nstages ? st : nstages) * kTm);
#pragma unroll
    for (int ii = 0; ii < kXB / 4096; ++ii) {
      const int i = ii * 4 + wave;
      const int row = 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ tn_swz<kXC>(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (lds_ptr_t)(sb + i * 1024), 16,
          static_cast<uint32_t>(((lane >> 4) * a.ldx) * 2 + c * 16),
          static_cast<int>((m_rel + 4 * i) * a.ldx * 2), 0, 0);
    }
    constexpr int ZROWS = 1024 / (kZC * 16);  // rows per instruction
    constexpr int ZINS = kZB / 1024;          // instructions per plane
#pragma unroll
    for (int ii = 0; ii < ZINS / 4; ++ii) {
      const int i = ii * 4 + wave;
      const int row = ZROWS * i + lane / kZC;
      const int c = (lane % kZC) ^ tn_swz<kZC>(row);
      const uint32_t voff = static_cast<uint32_t>((lane / kZC) * JP * 2 + c * 16);
      const int soff = static_cast<int>((m_rel + ZROWS * i) * JP * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(zhr, (lds_ptr_t)(sb + kXB + i * 1024), 16, voff,
                                               soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(zlr, (lds_ptr_t)(sb + kXB + kZB + i * 1024), 16,
                                               voff, soff, 0, 0);
    }
  };

  f32x4 acc[2][JG];
#pragma unroll
  for (int pg = 0; pg < 2; ++pg)
#pragma unroll
    for (int jg = 0; jg < JG; ++jg) acc[pg][jg] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage st sits in ring slot st % kRing.  The loads of stage st + kRing - 1
  // go into the slot of stage st - 1 after the barrier that ends its use;
  // every iteration issues them (past the share they read zeros), so the
  // wait before stage st always leaves exactly kRing - 2 stages in flight.
  // The stage loop is unrolled by kRing, so that each slot is a fixed array,
  // and runs whole turns of the ring: the stages past the share hold zeros
  // and add nothing.  (An early exit inside the turn makes the compiler merge
  // the pending loads of every slot at the loop head and wait for all of them
  // before the first read.)
  static_assert(kZB / 1024 % 4 == 0, "Z plane loads split evenly over the waves");
  if (nstages > 0) {
#pragma unroll
    for (int i = 0; i < kRing - 1; ++i)
      load_stage(i, i == 0 ? s0 : i == 1 ? s1 : s2);
  }
  for (int st0 = 0; st0 < nstages; st0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int st = st0 + i;
      // this wave's loads of stage st have landed and its reads of stage
      // st - 1 are done, then the waves meet (one asm block: a fence here
      // would wait for every direct-to-LDS load in flight)
      if constexpr (kRing == 4)  // 2 stages x (2 X + 2 Z) loads stay in flight
        __asm__ volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else  // 1 stage x (2 X + 4 Z) loads
        __asm__ volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const int nx = (i + kRing - 1) % kRing;
      load_stage(st + kRing - 1, nx == 0 ? s0 : nx == 1 ? s1 : nx == 2 ? s2 : s3);
      const uint8_t* xs = i == 0 ? s0 : i == 1 ? s1 : i == 2 ? s2 : s3;
      const uint8_t* zh = xs + kXB;
      const uint8_t* zl = xs + kXB + kZB;
#pragma unroll
      for (int kb = 0; kb < kTm; kb += 32) {
        u32x4 af[2];
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) af[pg] = tn_operand<kXC>(xs, kb + 8 * g, wave * 32 + pg * 16, l16);
#pragma unroll
        for (int jg = 0; jg < JG; ++jg) {
          const u32x4 bh = tn_operand<kZC>(zh, kb + 8 * g, jg * 16, l16);
          const u32x4 bl = tn_operand<kZC>(zl, kb + 8 * g, jg * 16, l16);
#pragma unroll
          for (int pg = 0; pg < 2; ++pg) {
            acc[pg][jg] = mfma16(af[pg], bh, acc[pg][jg]);
            acc[pg][jg] = mfma16(af[pg], bl, acc[pg][jg]);
          }
        }
      }
    }
  }

  // the loads issued past the share land in LDS before the workgroup ends
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // lane (l16, g) of tile (pg, jg) holds D[p = 32 w + 16 pg + 4 g + v][j = 16 jg + l16]
  const int S = a.splits;
  if (S > 1) {
    // partial layout [tile][split][wave][pg][jg][lane] x f32x4
    const int64_t per_wg = 4 * 2 * JG * 64 * 4;
    const rsrc_t pr = make_rsrc(a.partial);
    const int64_t mine = (static_cast<int64_t>(tile) * S + split) * per_wg;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int jg = 0; jg < JG; ++jg)
        st_sys16(pr, static_cast<uint32_t>((mine + (((wave * 2 + pg) * JG + jg) * 64 + lane) * 4) * 4),
                 acc[pg][jg]);
    if (publish_and_ticket(a.counters + tile, &s_ticket) != static_cast<uint32_t>(S - 1)) return;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int jg = 0; jg < JG; ++jg) acc[pg][jg] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < S; ++sp) {
      const int64_t base = (static_cast<int64_t>(tile) * S + sp) * per_wg;
      f32x4 v[2][JG];
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int jg = 0; jg < JG; ++jg)
          v[pg][jg] = ld_sys16(pr, static_cast<uint32_t>((base + (((wave * 2 + pg) * JG + jg) * 64 + lane) * 4) * 4));
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int jg = 0; jg < JG; ++jg) acc[pg][jg] += v[pg][jg];
    }
    if (tid == 0) a.counters[tile] = 0u;
  }
#pragma unroll
  for (int pg = 0; pg < 2; ++pg)
#pragma unroll
    for (int jg = 0; jg < JG; ++jg) {
      const int j = jg * 16 + l16;
      if (j >= a.J) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t p = p0 + wave * 32 + pg * 16 + 4 * g + v;
        if (p >= a.P) continue;
        const uint16_t o = f32_to_bf16(a.alpha * acc[pg][jg][v]);
        if (a.out_transposed)
          a.C[static_cast<int64_t>(j) * a.ldc + p] = o;
        else
          a.C[p * a.ldc + j] = o;
      }
    }
}

}  // namespace

int tn2_jp(int J) { return J <= 64 ? 64 : 128; }
int tn2_tiles(int64_t P) { return static_cast<int>((P + kTp - 1) / kTp); }
int64_t tn2_partial_floats(int64_t P, int J, int splits) {
  return splits > 1 ? static_cast<int64_t>(tn2_tiles(P)) * splits * 4 * 2 * (tn2_jp(J) / 16) * 64 * 4
                    : 0;
}

hipError_t launch_split_hl(const float* Z, int64_t M, int J, int64_t ldz, uint16_t* Zh,
                           uint16_t* Zl, hipStream_t stream) {
  const int JP = tn2_jp(J);
  const int64_t n = M * JP;
  hipLaunchKernelGGL(k_split_hl, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, stream,
                     Z, M, J, ldz, JP, Zh, Zl);
  return hipGetLastError();
}

hipError_t launch_tn2(const Tn2Args& a, hipStream_t stream) {
  const int grid = tn2_tiles(a.P) * a.splits;
  if (tn2_jp(a.J) == 64)
    hipLaunchKernelGGL(k_tn2<64>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_tn2<128>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlin
