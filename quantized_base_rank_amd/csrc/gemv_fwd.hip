// Few-token (M <= 16) forward, bound by streaming the packed 4-bit weight
// from HBM rather than by MFMA.
// [QLoRA "The QLoRA recipe" stage 3: decode each block to bf16 on the fly;
//  "Background: how LoRA works" for the adapter; QA-LoRA abstract for INT4
//  groups.]
//
//   y = x W_bf16^T + s u B^T,  u = x A^T
//
// A workgroup owns 16 output features over a share of K of at most 4096
// (the whole K for K <= 4096, so no cross-workgroup reduction at all).  Its
// 16 waves (four per SIMD; 8 with u fused) take interleaved 256-wide K
// chunks, one each (two with u fused).  Token (and adapter) chunks are staged through per-wave LDS slots
// with whole-line direct-to-LDS loads; packed codes are read as whole row
// segments and routed to their MFMA lanes with ds_bpermute; every lane
// decodes one 64-element block of one row per chunk.  The plain adapter's
// u = x A^T (r <= 16) is formed from the same token fragments.  Waves
// combine through LDS in fixed order.  With K > 4096 the K shares publish
// fp32 partial sums with write-through stores and the last workgroup of a
// tile (atomic ticket) adds them in fixed split order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

// ======================================================================
// forward
// ======================================================================
constexpr int kGfRows = 16;
constexpr int kGfChunk = 256;
constexpr int kGfKShare = 4096;  // K per workgroup at most (bounds activation re-reads)
// Waves per workgroup: 16 for the plain product (one chunk each: a wave
// starts as soon as its own chunk has landed, while later chunks still
// stream in), 8 with u fused (two rounds of a token and an adapter chunk).
template <bool FUSE_U>
struct GfShape {
  static constexpr int kWaves = FUSE_U ? 8 : 16;
  static constexpr int kPerWave = kGfKShare / kGfChunk / kWaves;  // chunks per wave
  static constexpr int kSlots = FUSE_U ? 2 : kPerWave;            // LDS slots per wave
  static constexpr int kThreads = 64 * kWaves;
};
constexpr int kGfSlot = kGfRows * kGfChunk * 2;               // one staged chunk: 8 KB

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Stage a [16][256] bf16 chunk (rows `src` + row * ld, columns k0..k0+255)
// into an 8 KB LDS slot with direct-to-LDS loads.  Each load instruction
// covers two rows of 512 B, whole 128 B lines per run of lanes.  A row's
// 16-byte pieces are XOR-swizzled by the row index so that the fragment
// reads below hit 16 distinct bank groups.  Rows past `rows` repeat the last
// row and columns past `kmax` repeat the last valid piece (both are masked
// or discarded by the caller).
__device__ __forceinline__ void stage_chunk(const uint16_t* src, int64_t ld, int rows, int64_t k0,
                                            int64_t kmax, uint8_t* slot, int lane) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int row = 2 * t + (lane >> 5);
    const int q = (lane & 31) ^ (row & 15);
    const int64_t rc = row < rows ? row : rows - 1;
    int64_t k = k0 + q * 8;
    k = k < kmax ? k : kmax - 8;
    __builtin_amdgcn_global_load_lds(src + rc * ld + k, (lds_ptr_t)(slot + t * 1024), 16, 0, 0);
  }
}

// The same chunk through registers: load_chunk_regs reads the pieces that
// stage_chunk would place, store_chunk_regs writes them to the same slot
// positions.  (Ordinary loads let the wave wait for exactly the data it
// needs; after a direct-to-LDS load the compiler waits for every load
// before any LDS access.)
__device__ __forceinline__ void load_chunk_regs(const uint16_t* src, int64_t ld, int rows, int64_t k0,
                                                int64_t kmax, int lane, u32x4 (&xr)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int row = 2 * t + (lane >> 5);
    const int q = (lane & 31) ^ (row & 15);
    const int64_t rc = row < rows ? row : rows - 1;
    int64_t k = k0 + q * 8;
    k = k < kmax ? k : kmax - 8;
    xr[t] = *reinterpret_cast<const u32x4*>(src + rc * ld + k);
  }
}
__device__ __forceinline__ void store_chunk_regs(const u32x4 (&xr)[8], uint8_t* slot, int lane) {
#pragma unroll
  for (int t = 0; t < 8; ++t) *reinterpret_cast<u32x4*>(slot + t * 1024 + lane * 16) = xr[t];
}

// MFMA fragment of a staged chunk: row l16, logical piece q (8 bf16).
__device__ __forceinline__ u32x4 chunk_frag(const uint8_t* slot, int l16, int q) {
  return *reinterpret_cast<const u32x4*>(slot + l16 * 512 + ((q ^ l16) << 4));
}

// Packed codes of a [16 rows][256 columns] chunk for lane (l16, g): the 32
// bytes of row l16, block g.  They are loaded as whole 128 B row segments
// (lane L reads row 8j + L/8, bytes 16 (L%8) .. +16 for j = 0, 1) and moved
// to their lane with ds_bpermute.
__device__ __forceinline__ void load_chunk_codes(const uint8_t* codes, int64_t ldc, int64_t n0,
                                                 int64_t N, int64_t byte0, int64_t bmax, int lane,
                                                 u32x4 (&raw)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int64_t n = n0 + 8 * j + (lane >> 3);
    n = n < N ? n : N - 1;
    int64_t b = byte0 + (lane & 7) * 16;
    b = b < bmax ? b : bmax - 16;
    raw[j] = *reinterpret_cast<const u32x4*>(codes + n * ldc + b);
  }
}
__device__ __forceinline__ void route_chunk_codes(const u32x4 (&raw)[2], int l16, int g,
                                                  u32x4 (&cw)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int src = (((l16 & 7) << 3) | (2 * g + h)) << 2;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t v0 = __builtin_amdgcn_ds_bpermute(src, static_cast<int>(raw[0][d]));
      const uint32_t v1 = __builtin_amdgcn_ds_bpermute(src, static_cast<int>(raw[1][d]));
      cw[h][d] = (l16 >> 3) ? v1 : v0;
    }
  }
}

template <int FMT, bool FUSE_U>
__global__ __launch_bounds__(GfShape<FUSE_U>::kThreads) void k_gemv_fwd(GemvFwdArgs a) {
  constexpr int kGfWaves = GfShape<FUSE_U>::kWaves;
  constexpr int kGfPerWave = GfShape<FUSE_U>::kPerWave;
  constexpr int kNT = GfShape<FUSE_U>::kThreads;
  constexpr int kAdapterIters = 2048 / kNT;  // 16 x 128 adapter elements at most
  // per wave: two 8 KB slots (token chunks i = 0, 1; or, with u fused, the
  // token and adapter chunk of one round); after the products the first
  // 2 KB of a wave's slots hold its partial y and u
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[kGfWaves][GfShape<FUSE_U>::kSlots * kGfSlot];
  __shared__ float s_fu[16 * 128];       // final u [16][r]
  __shared__ uint16_t s_b[16 * 128];     // B rows of this tile [16][r]
  __shared__ uint32_t s_ticket;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t N = a.w.N, K = a.w.K, M = a.M;
  const int r = a.r;
  const int S = a.splits;
  const int tiles = static_cast<int>((N + kGfRows - 1) / kGfRows);
  const int tile = static_cast<int>(blockIdx.x) % tiles;
  const int split = static_cast<int>(blockIdx.x) / tiles;
  const int64_t kr0 = static_cast<int64_t>(split) * a.kshare;
  const int64_t krlen = K - kr0 < a.kshare ? K - kr0 : a.kshare;
  const int nch = static_cast<int>((krlen + kGfChunk - 1) / kGfChunk);
  const int64_t n0 = static_cast<int64_t>(tile) * kGfRows;
  uint8_t* slot0 = s_stage[wave];
  uint8_t* slot1 = s_stage[wave] + (GfShape<FUSE_U>::kSlots > 1 ? kGfSlot : 0);

  // chunks of this wave (clamped; a chunk past the share is fully masked)
  int cc[kGfPerWave];
  bool live[kGfPerWave];
#pragma unroll
  for (int i = 0; i < kGfPerWave; ++i) {
    const int c = wave + i * kGfWaves;
    live[i] = c < nch;
    cc[i] = c < nch ? c : nch - 1;
  }
  auto chunk_k0 = [&](int i) { return kr0 + static_cast<int64_t>(cc[i]) * kGfChunk; };

  // (1) adapter operands of the epilogue (small, L2-resident)
  uint32_t breg[kAdapterIters];
  float ureg[kAdapterIters];
  if (a.adapter) {
#pragma unroll
    for (int i = 0; i < kAdapterIters; ++i) {
      const int idx = i * kNT + tid;
      const int nn = idx / r;
      const int64_t n = n0 + (nn < 16 ? nn : 15);
      breg[i] = a.B[(n < N ? n : N - 1) * r + idx % r];
      if (!FUSE_U) {
        const int64_t last = M * r - 1;
        ureg[i] = a.u_in[idx < last ? idx : last];
      }
    }
  }
  // (2) packed codes and block constants of this wave's chunks (HBM stream)
  const int64_t rowc = n0 + l16 < N ? n0 + l16 : N - 1;
  u32x4 raw[kGfPerWave][2];
  BlockParams bp[kGfPerWave];
  bool vblk[kGfPerWave];
#pragma unroll
  for (int i = 0; i < kGfPerWave; ++i) {
    load_chunk_codes(a.w.codes, K >> 1, n0, N, chunk_k0(i) >> 1, K >> 1, lane, raw[i]);
    const int64_t kl = static_cast<int64_t>(cc[i]) * kGfChunk + g * 64;
    vblk[i] = live[i] && kl < krlen;
    const int64_t kb = kr0 + (kl < krlen ? kl : 0);
    bp[i] = load_block_params<FMT>(a.w, rowc, kb >> 6, true);
  }
  // (3) token (and adapter) chunks straight into LDS, issued after the codes
  //     so that the decode (which needs only the codes) can start while the
  //     chunks still stream in
  //     (plain product, one chunk per wave: through registers)
  const int mrows = static_cast<int>(M < 16 ? M : 16);
  const int arows = r < 16 ? r : 16;
  constexpr bool kRegX = !FUSE_U && kGfPerWave == 1;
  u32x4 xr[8];
  if (kRegX) {
    load_chunk_regs(a.x, K, mrows, chunk_k0(0), K, lane, xr);
  } else {
    stage_chunk(a.x, K, mrows, chunk_k0(0), K, slot0, lane);
    if (FUSE_U)
      stage_chunk(a.A, K, arows, chunk_k0(0), K, slot1, lane);
    else if (kGfPerWave > 1)
      stage_chunk(a.x, K, mrows, chunk_k0(kGfPerWave - 1), K, slot1, lane);
  }
  // keep every load above ahead of the first use (the scheduler would
  // otherwise sink some next to their use, one round trip each)
  __builtin_amdgcn_sched_barrier(0);

  f32x4 accy = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 accu = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kGfPerWave; ++i) {
    // the weights first: they need only the codes.  A chunk past the share
    // decodes through an all-zero table.
    u32x4 cw[2];
    route_chunk_codes(raw[i], l16, g, cw);
    Lut16 lut[2];
    BlockParams p = bp[i];
    p.a = vblk[i] ? p.a : 0u;
    p.b = vblk[i] ? p.b : 0u;
    luts_from_params<FMT>(a.w, p, lut);
    u32x4 wf[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) wf[t] = lut_decode8(lut[t >> 2], cw[t >> 2][t & 3]);
    // token (and adapter) fragments of this chunk.  Slots filled by
    // direct-to-LDS loads are read only after an explicit wait for them: the
    // compiler's own wait for such loads can be placed after the first read.
    if (kRegX)
      store_chunk_regs(xr, slot0, lane);
    else
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint8_t* xs = (FUSE_U || i == 0) ? slot0 : slot1;
    u32x4 xf[8], af[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) xf[t] = chunk_frag(xs, l16, g * 8 + t);
    if (FUSE_U) {
#pragma unroll
      for (int t = 0; t < 8; ++t) af[t] = chunk_frag(slot1, l16, g * 8 + t);
      if (i + 1 < kGfPerWave) {
        // the slots are free once the fragments are in registers
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        stage_chunk(a.x, K, mrows, chunk_k0(i + 1), K, slot0, lane);
        stage_chunk(a.A, K, arows, chunk_k0(i + 1), K, slot1, lane);
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      accy = mfma16(wf[t], xf[t], accy);
      if (FUSE_U) accu = mfma16(xf[t], vblk[i] ? af[t] : u32x4{0, 0, 0, 0}, accu);
    }
  }

  // combine the waves: lane (l16, g) holds D[4g + v][l16]; each wave's
  // partials go to the start of its own (now unused) slot
  float* s_yw = reinterpret_cast<float*>(slot0);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    s_yw[lane * 4 + v] = accy[v];
    if (FUSE_U) s_yw[256 + lane * 4 + v] = accu[v];
  }
  if (a.adapter) {
#pragma unroll
    for (int i = 0; i < kAdapterIters; ++i) {
      const int idx = i * kNT + tid;
      if (idx < 16 * r) {
        s_b[idx] = static_cast<uint16_t>(breg[i]);
        if (!FUSE_U) s_fu[idx] = ureg[i];
      }
    }
  }
  __syncthreads();
  // threads 0..255 -> y element (n = tid >> 4, m = tid & 15) and u element
  // (m = tid >> 4, j = tid & 15); the waves are added in fixed order
  const int e8 = tid & 255;
  const int en = e8 >> 4, em = e8 & 15;
  const int ysrc = ((en >> 2) * 16 + em) * 4 + (en & 3);
  float ysum = 0.0f;
#pragma unroll
  for (int w = 0; w < kGfWaves; ++w) ysum += reinterpret_cast<const float*>(s_stage[w])[ysrc];
  const int um = e8 >> 4, uj = e8 & 15;
  const int usrc = ((um >> 2) * 16 + uj) * 4 + (um & 3);
  float usum = 0.0f;
  if (FUSE_U)
#pragma unroll
    for (int w = 0; w < kGfWaves; ++w) usum += reinterpret_cast<const float*>(s_stage[w])[256 + usrc];
  const bool owner = tid < 256;  // threads that finish one element each

  if (S > 1) {
    // publish this split's partial sums; the tile's last workgroup adds them
    float* part = a.partial + (static_cast<int64_t>(split) * tiles + tile) * 512;
    if (owner) {
      st_sys(part + e8, ysum);
      if (FUSE_U) st_sys(part + 256 + e8, usum);
    }
    if (publish_and_ticket(a.counters + tile, &s_ticket) != static_cast<uint32_t>(S - 1)) return;
    float yv[8], uv[8];
#pragma unroll
    for (int sp = 0; sp < 8; ++sp) {
      const float* ps = a.partial + (static_cast<int64_t>(sp < S ? sp : S - 1) * tiles + tile) * 512;
      yv[sp] = ld_sys(ps + e8);
      uv[sp] = FUSE_U ? ld_sys(ps + 256 + e8) : 0.0f;
    }
    ysum = 0.0f;
    usum = 0.0f;
#pragma unroll
    for (int sp = 0; sp < 8; ++sp)
      if (sp < S) {
        ysum += yv[sp];
        usum += uv[sp];
      }
    for (int sp = 8; sp < S; ++sp) {
      const float* ps = a.partial + (static_cast<int64_t>(sp) * tiles + tile) * 512;
      ysum += ld_sys(ps + e8);
      if (FUSE_U) usum += ld_sys(ps + 256 + e8);
    }
    if (tid == 0) a.counters[tile] = 0u;
  }
  if (FUSE_U) {
    if (owner && uj < r) {
      s_fu[um * r + uj] = usum;
      if (tile == 0 && a.u_out != nullptr && um < M) a.u_out[um * r + uj] = usum;
    }
    __syncthreads();
  }
  if (owner && em < M && n0 + en < N) {
    float yv = ysum;
    if (a.adapter) {
      float t = 0.0f;
      for (int j = 0; j < r; ++j) t += s_fu[em * r + j] * bf16_to_f32(s_b[en * r + j]);
      yv += a.s * t;
    }
    a.y[em * N + n0 + en] = f32_to_bf16(yv);
  }
}

}  // namespace

int gemv_fwd_tiles(int64_t N) { return static_cast<int>((N + kGfRows - 1) / kGfRows); }
int gemv_fwd_splits(int64_t K) { return static_cast<int>((K + kGfKShare - 1) / kGfKShare); }
int64_t gemv_fwd_kshare(int64_t K) {
  const int64_t per = (K + gemv_fwd_splits(K) - 1) / gemv_fwd_splits(K);
  return (per + kGfChunk - 1) / kGfChunk * kGfChunk;
}
int64_t gemv_fwd_partial_floats(int64_t N, int64_t K) {
  const int S = gemv_fwd_splits(K);
  return S > 1 ? static_cast<int64_t>(S) * gemv_fwd_tiles(N) * 512 : 0;
}

hipError_t launch_gemv_fwd(const GemvFwdArgs& a, int fmt, hipStream_t stream) {
  const int grid = gemv_fwd_tiles(a.w.N) * a.splits;
  const dim3 block(a.fuse_u ? GfShape<true>::kThreads : GfShape<false>::kThreads);
  if (fmt == kFmtNF4) {
    if (a.fuse_u)
      hipLaunchKernelGGL((k_gemv_fwd<kFmtNF4, true>), dim3(grid), block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_fwd<kFmtNF4, false>), dim3(grid), block, 0, stream, a);
  } else if (fmt == kFmtINT4) {
    if (a.fuse_u)
      hipLaunchKernelGGL((k_gemv_fwd<kFmtINT4, true>), dim3(grid), block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_fwd<kFmtINT4, false>), dim3(grid), block, 0, stream, a);
  } else {
    if (a.fuse_u)
      hipLaunchKernelGGL((k_gemv_fwd<kFmtNFG, true>), dim3(grid), block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_fwd<kFmtNFG, false>), dim3(grid), block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace qlin
