// Few-token (M <= 16) input gradient for large weights, bound by streaming
// the packed weight from HBM.  [QLoRA "The QLoRA recipe": the gradient flows
// through the dequantized weight to the input; "Background: how LoRA works"
// for the adapter term; QA-LoRA abstract for INT4 groups and the pooled
// adapter]
//
// k_gemv_dx_stream:  dX = dY W_bf16 + expand(du A)   (du = s dY B given)
//   The reduction runs over the rows of W.  A workgroup owns a panel of 256
//   columns of dX (four 64-column blocks, 128 contiguous bytes of every row
//   of codes) and a share of the rows, which it walks 128 rows per
//   iteration: wave w decodes block w % 4 of rows 64 (w / 4) .. + 63, one
//   row per lane, into its own LDS tile, and transposed LDS reads turn eight
//   consecutive rows of one column into the operand of a
//   v_mfma_f32_16x16x32_bf16 against the matching eight dY values.  Codes
//   and dY run one iteration ahead in registers; the block constants of the
//   next four iterations are loaded once (coalesced), turned into per-block
//   scales or group words and kept in an LDS table.  The two waves of a block
//   add their sums in fixed order; row shares publish fp32 partial sums
//   (write-through stores) and the last workgroup of a panel (atomic ticket)
//   adds them in fixed share order, adds du A with MFMAs (du split into bf16
//   hi + lo halves) and stores dX.  With an unpooled adapter every workgroup
//   also forms its share of dA = du^T x over the panel's columns (a slice of
//   the adapter rows; du is complete before the launch).
#include "device_common.hpp"
#include "kernels.hpp"

namespace qlin {

namespace {

constexpr int kDsWaves = 8;
constexpr int kDsThreads = 64 * kDsWaves;
constexpr int kDsCols = 256;                 // dX columns per workgroup
constexpr int kDsRows = 128;                 // rows of W per iteration
constexpr int kDsU = 4;                      // iterations per phase of block constants
constexpr int kDsTile = 64 * 128;            // a wave's 64 x 64 bf16 tile (bytes)
constexpr int kDsAStride = 544;              // staged adapter row (256 bf16 + pad) in bytes

// 16-byte chunk swizzle of a tile row (8 chunks of 8 columns): the eight
// lanes writing one chunk position hit eight different bank groups, and the
// four rows of a transposed read hit four different chunk pairs.
__device__ __forceinline__ int ds_swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

template <int FMT> struct DsEntry { typedef uint32_t type; };
template <> struct DsEntry<kFmtINT4> { typedef uint2 type; };
template <> struct DsEntry<kFmtNFG> { typedef uint2 type; };

template <int FMT>
constexpr int ds_lds_bytes() {
  return kDsWaves * kDsTile + 2 * kDsU * 4 * kDsRows * static_cast<int>(sizeof(typename DsEntry<FMT>::type));
}
static_assert(ds_lds_bytes<kFmtNF4>() <= 81920, "two NF4 workgroups per compute unit");
static_assert(128 * kDsAStride <= kDsWaves * kDsTile + 2 * kDsU * 4 * kDsRows * 4,
              "the staged adapter panel fits in the NF4 footprint");

// Per lane and iteration: 32 bytes of codes (its row's block) and the two dY
// operands (tokens x 8 rows) of the wave's two 32-row MFMA steps.
struct DsSlot {
  u32x4 c[2];
  u32x4 dy[2];
};

template <int FMT, bool DQ, bool AL>
__global__ __launch_bounds__(kDsThreads, FMT == kFmtNF4 ? 4 : 2) void k_gemv_dx_stream(DxStreamArgs a) {
  typedef typename DsEntry<FMT>::type Entry;
  __shared__ __attribute__((aligned(16))) uint8_t s_mem[ds_lds_bytes<FMT>()];
  uint8_t* const s_tiles = s_mem;
  Entry (*const s_tab)[kDsU][4][kDsRows] =
      reinterpret_cast<Entry (*)[kDsU][4][kDsRows]>(s_mem + kDsWaves * kDsTile);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int blk = wave & 3, half = wave >> 2;
  const int64_t N = a.w.N, K = a.w.K, M = a.M;
  const int64_t Kb = K >> 6;
  const int n_pan = static_cast<int>((K + kDsCols - 1) / kDsCols);
  const int pan = static_cast<int>(blockIdx.x) % n_pan;
  const int sh = static_cast<int>(blockIdx.x) / n_pan;
  const int S = a.splits;
  const int nit = static_cast<int>((N + kDsRows - 1) / kDsRows);
  const int per = (nit + S - 1) / S;
  const int i0 = sh * per;
  const int i1 = i0 + per < nit ? i0 + per : nit;
  const int ilast = i1 > i0 ? i1 - 1 : nit - 1;  // loads past the share repeat its last iteration
  auto clampi = [&](int it) { return it < ilast ? it : ilast; };
  const int64_t r0 = static_cast<int64_t>(i0) * kDsRows;  // the share's first row
  const int64_t rows_left = N - r0;                        // <= 0 for an empty share
  auto cap32 = [](int64_t v) {
    return static_cast<uint32_t>(v <= 0 ? 0 : (v < 0xFFFFFFFFll ? v : 0xFFFFFFFFll));
  };
  uint8_t* const tile = s_tiles + wave * kDsTile;

  // codes of the share's rows from the panel's first byte: rows past N and
  // bytes past the weight read as zeros; a block past K reads the next row's
  // codes (zero table entry)
  const rsrc_t rc = uniform_rsrc(a.w.codes + (rows_left > 0 ? r0 * (K >> 1) + pan * (kDsCols / 2) : 0),
                                 cap32(rows_left * (K >> 1) - pan * (kDsCols / 2)));
  const rsrc_t rdy = uniform_rsrc(a.dy, static_cast<uint32_t>(M * N * 2));
  const int64_t mrow = l16 < M ? l16 : M - 1;
  auto load_slot = [&](int it, DsSlot& sl) {
    const int ic = clampi(it);
    const uint32_t off = static_cast<uint32_t>((static_cast<int64_t>(ic - i0) * kDsRows + half * 64 + lane) * (K >> 1)) +
                         static_cast<uint32_t>(blk * 32);
    sl.c[0] = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
    sl.c[1] = __builtin_amdgcn_raw_buffer_load_b128(rc, off + 16, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int64_t n = static_cast<int64_t>(ic) * kDsRows + half * 64 + 32 * q + 8 * g;
      n = n < N ? n : N - 8;  // rows past N meet zero weights
      sl.dy[q] = __builtin_amdgcn_raw_buffer_load_b128(rdy, static_cast<uint32_t>((mrow * N + n) * 2), 0, 0);
    }
  };

  // Block constants of a phase (iterations ib .. ib + 3): thread t takes
  // row t % 128 of iteration ib + t / 128 and the panel's four blocks.
  const int fi = tid >> 7, frow = tid & 127;
  const int panb = pan * 4;  // the panel's first block in a row
  struct Raw {
    uint32_t v[FMT == kFmtNF4 ? (DQ ? 4 : 4) : 8];
  };
  auto frow_of = [&](int ib) {
    const int64_t n = static_cast<int64_t>(clampi(ib + fi)) * kDsRows + frow;
    return n < N ? n : N - 1;
  };
  auto load_raw = [&](int ib, Raw& r) {
    const int64_t n = frow_of(ib);
    if constexpr (FMT == kFmtNF4 && DQ) {
      // the two aligned dwords holding the four 8-bit constants (zeros past
      // the array), then the group constants of the first and last block
      const int64_t b0 = n * Kb + (panb < Kb ? panb : Kb - 1);
      const rsrc_t ra = uniform_rsrc(a.w.absmax, cap32(N * Kb));
      const uint32_t a0 = static_cast<uint32_t>(b0) & ~3u;
      r.v[0] = __builtin_amdgcn_raw_buffer_load_b32(ra, a0, 0, 0);
      r.v[1] = __builtin_amdgcn_raw_buffer_load_b32(ra, a0 + 4, 0, 0);
      const int64_t bl = n * Kb + (panb + 3 < Kb ? panb + 3 : Kb - 1);
      r.v[2] = __float_as_uint(a.w.absmax2[b0 >> 8]);
      r.v[3] = __float_as_uint(a.w.absmax2[bl >> 8]);
    } else if constexpr (FMT == kFmtNF4) {
      const float* am = static_cast<const float*>(a.w.absmax) + n * Kb;
#pragma unroll
      for (int i = 0; i < 4; ++i) r.v[i] = __float_as_uint(am[panb + i < Kb ? panb + i : Kb - 1]);
    } else {
      // the eight groups' fp16 scales, then zeros (zeros past the array)
      const int64_t G = K >> 5;
      const rsrc_t rs = uniform_rsrc(a.w.scale, cap32(N * G * 2));
      const rsrc_t rz = uniform_rsrc(a.w.zero, cap32(N * G * 2));
      const uint32_t off = static_cast<uint32_t>((n * G + 2 * panb) * 2);
      if constexpr (AL) {
        const u32x4 sv = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        const u32x4 zv = __builtin_amdgcn_raw_buffer_load_b128(rz, off, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r.v[e] = sv[e];
          r.v[4 + e] = zv[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r.v[e] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * e, 0, 0);
          r.v[4 + e] = __builtin_amdgcn_raw_buffer_load_b32(rz, off + 4 * e, 0, 0);
        }
      }
    }
  };
  auto write_tab = [&](int ib, const Raw& r, int buf) {
    const int64_t n = frow_of(ib);
    const bool row_ok = ib + fi < i1 && static_cast<int64_t>(ib + fi) * kDsRows + frow < N;
    [[maybe_unused]] uint32_t q4 = 0;
    [[maybe_unused]] int64_t b0 = 0;
    if constexpr (FMT == kFmtNF4 && DQ) {
      b0 = n * Kb + (panb < Kb ? panb : Kb - 1);
      q4 = __builtin_amdgcn_alignbyte(r.v[1], r.v[0], static_cast<uint32_t>(b0) & 3u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = row_ok && panb + i < Kb;
      Entry e;
      if constexpr (FMT == kFmtNF4 && DQ) {
        const int8_t q = static_cast<int8_t>((q4 >> (8 * i)) & 0xFFu);
        const float s2 = __uint_as_float(((b0 + i) >> 8) == (b0 >> 8) ? r.v[2] : r.v[3]);
        e = ok ? __float_as_uint(nf4_dq_scale(q, s2)) : 0u;
      } else if constexpr (FMT == kFmtNF4) {
        e = ok ? r.v[i] : 0u;
      } else {
        // groups 2 i, 2 i + 1: low / high halves of scale and zero dword i
        e.x = ok ? perm(r.v[4 + i], r.v[i], 0x05040100u) : 0u;
        e.y = ok ? perm(r.v[4 + i], r.v[i], 0x07060302u) : 0u;
      }
      s_tab[buf][fi][i][frow] = e;
    }
  };
  // transposed operand: rows kb .. kb + 7 of column c0 + l16 of a swizzled tile
  auto tile_operand = [&](const uint8_t* t, int kb, int c0) {
    const int row = kb + (l16 >> 2);
    const int ch = (c0 + 4 * (l16 & 3)) >> 3;
    const uint8_t* p0 = t + row * 128 + ((ch ^ ds_swz(row)) << 4) + 8 * (l16 & 1);
    const uint8_t* p1 = t + (row + 4) * 128 + ((ch ^ ds_swz(row + 4)) << 4) + 8 * (l16 & 1);
    const u32x2 lo = ds_read_tr16(p0), hi = ds_read_tr16(p1);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  };

  // lane (l16, g) accumulates dX[m = 4 g + v][64 blk + 16 c + l16] of the panel
  f32x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // dA over the panel's columns (unpooled adapter; du is complete before
  // this launch): dA[j][k] = sum_m du[m][j] x[m][k], fp32 fma over the tokens
  // in order.  The row shares of a panel split the adapter rows between
  // them; a wave's rows are uniform, so du is read through scalar loads.
  // The token loads go out ahead of the pipeline's first loads and the sums
  // run while those are in flight.
  const int r = a.r;
  const bool do_da = a.dA != nullptr;
  const int64_t kda = static_cast<int64_t>(pan) * kDsCols + (tid & (kDsCols - 1));
  const int64_t kdc = kda < K ? kda : K - 1;
  // (branch-free: a branch join here would wait for these loads before the
  // pipeline's go out; without dA they re-read the first dY element)
  const uint16_t* const xsrc = do_da ? a.x : a.dy;
  uint16_t xraw[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) xraw[m] = xsrc[do_da ? (m < M ? m : M - 1) * K + kdc : 0];
  DsSlot ring[2];
  {
    Raw raw;
    load_raw(i0, raw);
    load_slot(i0, ring[0]);
    load_slot(i0 + 1, ring[1]);
    if (do_da) {
      const int jper = (r + S - 1) / S, jlo = sh * jper, jhi = jlo + jper < r ? jlo + jper : r;
#pragma unroll 1
      for (int j = jlo + __builtin_amdgcn_readfirstlane(tid / kDsCols); j < jhi; j += kDsThreads / kDsCols) {
        float sa = 0.0f;
#pragma unroll
        for (int m = 0; m < 16; ++m)
          if (m < M) sa = __builtin_fmaf(a.du[m * r + j], bf16_to_f32(xraw[m]), sa);
        if (kda < K) a.dA[j * K + kda] = f32_to_bf16(sa);
      }
    }
    write_tab(i0, raw, 0);
  }
  __syncthreads();

  int tb = 0;
  for (int ib = i0; ib < i1; ib += kDsU, tb ^= 1) {
    Raw raw;
    load_raw(ib + kDsU, raw);
#pragma unroll
    for (int d = 0; d < kDsU; ++d) {
      const int it = ib + d;
      DsSlot& sl = ring[d & 1];
      // iterations past the share (the last phase's tail) skip the
      // arithmetic; the branch is uniform and holds no global loads
      if (it < i1) {
        const Entry e = s_tab[tb][d][blk][half * 64 + lane];
        Lut16 lut[2];
        if constexpr (FMT == kFmtNF4) {
          lut[0] = lut_nf4(a.w.cb, __uint_as_float(e));
          lut[1] = lut[0];
        } else {
          lut[0] = lut_group32<FMT>(a.w.cb, e.x);
          lut[1] = lut_group32<FMT>(a.w.cb, e.y);
        }
        // this lane's row of the tile: chunk j = columns 8 j .. 8 j + 7
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4 wf = lut_decode8(lut[j >> 2], sl.c[j >> 2][j & 3]);
          *reinterpret_cast<u32x4*>(tile + lane * 128 + ((j ^ ds_swz(lane)) << 4)) = wf;
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] = mfma16(sl.dy[q], tile_operand(tile, 32 * q + 8 * g, 16 * c), acc[c]);
        }
      }
      if (d == kDsU - 1) write_tab(ib + kDsU, raw, tb ^ 1);
      load_slot(it + 2, sl);
      __builtin_amdgcn_sched_barrier(0);  // keep the refill here, ahead of later iterations' work
    }
    __syncthreads();
  }

  // the two waves of a block: rows 0..63 of each iteration, then 64..127
  float* s_red = reinterpret_cast<float*>(s_tiles);
  if (half == 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<f32x4*>(&s_red[((blk * 64 + lane) * 4 + c) * 4]) = acc[c];
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += *reinterpret_cast<const f32x4*>(&s_red[((blk * 64 + lane) * 4 + c) * 4]);
  }

  // lane (l16, g) holds tokens 4 g .. 4 g + 3: lanes whose tokens all lie
  // past M hold no output and move no partial sums
  const bool live = 4 * g < M;
  if (S > 1) {
    const rsrc_t pr = make_rsrc(a.partial);
    auto slot_off = [&](int share, int c) {
      return static_cast<uint32_t>((((static_cast<int64_t>(share) * n_pan + pan) * 256 + tid) * 4 + c) * 16);
    };
    if (half == 0 && live) {
#pragma unroll
      for (int c = 0; c < 4; ++c) st_sys16(pr, slot_off(sh, c), acc[c]);
    }
    uint32_t* s_ticket = reinterpret_cast<uint32_t*>(s_mem + kDsWaves * kDsTile);
    if (__builtin_amdgcn_readfirstlane(publish_and_ticket(a.counters + pan, s_ticket)) !=
        static_cast<uint32_t>(S - 1))
      return;
    if (half == 0 && live) {
      // shares in order, two at a time
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < S; s0 += 2) {
        f32x4 part[2][4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int sc = s0 + q < S ? s0 + q : S - 1;
#pragma unroll
          for (int c = 0; c < 4; ++c) part[q][c] = ld_sys16(pr, slot_off(sc, c));
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if (s0 + q < S) {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] += part[q][c];
          }
      }
    }
    if (tid == 0) a.counters[pan] = 0u;
  }

  // adapter term du A over the panel: A staged in LDS as rows of the panel's
  // 256 columns (pooled A expanded: column k reads A[.][k >> pool_shift]),
  // zero past r (to the next multiple of 32) and past K
  if (a.adapter) {
    __syncthreads();  // the reduction buffer is free again
    const int rp = (r + 31) & ~31;
    const int64_t Kp = K >> a.pool_shift;
    for (int idx = tid; idx < rp * 32; idx += kDsThreads) {
      const int j = idx >> 5, c8 = (idx & 31) * 8;  // row j, columns c8 .. c8 + 7
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t lohi[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t k = static_cast<int64_t>(pan) * kDsCols + c8 + 2 * e + h;
          const int64_t kp = k >> a.pool_shift;
          lohi[h] = (j < r && k < K) ? a.A[static_cast<int64_t>(j) * Kp + kp] : 0u;
        }
        w[e] = lohi[0] | (lohi[1] << 16);
      }
      *reinterpret_cast<u32x4*>(s_tiles + j * kDsAStride + c8 * 2) = u32x4{w[0], w[1], w[2], w[3]};
    }
    __syncthreads();
    if (half == 0) {
      const float* durow = a.du + mrow * r;
      for (int j0 = 0; j0 < r; j0 += 32) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + 8 * g + 2 * e;
          float h0, l0, h1, l1;
          split_bf16(j < r ? durow[j] : 0.0f, h0, l0);
          split_bf16(j + 1 < r ? durow[j + 1] : 0.0f, h1, l1);
          hw[e] = pack_bf16x2(h0, h1);
          lw[e] = pack_bf16x2(l0, l1);
        }
        const u32x4 hop = {hw[0], hw[1], hw[2], hw[3]}, lop = {lw[0], lw[1], lw[2], lw[3]};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // rows j0 + 8 g .. + 7 of column 64 blk + 16 c + l16 of the staged panel
          const uint8_t* p0 = s_tiles + (j0 + 8 * g + (l16 >> 2)) * kDsAStride + (64 * blk + 16 * c + 4 * (l16 & 3)) * 2;
          const u32x2 lo = ds_read_tr16(p0), hi = ds_read_tr16(p0 + 4 * kDsAStride);
          const u32x4 bop = {lo.x, lo.y, hi.x, hi.y};
          acc[c] = mfma16(hop, bop, acc[c]);
          acc[c] = mfma16(lop, bop, acc[c]);
        }
      }
    }
  }
  if (half == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t k = static_cast<int64_t>(pan) * kDsCols + 64 * blk + 16 * c + l16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M && k < K) a.dx[m * K + k] = f32_to_bf16(acc[c][v]);
      }
    }
  }

}

}  // namespace

int dx_stream_panels(int64_t K) { return static_cast<int>((K + kDsCols - 1) / kDsCols); }
int dx_stream_splits(int64_t N, int64_t K, int fmt) {
  const int64_t nit = (N + kDsRows - 1) / kDsRows;
  const int64_t slots = 256 * (fmt == kFmtNF4 ? 2 : 1);  // resident workgroups
  int64_t s = slots / dx_stream_panels(K);
  if (s > nit) s = nit;
  return static_cast<int>(s < 1 ? 1 : s);
}
int64_t dx_stream_partial_floats(int64_t N, int64_t K, int fmt) {
  const int S = dx_stream_splits(N, K, fmt);
  return S > 1 ? static_cast<int64_t>(S) * dx_stream_panels(K) * 256 * 16 : 0;
}
// rows of one share times the row pitch of the codes stay within a 32-bit offset
bool dx_stream_fits(int64_t N, int64_t K, int fmt) {
  const int64_t nit = (N + kDsRows - 1) / kDsRows;
  const int S = dx_stream_splits(N, K, fmt);
  const int64_t per = (nit + S - 1) / S;
  return (per + 1) * kDsRows * (K >> 1) < (int64_t{1} << 31) && N * (K >> 6) < 0xFFFFFFFFll &&
         N * (K >> 5) * 2 < 0xFFFFFFFFll;
}

hipError_t launch_gemv_dx_stream(const DxStreamArgs& a, int fmt, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(dx_stream_panels(a.w.K) * a.splits)), block(kDsThreads);
  const bool al = a.w.K % 256 == 0;
  if (fmt == kFmtNF4) {
    if (a.w.dq)
      hipLaunchKernelGGL((k_gemv_dx_stream<kFmtNF4, true, false>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_dx_stream<kFmtNF4, false, false>), grid, block, 0, stream, a);
  } else if (fmt == kFmtINT4) {
    if (al)
      hipLaunchKernelGGL((k_gemv_dx_stream<kFmtINT4, false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_dx_stream<kFmtINT4, false, false>), grid, block, 0, stream, a);
  } else {
    if (al)
      hipLaunchKernelGGL((k_gemv_dx_stream<kFmtNFG, false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemv_dx_stream<kFmtNFG, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace qlin
