// Expert grouped GEMM on bf16 MFMA for prefill-sized token counts.
//
// At prefill sizes (about 915 tokens per routed expert, every token for each
// shared expert) the experts are bound by MFMA throughput, not HBM.  Work item
// = (expert slot, tile of 128 output features, tile of 256 of the slot's
// tokens).  A 256-thread workgroup computes one item: its operands for a
// 64-wide slice of the reduction dimension -- 16 weight row tiles (already in
// MFMA operand order in HBM) and 16 token tiles gathered through the
// permutation -- are staged in LDS (double buffered, 128 KiB), and each of
// the four wavefronts accumulates a 128 x 128 (rows x tokens) tile with
// 16x16x32 bf16 MFMAs (256 accumulators per lane).
//   up:   rows are 8 gate + 8 up tiles of the same 128 features; epilogue
//         a = round(silu(g) * u) written per pair (bf16)
//   down: rows are 16 tiles of 16 hidden features; epilogue y (fp32) per pair
// Items are numbered slot-major, feature-tile, token-tile, and handed out so
// that each XCD works through a contiguous range of them: the workgroups that
// share a weight tile run together on one XCD and hit in its L2.
// Shared experts occupy slots 0..S-1.  The 64 routed + 2 shared experts with
// top-6 routing follow the page "Jina AI releases lightweight OCR model with
// built-in speculative decoding", section "Lean architecture with a
// compressed encoder"; a page holds at most 1,156 visual tokens (same
// section), which makes a multi-page prefill thousands of rows.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBT = 256;          // tokens per item
constexpr int kRowTiles = 16;     // MFMA row tiles per item
constexpr int kTokTiles = kBT / kTile;
constexpr int kSlabK = 2;         // k-steps (of 32) per LDS slab
constexpr int kFragsPerSlab = (kRowTiles + kTokTiles) * kSlabK;     // 64
constexpr int kPiecesPerThread = kFragsPerSlab * kWave / kBlock;    // 16
constexpr int kSlabElems = kFragsPerSlab * kFragElems;              // bf16 per slab
constexpr int kXcds = 8;

// Tile table: one entry per (slot, token tile), shared slots first, then the
// routed experts in ascending order.  Built on the device after the
// permutation by one wavefront (lane e counts expert e's tiles).
__global__ __launch_bounds__(64) void k_tile_list(Dims d, GemmTileParams p) {
  const int lane = threadIdx.x;
  const int per_shared = (p.T + kBT - 1) / kBT;
  const int c = lane < d.E ? p.cnt[lane] : 0;
  const int mine = (c + kBT - 1) / kBT;
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  const int n_shared = d.S * per_shared;
  for (int i = lane; i < n_shared; i += kWave) {
    const int slot = i / per_shared, m0 = (i % per_shared) * kBT;
    p.tiles[i] = make_int4(d.E + slot, slot, m0, min(kBT, p.T - m0));
  }
  if (lane < d.E) {
    const int base = p.off[lane];
    int n = n_shared + incl - mine;
    for (int m0 = 0; m0 < c; m0 += kBT) p.tiles[n++] = make_int4(lane, -1 - base, m0, min(kBT, c - m0));
  }
  if (lane == kWave - 1) *p.n_tiles = n_shared + incl;
}

template <bool UP>
__global__ __launch_bounds__(kBlock) void k_grouped_gemm(Dims d, GemmParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* lds = reinterpret_cast<bf16_t*>(smem);  // [2][kFragsPerSlab][64][8]
  __shared__ int pairs[kBT];

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wr = wave / 2, wt = wave % 2;         // wavefront's row half / token half
  const int n_ft = UP ? d.I / 128 : d.H / 256;     // feature tiles per slot
  const int n_items = *p.n_tiles * n_ft;
  const int chunk = (n_items + kXcds - 1) / kXcds;
  const int b = blockIdx.x;
  if (b / kXcds >= chunk) return;
  const int item = (b % kXcds) * chunk + b / kXcds;
  if (item >= n_items) return;
  const int4 tile = p.tiles[item / n_ft];
  const int ft = item % n_ft;
  const int expert = tile.x, m0 = tile.z, ntok = tile.w;
  const bool shared = tile.y >= 0;
  const int base = shared ? 0 : -1 - tile.y;

  // pair ids of this item's tokens
  for (int i = threadIdx.x; i < kBT; i += kBlock) {
    int pr = -1;
    if (i < ntok) pr = shared ? p.T * d.k + tile.y * p.T + m0 + i : p.perm[base + m0 + i];
    pairs[i] = pr;
  }
  __syncthreads();

  const int Kd = UP ? d.H : d.I;                   // reduction length
  const int KT = Kd / kKStep;
  const int nslab = KT / kSlabK;
  const bf16_t* wa = reinterpret_cast<const bf16_t*>(UP ? p.w_gate : p.w_down);
  const bf16_t* wu = reinterpret_cast<const bf16_t*>(p.w_up);
  const bf16_t* src = reinterpret_cast<const bf16_t*>(UP ? p.xhat : p.act);
  const int rows_per_expert_tiles = UP ? d.I / kTile : d.H / kTile;

  // per-thread staging pieces: q = threadIdx.x + kBlock * j; frag q/64, lane q%64.
  // Pieces j < 8 are weight fragments (frag = r*kSlabK + kk, r < 16), j >= 8
  // token fragments; their addresses advance by a fixed stride per slab.
  const bf16_t* pbase[kPiecesPerThread];
#pragma unroll
  for (int j = 0; j < kPiecesPerThread; ++j) {
    const int q = threadIdx.x + kBlock * j;
    const int f = q / kWave, ln = q % kWave;
    const int kk = f % kSlabK, r = f / kSlabK;
    if (r < kRowTiles) {
      const bf16_t* mat;
      int row_tile;
      if (UP) {
        const int half = r / 8, qq = r % 8;
        mat = (qq / 4) ? wu : wa;
        row_tile = ft * 8 + half * 4 + qq % 4;
      } else {
        mat = wa;
        row_tile = ft * 16 + r;
      }
      pbase[j] = mat + ((static_cast<int64_t>(expert) * rows_per_expert_tiles + row_tile) * KT + kk) * kFragElems + ln * 8;
    } else {
      const int tt = r - kRowTiles;
      const int pr = pairs[tt * kTile + ln % kTile];
      if (pr < 0) {
        pbase[j] = nullptr;
      } else {
        const int64_t row = UP ? static_cast<int64_t>(shared ? pr - p.T * d.k - tile.y * p.T : pr / d.k) : pr;
        pbase[j] = src + row * Kd + kk * kKStep + (ln / kTile) * 8;
      }
    }
  }
  static_assert(kRowTiles * kSlabK * kWave == 8 * kBlock, "weight pieces are j < 8");

  bf16x8_t st[kPiecesPerThread];
  auto load_slab = [&](int slab) {
#pragma unroll
    for (int j = 0; j < kPiecesPerThread; ++j) {
      const int64_t step = j < 8 ? static_cast<int64_t>(kSlabK) * kFragElems : kSlabK * kKStep;
      st[j] = pbase[j] ? load_frag(pbase[j] + slab * step) : zero_frag();
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kPiecesPerThread; ++j) {
      const int q = threadIdx.x + kBlock * j;
      *reinterpret_cast<bf16x8_t*>(lds + buf * kSlabElems + q * 8) = st[j];
    }
  };

  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_slab(0);
  store_slab(0);
  __syncthreads();
  for (int s = 0; s < nslab; ++s) {
    const bool more = s + 1 < nslab;
    if (more) load_slab(s + 1);
    const bf16_t* buf = lds + (s & 1) * kSlabElems;
#pragma unroll
    for (int kk = 0; kk < kSlabK; ++kk) {
      bf16x8_t a[8], bt[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(buf + (((wr * 8 + i) * kSlabK + kk) * kWave + lane) * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bt[j] = *reinterpret_cast<const bf16x8_t*>(
            buf + (((kRowTiles + wt * 8 + j) * kSlabK + kk) * kWave + lane) * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(a[i], bt[j], acc[i][j]);
    }
    if (more) store_slab((s + 1) & 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane/16)+i of each row tile, token lane%16
  if (UP) {
    bf16_t* act = reinterpret_cast<bf16_t*>(p.act);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int feat = (ft * 8 + wr * 4 + f) * kTile + 4 * (lane / kTile);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int pr = pairs[(wt * 8 + j) * kTile + lane % kTile];
        if (pr < 0) continue;
        ushort4 v;
        v.x = f32_to_bf16(silu_mul(acc[f][j][0], acc[f + 4][j][0]));
        v.y = f32_to_bf16(silu_mul(acc[f][j][1], acc[f + 4][j][1]));
        v.z = f32_to_bf16(silu_mul(acc[f][j][2], acc[f + 4][j][2]));
        v.w = f32_to_bf16(silu_mul(acc[f][j][3], acc[f + 4][j][3]));
        *reinterpret_cast<ushort4*>(act + static_cast<int64_t>(pr) * d.I + feat) = v;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int feat = (ft * 16 + wr * 8 + i) * kTile + 4 * (lane / kTile);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int pr = pairs[(wt * 8 + j) * kTile + lane % kTile];
        if (pr < 0) continue;
        *reinterpret_cast<float4*>(p.y + static_cast<int64_t>(pr) * d.H + feat) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
  }
}

}  // namespace

int gemm_max_tiles(const Dims& d, int T) {
  // routed: at most one partial tile per expert beyond the full ones
  return d.S * ((T + kBT - 1) / kBT) + (T * d.k) / kBT + d.E;
}

size_t gemm_lds_bytes() { return 2ull * kSlabElems * sizeof(bf16_t); }

hipError_t launch_tile_list(const Dims& d, const GemmTileParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_tile_list, dim3(1), dim3(64), 0, s, d, p);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const Dims& d, const GemmParams& p, int up, hipStream_t s) {
  if (d.I % 128 != 0 || d.H % 256 != 0 || (d.H / kKStep) % kSlabK != 0 || (d.I / kKStep) % kSlabK != 0)
    return hipErrorInvalidValue;
  const int n_ft = up ? d.I / 128 : d.H / 256;
  const int64_t items = static_cast<int64_t>(gemm_max_tiles(d, p.T)) * n_ft;
  const int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
  const size_t smem = gemm_lds_bytes();
  if (up)
    hipLaunchKernelGGL(k_grouped_gemm<true>, dim3(static_cast<unsigned>(grid)), dim3(kBlock), smem, s, d, p);
  else
    hipLaunchKernelGGL(k_grouped_gemm<false>, dim3(static_cast<unsigned>(grid)), dim3(kBlock), smem, s, d, p);
  return hipGetLastError();
}

}  // namespace moe
