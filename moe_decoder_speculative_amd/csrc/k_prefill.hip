// Expert grouped GEMM on bf16 MFMA for prefill-sized token counts.
//
// At prefill sizes (about 915 tokens per routed expert, every token for each
// shared expert) the experts are bound by MFMA throughput, not HBM.  Work item
// = (expert slot, tile of 128 output features, tile of 256 of the slot's
// tokens).  A 512-thread workgroup computes one item: its operands for each
// 32-wide step of the reduction dimension -- 16 weight row tiles (already in
// MFMA operand order in HBM) and 16 token tiles gathered through the
// permutation (padding lanes read an all-zero row) -- go straight from global
// memory into a 4-stage LDS ring with gfx950's direct-to-LDS 16-byte loads
// (no registers, three steps in flight), and each of the eight wavefronts
// (two per SIMD, so one's MFMAs cover the other's waits) accumulates a
// 128 x 64 (rows x tokens) tile with 16x16x32 bf16 MFMAs (128 accumulators
// per lane).
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
constexpr int kStages = 4;        // LDS ring depth (one 32-wide k-step per stage), 128 KiB
constexpr int kStageBytes = (kRowTiles + kTokTiles) * kFragElems * 2;   // 32 KiB
constexpr int kXcds = 8;
constexpr int kGemmThreads = 512;  // 8 wavefronts: two per SIMD

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
__global__ __launch_bounds__(kGemmThreads) void k_grouped_gemm(Dims d, GemmParams p) {
  // LDS ring of kStages stages; a stage holds one 32-wide k-step: 16 weight
  // fragments then 16 token fragments, 1 KiB each, in MFMA operand order.
  extern __shared__ __align__(16) unsigned char smem[];

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wr = wave / 4, wt = wave % 4;         // wavefront's row half / token quarter
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

  // pair id of the item's i-th token (-1: padding); its result row.  Read from
  // the permutation when needed (the LDS is all ring).
  auto pair_of = [&](int i) -> int {
    if (i >= ntok) return -1;
    return shared ? p.T * d.k + tile.y * p.T + m0 + i : p.perm[base + m0 + i];
  };

  const int Kd = UP ? d.H : d.I;                   // reduction length
  const int KT = Kd / kKStep;
  const bf16_t* wa = reinterpret_cast<const bf16_t*>(UP ? p.w_gate : p.w_down);
  const bf16_t* wu = reinterpret_cast<const bf16_t*>(p.w_up);
  const bf16_t* src = reinterpret_cast<const bf16_t*>(UP ? p.xhat : p.act);
  const int zero_row = UP ? p.xhat_zero_row : p.act_zero_row;
  const int rows_per_expert_tiles = UP ? d.I / kTile : d.H / kTile;

  // this wavefront fills weight fragments 2w, 2w+1 and token fragments
  // 2w, 2w+1 of every stage; lane offsets (elements, 32-bit) advance by one
  // k-step per stage
  int woff[2], toff[2];
  const bf16_t* wmat[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = wave * 2 + q;  // weight row tile of the item
    int row_tile;
    if (UP) {
      const int half = r / 8, qq = r % 8;
      wmat[q] = (qq / 4) ? wu : wa;
      row_tile = ft * 8 + half * 4 + qq % 4;
    } else {
      wmat[q] = wa;
      row_tile = ft * 16 + r;
    }
    woff[q] = ((expert * rows_per_expert_tiles + row_tile) * KT) * kFragElems + lane * 8;
    const int pr = pair_of(r * kTile + lane % kTile);  // token tile r of the item
    int row = zero_row;
    if (pr >= 0) row = UP ? (shared ? pr - p.T * d.k - tile.y * p.T : pr / d.k) : pr;
    toff[q] = row * Kd + (lane / kTile) * 8;
  }
  auto issue = [&](int kt) {
    unsigned char* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      __builtin_amdgcn_global_load_lds((void*)(wmat[q] + woff[q] + kt * kFragElems),
                                       (lds_ptr_t)(st + (wave * 2 + q) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((void*)(src + toff[q] + kt * kKStep),
                                       (lds_ptr_t)(st + (kRowTiles + wave * 2 + q) * 1024), 16, 0, 0);
    }
  };

  // result rows of this wavefront's 64 tokens, looked up while the loop runs
  int out_pair[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) out_pair[j] = pair_of((wt * 4 + j) * kTile + lane % kTile);

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragment registers, double buffered: step k+1 is read from LDS while the
  // 32 MFMAs of step k run.  KT is even (H and I are multiples of 128), so the
  // loop runs in pairs with the two register sets in fixed roles.
  //
  // The barriers are bare: a fenced barrier would wait for every load in
  // flight, later steps included, and drain the ring.  LDS-DMA writes are
  // complete once vmcnt says so; each wavefront waits for its own loads of a
  // step before the barrier, so after it every wavefront's share has landed.
  bf16x8_t a0[8], b0[4], a1[8], b1[4];
#define MOE_READ_STEP(K, A, B)                                                                     \
  {                                                                                                \
    const unsigned char* st_ = smem + ((K) % kStages) * kStageBytes;                               \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) B[j] =                                           \
        *reinterpret_cast<const bf16x8_t*>(st_ + (kRowTiles + wt * 4 + j) * 1024 + lane * 16);     \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) A[i] =                                           \
        *reinterpret_cast<const bf16x8_t*>(st_ + (wr * 8 + i) * 1024 + lane * 16);                 \
  }
#define MOE_MMA_STEP(A, B)                                                                         \
  _Pragma("unroll") for (int i = 0; i < 8; ++i)                                                    \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(A[i], B[j], acc[i][j]);
  // wait for this wavefront's loads of step k+1 at iteration k: the steps
  // issued after it (up to two) may stay in flight, 4 loads each
#define MOE_WAIT_NEXT(K)                                                                           \
  {                                                                                                \
    const int later_ = min(KT, (K) + kStages) - (K) - 2;                                           \
    if (later_ >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));                                    \
    else if (later_ == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));                               \
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));                                                \
  }
// One step: make step K+1 available (wait for this wavefront's loads, bare
// barrier, refill the ring), then run step K's 32 MFMAs with step K+1's 12
// fragment reads interleaved (a read after every 2 or 3 MFMAs).  Interleaving
// matters: with all reads ahead of the MFMAs, the first MFMA waits for all of
// them (the LDS counter cannot express "16 newer reads may stay in flight").
// At the last step the reads fetch a stale stage that is never used.
#define MOE_STEP(K, CA, CB, NA, NB)                                                                \
  {                                                                                                \
    if ((K) + 1 < KT) {                                                                            \
      MOE_WAIT_NEXT(K)                                                                             \
      __builtin_amdgcn_s_barrier(); /* step K+1 landed; everyone has read step K */                \
      if ((K) + kStages < KT) issue((K) + kStages); /* into step K's buffer */                     \
    }                                                                                              \
    MOE_MMA_STEP(CA, CB)                                                                           \
    MOE_READ_STEP((K) + 1, NA, NB)                                                                 \
    _Pragma("unroll") for (int g_ = 0; g_ < 8; ++g_) {                                             \
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0); /* 3 MFMA */                              \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); /* 1 LDS read */                          \
    }                                                                                              \
    _Pragma("unroll") for (int g_ = 0; g_ < 4; ++g_) {                                             \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); /* 2 MFMA */                              \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); /* 1 LDS read */                          \
    }                                                                                              \
  }

#pragma unroll
  for (int s = 0; s < kStages; ++s)
    if (s < KT) issue(s);
  // step 0 landed once the other issued steps (up to kStages - 1) remain
  static_assert(kStages == 4, "wait counts below assume a 4-stage ring");
  switch (min(KT, kStages) - 1) {
    case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm(12)); break;
    case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(8)); break;
    case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(4)); break;
    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
  }
  __builtin_amdgcn_s_barrier();
  MOE_READ_STEP(0, a0, b0)
  for (int k = 0; k < KT; k += 2) {
    MOE_STEP(k, a0, b0, a1, b1)
    MOE_STEP(k + 1, a1, b1, a0, b0)
  }
#undef MOE_STEP
#undef MOE_WAIT_NEXT
#undef MOE_MMA_STEP
#undef MOE_READ_STEP

  // epilogue: lane holds rows 4*(lane/16)+i of each row tile, token lane%16
  if (UP) {
    bf16_t* act = reinterpret_cast<bf16_t*>(p.act);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int feat = (ft * 8 + wr * 4 + f) * kTile + 4 * (lane / kTile);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pr = out_pair[j];
        if (pr < 0) continue;
        uint2 v;
        v.x = pack_bf16x2(silu_mul(acc[f][j][0], acc[f + 4][j][0]), silu_mul(acc[f][j][1], acc[f + 4][j][1]));
        v.y = pack_bf16x2(silu_mul(acc[f][j][2], acc[f + 4][j][2]), silu_mul(acc[f][j][3], acc[f + 4][j][3]));
        *reinterpret_cast<uint2*>(act + static_cast<int64_t>(pr) * d.I + feat) = v;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int feat = (ft * 16 + wr * 8 + i) * kTile + 4 * (lane / kTile);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pr = out_pair[j];
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

size_t gemm_lds_bytes() { return static_cast<size_t>(kStages) * kStageBytes; }

hipError_t launch_tile_list(const Dims& d, const GemmTileParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_tile_list, dim3(1), dim3(64), 0, s, d, p);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const Dims& d, const GemmParams& p, int up, hipStream_t s) {
  // the step loop runs in pairs (H and I are multiples of 128)
  if (d.I % 128 != 0 || d.H % 256 != 0) return hipErrorInvalidValue;
  const int n_ft = up ? d.I / 128 : d.H / 256;
  const int64_t items = static_cast<int64_t>(gemm_max_tiles(d, p.T)) * n_ft;
  const int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
  const size_t smem = gemm_lds_bytes();
  if (up)
    hipLaunchKernelGGL(k_grouped_gemm<true>, dim3(static_cast<unsigned>(grid)), dim3(kGemmThreads), smem, s, d, p);
  else
    hipLaunchKernelGGL(k_grouped_gemm<false>, dim3(static_cast<unsigned>(grid)), dim3(kGemmThreads), smem, s, d, p);
  return hipGetLastError();
}

}  // namespace moe
