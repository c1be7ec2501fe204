// Expert grouped GEMM on bf16 MFMA for prefill-sized token counts, and the
// combine of its bf16 expert rows.
//
// At prefill sizes (about 915 tokens per routed expert, every token for each
// shared expert) the experts are bound by MFMA throughput, not HBM.  Work item
// = (expert slot, tile of 256 weight rows, tile of 256 of the slot's tokens).
// A 512-thread workgroup computes one item, two wavefronts per SIMD, each
// wavefront a 128 x 64 (rows x tokens) block of 32x32x16 bf16 MFMAs (128
// accumulators per lane); one workgroup per CU (128 KiB of LDS).  The operands
// of each 32-wide step of the reduction -- 16 weight row tiles (already in
// 16x32 MFMA operand order in HBM) and 16 token tiles -- go straight from
// global memory into a 4-stage LDS ring with gfx950's direct-to-LDS 16-byte
// loads (three steps in flight), placed between the MFMAs; the 32x32x16
// fragments are read out of the 16x32 tiles with a lane-dependent offset,
// double buffered by half step.  The vector-memory path bounds the loop: a
// CU moves about 32 bytes of operands per cycle with 8 wavefronts issuing,
// so the 256 x 256 item (32 KiB per step for 1,024 MFMA cycles per SIMD) is
// the smallest that does not leave the MFMAs waiting on it, and a 16x32
// token tile gathered from 16 rows costs it more than a contiguous 1 KiB
// tile -- the down GEMM reads activation tiles that the up GEMM wrote in
// operand-tile order.
//   up:   rows are 8 gate + 8 up tiles of the same 128 features; token rows
//         of xhat gathered through the permutation (padding lanes read an
//         all-zero row); epilogue a = round(silu(g) * u) written in
//         operand-tile order at row 256 * (item's token tile) + token
//   down: rows are 16 tiles of 16 hidden features; epilogue per pair either
//         y (fp32; a verify step, whose next router must see the exact sum)
//         or round(w * y) (bf16, the pair's gate weight applied; the prefill
//         block, which the 2e-2 tolerance of its output covers)
// Items are numbered slot-major, token tile, feature tile, and handed out so
// that each XCD works through a contiguous range of them: the workgroups that
// share a token tile or a weight tile run together on one XCD and hit in its
// L2.  With a reduction of 16 steps or more (H >= 512) the gate+up GEMM runs
// as a persistent kernel (k_gemm_up_persist) whose ring carries on from one
// item into the next; the down GEMM, whose epilogue stages its rows in the
// ring, keeps one item per workgroup.  Shared experts occupy slots 0..S-1.
// The 64 routed + 2 shared experts
// with top-6 routing follow the page "Jina AI releases lightweight OCR model
// with built-in speculative decoding", section "Lean architecture with a
// compressed encoder"; a page holds at most 1,156 visual tokens (same
// section), which makes a multi-page prefill thousands of rows.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBT = kGemmTokens;  // tokens per item
constexpr int kRowTiles = 16;     // MFMA row tiles per item (256 rows)
constexpr int kTokTiles = kBT / kTile;
constexpr int kStages = 4;        // LDS ring depth (one 32-wide k-step per stage, 32 KiB each)
constexpr int kStageBytes = (kRowTiles + kTokTiles) * kFragElems * 2;
constexpr int kXcds = 8;
constexpr int kGemmThreads = 512;  // 8 wavefronts: two per SIMD; one workgroup per CU
constexpr int kGemmWaves = kGemmThreads / kWave;
constexpr int kLoadsA = kRowTiles / kGemmWaves;  // weight fragments a wavefront stages per step
constexpr int kLoadsB = kTokTiles / kGemmWaves;  // token fragments a wavefront stages per step
constexpr int kLoads = kLoadsA + kLoadsB;
// Down epilogue of a prefill block: the item's 256 tokens x 256 features in
// bf16, staged in the (then idle) LDS ring with rows padded by 8 bytes (the
// staging writes of 32 token columns then fall in distinct banks), plus the
// item's 256 pair ids.
constexpr int kStagePitch = 256 + 4;  // bf16 elements per staged token row
constexpr size_t kEpiLds = static_cast<size_t>(kBT) * kStagePitch * 2 + kBT * sizeof(int);
constexpr size_t kRingLds = static_cast<size_t>(kStages) * kStageBytes;

// OUT: 0 act (up), 1 fp32 y (down), 2 bf16 gate-weighted y (down)
template <bool UP, int OUT>
__global__ __launch_bounds__(kGemmThreads, 1) void k_grouped_gemm(Dims d, GemmParams p) {
  // LDS ring of kStages stages; a stage holds one 32-wide k-step: 16 weight
  // fragments then 16 token fragments, 1 KiB each, in MFMA operand order.
  extern __shared__ __align__(16) unsigned char smem[];

  // the wavefront index is uniform: keeping it in a scalar register makes the
  // LDS destinations and weight pointers of the loads scalar
  const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wr = wave / (kGemmWaves / 2), wt = wave % (kGemmWaves / 2);  // wavefront's row half / token quarter
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

  // pair id of the item's i-th token (-1: padding); its result row
  auto pair_of = [&](int i) -> int {
    if (i >= ntok) return -1;
    return shared ? p.T * d.k + tile.y * p.T + m0 + i : p.perm[base + m0 + i];
  };

  const int Kd = UP ? d.H : d.I;                   // reduction length
  const int KT = Kd / kKStep;
  const bf16_t* wa = reinterpret_cast<const bf16_t*>(UP ? p.w_gate : p.w_down);
  const bf16_t* wu = reinterpret_cast<const bf16_t*>(p.w_up);
  const bf16_t* src = reinterpret_cast<const bf16_t*>(UP ? p.xhat : p.act);
  const int rows_per_expert_tiles = UP ? d.I / kTile : d.H / kTile;

  // this wavefront stages weight fragments kLoadsA*w .. +kLoadsA and token
  // fragments kLoadsB*w .. +kLoadsB of every stage; lane offsets (elements)
  // from scalar bases
  uint32_t woff = lane * 8, toff[kLoadsB];
  const bf16_t* wmat[kLoadsA];
#pragma unroll
  for (int q = 0; q < kLoadsA; ++q) {
    const int r = wave * kLoadsA + q;  // weight row tile of the item
    int row_tile;
    if (UP) {
      const int half = r / 8, qq = r % 8;
      wmat[q] = (qq / 4) ? wu : wa;
      row_tile = ft * 8 + half * 4 + qq % 4;
    } else {
      wmat[q] = wa;
      row_tile = ft * 16 + r;
    }
    wmat[q] += static_cast<int64_t>(expert * rows_per_expert_tiles + row_tile) * KT * kFragElems;
  }
  // up: token rows of xhat gathered through the permutation (padding lanes
  // read an all-zero row), 64 contiguous bytes per row and k-step;
  // down: the item's activation tiles, 1 KiB contiguous per fragment (the up
  // GEMM writes them in operand-tile order at the item's tile index)
  const int tix = item / n_ft;
#pragma unroll
  for (int q = 0; q < kLoadsB; ++q) {
    const int r = wave * kLoadsB + q;  // token tile of the item
    if constexpr (UP) {
      const int pr = pair_of(r * kTile + lane % kTile);
      int row = p.xhat_zero_row;
      if (pr >= 0) row = shared ? pr - p.T * d.k - tile.y * p.T : pr / d.k;
      toff[q] = static_cast<uint32_t>(row) * Kd + (lane / kTile) * 8;
    } else {
      toff[q] = static_cast<uint32_t>((tix * kTokTiles + r) * KT) * kFragElems + lane * 8;
    }
  }
  auto issue = [&](int kt) {
    unsigned char* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int q = 0; q < kLoadsA; ++q)
      __builtin_amdgcn_global_load_lds((void*)((wmat[q] + kt * kFragElems) + woff),
                                       (lds_ptr_t)(st + (wave * kLoadsA + q) * 1024), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < kLoadsB; ++q)
      __builtin_amdgcn_global_load_lds((void*)((src + kt * (UP ? kKStep : kFragElems)) + toff[q]),
                                       (lds_ptr_t)(st + (kRowTiles + wave * kLoadsB + q) * 1024), 16, 0, 0);
  };

  // result rows of this wavefront's 64 tokens (token blocks of 32), looked up
  // while the loop runs
  int out_pair[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) out_pair[n] = pair_of(wt * 64 + n * 32 + lane % 32);

  // 32x32x16 MFMAs on fragments read from the 16x32 operand tiles of the
  // ring: the fragment of 32 rows (tiles 2b, 2b+1) and reduction half kk of a
  // step gives lane L row L%32, reduction elements 16kk + 8(L/32) .. +8, which
  // sit in tile 2b + (L%32)/16 at lane slot L%16 + 16(2kk + L/32).
  const int lane_off = ((lane >> 4) & 1) * 1024 + ((lane & 15) + 16 * (lane >> 5)) * 16;
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  // Fragment registers, double buffered by half step: x holds reduction half
  // 0 of a step, y half 1.  While the 8 MFMAs of (k, 0) run, (k, 1) is read
  // from the ring; while those of (k, 1) run, (k+1, 0) is.  48 registers
  // instead of 96 for whole steps, which leaves the allocator room to keep
  // the two sets apart (shared registers would order each read after the
  // MFMA that last used them).
  //
  // The barriers are bare: a fenced barrier would wait for every load in
  // flight, later steps included, and drain the ring.  LDS-DMA writes are
  // complete once vmcnt says so; each wavefront waits for its own loads of a
  // step before the barrier, so after it every wavefront's share has landed.
  // Each wavefront also waits for its own reads of step k (both halves)
  // before it arrives, so the refill of step k's stage, issued after the
  // barrier, cannot overtake a read of it.
  bf16x8_t xa[4], xb[2], ya[4], yb[2];
#define MOE_READ_HALF(K, KK, FA, FB)                                                               \
  {                                                                                                \
    const unsigned char* st_ = smem + ((K) % kStages) * kStageBytes + lane_off + (KK) * 512;       \
    _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                  \
      FB[j] = *reinterpret_cast<const bf16x8_t*>(st_ + (kRowTiles + wt * 4 + 2 * j) * 1024);       \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                  \
      FA[i] = *reinterpret_cast<const bf16x8_t*>(st_ + (wr * 8 + 2 * i) * 1024);                   \
  }
#define MOE_MMA_HALF(FA, FB)                                                                       \
  _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                    \
  _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(FA[i], FB[j], acc[i][j]);
// 8 MFMAs with the 6 fragment reads of the other half (and the ring loads)
// between them
#define MOE_INTERLEAVE(LOADS)                                                                      \
  _Pragma("unroll") for (int g_ = 0; g_ < 6; ++g_) {                                               \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* 1 MFMA */                                \
    if (g_ < (LOADS)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); /* 1 ring load */        \
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); /* 1 LDS read */                            \
  }                                                                                                \
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
// One step K: read (K, 1) during the MFMAs of (K, 0); then make step K+1
// available -- wait until at most VM of this wavefront's loads (the steps
// issued after K+1) are in flight and its reads of step K are done, bare
// barrier, refill step K's stage with step K+4 when ISSUE -- and read
// (K+1, 0) during the MFMAs of (K, 1).
#define MOE_STEP(K, VM, ISSUE, NEXT)                                                               \
  {                                                                                                \
    MOE_READ_HALF(K, 1, ya, yb)                                                                    \
    MOE_MMA_HALF(xa, xb)                                                                           \
    MOE_INTERLEAVE(0)                                                                              \
    if (NEXT) {                                                                                    \
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM));                                                  \
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0);                                                   \
      __builtin_amdgcn_s_barrier();                                                                \
      if (ISSUE) issue((K) + kStages);                                                             \
      MOE_READ_HALF((K) + 1, 0, xa, xb)                                                            \
    }                                                                                              \
    MOE_MMA_HALF(ya, yb)                                                                           \
    if (NEXT) { MOE_INTERLEAVE((ISSUE) ? kLoads : 0) }                                             \
  }

  // KT is a multiple of 4 (H and I are multiples of 128).  Steps 0..KT-5
  // refill the ring (issue step k+4) and wait until two later steps may stay
  // in flight; steps KT-4..KT-1 drain it.
  static_assert(kLoads <= 6, "ring loads are placed between the MFMAs of a half step");
#pragma unroll
  for (int s = 0; s < kStages; ++s) issue(s);
  // the pairs' gate weights, requested now (behind the ring's first steps)
  // rather than at the epilogue, where they were a dependent round trip
  // (unconditional, clamped into the routed pairs: the wait counts below are
  // constants; a shared item uses weight 1 and ignores them; the loop's first
  // waits then also cover these two loads, which only makes them stricter)
  float gw[2] = {1.0f, 1.0f};
  if constexpr (OUT == 2) {
#pragma unroll
    for (int n = 0; n < 2; ++n) gw[n] = p.gate_w[min(max(out_pair[n], 0), p.T * d.k - 1)];
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * kLoads + (OUT == 2 ? 2 : 0)));  // step 0 landed, 1..3 may be in flight
  __builtin_amdgcn_s_barrier();
  MOE_READ_HALF(0, 0, xa, xb)
  if (KT >= 8) {
    for (int k = 0; k < KT - kStages; ++k) MOE_STEP(k, 2 * kLoads, true, true)
    MOE_STEP(KT - 4, 2 * kLoads, false, true)
  } else {  // KT == 4: every step is in the ring already
    MOE_STEP(0, 2 * kLoads, false, true)
  }
  MOE_STEP(KT - 3, kLoads, false, true)
  MOE_STEP(KT - 2, 0, false, true)
  MOE_STEP(KT - 1, 0, false, false)
#undef MOE_STEP
#undef MOE_INTERLEAVE
#undef MOE_MMA_HALF
#undef MOE_READ_HALF

  // epilogue: lane holds, of each 32 x 32 block, column (token) lane%32 and
  // rows 8g + 4(lane/32) + r for g, r in 0..3 (element 4g + r)
  if constexpr (UP) {
    // a in operand-tile order at the item's tile index: row R = 128 tix + token,
    // feature f sit in tile (R/16, f/32), lane slot R%16 + 16((f%32)/8),
    // element f%8 (padding tokens are not written and never read back into
    // a result column that is stored)
    bf16_t* act = reinterpret_cast<bf16_t*>(p.act);
    const int IT = d.I / kKStep;
#pragma unroll
    for (int bl = 0; bl < 2; ++bl)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        if (out_pair[n] < 0) continue;
        const int rt = tix * kTokTiles + wt * 4 + n * 2 + (lane % 32) / 16;   // R / 16
        const int ct = ft * 4 + wr * 2 + bl;                                    // f / 32
        bf16_t* dst = act + (static_cast<int64_t>(rt) * IT + ct) * kFragElems + (lane % 16) * 8 + 4 * (lane / 32);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& gt = acc[bl][n];
          const f32x16_t& up = acc[bl + 2][n];
          uint2 v;
          v.x = pack_bf16x2(silu_mul(gt[4 * g], up[4 * g]), silu_mul(gt[4 * g + 1], up[4 * g + 1]));
          v.y = pack_bf16x2(silu_mul(gt[4 * g + 2], up[4 * g + 2]), silu_mul(gt[4 * g + 3], up[4 * g + 3]));
          *reinterpret_cast<uint2*>(dst + g * 16 * 8) = v;
        }
      }
  } else if constexpr (OUT == 2) {
    // gate-weighted rows through LDS: every wavefront has finished reading
    // the ring, its 128 x 64 block goes to the staged [token][feature] tile,
    // then each wavefront writes 32 whole token rows (512 contiguous bytes,
    // 8 per lane) instead of 16-byte pieces of 32 rows per store
    bf16_t* stg = reinterpret_cast<bf16_t*>(smem);
    int* prs = reinterpret_cast<int*>(smem + static_cast<size_t>(kBT) * kStagePitch * 2);
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int tcol = wt * 64 + n * 32 + lane % 32;
      if (wr == 0 && lane < 32) prs[tcol] = out_pair[n];
#pragma unroll
      for (int bl = 0; bl < 4; ++bl)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int fcol = wr * 128 + bl * 32 + 8 * g + 4 * (lane / 32);
          const f32x16_t& c = acc[bl][n];
          const float w = shared ? 1.0f : gw[n];
          uint2 v;
          v.x = pack_bf16x2(w * c[4 * g], w * c[4 * g + 1]);
          v.y = pack_bf16x2(w * c[4 * g + 2], w * c[4 * g + 3]);
          *reinterpret_cast<uint2*>(stg + tcol * kStagePitch + fcol) = v;
        }
    }
    __syncthreads();
#pragma unroll 4
    for (int i = 0; i < kBT / kGemmWaves; ++i) {
      const int tok = wave * (kBT / kGemmWaves) + i;
      const int pr = prs[tok];
      if (pr >= 0)
        *reinterpret_cast<uint2*>(p.yb + static_cast<int64_t>(pr) * d.H + ft * 256 + lane * 4) =
            *reinterpret_cast<const uint2*>(stg + tok * kStagePitch + lane * 4);
    }
  } else {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int pr = out_pair[n];
      if (pr < 0) continue;
#pragma unroll
      for (int bl = 0; bl < 4; ++bl)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int feat = ft * 256 + wr * 128 + bl * 32 + 8 * g + 4 * (lane / 32);
          const f32x16_t& c = acc[bl][n];
          *reinterpret_cast<float4*>(p.y + static_cast<int64_t>(pr) * d.H + feat) =
              make_float4(c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]);
        }
    }
  }
}

// Gate+up GEMM as a persistent kernel: one workgroup per CU works through the
// items of its XCD's range (items c, c + 32, c + 64, ... of the range for the
// XCD's c-th workgroup), and the LDS ring runs on from one item into the next:
// the last four steps of an item issue the first four steps of the next, so
// those loads are in flight during the epilogue, and a new item starts
// without a launch, a lookup or an empty ring.  What the next item's loads
// need is fetched one item ahead through the same direct-to-LDS path as the
// operands -- its tile-table entry at step 0, its token pairs at step 4 (once
// the entry is in), read back at step 8 -- so the only vector memory
// operations in flight are ring loads, those two fetches and the epilogue's
// stores, and every wait in the loop is an exact constant; a lookup into
// registers would make the compiler wait for it with the ring loads behind it.
// Same items, same arithmetic and the same activation layout as
// k_grouped_gemm<true, 0>, except that padding token columns are stored too
// (their zero rows give zero activations in rows no result reads), so the
// epilogue's store count is fixed.
constexpr int kMetaBytes = 512;   // per wavefront: a tile-table entry (256 B) and 64 token pairs (256 B)
constexpr size_t kPersistLds = kRingLds + kGemmWaves * kMetaBytes;
constexpr int kUpEpiStores = 16;  // global stores per lane of one up epilogue (2 x 2 x 4, none skipped)
constexpr int kPersistWgs = 256;  // one workgroup per CU
constexpr int kPersistMinSteps = 16;  // steps 0..8 are scheduled one by one; the next item's loads start at KT-4

__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_up_persist(Dims d, GemmParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wr = wave / (kGemmWaves / 2), wt = wave % (kGemmWaves / 2);
  const int n_ft = d.I / 128;
  const int n_items = *p.n_tiles * n_ft;
  const int chunk = (n_items + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, stride = gridDim.x / kXcds;
  const int item_end = min((xcd + 1) * chunk, n_items);
  int item = xcd * chunk + blockIdx.x / kXcds;
  if (item >= item_end) return;

  const int KT = d.H / kKStep;
  const bf16_t* wg = reinterpret_cast<const bf16_t*>(p.w_gate);
  const bf16_t* wu = reinterpret_cast<const bf16_t*>(p.w_up);
  const bf16_t* src = reinterpret_cast<const bf16_t*>(p.xhat);
  const int rpe = d.I / kTile;  // weight row tiles per expert
  unsigned char* meta = smem + kRingLds + wave * kMetaBytes;

  // weight fragments kLoadsA*wave .. +kLoadsA of an item (8 gate + 8 up row
  // tiles of feature tile ft) and the lane's row offsets of the token
  // fragments kLoadsB*wave .. +kLoadsB (64 contiguous bytes per row and step)
  auto weights = [&](int expert, int ft, const bf16_t* (&w)[kLoadsA]) {
#pragma unroll
    for (int q = 0; q < kLoadsA; ++q) {
      const int r = wave * kLoadsA + q, half = r / 8, qq = r % 8;
      w[q] = ((qq / 4) ? wu : wg) + static_cast<int64_t>(expert * rpe + ft * 8 + half * 4 + qq % 4) * KT * kFragElems;
    }
  };
  auto row_off = [&](bool shared, int m0, int ntok, int t, int pair) -> uint32_t {
    int row = p.xhat_zero_row;  // padding tokens read an all-zero row
    if (t < ntok) row = shared ? m0 + t : pair / d.k;
    return static_cast<uint32_t>(row) * d.H + (lane / kTile) * 8;
  };
  auto issue = [&](const bf16_t* const (&w)[kLoadsA], const uint32_t (&to)[kLoadsB], int kt) {
    unsigned char* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int q = 0; q < kLoadsA; ++q)
      __builtin_amdgcn_global_load_lds((void*)((w[q] + kt * kFragElems) + lane * 8),
                                       (lds_ptr_t)(st + (wave * kLoadsA + q) * 1024), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < kLoadsB; ++q)
      __builtin_amdgcn_global_load_lds((void*)((src + kt * kKStep) + to[q]),
                                       (lds_ptr_t)(st + (kRowTiles + wave * kLoadsB + q) * 1024), 16, 0, 0);
  };
  // one-item-ahead fetches into the wavefront's meta area: the 4 words of a
  // tile-table entry (lane i loads word i % 4; clamped to a valid entry), and
  // the pairs of the wavefront's 32 tokens of an item (lane i the pair of
  // token 32 * wave + i % 32, clamped into the item's tokens; a shared item
  // needs none and reads a valid word)
  auto fetch_entry = [&](int it) {
    const int* e = reinterpret_cast<const int*>(p.tiles + min(it, n_items - 1) / n_ft) + lane % 4;
    __builtin_amdgcn_global_load_lds((void*)e, (lds_ptr_t)meta, 4, 0, 0);
  };
  auto fetch_pairs = [&](bool shared, int base, int m0, int ntok) {
    const int t = min(wave * 32 + lane % 32, ntok - 1);
    const int* e = p.perm + (shared ? 0 : base + m0 + t);
    __builtin_amdgcn_global_load_lds((void*)e, (lds_ptr_t)(meta + 256), 4, 0, 0);
  };

  // the current item's loads; the first item's lookups are ordinary loads
  const bf16_t* cw[kLoadsA];
  uint32_t ct[kLoadsB];
  {
    const int4 tile = p.tiles[item / n_ft];
    const bool shared = tile.y >= 0;
    const int base = shared ? 0 : -1 - tile.y;
    weights(tile.x, item % n_ft, cw);
#pragma unroll
    for (int q = 0; q < kLoadsB; ++q) {
      const int t = (wave * kLoadsB + q) * kTile + lane % kTile;
      const int pair = (!shared && t < tile.w) ? p.perm[base + tile.z + t] : 0;
      ct[q] = row_off(shared, tile.z, tile.w, t, pair);
    }
  }
  const bf16_t* nw[kLoadsA];
  uint32_t nt[kLoadsB];
  bool n_shared = false;
  int n_base = 0, n_m0 = 0, n_ntok = 1, n_expert = 0;

  const int lane_off = ((lane >> 4) & 1) * 1024 + ((lane & 15) + 16 * (lane >> 5)) * 16;
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
  bf16x8_t xa[4], xb[2], ya[4], yb[2];

#define MOE_READ_HALF(K, KK, FA, FB)                                                               \
  {                                                                                                \
    const unsigned char* st_ = smem + ((K) % kStages) * kStageBytes + lane_off + (KK) * 512;       \
    _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                  \
      FB[j] = *reinterpret_cast<const bf16x8_t*>(st_ + (kRowTiles + wt * 4 + 2 * j) * 1024);       \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                  \
      FA[i] = *reinterpret_cast<const bf16x8_t*>(st_ + (wr * 8 + 2 * i) * 1024);                   \
  }
#define MOE_MMA_HALF(FA, FB)                                                                       \
  _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                    \
  _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(FA[i], FB[j], acc[i][j]);
#define MOE_INTERLEAVE(LOADS)                                                                      \
  _Pragma("unroll") for (int g_ = 0; g_ < 6; ++g_) {                                               \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             \
    if (g_ < (LOADS)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                           \
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                             \
  }                                                                                                \
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
// One step K as in k_grouped_gemm, with the refill (and whatever rides with
// it) given as the statement ISSUE; LOADS: vector memory operations it issues
#define MOE_STEP(K, VM, LOADS, ISSUE, NEXT)                                                        \
  {                                                                                                \
    MOE_READ_HALF(K, 1, ya, yb)                                                                    \
    MOE_MMA_HALF(xa, xb)                                                                           \
    MOE_INTERLEAVE(0)                                                                              \
    if (NEXT) {                                                                                    \
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM));                                                  \
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0);                                                   \
      __builtin_amdgcn_s_barrier();                                                                \
      ISSUE;                                                                                       \
      MOE_READ_HALF((K) + 1, 0, xa, xb)                                                            \
    }                                                                                              \
    MOE_MMA_HALF(ya, yb)                                                                           \
    if (NEXT) { MOE_INTERLEAVE(LOADS) }                                                            \
  }

  // Wait counts.  At step K's wait, the operations younger than step K+1's
  // loads may stay in flight: steps K+2 and K+3 (2 kLoads); at steps 0..2 of
  // an item after the first also the previous epilogue's stores (issued after
  // this item's steps 0..3); the entry and pair fetches (one operation each,
  // at steps 0 and 4) are left out of the counts, which only makes the three
  // waits after each of them stricter by one operation.
  constexpr int kVm = 2 * kLoads, kVmEpi = 2 * kLoads + kUpEpiStores;
  for (int s = 0; s < kStages; ++s) issue(cw, ct, s);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * kLoads));  // step 0 landed, 1..3 may be in flight
  __builtin_amdgcn_s_barrier();
  MOE_READ_HALF(0, 0, xa, xb)
  bool first = true;
  for (;;) {
    const int nxt = item + stride;
    const bool has_next = nxt < item_end;
    const int tix = item / n_ft, ft = item % n_ft;
    if (first) {
      MOE_STEP(0, kVm, kLoads + 1, (issue(cw, ct, 4), fetch_entry(nxt)), true)
      MOE_STEP(1, kVm, kLoads, issue(cw, ct, 5), true)
      MOE_STEP(2, kVm, kLoads, issue(cw, ct, 6), true)
    } else {
      MOE_STEP(0, kVmEpi, kLoads + 1, (issue(cw, ct, 4), fetch_entry(nxt)), true)
      MOE_STEP(1, kVmEpi, kLoads, issue(cw, ct, 5), true)
      MOE_STEP(2, kVmEpi, kLoads, issue(cw, ct, 6), true)
    }
    MOE_STEP(3, kVm, kLoads, issue(cw, ct, 7), true)
    // step 4: the entry fetched at step 0 is in (it is older than step 5)
    MOE_STEP(4, kVm, kLoads + 1,
             {
               issue(cw, ct, 8);
               asm volatile("" ::: "memory");
               const int e = *reinterpret_cast<const int*>(meta + 4 * (lane % 4));
               n_expert = __builtin_amdgcn_readlane(e, 0);
               const int ey = __builtin_amdgcn_readlane(e, 1);
               n_shared = ey >= 0;
               n_base = n_shared ? 0 : -1 - ey;
               n_m0 = __builtin_amdgcn_readlane(e, 2);
               n_ntok = __builtin_amdgcn_readlane(e, 3);
               fetch_pairs(n_shared, n_base, n_m0, n_ntok);
             },
             true)
    MOE_STEP(5, kVm, kLoads, issue(cw, ct, 9), true)
    MOE_STEP(6, kVm, kLoads, issue(cw, ct, 10), true)
    MOE_STEP(7, kVm, kLoads, issue(cw, ct, 11), true)
    // step 8: the pairs fetched at step 4 are in (older than step 9)
    MOE_STEP(8, kVm, kLoads,
             {
               issue(cw, ct, 12);
               asm volatile("" ::: "memory");
               weights(n_expert, nxt % n_ft, nw);
               _Pragma("unroll") for (int q = 0; q < kLoadsB; ++q) {
                 const int t = (wave * kLoadsB + q) * kTile + lane % kTile;
                 const int pair = *reinterpret_cast<const int*>(meta + 256 + 4 * (q * kTile + lane % kTile));
                 nt[q] = row_off(n_shared, n_m0, n_ntok, t, pair);
               }
             },
             true)
    for (int k = 9; k < KT - kStages; ++k) MOE_STEP(k, kVm, kLoads, issue(cw, ct, k + kStages), true)
    // the last four steps always issue an item's first four steps: the next
    // one's, or after the last item those of the clamped entry fetched above
    // (valid memory, never read), so both cases share one schedule
    MOE_STEP(KT - 4, kVm, kLoads, issue(nw, nt, 0), true)
    MOE_STEP(KT - 3, kVm, kLoads, issue(nw, nt, 1), true)
    MOE_STEP(KT - 2, kVm, kLoads, issue(nw, nt, 2), true)
    MOE_STEP(KT - 1, kVm, kLoads, issue(nw, nt, 3), true)  // reads the next item's (0, 0)

    // epilogue as k_grouped_gemm<true, 0>: a = round(silu(g) * u) in
    // operand-tile order at row 256 tix + token; all 16 stores made
    bf16_t* act = reinterpret_cast<bf16_t*>(p.act);
    const int IT = d.I / kKStep;
#pragma unroll
    for (int bl = 0; bl < 2; ++bl)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int rt = tix * kTokTiles + wt * 4 + n * 2 + (lane % 32) / 16;
        const int ctile = ft * 4 + wr * 2 + bl;
        bf16_t* dst = act + (static_cast<int64_t>(rt) * IT + ctile) * kFragElems + (lane % 16) * 8 + 4 * (lane / 32);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& gt = acc[bl][n];
          const f32x16_t& up = acc[bl + 2][n];
          uint2 v;
          v.x = pack_bf16x2(silu_mul(gt[4 * g], up[4 * g]), silu_mul(gt[4 * g + 1], up[4 * g + 1]));
          v.y = pack_bf16x2(silu_mul(gt[4 * g + 2], up[4 * g + 2]), silu_mul(gt[4 * g + 3], up[4 * g + 3]));
          *reinterpret_cast<uint2*>(dst + g * 16 * 8) = v;
        }
      }
    if (!has_next) break;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
#pragma unroll
    for (int q = 0; q < kLoadsA; ++q) cw[q] = nw[q];
#pragma unroll
    for (int q = 0; q < kLoadsB; ++q) ct[q] = nt[q];
    item = nxt;
    first = false;
  }
  // the ring loads of the last four steps land before the workgroup's LDS is
  // released
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
#undef MOE_STEP
#undef MOE_INTERLEAVE
#undef MOE_MMA_HALF
#undef MOE_READ_HALF
}

// Combine of a prefill block from bf16 gate-weighted expert rows: one
// wavefront per token row, m = sum of the shared rows then the routed rows in
// ascending expert order (fp32, fixed order), x' = round(x + m).  A token's
// routed rows are rows t*k .. t*k+k-1 whatever their experts, so every row is
// requested at once together with the selection (one memory round trip); the
// selection, uniform over the wavefront, then only decides the order of the
// adds, by uniform branches over register-resident rows.
constexpr int kCombineRows = 4;   // token rows (wavefronts) per workgroup
constexpr int kCombineChunks = 3; // 8-element chunks per lane: H <= 1536
constexpr int kCombineShared = 4; // most shared experts

__device__ __forceinline__ void add_bf16x8(float (&m)[8], const uint4& v) {
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m[2 * e] = __fadd_rn(m[2 * e], __uint_as_float(w4[e] << 16));
    m[2 * e + 1] = __fadd_rn(m[2 * e + 1], __uint_as_float(w4[e] & 0xffff0000u));
  }
}

__global__ __launch_bounds__(kCombineRows * kWave) void k_combine_bf16(Dims d, CombineParams p) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kCombineRows + threadIdx.x / kWave;
  if (t >= p.T) return;
  const int H = d.H, k = d.k, S = d.S, nch = H / 8;
  // lane j < k holds the expert of routed slot j (requested first: loads
  // complete in order, and it is the first value needed)
  const int my_e = p.idx[static_cast<int64_t>(t) * k + min(lane, k - 1)];
  uint4 xv[kCombineChunks];
  uint4 ys[kCombineChunks][kCombineShared];
  uint4 yr[kCombineChunks][kMaxTopK];
  const bf16_t* xr = reinterpret_cast<const bf16_t*>(p.x_in) + static_cast<int64_t>(t) * H;
#pragma unroll
  for (int c = 0; c < kCombineChunks; ++c) {
    const int ch = lane + c * kWave;
    if (ch < nch) xv[c] = *reinterpret_cast<const uint4*>(xr + 8 * ch);
  }
#pragma unroll
  for (int r = 0; r < kCombineShared; ++r) {
    if (r < S) {
      const bf16_t* yrow = p.yb + (static_cast<int64_t>(p.T) * k + static_cast<int64_t>(r) * p.T + t) * H;
#pragma unroll
      for (int c = 0; c < kCombineChunks; ++c) {
        const int ch = lane + c * kWave;
        if (ch < nch) ys[c][r] = *reinterpret_cast<const uint4*>(yrow + 8 * ch);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      const bf16_t* yrow = p.yb + (static_cast<int64_t>(t) * k + j) * H;
#pragma unroll
      for (int c = 0; c < kCombineChunks; ++c) {
        const int ch = lane + c * kWave;
        if (ch < nch) yr[c][j] = *reinterpret_cast<const uint4*>(yrow + 8 * ch);
      }
    }
  }
  // order[q]: the routed slot holding the q-th smallest expert of the token
  // (the experts of a token are distinct)
  int rank = 0;
  for (int jj = 0; jj < k; ++jj) rank += __shfl(my_e, jj, kWave) < my_e ? 1 : 0;
  int order[kMaxTopK];
#pragma unroll
  for (int q = 0; q < kMaxTopK; ++q) {
    const unsigned long long m = __ballot(lane < k && rank == q);
    order[q] = __builtin_amdgcn_readfirstlane(m ? static_cast<int>(__builtin_ctzll(m)) : 0);
  }

  bf16_t* xo = reinterpret_cast<bf16_t*>(p.x_out) + static_cast<int64_t>(t) * H;
  float* mo = p.m_out ? p.m_out + static_cast<int64_t>(t) * H : nullptr;
#pragma unroll
  for (int c = 0; c < kCombineChunks; ++c) {
    const int ch = lane + c * kWave;
    if (ch >= nch) continue;
    float m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = 0.0f;
#pragma unroll
    for (int r = 0; r < kCombineShared; ++r)
      if (r < S) add_bf16x8(m, ys[c][r]);
#pragma unroll
    for (int q = 0; q < kMaxTopK; ++q) {
      if (q >= k) break;
      const int j = order[q];
#pragma unroll
      for (int jj = 0; jj < kMaxTopK; ++jj)
        if (jj == j) add_bf16x8(m, yr[c][jj]);
    }
    const uint32_t x4[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
    uint32_t o4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o4[e] = pack_bf16x2(__fadd_rn(__uint_as_float(x4[e] << 16), m[2 * e]),
                          __fadd_rn(__uint_as_float(x4[e] & 0xffff0000u), m[2 * e + 1]));
    *reinterpret_cast<uint4*>(xo + 8 * ch) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
    if (mo) {
      *reinterpret_cast<float4*>(mo + 8 * ch) = make_float4(m[0], m[1], m[2], m[3]);
      *reinterpret_cast<float4*>(mo + 8 * ch + 4) = make_float4(m[4], m[5], m[6], m[7]);
    }
  }
}

}  // namespace

int64_t gemm_act_rows(const Dims& d, int T) { return static_cast<int64_t>(gemm_max_tiles(d, T)) * kBT; }

int gemm_max_tiles(const Dims& d, int T) {
  // routed: at most one partial tile per expert beyond the full ones
  return d.S * ((T + kBT - 1) / kBT) + (T * d.k) / kBT + d.E;
}

size_t gemm_lds_bytes() {
  const size_t a = kRingLds > kEpiLds ? kRingLds : kEpiLds;
  return a > kPersistLds ? a : kPersistLds;
}

hipError_t launch_grouped_gemm(const Dims& d, const GemmParams& p, int up, hipStream_t s) {
  // the step schedule needs a multiple of 4 steps (H and I multiples of 128)
  if (d.I % 128 != 0 || d.H % 256 != 0) return hipErrorInvalidValue;
  const int n_ft = up ? d.I / 128 : d.H / 256;
  const int64_t items = static_cast<int64_t>(gemm_max_tiles(d, p.T)) * n_ft;
  const int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
  const size_t smem = gemm_lds_bytes();
  const dim3 g(static_cast<unsigned>(grid)), b(kGemmThreads);
  if (up && d.H / kKStep >= kPersistMinSteps) {
    hipLaunchKernelGGL(k_gemm_up_persist, dim3(kPersistWgs), b, kPersistLds, s, d, p);
  } else if (up)
    hipLaunchKernelGGL((k_grouped_gemm<true, 0>), g, b, smem, s, d, p);
  else if (p.yb)
    hipLaunchKernelGGL((k_grouped_gemm<false, 2>), g, b, smem, s, d, p);
  else
    hipLaunchKernelGGL((k_grouped_gemm<false, 1>), g, b, smem, s, d, p);
  return hipGetLastError();
}

hipError_t launch_combine_bf16(const Dims& d, const CombineParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  if (d.H % 8 != 0 || d.H / 8 > kCombineChunks * kWave || d.S > kCombineShared || d.k > kMaxTopK || d.k < 1)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_combine_bf16, dim3((p.T + kCombineRows - 1) / kCombineRows), dim3(kCombineRows * kWave), 0,
                     s, d, p);
  return hipGetLastError();
}

}  // namespace moe
