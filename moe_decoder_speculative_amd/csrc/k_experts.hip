// Expert SwiGLU on the decode path (a few to a few hundred token rows).
//
// At decode sizes the experts are bound by streaming their weights from HBM:
// each selected expert's 3 x I x H weights are read once per step, whatever
// the number of its tokens.  One workgroup owns (expert slot, RPW tiles of 16
// output rows: two for the gate/up projection, four for the down projection
// above 16 rows, as many as fit in 256 registers, so that two workgroups per
// CU keep the most weight bytes in flight).  Its four wavefronts split the
// reduction dimension in four and each loads its quarter of the weight tiles
// straight into registers with coalesced 1 KiB reads (weights are pre-tiled in
// MFMA operand order; non-temporal, being read once per step, so the stream
// does not evict the activation rows every token tile re-reads from L2),
// keeps them there, and loops over the expert's tokens 16
// at a time (tokens gathered from
// the permutation; columns past the expert's tokens repeat its last token, so
// they compute that token's values bit for bit and store them to its row
// again), issuing 16x16x32 bf16 MFMAs; with several token tiles the next
// tile's activation fragments are requested before the current tile's MFMAs.
// The four partial sums are added through LDS.  For steps sorted by
// the permutation kernel the slots are launched busiest first (the active
// list is ordered by token count), so the longest workgroups do not trail
// the kernel; the shared experts, which see every token, split their token
// tiles over more workgroups only beyond eight tiles (see split_index and
// token_split).
//   up:   a[pair][i] = round(silu(Wg x)[i] * (Wu x)[i])        (pairs of the slot)
//   down: y[pair][h] = (Wd a)[h]                                 (float32)
// Shared experts occupy slots 0..S-1 and see every token.  The page "Jina AI
// releases lightweight OCR model with built-in speculative decoding", section
// "Lean architecture with a compressed encoder", fixes 64 routed and 2 shared
// experts with top-6 routing; SwiGLU is this library's reading of the expert.
#include <algorithm>

#include "kernels.h"

namespace moe {

namespace {

struct SlotInfo {
  int expert;    // weight index 0..E+S-1 (shared experts after the routed ones)
  int ntok;
  int base;      // offset into perm (routed)
  int shared;    // shared slot index or -1
};

// A shared slot needs no lookup; a routed slot reads its one descriptor
// (expert, tokens, first pair), written by the sort.
__device__ __forceinline__ bool slot_info(const Dims& d, const ExpertParams& p, int slot, SlotInfo& si) {
  if (slot < d.S) {
    si.expert = d.E + slot;
    si.ntok = p.T;
    si.base = 0;
    si.shared = slot;
    return true;
  }
  if (slot >= d.S + d.E) return false;
  const int4 ds = p.desc[slot - d.S];
  // all three fields are used before the validity test, so the descriptor
  // arrives in one scalar load instead of the expert id first and the rest
  // in a second, dependent one
  asm volatile("" ::"s"(ds.x), "s"(ds.y), "s"(ds.z));
  if (ds.x < 0) return false;
  si.expert = ds.x;
  si.ntok = ds.y;
  si.base = ds.z;
  si.shared = -1;
  return true;
}

// pair id of the n-th token of a slot (activation / output row)
__device__ __forceinline__ int slot_pair(const Dims& d, const ExpertParams& p, const SlotInfo& si, int n) {
  return si.shared >= 0 ? p.T * d.k + si.shared * p.T + n : p.perm[si.base + n];
}

// ---------------------------------------------------------------- bf16 ----

// Token tiles t, t + s, ... (below nt) of one workgroup: tile t + s's rows
// are requested before tile t's MFMAs and the pairs they need one tile
// earlier still, so that no tile waits for a pair and then for its rows;
// nothing is requested past the last tile.  On entry tile t's rows are in b
// (its lane's pair in pair) and the pairs of tile t + s in pr1 (requested).
// pair_at(tile) requests the lane's pair of a tile, rows(tile, pr, b) its
// rows, do_tile(pair, b) consumes a tile.  Every store of do_tile is made by
// every lane (no branch around it): the compiler can then count the memory
// operations in flight exactly, and waiting for a tile's rows does not mean
// waiting for the previous tile's stores.
template <int KW, class PairAt, class Rows, class DoTile>
__device__ __forceinline__ void token_tiles(int t, int s, int nt, int pair, bf16x8_t (&b)[KW], int pr1,
                                            PairAt pair_at, Rows rows, DoTile do_tile) {
  for (;;) {
    if (t + s >= nt) {
      do_tile(pair, b);
      return;
    }
    const int pr2 = pair_at(t + 2 * s);  // clamped: a valid read past the end
    bf16x8_t bn[KW];
    rows(t + s, pr1, bn);
    do_tile(pair, b);
    pair = pr1;
#pragma unroll
    for (int i = 0; i < KW; ++i) b[i] = bn[i];
    pr1 = pr2;
    t += s;
  }
}

// token_tiles with the lane's pair of a tile read from the permutation
// (routed slot) or computed (shared slot) without a branch: a shared slot
// reads a word of `any` (valid memory) and multiplies it by zero.  A register
// loaded on one path and computed on the other would make the compiler wait
// for every load in flight where the paths meet.
template <int KW, class Rows, class DoTile>
__device__ __forceinline__ void slot_tiles(const Dims& d, const ExpertParams& p, const SlotInfo& si, const void* any,
                                           int lane, int t, int s, int nt, int pair, bf16x8_t (&b)[KW], int pr1,
                                           Rows rows, DoTile do_tile) {
  const bool shared = si.shared >= 0;
  const int* src = shared ? static_cast<const int*>(any) : p.perm + si.base;
  const int mul = shared ? 0 : 1, add = shared ? p.T * d.k + si.shared * p.T : 0;
  token_tiles<KW>(t, s, nt, pair, b, pr1,
                  [&](int tl) {
                    const int n = min(tl * kTile + lane % kTile, si.ntok - 1);
                    return src[n * mul] * mul + (add + n) * (1 - mul);
                  },
                  rows, do_tile);
}

// Workgroup b -> (slot, row tile r, chunk c, chunks n) for R row tiles.  The
// shared experts see all T tokens, the most of any slot, and their workgroups
// would run several times longer than the rest (latency-bound, one token tile
// after another); so the first workgroups split each shared (slot, row tile)
// `split` ways -- chunk c takes token tiles c, c + split, ... -- with the
// chunks of one pair eight workgroups apart, i.e. on one XCD at about the
// same time, where the weight tile they all read comes from L2.  The routed
// slots follow, one workgroup per (slot, row tile), busiest first.  (The
// shared part covers whole groups of 8; indices past it exit.)
__device__ __forceinline__ void split_index(const Dims& d, int R, int b, int split, int& slot, int& r, int& c,
                                           int& n) {
  const int shared_wgs = (d.S * R + 7) / 8 * 8 * split;
  if (b < shared_wgs) {
    const int q = (b / (8 * split)) * 8 + b % 8;
    c = (b / 8) % split;
    n = split;
    slot = q < d.S * R ? q / R : d.S + d.E;  // past the shared pairs: no slot
    r = q % R;
  } else {
    const int q = b - shared_wgs;
    c = 0;
    n = 1;
    slot = d.S + q / R;
    r = q % R;
  }
}

// KW: k-steps per wavefront (H / 32 / 4); RPW: row tiles per workgroup (with
// two, the launch bound holds the kernel to 256 registers: two wavefronts per
// SIMD)
template <int KW, int RPW>
__global__ __launch_bounds__(kBlock, RPW == 1 ? 1 : 2) void k_up_mfma(Dims d, ExpertParams p, int split) {
  __shared__ float red[4][RPW][2][kWave][4];
  __shared__ int pairs[kTile];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int RB = d.I / (kTile * RPW), KT = d.H / kKStep;
  int slot, rb, c, split_;
  split_index(d, RB, blockIdx.x, split, slot, rb, c, split_);
  if (slot < d.S && c * kTile >= p.T) return;  // a chunk past the shared tokens
  SlotInfo si;
  if (!slot_info(d, p, slot, si)) return;
  const int nt = (si.ntok + kTile - 1) / kTile;

  const int kt0 = wave * KW;
  const bf16_t* xh = reinterpret_cast<const bf16_t*>(p.xhat);
  bf16_t* act = reinterpret_cast<bf16_t*>(p.act);
  // the first token tile's pairs are requested before the weights: loads
  // complete in order, and the activation rows they address can then be
  // requested while the weights are in flight instead of after them
  const int n0 = c * kTile + lane % kTile, nc0 = min(n0, si.ntok - 1);
  const int pr0 = slot_pair(d, p, si, nc0);
  // and those of the workgroup's next tile (clamped: a valid read)
  const int pr1 = slot_pair(d, p, si, min(n0 + split_ * kTile, si.ntok - 1));
  bf16x8_t ag[RPW][KW], au[RPW][KW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int64_t tile = (static_cast<int64_t>(si.expert) * (d.I / kTile) + rb * RPW + r) * KT + kt0;
    const bf16_t* g = reinterpret_cast<const bf16_t*>(p.w_gate) + tile * kFragElems + lane * 8;
    const bf16_t* u = reinterpret_cast<const bf16_t*>(p.w_up) + tile * kFragElems + lane * 8;
#pragma unroll
    for (int i = 0; i < KW; ++i) {
      ag[r][i] = load_frag_stream(g + i * kFragElems);
      au[r][i] = load_frag_stream(u + i * kFragElems);
    }
  }

  // activation fragments of a token tile (column lane % 16) given the pair of
  // its n-th token clamped to the last (nc); a column past the slot's tokens
  // repeats its last token
  auto load_rows = [&](int nc, int pr, bf16x8_t (&b)[KW]) {
    const int tok = si.shared >= 0 ? nc : pr / d.k;
    const bf16_t* xr = xh + static_cast<int64_t>(tok) * d.H + kt0 * kKStep + (lane / kTile) * 8;
#pragma unroll
    for (int i = 0; i < KW; ++i) b[i] = load_frag(xr + i * kKStep);
  };
  auto rows = [&](int tl, int pr, bf16x8_t (&b)[KW]) { load_rows(min(tl * kTile + lane % kTile, si.ntok - 1), pr, b); };
  auto do_tile = [&](int pair, const bf16x8_t (&b)[KW]) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      f32x4_t cg = {0.f, 0.f, 0.f, 0.f}, cu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KW; ++i) {
        cg = mfma16(ag[r][i], b[i], cg);
        cu = mfma16(au[r][i], b[i], cu);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red[wave][r][0][lane][i] = cg[i];
        red[wave][r][1][lane][i] = cu[i];
      }
    }
    if (wave == 0 && lane < kTile) pairs[lane] = pair;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int L = threadIdx.x % kWave, i = threadIdx.x / kWave;
      const int col = L % kTile, row = 4 * (L / kTile) + i;
      const int pr = pairs[col];
      const float gs = ((red[0][r][0][L][i] + red[1][r][0][L][i]) + red[2][r][0][L][i]) + red[3][r][0][L][i];
      const float us = ((red[0][r][1][L][i] + red[1][r][1][L][i]) + red[2][r][1][L][i]) + red[3][r][1][L][i];
      act[static_cast<int64_t>(pr) * d.I + (rb * RPW + r) * kTile + row] = f32_to_bf16(silu_mul(gs, us));
    }
    __syncthreads();
  };

  bf16x8_t b[KW];
  load_rows(nc0, pr0, b);
  if (c + split_ >= nt) {
    do_tile(pr0, b);
    return;
  }
  slot_tiles<KW>(d, p, si, p.xhat, lane, c, split_, nt, pr0, b, pr1, rows, do_tile);
}

// Epilogue of the down kernel when it serves as a plain linear layer over
// shared-slot rows (EPI 1: the attention's q/k/v projection, slots 0, 1, 2
// reading the same rows; EPI 2: the attention's output projection with the
// residual add).  Adjacent output features (2i, 2i+1) sit in one lane, which
// is the pair the rotary embedding turns.
template <int EPI>
__device__ __forceinline__ void linear_epilogue(const Dims& d, const ExpertParams& p, const EpiParams& e, int slot,
                                                int n, int f, float v0, float v1) {
  if constexpr (EPI == 1) {
    const int b = n / e.K1, j = n % e.K1;
    const int pos = step_position(e.positions, b, e.P, e.K1) + j;  // the attention's clamp
    const int h = f / kHeadDim, dd = f % kHeadDim;
    if (slot < 2) {  // rotate q and k by pos * inv_freq of the pair
      float sn, cs;
      sincosf(static_cast<float>(pos) * e.inv_freq[dd / 2], &sn, &cs);
      const float r0 = __fsub_rn(__fmul_rn(v0, cs), __fmul_rn(v1, sn));
      const float r1 = __fadd_rn(__fmul_rn(v0, sn), __fmul_rn(v1, cs));
      v0 = r0;
      v1 = r1;
    }
    const uint32_t packed = pack_bf16x2(v0, v1);
    if (slot == 0) {
      *reinterpret_cast<uint32_t*>(e.q + static_cast<int64_t>(n) * d.H + f) = packed;
    } else {
      bf16_t* cache = slot == 1 ? e.kc : e.vc;
      *reinterpret_cast<uint32_t*>(cache + ((static_cast<int64_t>(b) * e.nh + h) * e.P + pos) * kHeadDim + dd) =
          packed;
    }
  } else {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(e.x_in + static_cast<int64_t>(n) * d.H + f);
    const float x0 = __uint_as_float(x << 16), x1 = __uint_as_float(x & 0xffff0000u);
    *reinterpret_cast<uint32_t*>(e.x_out + static_cast<int64_t>(n) * d.H + f) =
        pack_bf16x2(__fadd_rn(x0, v0), __fadd_rn(x1, v1));
  }
}

template <int KW, int RPW, int EPI = 0>  // KW: k-steps per wavefront (I/32/4); RPW: row tiles per workgroup
__global__ __launch_bounds__(kBlock) void k_down_mfma(Dims d, ExpertParams p, int split, EpiParams e) {
  __shared__ float red[4][RPW][kWave][4];
  __shared__ int pairs[kTile];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int RB = d.H / (kTile * RPW), KT = d.I / kKStep;
  int slot, rb, c, split_;
  split_index(d, RB, blockIdx.x, split, slot, rb, c, split_);
  if (slot < d.S && c * kTile >= p.T) return;  // a chunk past the shared tokens
  SlotInfo si;
  if (!slot_info(d, p, slot, si)) return;
  const int nt = (si.ntok + kTile - 1) / kTile;

  const int kt0 = wave * KW;
  const bf16_t* act = reinterpret_cast<const bf16_t*>(p.act);
  // the first token tile's pairs before the weights (see the up kernel)
  const int n0 = c * kTile + lane % kTile;
  const int pr0 = slot_pair(d, p, si, min(n0, si.ntok - 1));
  const int pr1 = slot_pair(d, p, si, min(n0 + split_ * kTile, si.ntok - 1));
  bf16x8_t a[RPW][KW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int64_t tile = (static_cast<int64_t>(si.expert) * (d.H / kTile) + rb * RPW + r) * KT + kt0;
    const bf16_t* w = reinterpret_cast<const bf16_t*>(p.w_down) + tile * kFragElems + lane * 8;
#pragma unroll
    for (int i = 0; i < KW; ++i) a[r][i] = load_frag_stream(w + i * kFragElems);
  }

  // activation fragments of a token tile (column lane % 16) given the pair of
  // its n-th token clamped to the last (nc); a column past the slot's tokens
  // repeats its last pair
  auto load_rows = [&](int nc, int pr, bf16x8_t (&b)[KW]) {
    // a linear layer's slots all read the token's own row
    const int arow = EPI == 0 ? pr : nc;
    const bf16_t* ar = act + static_cast<int64_t>(arow) * d.I + kt0 * kKStep + (lane / kTile) * 8;
#pragma unroll
    for (int i = 0; i < KW; ++i) b[i] = load_frag(ar + i * kKStep);
  };
  auto rows = [&](int tl, int pr, bf16x8_t (&b)[KW]) { load_rows(min(tl * kTile + lane % kTile, si.ntok - 1), pr, b); };
  auto do_tile = [&](int pair, const bf16x8_t (&b)[KW]) {
    f32x4_t c[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      c[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KW; ++i) c[r] = mfma16(a[r][i], b[i], c[r]);
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][r][lane][i] = c[r][i];
    }
    if (wave == 0 && lane < kTile) pairs[lane] = pair;
    __syncthreads();
    if constexpr (EPI == 0) {
      static_assert(RPW * kWave * 4 % kBlock == 0, "whole passes of the workgroup over the outputs");
#pragma unroll
      for (int j = 0; j < RPW * kWave * 4 / kBlock; ++j) {
        const int q = threadIdx.x + j * kBlock;
        const int r = q / (kWave * 4), L = (q / 4) % kWave, i = q % 4;
        const int col = L % kTile, row = 4 * (L / kTile) + i;
        const int pr = pairs[col];
        const float v = ((red[0][r][L][i] + red[1][r][L][i]) + red[2][r][L][i]) + red[3][r][L][i];
        p.y[static_cast<int64_t>(pr) * d.H + (rb * RPW + r) * kTile + row] = v;
      }
    } else {
      // feature pairs (row, row + 1) of one token per thread
      for (int q = threadIdx.x; q < RPW * kWave * 2; q += kBlock) {
        const int r = q / (kWave * 2), L = (q / 2) % kWave, i = 2 * (q % 2);
        const int col = L % kTile, row = 4 * (L / kTile) + i;
        const int pr = pairs[col];
        const float v0 = ((red[0][r][L][i] + red[1][r][L][i]) + red[2][r][L][i]) + red[3][r][L][i];
        const float v1 = ((red[0][r][L][i + 1] + red[1][r][L][i + 1]) + red[2][r][L][i + 1]) + red[3][r][L][i + 1];
        const int n = pr - si.shared * p.T;  // token of the shared-slot row (no routed slots)
        linear_epilogue<EPI>(d, p, e, si.shared, n, (rb * RPW + r) * kTile + row, v0, v1);
      }
    }
    __syncthreads();
  };

  bf16x8_t b[KW];
  load_rows(min(n0, si.ntok - 1), pr0, b);
  if (c + split_ >= nt) {
    do_tile(pr0, b);
    return;
  }
  slot_tiles<KW>(d, p, si, p.act, lane, c, split_, nt, pr0, b, pr1, rows, do_tile);
}

// ------------------------------------------------------------- float32 ----
// Plain FMAs, one thread per output row; used for float32 storage.

__global__ __launch_bounds__(kBlock) void k_up_f32(Dims d, ExpertParams p) {
  const int RB = (d.I + kBlock - 1) / kBlock;
  const int slot = blockIdx.x / RB, row = (blockIdx.x % RB) * kBlock + threadIdx.x;
  SlotInfo si;
  if (!slot_info(d, p, slot, si) || row >= d.I) return;
  const float* wg = reinterpret_cast<const float*>(p.w_gate) + (static_cast<int64_t>(si.expert) * d.I + row) * d.H;
  const float* wu = reinterpret_cast<const float*>(p.w_up) + (static_cast<int64_t>(si.expert) * d.I + row) * d.H;
  const float* xh = reinterpret_cast<const float*>(p.xhat);
  float* act = reinterpret_cast<float*>(p.act);
  for (int n = 0; n < si.ntok; ++n) {
    const int pair = slot_pair(d, p, si, n);
    const int tok = si.shared >= 0 ? n : pair / d.k;
    const float* x = xh + static_cast<int64_t>(tok) * d.H;
    float g = 0.f, u = 0.f;
    for (int h = 0; h < d.H; ++h) {
      g = __fadd_rn(g, __fmul_rn(wg[h], x[h]));
      u = __fadd_rn(u, __fmul_rn(wu[h], x[h]));
    }
    act[static_cast<int64_t>(pair) * d.I + row] = silu_mul(g, u);
  }
}

__global__ __launch_bounds__(kBlock) void k_down_f32(Dims d, ExpertParams p) {
  const int RB = (d.H + kBlock - 1) / kBlock;
  const int slot = blockIdx.x / RB, row = (blockIdx.x % RB) * kBlock + threadIdx.x;
  SlotInfo si;
  if (!slot_info(d, p, slot, si) || row >= d.H) return;
  const float* wd = reinterpret_cast<const float*>(p.w_down) + (static_cast<int64_t>(si.expert) * d.H + row) * d.I;
  const float* act = reinterpret_cast<const float*>(p.act);
  for (int n = 0; n < si.ntok; ++n) {
    const int pair = slot_pair(d, p, si, n);
    const float* a = act + static_cast<int64_t>(pair) * d.I;
    float acc = 0.f;
    for (int i = 0; i < d.I; ++i) acc = __fadd_rn(acc, __fmul_rn(wd[i], a[i]));
    p.y[static_cast<int64_t>(pair) * d.H + row] = acc;
  }
}

// Ways to split a shared expert's T tokens over workgroups: one up to eight
// token tiles (128 rows), then as many as keep a workgroup at eight tiles, at
// most four.  With the token-tile loop pipelined and the weights streamed
// non-temporally (the activation rows stay in L2) a tile costs well under one
// HBM round trip, and at 128 rows one workgroup per (shared slot, row tile)
// beat two (the second fetches its weights from L2 and then only runs tiles).
int token_split(int T) { return std::min(4, std::max(1, (T + 8 * kTile - 1) / (8 * kTile))); }
// A linear layer's few slots (three for q/k/v, one for the output
// projection) give too few workgroups to fill the chip at one per (slot, row
// tile): a way per two token tiles, at most four (one attention layer at
// batch 32 took 286 us with one way, 274 us with two, 269 us with four).
int linear_split(int T) { return std::min(4, std::max(1, (T + 2 * kTile - 1) / (2 * kTile))); }
// grid for R row tiles: the shared part (whole groups of 8 pairs, `split`
// ways), then one workgroup per routed (slot, row tile) -- for at most T*k
// routed slots, as many as T tokens can activate (the rest would only read
// the active count and exit, holding a CU slot for a memory round trip)
int split_grid(const Dims& d, int R, int split, int T) {
  const int routed = std::min(d.E, std::max(0, T) * d.k);
  return (d.S * R + 7) / 8 * 8 * split + routed * R;
}

template <int KW>
hipError_t up_kw(const Dims& d, const ExpertParams& p, hipStream_t s) {
  // two row tiles per workgroup (twice the weights in flight per CU at two
  // workgroups per CU) while their fragments fit in 256 registers
  constexpr int RPW = KW <= 10 ? 2 : 1;
  const int split = token_split(p.T);
  if ((d.I / kTile) % RPW == 0) {
    const int grid = split_grid(d, d.I / (kTile * RPW), split, p.T);
    hipLaunchKernelGGL((k_up_mfma<KW, RPW>), dim3(grid), dim3(kBlock), 0, s, d, p, split);
  } else {
    const int grid = split_grid(d, d.I / kTile, split, p.T);
    hipLaunchKernelGGL((k_up_mfma<KW, 1>), dim3(grid), dim3(kBlock), 0, s, d, p, split);
  }
  return hipGetLastError();
}

template <int KW, int RPW>
void down_rpw(const Dims& d, const ExpertParams& p, hipStream_t s) {
  const int split = token_split(p.T);
  const int grid = split_grid(d, d.H / (kTile * RPW), split, p.T);
  hipLaunchKernelGGL((k_down_mfma<KW, RPW>), dim3(grid), dim3(kBlock), 0, s, d, p, split, EpiParams{});
}

// Four row tiles per workgroup once a slot can hold more than one token tile
// and their fragments fit in 256 registers (two at most 16 rows: there a
// step is short enough that spreading its few slots' weights over more
// workgroups wins).
template <int KW>
hipError_t down_kw(const Dims& d, const ExpertParams& p, hipStream_t s) {
  const int tiles = d.H / kTile;
  if (KW <= 10 && p.T > kTile && tiles % 4 == 0) {
    down_rpw<KW, 4>(d, p, s);
  } else if (tiles % 2 == 0) {
    down_rpw<KW, 2>(d, p, s);
  } else {
    down_rpw<KW, 1>(d, p, s);
  }
  return hipGetLastError();
}

// A linear layer (H x H per slot) on the down kernel: the slots are shared
// expert slots over T token rows, the epilogue writes q/k/v or x + W x.
template <int EPI>
hipError_t linear_launch(const Dims& d, const ExpertParams& p, const EpiParams& e, hipStream_t s) {
  constexpr int RPW = 2;
  if (d.E != 0 || d.k != 0 || d.I != d.H || d.H % (kTile * RPW) != 0 || d.H % kHeadDim != 0) return hipErrorInvalidValue;
  const int split = linear_split(p.T);
  const int grid = split_grid(d, d.H / (kTile * RPW), split, p.T);
  switch (d.I / (kKStep * 4)) {
    case 2: hipLaunchKernelGGL((k_down_mfma<2, RPW, EPI>), dim3(grid), dim3(kBlock), 0, s, d, p, split, e); break;
    case 4: hipLaunchKernelGGL((k_down_mfma<4, RPW, EPI>), dim3(grid), dim3(kBlock), 0, s, d, p, split, e); break;
    case 8: hipLaunchKernelGGL((k_down_mfma<8, RPW, EPI>), dim3(grid), dim3(kBlock), 0, s, d, p, split, e); break;
    case 10: hipLaunchKernelGGL((k_down_mfma<10, RPW, EPI>), dim3(grid), dim3(kBlock), 0, s, d, p, split, e); break;
    case 12: hipLaunchKernelGGL((k_down_mfma<12, RPW, EPI>), dim3(grid), dim3(kBlock), 0, s, d, p, split, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#define MOE_KW_CASES(F)                                                                  \
  switch (kw) {                                                                         \
    case 1: return F<1>(d, p, s);   case 2: return F<2>(d, p, s);                       \
    case 3: return F<3>(d, p, s);   case 4: return F<4>(d, p, s);                       \
    case 5: return F<5>(d, p, s);   case 6: return F<6>(d, p, s);                       \
    case 7: return F<7>(d, p, s);   case 8: return F<8>(d, p, s);                       \
    case 9: return F<9>(d, p, s);   case 10: return F<10>(d, p, s);                     \
    case 11: return F<11>(d, p, s); case 12: return F<12>(d, p, s);                     \
    case 13: return F<13>(d, p, s); case 14: return F<14>(d, p, s);                     \
    case 15: return F<15>(d, p, s); case 16: return F<16>(d, p, s);                     \
    default: return hipErrorInvalidValue;                                               \
  }

}  // namespace

hipError_t launch_expert_up(const Dims& d, const ExpertParams& p, hipStream_t s) {
  if (!d.bf16) {
    const int grid = (d.S + d.E) * ((d.I + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(k_up_f32, dim3(grid), dim3(kBlock), 0, s, d, p);
    return hipGetLastError();
  }
  const int kw = d.H / (kKStep * 4);
  MOE_KW_CASES(up_kw)
}

hipError_t launch_linear_qkv(const Dims& d, const ExpertParams& p, const EpiParams& e, hipStream_t s) {
  if (!d.bf16 || d.S != 3) return hipErrorInvalidValue;
  return linear_launch<1>(d, p, e, s);
}

hipError_t launch_linear_resid(const Dims& d, const ExpertParams& p, const EpiParams& e, hipStream_t s) {
  if (!d.bf16 || d.S != 1) return hipErrorInvalidValue;
  return linear_launch<2>(d, p, e, s);
}

hipError_t launch_expert_down(const Dims& d, const ExpertParams& p, hipStream_t s) {
  if (!d.bf16) {
    const int grid = (d.S + d.E) * ((d.H + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(k_down_f32, dim3(grid), dim3(kBlock), 0, s, d, p);
    return hipGetLastError();
  }
  const int kw = d.I / (kKStep * 4);
  MOE_KW_CASES(down_kw)
}

}  // namespace moe
