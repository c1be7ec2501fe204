// Stable counting sort of the (token, slot) pairs by expert, in LDS.
//
// Used for large steps (prefill).  One 1024-thread workgroup per expert e
// (grid = E).  Every workgroup first copies the expert id of every pair into
// LDS as one byte (coalesced 16-byte reads, eight in flight per thread) and
// adds them, from registers, to the full 64-bin histogram with LDS atomics
// (it needs the counts of all experts below it for its offset and its rank
// among the active experts), then gathers the pairs routed to e in
// increasing pair order: each thread scans a contiguous run of pairs, four
// ids per LDS word,
// a block-wide exclusive scan of the per-thread match counts gives every
// thread its output position, and the thread writes its matches in order.
// Outputs cnt[e], off[e] (and off[E] = P), perm[off[e] ..] and the list of
// active experts, busiest first.  Grouping tokens by expert is what lets a
// top-k mixture of experts touch each selected expert's weights once per step
// (page "Jina AI lance jina-ocr-v1 ...", section "Architecture MoE et
// economies de parametres": only a fraction of the parameters is active per
// token).
#include "kernels.h"

namespace moe {

namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

__global__ __launch_bounds__(kPermThreads) void k_permute(int E, PermuteParams p, int cache_in_lds) {
  // expert id of every pair as one byte (E <= 64), cached in LDS when it fits
  extern __shared__ unsigned char ids[];
  __shared__ int hist[kMaxExperts];
  __shared__ int wave_tot[kPermWaves];
  __shared__ int base_e;
  __shared__ int cnt_e;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int P = p.P;

  if (tid < kMaxExperts) hist[tid] = 0;
  __syncthreads();
  if (cache_in_lds) {
    // batches of 16-byte reads in flight at once; each 4 ids become one
    // 32-bit LDS word and go straight into the histogram from registers
    constexpr int kBatch = 8;
    const int P4 = P / 4;
    const int4* src = reinterpret_cast<const int4*>(p.idx);
    uint32_t* ids32 = reinterpret_cast<uint32_t*>(ids);
    for (int i0 = tid; i0 < P4; i0 += kBatch * kPermThreads) {
      int4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = src[min(i0 + u * kPermThreads, P4 - 1)];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (i0 + u * kPermThreads < P4) {
          ids32[i0 + u * kPermThreads] = (static_cast<uint32_t>(v[u].x) & 255u) |
                                         ((static_cast<uint32_t>(v[u].y) & 255u) << 8) |
                                         ((static_cast<uint32_t>(v[u].z) & 255u) << 16) |
                                         (static_cast<uint32_t>(v[u].w) << 24);
          atomicAdd(&hist[v[u].x], 1);
          atomicAdd(&hist[v[u].y], 1);
          atomicAdd(&hist[v[u].z], 1);
          atomicAdd(&hist[v[u].w], 1);
        }
      }
    }
    for (int i = 4 * P4 + tid; i < P; i += kPermThreads) {
      const int e_i = p.idx[i];
      ids[i] = static_cast<unsigned char>(e_i);
      atomicAdd(&hist[e_i], 1);
    }
  } else {
    for (int i = tid; i < P; i += kPermThreads) atomicAdd(&hist[p.idx[i]], 1);
  }
  __syncthreads();

  if (e == 0 && wave == 1 && p.tiles) {
    // the grouped GEMM's tile table from the same histogram: lane e counts
    // expert e's token tiles
    const int c = lane < E ? hist[lane] : 0;
    int off = c;  // inclusive prefix of the counts, then of the tiles
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(off, o, kWave);
      if (lane >= o) off += v;
    }
    off -= c;
    const int mine = (c + kGemmTokens - 1) / kGemmTokens;
    int incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    const int T = p.tile_T, S = p.n_shared;
    const int per_shared = (T + kGemmTokens - 1) / kGemmTokens;
    const int n_shared = S * per_shared;
    for (int i = lane; i < n_shared; i += kWave) {
      const int slot = i / per_shared, m0 = (i % per_shared) * kGemmTokens;
      p.tiles[i] = make_int4(E + slot, slot, m0, min(kGemmTokens, T - m0));
    }
    if (lane < E) {
      int n = n_shared + incl - mine;
      for (int m0 = 0; m0 < c; m0 += kGemmTokens) p.tiles[n++] = make_int4(lane, -1 - off, m0, min(kGemmTokens, c - m0));
    }
    if (lane == kWave - 1) *p.n_tiles = n_shared + incl;
  }
  if (wave == 0) {
    const int c = lane < E ? hist[lane] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    const unsigned long long act = __ballot(c > 0);
    // active experts, busiest first (ties: lower id first): the expert kernels
    // start the longest slots first
    int rank = 0;
#pragma unroll
    for (int q = 0; q < kWave; ++q) {
      const int cq = __builtin_amdgcn_readlane(c, q);
      rank += (cq > c || (cq == c && q < lane)) ? 1 : 0;
    }
    if (lane == e) {
      base_e = incl - c;
      cnt_e = c;
      p.cnt[e] = c;
      p.off[e] = incl - c;
      if (c > 0) p.active[rank] = e;
      // every rank gets a descriptor: inactive experts rank last
      p.desc[rank] = c > 0 ? make_int4(e, c, incl - c, 0) : make_int4(-1, 0, 0, 0);
    }
    if (e == E - 1 && lane == E - 1) {
      p.off[E] = incl;
      *p.n_active = static_cast<int>(__popcll(act));
    }
  }
  __syncthreads();
  if (cnt_e == 0) return;

  // contiguous run of pairs per thread (a multiple of 4, so a cached run is
  // whole LDS words); a block-wide exclusive scan of the per-thread match
  // counts gives each thread its output position
  const int run = (P + 4 * kPermThreads - 1) / (4 * kPermThreads) * 4;
  const int lo = min(P, tid * run), hi = min(P, lo + run);
  const uint32_t* ids32 = reinterpret_cast<const uint32_t*>(ids);
  int mine = 0;
  if (cache_in_lds) {
    for (int i = lo; i < hi; i += 4) {
      const uint32_t w4 = ids32[i / 4];
#pragma unroll
      for (int q = 0; q < 4; ++q) mine += (i + q < hi && static_cast<int>((w4 >> (8 * q)) & 255u) == e) ? 1 : 0;
    }
  } else {
    for (int i = lo; i < hi; ++i) mine += (p.idx[i] == e);
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int pos = base_e + incl - mine;
  for (int w = 0; w < wave; ++w) pos += wave_tot[w];
  if (mine == 0) return;
  if (cache_in_lds) {
    for (int i = lo; i < hi; i += 4) {
      const uint32_t w4 = ids32[i / 4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (i + q < hi && static_cast<int>((w4 >> (8 * q)) & 255u) == e) p.perm[pos++] = i + q;
    }
  } else {
    for (int i = lo; i < hi; ++i)
      if (p.idx[i] == e) p.perm[pos++] = i;
  }
}

}  // namespace

hipError_t launch_permute(const Dims& d, const PermuteParams& p, hipStream_t s) {
  // byte cache of the expert ids in LDS (16-byte aligned pair arrays only)
  const int cache = p.P <= 96 * 1024 && (reinterpret_cast<uintptr_t>(p.idx) & 15u) == 0;
  const size_t smem = cache ? static_cast<size_t>(p.P + 15) / 16 * 16 : 0;
  hipLaunchKernelGGL(k_permute, dim3(d.E), dim3(kPermThreads), smem, s, d.E, p, cache);
  return hipGetLastError();
}

}  // namespace moe
