// Stable counting sort of the (token, slot) pairs by expert, in LDS.
//
// Used for large steps (prefill).  One 1024-thread workgroup per expert e
// (grid = E).  Every workgroup first copies the expert id of every pair into
// LDS as one byte (coalesced 16-byte reads), builds the full 64-bin histogram
// with LDS atomics (it needs the counts of all experts below it for its
// offset and its rank among the active experts), then gathers the pairs routed
// to e in increasing pair order: each thread scans a contiguous run of pairs,
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
  auto id_of = [&](int i) -> int { return cache_in_lds ? ids[i] : p.idx[i]; };

  if (tid < kMaxExperts) hist[tid] = 0;
  if (cache_in_lds) {
    const int P4 = P / 4;
    const int4* src = reinterpret_cast<const int4*>(p.idx);
    for (int i = tid; i < P4; i += kPermThreads) {
      const int4 v = src[i];
      ids[4 * i] = static_cast<unsigned char>(v.x);
      ids[4 * i + 1] = static_cast<unsigned char>(v.y);
      ids[4 * i + 2] = static_cast<unsigned char>(v.z);
      ids[4 * i + 3] = static_cast<unsigned char>(v.w);
    }
    for (int i = 4 * P4 + tid; i < P; i += kPermThreads) ids[i] = static_cast<unsigned char>(p.idx[i]);
  }
  __syncthreads();
  for (int i = tid; i < P; i += kPermThreads) atomicAdd(&hist[id_of(i)], 1);
  __syncthreads();

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

  // contiguous run of pairs per thread; a block-wide exclusive scan of the
  // per-thread match counts gives each thread its output position
  const int run = (P + kPermThreads - 1) / kPermThreads;
  const int lo = min(P, tid * run), hi = min(P, lo + run);
  int mine = 0;
  for (int i = lo; i < hi; ++i) mine += (id_of(i) == e);
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
  for (int i = lo; i < hi; ++i)
    if (id_of(i) == e) p.perm[pos++] = i;
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
