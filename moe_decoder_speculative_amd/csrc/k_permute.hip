// Stable counting sort of the (token, slot) pairs by expert, in LDS.
//
// One workgroup per expert e (grid = E).  Every workgroup builds the full
// 64-bin histogram with LDS atomics (it needs the counts of all experts below
// it for its offset and its rank among the active experts), then gathers the
// pairs routed to e in increasing pair order: each thread scans a contiguous
// run of pairs, a block-wide exclusive scan of the per-thread match counts
// gives every thread its output position, and the thread writes its matches in
// order.  Outputs cnt[e], off[e] (and off[E] = P), perm[off[e] ..] and the
// ascending list of active experts.  Grouping tokens by expert is what lets a
// top-k mixture of experts touch each selected expert's weights once per step
// (page "Jina AI lance jina-ocr-v1 ...", section "Architecture MoE et
// economies de parametres": only a fraction of the parameters is active per
// token).
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(kBlock) void k_permute(int E, PermuteParams p) {
  __shared__ int hist[kMaxExperts];
  __shared__ int wave_tot[4];
  __shared__ int base_e;
  __shared__ int cnt_e;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int P = p.P;

  if (tid < kMaxExperts) hist[tid] = 0;
  __syncthreads();
  for (int i = tid; i < P; i += kBlock) atomicAdd(&hist[p.idx[i]], 1);
  __syncthreads();

  if (wave == 0) {
    const int c = lane < E ? hist[lane] : 0;
    // inclusive scan over the 64 lanes
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    const unsigned long long act = __ballot(c > 0);
    if (lane == e) {
      base_e = incl - c;
      cnt_e = c;
      p.cnt[e] = c;
      p.off[e] = incl - c;
      if (c > 0) p.active[__popcll(act & ((1ull << lane) - 1ull))] = e;
    }
    if (e == E - 1 && lane == E - 1) {
      p.off[E] = incl;
      *p.n_active = static_cast<int>(__popcll(act));
    }
  }
  __syncthreads();
  if (cnt_e == 0) return;

  // contiguous run of pairs per thread
  const int run = (P + kBlock - 1) / kBlock;
  const int lo = min(P, tid * run), hi = min(P, lo + run);
  int mine = 0;
  for (int i = lo; i < hi; ++i) mine += (p.idx[i] == e);
  // exclusive scan of `mine` over the workgroup
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
    if (p.idx[i] == e) p.perm[pos++] = i;
}

}  // namespace

hipError_t launch_permute(const Dims& d, const PermuteParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_permute, dim3(d.E), dim3(kBlock), 0, s, d.E, p);
  return hipGetLastError();
}

}  // namespace moe
