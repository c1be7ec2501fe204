// Decode attention of the verify step: each sequence's K1 = K+1 query rows
// (the last committed token and the drafts, already rotated and with their
// keys and values written to the cache) against cache positions 0..p_b+j.
//
// At decode sizes attention is a stream over the KV cache (512 B per position
// and head), so the work is split over positions: workgroup (g, h, b) takes
// the 64-position tiles g*4 + w, g*4 + w + 4G, ... of sequence b and head h,
// one tile per wavefront at a time, every load of a tile issued first (with
// the default cache policy: a key row's 128-byte lines are read in two halves
// by two loads, and with the non-temporal hint a line could leave the cache
// between them -- 10 % more HBM traffic, no faster):
//   scores: 16 MFMAs 16x16x32 per tile with the keys as the A operand (bf16
//           rows as cached, 16 B a lane) and the bf16 queries as B (columns
//           >= K1 zero), float32 accumulation;
//   softmax: per query the tile's maximum and sum (16 values in a lane, then
//           across the four lane groups), folded into a running (max, sum)
//           with the usual rescaling;
//   values:  float32; a lane reads 16 bytes (eight dimensions) of every fourth
//           value row, so a tile is 16 loads and all 32 of a tile's loads fit
//           in flight at once; weights come from LDS, and the four lane
//           groups' partial sums are added once at the end.
// The four wavefronts' states meet in LDS and the workgroup writes one
// partial (max, sum, weighted values) per query; k_attn_combine merges the G
// partials of every (row, head) and rounds the result to bfloat16.  Reading of
// the pages: attention is not described there; multi-head attention with
// rotary positions and a KV cache is this library's reading of the decoder
// named on the page "Jina AI releases lightweight OCR model with built-in
// speculative decoding", section "Lean architecture with a compressed
// encoder" (12 layers, 32,768 positions).
#include <algorithm>

#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxK1 = 8;
constexpr int kPosTile = 64;
constexpr int kPartStride = 2 + kHeadDim;
constexpr int kMaxGroups = 64;  // position groups per (sequence, head), at most
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// position groups of a sequence that hold cache rows (the others exit)
__device__ __forceinline__ int used_groups(int len, int G) { return min(G, (len + 4 * kPosTile - 1) / (4 * kPosTile)); }

__device__ __forceinline__ int clamped_pos(const AttnParams& p, int b, int K1) {
  return step_position(p.positions, b, p.P, K1);
}

template <int K1>
__global__ __launch_bounds__(kBlock) void k_attn_split(AttnParams p) {
  __shared__ __align__(16) bf16_t qb[16][kHeadDim];       // queries, rows >= K1 zero (MFMA B operand)
  __shared__ __align__(16) float wsm[4][K1][kPosTile];     // a wavefront's softmax weights of one tile
  __shared__ float wm[4][K1], wl[4][K1];
  __shared__ float wacc[4][K1][kHeadDim];
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int H = p.nh * kHeadDim;
  // positions are clamped so every access stays inside the cache
  const int pos0 = clamped_pos(p, b, K1);
  const int len = pos0 + K1;
  if (g >= used_groups(len, p.G)) return;
  for (int i = threadIdx.x; i < 16 * kHeadDim / 8; i += kBlock) {
    const int j = i / (kHeadDim / 8), c = i % (kHeadDim / 8);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < K1) v = *reinterpret_cast<const uint4*>(p.q + static_cast<int64_t>(b * K1 + j) * H + h * kHeadDim + 8 * c);
    *reinterpret_cast<uint4*>(&qb[j][8 * c]) = v;
  }
  __syncthreads();
  // query fragments of the four k-steps: column lane % 16, dimensions (lane / 16) * 8 + 32 ks
  bf16x8_t qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8_t*>(&qb[lane % 16][ks * 32 + (lane / 16) * 8]);
  const int64_t base = (static_cast<int64_t>(b) * p.nh + h) * p.P;
  const bf16_t* kc = p.kc + base * kHeadDim;
  const bf16_t* vc = p.vc + base * kHeadDim;
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
  const int jq = lane % 16;                    // the query this lane's scores belong to

  float m = kNegBig, l = 0.0f;  // running max and sum of query jq
  // weighted values: lane sums dimensions 8 (lane % 16) .. + 8 over the rows
  // 4 i + lane / 16 of each tile; the four lane groups are added at the end
  float acc[K1][8];
#pragma unroll
  for (int j = 0; j < K1; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
  for (int tile = g * 4 + wave; tile * kPosTile < len; tile += p.G * 4) {
    const int t0 = tile * kPosTile;
    // every load of the tile first: key fragments (A operand: row = position
    // t0 + 16 pt + lane % 16, dimensions (lane / 16) * 8 + 32 ks) and the 64
    // value-row words of this lane's two dimensions; rows past the cache length
    // repeat the last row and get weight zero
    uint4 kf[4][4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16_t* krow = kc + static_cast<int64_t>(min(t0 + pt * 16 + lane % 16, len - 1)) * kHeadDim;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[pt][ks] = *reinterpret_cast<const uint4*>(krow + ks * 32 + (lane / 16) * 8);
    }
    // value rows 4 i + lane / 16, 16 bytes a lane: 16 loads cover the tile, so
    // a tile's 32 loads stay under the per-wavefront limit of loads in flight
    uint4 vv[kPosTile / 4];
#pragma unroll
    for (int i = 0; i < kPosTile / 4; ++i)
      vv[i] = *reinterpret_cast<const uint4*>(
          vc + static_cast<int64_t>(min(t0 + 4 * i + lane / 16, len - 1)) * kHeadDim + 8 * (lane % 16));
    // scores: sc[pt][i] = q_jq . k at position t0 + 16 pt + 4 (lane / 16) + i
    f32x4_t sc[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      sc[pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[pt] = mfma16(__builtin_bit_cast(bf16x8_t, kf[pt][ks]), qf[ks], sc[pt]);
    }
    float M = kNegBig;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pp = t0 + pt * 16 + 4 * (lane / 16) + i;
        const bool ok = jq < K1 && pp < len && pp <= pos0 + jq;  // causal: query j sees up to pos0 + j
        sc[pt][i] = ok ? sc[pt][i] * scale : kNegBig;
        M = fmaxf(M, sc[pt][i]);
      }
    M = fmaxf(M, __shfl_xor(M, 16, kWave));
    M = fmaxf(M, __shfl_xor(M, 32, kWave));
    float L = 0.0f;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = sc[pt][i] > 0.5f * kNegBig ? exp_f(sc[pt][i] - M) : 0.0f;
        sc[pt][i] = e;
        L += e;
      }
    L += __shfl_xor(L, 16, kWave);
    L += __shfl_xor(L, 32, kWave);
    const float mn = fmaxf(m, M);
    const float a = exp_f(m - mn), c = exp_f(M - mn);
    l = l * a + L * c;
    m = mn;
    if (jq < K1) {
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i) wsm[wave][jq][pt * 16 + 4 * (lane / 16) + i] = sc[pt][i] * c;
    }
    // the weights cross lanes of this wavefront through LDS: its stores are
    // complete and visible before any lane reads them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // values: every lane rescales its accumulators by query j's factor (held
    // by lane j) and adds the tile's weighted value rows
#pragma unroll
    for (int j = 0; j < K1; ++j) {
      const float aj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), j));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= aj;
    }
#pragma unroll
    for (int i = 0; i < kPosTile / 4; ++i) {
      const float vf[8] = {__uint_as_float(vv[i].x << 16), __uint_as_float(vv[i].x & 0xffff0000u),
                           __uint_as_float(vv[i].y << 16), __uint_as_float(vv[i].y & 0xffff0000u),
                           __uint_as_float(vv[i].z << 16), __uint_as_float(vv[i].z & 0xffff0000u),
                           __uint_as_float(vv[i].w << 16), __uint_as_float(vv[i].w & 0xffff0000u)};
#pragma unroll
      for (int j = 0; j < K1; ++j) {
        const float wq = wsm[wave][j][4 * i + lane / 16];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(wq, vf[e], acc[j][e]);
      }
    }
    // every lane has read this tile's weights before the next tile's stores
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // the four lane groups' partial sums of every dimension
#pragma unroll
  for (int j = 0; j < K1; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[j][e] += __shfl_xor(acc[j][e], 16, kWave);
      acc[j][e] += __shfl_xor(acc[j][e], 32, kWave);
    }
  // the four wavefronts' states -> one partial per query
  if (lane < K1) {
    wm[wave][lane] = m;
    wl[wave][lane] = l;
  }
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < K1; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) wacc[wave][j][8 * lane + e] = acc[j][e];
  }
  __syncthreads();
  float* out = p.part + ((static_cast<int64_t>(b) * p.nh + h) * p.G + g) * K1 * kPartStride;
  for (int i = threadIdx.x; i < K1 * kHeadDim; i += kBlock) {
    const int j = i / kHeadDim, dd = i % kHeadDim;
    const float Mx = fmaxf(fmaxf(wm[0][j], wm[1][j]), fmaxf(wm[2][j], wm[3][j]));
    float Ls = 0.0f, A = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float f = exp_f(wm[q][j] - Mx);
      Ls += f * wl[q][j];
      A += f * wacc[q][j][dd];
    }
    out[j * kPartStride + 2 + dd] = A;
    if (dd == 0) {
      out[j * kPartStride] = Mx;
      out[j * kPartStride + 1] = Ls;
    }
  }
}

// One 128-thread workgroup per (query row, head), a thread per dimension:
// merge the partials of the groups that hold positions, divide, round.
__global__ __launch_bounds__(kHeadDim) void k_attn_combine(AttnParams p) {
  __shared__ float sm[kMaxGroups], sl[kMaxGroups], sf[kMaxGroups];
  const int t = blockIdx.x, h = blockIdx.y, b = t / p.K1, j = t % p.K1;
  const int dd = threadIdx.x;
  const int len = clamped_pos(p, b, p.K1) + p.K1;
  const int ng = used_groups(len, p.G);
  const float* part = p.part + ((static_cast<int64_t>(b) * p.nh + h) * p.G) * p.K1 * kPartStride + j * kPartStride;
  const int64_t gs = static_cast<int64_t>(p.K1) * kPartStride;
  // every load first (one memory round trip): group dd's max and sum, and
  // this dimension's weighted sum of every group
  float av[kMaxGroups];
#pragma unroll
  for (int g = 0; g < kMaxGroups; ++g) av[g] = g < ng ? part[g * gs + 2 + dd] : 0.0f;
  if (dd < ng) {
    sm[dd] = part[dd * gs];
    sl[dd] = part[dd * gs + 1];
  }
  __syncthreads();
  float M = kNegBig;
  for (int g = 0; g < ng; ++g) M = fmaxf(M, sm[g]);
  if (dd < ng) sf[dd] = exp_f(sm[dd] - M);
  __syncthreads();
  float L = 0.0f, A = 0.0f;
#pragma unroll
  for (int g = 0; g < kMaxGroups; ++g) {
    if (g < ng) {
      L = fmaf(sf[g], sl[g], L);
      A = fmaf(sf[g], av[g], A);
    }
  }
  p.ctx[static_cast<int64_t>(t) * (p.nh * kHeadDim) + h * kHeadDim + dd] = f32_to_bf16(A / L);
}

}  // namespace

int attn_groups(const Dims& d, int B, int nh) {
  // about one workgroup per CU, at least two groups: at B = 1 (10 heads)
  // twice that many groups (52) was 3 us slower -- more partials to combine
  // -- and one group at B = 32 12 us slower
  const int target = d.n_cu;
  return std::min(kMaxGroups, std::max(2, (target + B * nh - 1) / (B * nh)));
}

size_t attn_part_floats(int T, int nh, int G) { return static_cast<size_t>(T) * nh * G * kPartStride; }

hipError_t launch_attention(const Dims& d, const AttnParams& p, hipStream_t s) {
  const hipError_t e = launch_attention_split(d, p, s);
  return e != hipSuccess ? e : launch_attention_combine(p, s);
}

hipError_t launch_attention_combine(const AttnParams& p, hipStream_t s) {
  if (p.G > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_combine, dim3(p.B * p.K1, p.nh), dim3(kHeadDim), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attention_split(const Dims& d, const AttnParams& p, hipStream_t s) {
  if (p.K1 < 1 || p.K1 > kMaxK1 || p.B < 1 || p.G < 1 || p.P < p.K1 || d.H != p.nh * kHeadDim)
    return hipErrorInvalidValue;
  const dim3 grid(p.G, p.nh, p.B);
  switch (p.K1) {
    case 1: hipLaunchKernelGGL(k_attn_split<1>, grid, dim3(kBlock), 0, s, p); break;
    case 2: hipLaunchKernelGGL(k_attn_split<2>, grid, dim3(kBlock), 0, s, p); break;
    case 3: hipLaunchKernelGGL(k_attn_split<3>, grid, dim3(kBlock), 0, s, p); break;
    case 4: hipLaunchKernelGGL(k_attn_split<4>, grid, dim3(kBlock), 0, s, p); break;
    case 5: hipLaunchKernelGGL(k_attn_split<5>, grid, dim3(kBlock), 0, s, p); break;
    case 6: hipLaunchKernelGGL(k_attn_split<6>, grid, dim3(kBlock), 0, s, p); break;
    case 7: hipLaunchKernelGGL(k_attn_split<7>, grid, dim3(kBlock), 0, s, p); break;
    case 8: hipLaunchKernelGGL(k_attn_split<8>, grid, dim3(kBlock), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
