// Decode attention of the verify step: each sequence's K1 = K+1 query rows
// (the last committed token and the drafts, already rotated and with their
// keys and values written to the cache) against cache positions 0..p_b+j.
//
// At decode sizes attention is a stream over the KV cache (512 B per position
// and head), so the work is split over positions: workgroup (g, h, b) takes
// the 64-position tiles g*4 + w, g*4 + w + 4G, ... of sequence b and head h,
// one tile per wavefront at a time, in float32 on the vector ALUs:
//   scores: lane = position, the lane streams its 256-byte key row and dots
//           it with the K1 queries held in LDS (broadcast reads);
//   softmax: per query the tile's maximum and sum across the wavefront, folded
//           into a running (max, sum) with the usual rescaling;
//   values:  lane = two head dimensions, each position's value row is one
//           coalesced 256-byte read, its weights broadcast from the lane that
//           scored it (readlane).
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
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

template <int K1>
__global__ __launch_bounds__(kBlock) void k_attn_split(AttnParams p) {
  __shared__ __align__(16) float qs[K1][kHeadDim];
  __shared__ float wm[4][K1], wl[4][K1];
  __shared__ float wacc[4][K1][kHeadDim];
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int H = p.nh * kHeadDim;
  // positions are clamped so every access stays inside the cache
  const int pos0 = min(max(p.positions[b], 0), p.P - K1);
  const int len = pos0 + K1;
  for (int i = threadIdx.x; i < K1 * kHeadDim; i += kBlock) {
    const int j = i / kHeadDim, dd = i % kHeadDim;
    qs[j][dd] = bf16_to_f32(p.q[static_cast<int64_t>(b * K1 + j) * H + h * kHeadDim + dd]);
  }
  __syncthreads();
  const int64_t base = (static_cast<int64_t>(b) * p.nh + h) * p.P;
  const bf16_t* kc = p.kc + base * kHeadDim;
  const bf16_t* vc = p.vc + base * kHeadDim;
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)

  float m[K1], l[K1], acc[K1][2];
#pragma unroll
  for (int j = 0; j < K1; ++j) {
    m[j] = kNegBig;
    l[j] = 0.0f;
    acc[j][0] = acc[j][1] = 0.0f;
  }
  for (int tile = g * 4 + wave; tile * kPosTile < len; tile += p.G * 4) {
    const int pp = tile * kPosTile + lane;
    const bool valid = pp < len;
    const bf16_t* krow = kc + static_cast<int64_t>(min(pp, len - 1)) * kHeadDim;
    float s[K1];
#pragma unroll
    for (int j = 0; j < K1; ++j) s[j] = 0.0f;
#pragma unroll 4
    for (int c = 0; c < kHeadDim / 8; ++c) {
      const uint4 kv = *reinterpret_cast<const uint4*>(krow + c * 8);
      const float kf[8] = {__uint_as_float(kv.x << 16), __uint_as_float(kv.x & 0xffff0000u),
                           __uint_as_float(kv.y << 16), __uint_as_float(kv.y & 0xffff0000u),
                           __uint_as_float(kv.z << 16), __uint_as_float(kv.z & 0xffff0000u),
                           __uint_as_float(kv.w << 16), __uint_as_float(kv.w & 0xffff0000u)};
#pragma unroll
      for (int j = 0; j < K1; ++j) {
        const float4 qa = *reinterpret_cast<const float4*>(&qs[j][c * 8]);
        const float4 qb = *reinterpret_cast<const float4*>(&qs[j][c * 8 + 4]);
        s[j] = fmaf(kf[0], qa.x, s[j]);
        s[j] = fmaf(kf[1], qa.y, s[j]);
        s[j] = fmaf(kf[2], qa.z, s[j]);
        s[j] = fmaf(kf[3], qa.w, s[j]);
        s[j] = fmaf(kf[4], qb.x, s[j]);
        s[j] = fmaf(kf[5], qb.y, s[j]);
        s[j] = fmaf(kf[6], qb.z, s[j]);
        s[j] = fmaf(kf[7], qb.w, s[j]);
      }
    }
    float w[K1];
#pragma unroll
    for (int j = 0; j < K1; ++j) {
      const bool ok = valid && pp <= pos0 + j;  // causal: query j sees positions up to pos0 + j
      const float sj = ok ? s[j] * scale : kNegBig;
      const float M = wave_max(sj);
      const float e = ok ? exp_f(sj - M) : 0.0f;
      const float L = wave_sum(e);
      const float mn = fmaxf(m[j], M);
      const float a = exp_f(m[j] - mn), c = exp_f(M - mn);
      l[j] = l[j] * a + L * c;
      acc[j][0] *= a;
      acc[j][1] *= a;
      m[j] = mn;
      w[j] = e * c;
    }
    const int n = min(kPosTile, len - tile * kPosTile);
    const bf16_t* vrow = vc + static_cast<int64_t>(tile * kPosTile) * kHeadDim + 2 * lane;
    for (int q = 0; q < n; ++q) {
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(vrow + static_cast<int64_t>(q) * kHeadDim);
      const float v0 = __uint_as_float(vv << 16), v1 = __uint_as_float(vv & 0xffff0000u);
#pragma unroll
      for (int j = 0; j < K1; ++j) {
        const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[j]), q));
        acc[j][0] = fmaf(wq, v0, acc[j][0]);
        acc[j][1] = fmaf(wq, v1, acc[j][1]);
      }
    }
  }
  // the four wavefronts' states -> one partial per query
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < K1; ++j) {
      wm[wave][j] = m[j];
      wl[wave][j] = l[j];
    }
  }
#pragma unroll
  for (int j = 0; j < K1; ++j) {
    wacc[wave][j][2 * lane] = acc[j][0];
    wacc[wave][j][2 * lane + 1] = acc[j][1];
  }
  __syncthreads();
  float* out = p.part + ((static_cast<int64_t>(b) * p.nh + h) * p.G + g) * K1 * kPartStride;
  for (int i = threadIdx.x; i < K1 * kHeadDim; i += kBlock) {
    const int j = i / kHeadDim, dd = i % kHeadDim;
    const float M = fmaxf(fmaxf(wm[0][j], wm[1][j]), fmaxf(wm[2][j], wm[3][j]));
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float f = exp_f(wm[q][j] - M);
      L += f * wl[q][j];
      A += f * wacc[q][j][dd];
    }
    out[j * kPartStride + 2 + dd] = A;
    if (dd == 0) {
      out[j * kPartStride] = M;
      out[j * kPartStride + 1] = L;
    }
  }
}

// One workgroup per query row: merge the G partials of each head, divide,
// round to bfloat16.
__global__ __launch_bounds__(kBlock) void k_attn_combine(AttnParams p) {
  const int t = blockIdx.x, b = t / p.K1, j = t % p.K1;
  const int H = p.nh * kHeadDim;
  for (int i = threadIdx.x; i < H; i += kBlock) {
    const int h = i / kHeadDim, dd = i % kHeadDim;
    const float* part = p.part + ((static_cast<int64_t>(b) * p.nh + h) * p.G) * p.K1 * kPartStride + j * kPartStride;
    float M = kNegBig;
    for (int g = 0; g < p.G; ++g) M = fmaxf(M, part[static_cast<int64_t>(g) * p.K1 * kPartStride]);
    float L = 0.0f, A = 0.0f;
    for (int g = 0; g < p.G; ++g) {
      const float* pg = part + static_cast<int64_t>(g) * p.K1 * kPartStride;
      const float f = exp_f(pg[0] - M);
      L += f * pg[1];
      A += f * pg[2 + dd];
    }
    p.ctx[static_cast<int64_t>(t) * H + i] = f32_to_bf16(A / L);
  }
}

}  // namespace

int attn_groups(const Dims& d, int B, int nh) {
  const int target = 2 * d.n_cu;
  return std::min(64, std::max(1, (target + B * nh - 1) / (B * nh)));
}

size_t attn_part_floats(int T, int nh, int G) { return static_cast<size_t>(T) * nh * G * kPartStride; }

hipError_t launch_attention(const Dims& d, const AttnParams& p, hipStream_t s) {
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
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(p.B * p.K1), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
