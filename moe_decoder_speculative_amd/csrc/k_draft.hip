// Draft head: the row kernels around one recursive dense-block step.
//
// A draft step for B sequences is eight launches on one stream:
//   k_draft_in (first step only) / k_draft_pick (later steps): the normalised
//       state and token-embedding rows a, e that the projection reads;
//   projection: the expert "down" kernel with two shared slots of width H
//       (slot 0 = W_proj[:, :H] on a, slot 1 = W_proj[:, H:] on e);
//   k_draft_mid: u = round(y0 + y1) and the FFN input RMSNorm(u);
//   FFN: the expert "up" and "down" kernels with the dense width split into Sf
//       shared slots of width If (the dense SwiGLU is the sum of its column
//       blocks, so the slots' outputs add up to W_down act);
//   k_draft_out: v = round(u + sum of the slots' outputs), the step output,
//       RMSNorm(v) for the head and, unless this is the last step, the next
//       step's normalised state;
//   the LM-head kernel (arg-max keys) and k_draft_pick: the draft token, and
//       for the next step the normalised embedding of that token.
// Each row kernel is one 256-thread workgroup per sequence: the row's loads,
// and the gains its RMSNorm multiplies by, are all issued before the sum of
// squares is reduced (a load after the reduction is one more memory round
// trip), and H <= 2048 gives at most two 4-element chunks per thread.  The block is the page "Jina AI
// releases lightweight OCR model with built-in speculative decoding", section
// "Speculative decoding without accuracy loss" (one draft block applied K
// times); its internals are this library's reading.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kCPB = 2;  // 4-element chunks per thread: H / 4 <= 2 * kBlock

struct Row {
  float v[kCPB][4];
};

__device__ __forceinline__ void load_bf16_row(const bf16_t* src, int nchunks, Row& r) {
#pragma unroll
  for (int c = 0; c < kCPB; ++c) {
    const int ch = threadIdx.x + c * kBlock;
    uint2 q = make_uint2(0u, 0u);
    if (ch < nchunks && src) q = *reinterpret_cast<const uint2*>(src + 4 * ch);
    r.v[c][0] = __uint_as_float(q.x << 16);
    r.v[c][1] = __uint_as_float(q.x & 0xffff0000u);
    r.v[c][2] = __uint_as_float(q.y << 16);
    r.v[c][3] = __uint_as_float(q.y & 0xffff0000u);
  }
}

__device__ __forceinline__ float row_sumsq(const Row& r, int nchunks) {
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < kCPB; ++c) {
    if (static_cast<int>(threadIdx.x) + c * kBlock < nchunks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ss = __fadd_rn(ss, __fmul_rn(r.v[c][i], r.v[c][i]));
    }
  }
  return ss;
}

// Workgroup sums of up to two per-thread partials (red: 2 x 4 floats of LDS).
__device__ __forceinline__ void block_sum2(float& a, float& b, float (*red)[kBlock / kWave]) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) {
    red[0][w] = a;
    red[1][w] = b;
  }
  __syncthreads();
  a = red[0][0];
  b = red[1][0];
#pragma unroll
  for (int q = 1; q < kBlock / kWave; ++q) {
    a += red[0][q];
    b += red[1][q];
  }
}

// A gain vector's chunks of this thread, loaded with the row.
struct Gain {
  uint2 g[kCPB];
};

__device__ __forceinline__ Gain load_gain(const bf16_t* gamma, int nchunks) {
  Gain r;
#pragma unroll
  for (int c = 0; c < kCPB; ++c) {
    const int ch = threadIdx.x + c * kBlock;
    r.g[c] = ch < nchunks ? *reinterpret_cast<const uint2*>(gamma + 4 * ch) : make_uint2(0u, 0u);
  }
  return r;
}

// dst = round(r / rms * gamma), rms = sqrt(ss / H + eps)
__device__ __forceinline__ void store_norm(const Row& r, int nchunks, float ss, const Dims& d, const Gain& gamma,
                                           bf16_t* dst) {
  const float rms = sqrtf(ss / static_cast<float>(d.H) + d.eps);
#pragma unroll
  for (int c = 0; c < kCPB; ++c) {
    const int ch = threadIdx.x + c * kBlock;
    if (ch < nchunks) {
      const uint2 g = gamma.g[c];
      const float gg[4] = {__uint_as_float(g.x << 16), __uint_as_float(g.x & 0xffff0000u),
                           __uint_as_float(g.y << 16), __uint_as_float(g.y & 0xffff0000u)};
      uint2 o;
      o.x = pack_bf16x2(__fmul_rn(r.v[c][0] / rms, gg[0]), __fmul_rn(r.v[c][1] / rms, gg[1]));
      o.y = pack_bf16x2(__fmul_rn(r.v[c][2] / rms, gg[2]), __fmul_rn(r.v[c][3] / rms, gg[3]));
      *reinterpret_cast<uint2*>(dst + 4 * ch) = o;
    }
  }
}

__device__ __forceinline__ void store_row(const Row& r, int nchunks, bf16_t* dst) {
#pragma unroll
  for (int c = 0; c < kCPB; ++c) {
    const int ch = threadIdx.x + c * kBlock;
    if (ch < nchunks) {
      uint2 o;
      o.x = pack_bf16x2(r.v[c][0], r.v[c][1]);
      o.y = pack_bf16x2(r.v[c][2], r.v[c][3]);
      *reinterpret_cast<uint2*>(dst + 4 * ch) = o;
    }
  }
}

__device__ __forceinline__ const bf16_t* embed_row(const DraftParams& p, const Dims& d, int tok) {
  return tok >= 0 && tok < p.V ? p.embed + static_cast<int64_t>(tok) * d.H : nullptr;
}

// First step: the state row and token each sequence continues from.
__global__ __launch_bounds__(kBlock) void k_draft_in(Dims d, DraftParams p) {
  __shared__ float red[2][kBlock / kWave];
  const int b = blockIdx.x, nchunks = d.H / 4;
  const Gain gh = load_gain(p.gamma_h, nchunks), ge = load_gain(p.gamma_e, nchunks);
  const int j = p.counts ? min(max(p.counts[b] - 1, 0), p.R - 1) : p.R - 1;
  const int64_t row = static_cast<int64_t>(b) * p.R + j;
  const int tok = p.committed[row];
  Row h, e;
  load_bf16_row(p.hidden + row * d.H, nchunks, h);
  load_bf16_row(embed_row(p, d, tok), nchunks, e);
  float sh = row_sumsq(h, nchunks), se = row_sumsq(e, nchunks);
  block_sum2(sh, se, red);
  store_norm(h, nchunks, sh, d, gh, p.x + static_cast<int64_t>(b) * d.H);
  store_norm(e, nchunks, se, d, ge, p.x + static_cast<int64_t>(p.B + b) * d.H);
}

// u = round(y0 + y1); FFN input RMSNorm(u; gamma_f)
__global__ __launch_bounds__(kBlock) void k_draft_mid(Dims d, DraftParams p) {
  __shared__ float red[2][kBlock / kWave];
  const int b = blockIdx.x, nchunks = d.H / 4;
  const float* y0 = p.yp + static_cast<int64_t>(b) * d.H;
  const float* y1 = p.yp + static_cast<int64_t>(p.B + b) * d.H;
  const Gain gf = load_gain(p.gamma_f, nchunks);
  Row u;
#pragma unroll
  for (int c = 0; c < kCPB; ++c) {
    const int ch = threadIdx.x + c * kBlock;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), q = a;
    if (ch < nchunks) {
      a = *reinterpret_cast<const float4*>(y0 + 4 * ch);
      q = *reinterpret_cast<const float4*>(y1 + 4 * ch);
    }
    u.v[c][0] = bf16_to_f32(f32_to_bf16(__fadd_rn(a.x, q.x)));
    u.v[c][1] = bf16_to_f32(f32_to_bf16(__fadd_rn(a.y, q.y)));
    u.v[c][2] = bf16_to_f32(f32_to_bf16(__fadd_rn(a.z, q.z)));
    u.v[c][3] = bf16_to_f32(f32_to_bf16(__fadd_rn(a.w, q.w)));
  }
  store_row(u, nchunks, p.u + static_cast<int64_t>(b) * d.H);
  float ss = row_sumsq(u, nchunks), unused = 0.0f;
  block_sum2(ss, unused, red);
  store_norm(u, nchunks, ss, d, gf, p.uh + static_cast<int64_t>(b) * d.H);
}

// v = round(u + sum_s y_s) (slots in ascending order); the step output, the
// head input RMSNorm(v; gamma_o) and the next step's RMSNorm(v; gamma_h)
__global__ __launch_bounds__(kBlock) void k_draft_out(Dims d, DraftParams p) {
  __shared__ float red[2][kBlock / kWave];
  const int b = blockIdx.x, nchunks = d.H / 4;
  const Gain go = load_gain(p.gamma_o, nchunks), gh = load_gain(p.gamma_h, nchunks);
  Row v;
  load_bf16_row(p.u + static_cast<int64_t>(b) * d.H, nchunks, v);
  // the slots' outputs, added in ascending slot order; each group of eight
  // slots has all its loads in flight before the first add
  constexpr int kG = 8;
  float m[kCPB][4] = {};
  for (int s0 = 0; s0 < p.Sf; s0 += kG) {
    float4 y[kG][kCPB];
#pragma unroll
    for (int q = 0; q < kG; ++q)
#pragma unroll
      for (int c = 0; c < kCPB; ++c) {
        const int ch = threadIdx.x + c * kBlock;
        y[q][c] = s0 + q < p.Sf && ch < nchunks
                      ? *reinterpret_cast<const float4*>(p.y + (static_cast<int64_t>(s0 + q) * p.B + b) * d.H + 4 * ch)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int q = 0; q < kG; ++q)
#pragma unroll
      for (int c = 0; c < kCPB; ++c)
        if (s0 + q < p.Sf) {
          m[c][0] = __fadd_rn(m[c][0], y[q][c].x);
          m[c][1] = __fadd_rn(m[c][1], y[q][c].y);
          m[c][2] = __fadd_rn(m[c][2], y[q][c].z);
          m[c][3] = __fadd_rn(m[c][3], y[q][c].w);
        }
  }
#pragma unroll
  for (int c = 0; c < kCPB; ++c)
    if (static_cast<int>(threadIdx.x) + c * kBlock < nchunks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v.v[c][i] = bf16_to_f32(f32_to_bf16(__fadd_rn(v.v[c][i], m[c][i])));
    }
  if (p.states) store_row(v, nchunks, p.states + (static_cast<int64_t>(p.step) * p.B + b) * d.H);
  float ss = row_sumsq(v, nchunks), unused = 0.0f;
  block_sum2(ss, unused, red);
  store_norm(v, nchunks, ss, d, go, p.xf + static_cast<int64_t>(b) * d.H);
  if (!p.last) store_norm(v, nchunks, ss, d, gh, p.x + static_cast<int64_t>(b) * d.H);
}

// The draft token from the arg-max keys (which are cleared for the next use)
// and, unless this is the last step, the next step's normalised embedding.
__global__ __launch_bounds__(kBlock) void k_draft_pick(Dims d, DraftParams p) {
  __shared__ float red[2][kBlock / kWave];
  __shared__ int tok_s;
  const int b = blockIdx.x, nchunks = d.H / 4;
  const Gain ge = load_gain(p.gamma_e, nchunks);
  if (threadIdx.x < kWave) {
    unsigned long long key = 0ull;
    if (threadIdx.x < kKeySlots) {
      unsigned long long* kp = p.keys + static_cast<int64_t>(threadIdx.x) * p.key_stride + b;
      key = *kp;
      *kp = 0ull;
    }
    key = wave_max_u64(key);
    if (threadIdx.x == 0) {
      const uint32_t row = argmax_key_index(key);
      const int tok = row < static_cast<uint32_t>(p.Vd) ? (p.head_ids ? p.head_ids[row] : static_cast<int>(row)) : -1;
      p.drafts[b * p.K + p.step] = tok;
      tok_s = tok;
    }
  }
  if (p.last) return;
  __syncthreads();
  Row e;
  load_bf16_row(embed_row(p, d, tok_s), nchunks, e);
  float ss = row_sumsq(e, nchunks), unused = 0.0f;
  block_sum2(ss, unused, red);
  store_norm(e, nchunks, ss, d, ge, p.x + static_cast<int64_t>(p.B + b) * d.H);
}

}  // namespace

static hipError_t draft_rows_ok(const Dims& d, const DraftParams& p) {
  return (p.B >= 1 && d.H % 4 == 0 && d.H / 4 <= kCPB * kBlock) ? hipSuccess : hipErrorInvalidValue;
}

hipError_t launch_draft_in(const Dims& d, const DraftParams& p, hipStream_t s) {
  if (draft_rows_ok(d, p) != hipSuccess) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_draft_in, dim3(p.B), dim3(kBlock), 0, s, d, p);
  return hipGetLastError();
}

hipError_t launch_draft_mid(const Dims& d, const DraftParams& p, hipStream_t s) {
  if (draft_rows_ok(d, p) != hipSuccess) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_draft_mid, dim3(p.B), dim3(kBlock), 0, s, d, p);
  return hipGetLastError();
}

hipError_t launch_draft_out(const Dims& d, const DraftParams& p, hipStream_t s) {
  if (draft_rows_ok(d, p) != hipSuccess) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_draft_out, dim3(p.B), dim3(kBlock), 0, s, d, p);
  return hipGetLastError();
}

hipError_t launch_draft_pick(const Dims& d, const DraftParams& p, hipStream_t s) {
  if (draft_rows_ok(d, p) != hipSuccess) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_draft_pick, dim3(p.B), dim3(kBlock), 0, s, d, p);
  return hipGetLastError();
}

}  // namespace moe
