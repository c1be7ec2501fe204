// Combine + RMSNorm + top-k softmax router, one workgroup per 16 token rows.
//
// Phase 1 (one wavefront per token row): optionally finish the previous block
//   (m = shared outputs + gate-weighted routed outputs in ascending expert
//   order, x' = round(x + m)), then RMSNorm xh = round(x / sqrt(mean(x^2)+eps) * gamma).
// Phase 2: router logits z = W_r xh for the 16 rows.  bfloat16 storage uses
//   16x16x32 MFMA (wavefront w owns experts 16w..16w+15, the rows' xh sit in
//   LDS in operand layout); float32 storage uses plain FMAs.
// Phase 3 (one wavefront per token row, one lane per expert): k rounds of a
//   wavefront arg-max over (logit, lower expert first), then the softmax over
//   the k selected logits.
// The mixture of 64 routed experts with top-6 routing is the decoder of the
// page "Jina AI releases lightweight OCR model with built-in speculative
// decoding", section "Lean architecture with a compressed encoder"; the norm,
// softmax-over-selection and combine order are this library's reading.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRows = 16;        // token rows per workgroup
constexpr int kMaxChunks = 16;   // H <= 4096: 4-element chunks per lane

template <typename ST>
struct alignas(8) Vec4 { ST v[4]; };

template <typename ST>
__device__ __forceinline__ void load4(const ST* p, float out[4]) {
  Vec4<ST> v = *reinterpret_cast<const Vec4<ST>*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = Storage<ST>::load(v.v, i);
}

template <typename ST>
__device__ __forceinline__ void store4(ST* p, const float in[4]) {
  Vec4<ST> v;
#pragma unroll
  for (int i = 0; i < 4; ++i) Storage<ST>::store(v.v, i, in[i]);
  *reinterpret_cast<Vec4<ST>*>(p) = v;
}

template <typename ST>
__global__ __launch_bounds__(kBlock) void k_norm_router(Dims d, NormRouterParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  // bf16: xh operand tiles [H/32][64 lanes][8]; f32: xh rows [16][H]
  __shared__ float zl[kRows][kMaxExperts + 1];

  const int H = d.H, k = d.k, T = p.T;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kRows;
  const int nchunks = H / 4;  // 4-element chunks per row

  // ------------------------------------------------------------ phase 1
  for (int n = wave; n < kRows; n += 4) {
    const int t = t0 + n;
    if (t >= T) break;
    float x[kMaxChunks][4];
    const ST* xin = reinterpret_cast<const ST*>(p.x_in) + static_cast<int64_t>(t) * H;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int ch = lane + c * kWave;
      if (ch < nchunks) load4<ST>(xin + 4 * ch, x[c]);
    }
    if (p.combine) {
      float m[kMaxChunks][4];
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) m[c][i] = 0.0f;
      const int P = T * k;
      for (int s = 0; s < d.S; ++s) {
        const float* yr = p.y + static_cast<int64_t>(P + s * T + t) * H;
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
          const int ch = lane + c * kWave;
          if (ch < nchunks) {
            float4 v = *reinterpret_cast<const float4*>(yr + 4 * ch);
            m[c][0] = __fadd_rn(m[c][0], v.x);
            m[c][1] = __fadd_rn(m[c][1], v.y);
            m[c][2] = __fadd_rn(m[c][2], v.z);
            m[c][3] = __fadd_rn(m[c][3], v.w);
          }
        }
      }
      // routed experts of this row in ascending expert order
      int ids[kMaxTopK];
      float ws[kMaxTopK];
      int js[kMaxTopK];
      for (int j = 0; j < k; ++j) {
        ids[j] = p.prev_idx[t * k + j];
        ws[j] = p.prev_w[t * k + j];
        js[j] = j;
      }
      for (int a = 1; a < k; ++a) {  // insertion sort by expert id
        int ia = ids[a], ja = js[a];
        float wa = ws[a];
        int b = a - 1;
        while (b >= 0 && ids[b] > ia) {
          ids[b + 1] = ids[b];
          js[b + 1] = js[b];
          ws[b + 1] = ws[b];
          --b;
        }
        ids[b + 1] = ia;
        js[b + 1] = ja;
        ws[b + 1] = wa;
      }
      for (int a = 0; a < k; ++a) {
        const float* yr = p.y + static_cast<int64_t>(t * k + js[a]) * H;
        const float g = ws[a];
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
          const int ch = lane + c * kWave;
          if (ch < nchunks) {
            float4 v = *reinterpret_cast<const float4*>(yr + 4 * ch);
            m[c][0] = __fadd_rn(m[c][0], __fmul_rn(g, v.x));
            m[c][1] = __fadd_rn(m[c][1], __fmul_rn(g, v.y));
            m[c][2] = __fadd_rn(m[c][2], __fmul_rn(g, v.z));
            m[c][3] = __fadd_rn(m[c][3], __fmul_rn(g, v.w));
          }
        }
      }
      ST* xout = reinterpret_cast<ST*>(p.x_out) + static_cast<int64_t>(t) * H;
      float* mo = p.m_out ? p.m_out + static_cast<int64_t>(t) * H : nullptr;
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) {
        const int ch = lane + c * kWave;
        if (ch < nchunks) {
#pragma unroll
          for (int i = 0; i < 4; ++i) x[c][i] = Storage<ST>::round(__fadd_rn(x[c][i], m[c][i]));
          store4<ST>(xout + 4 * ch, x[c]);
          if (mo) *reinterpret_cast<float4*>(mo + 4 * ch) = make_float4(m[c][0], m[c][1], m[c][2], m[c][3]);
        }
      }
    }
    if (!p.norm) continue;
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int ch = lane + c * kWave;
      if (ch < nchunks)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = __fadd_rn(ss, __fmul_rn(x[c][i], x[c][i]));
    }
    ss = wave_sum(ss);
    const float rms = sqrtf(ss / static_cast<float>(H) + d.eps);
    const ST* gam = reinterpret_cast<const ST*>(p.gamma);
    ST* xh = reinterpret_cast<ST*>(p.xhat) + static_cast<int64_t>(t) * H;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int ch = lane + c * kWave;
      if (ch < nchunks) {
        float g[4], v[4];
        load4<ST>(gam + 4 * ch, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = Storage<ST>::round(__fmul_rn(x[c][i] / rms, g[i]));
        store4<ST>(xh + 4 * ch, v);
        if (p.route) {
          const int h = 4 * ch;
          if constexpr (sizeof(ST) == 2) {
            // operand tile kt = h/32; lane n + 16*((h%32)/8); element h%8
            bf16_t* tile = reinterpret_cast<bf16_t*>(smem);
            const int kt = h / 32, ln = n + 16 * ((h % 32) / 8);
            store4<bf16_t>(tile + (kt * kWave + ln) * 8 + (h % 8), v);
          } else {
            float* rows = reinterpret_cast<float*>(smem);
            *reinterpret_cast<float4*>(rows + n * H + h) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
    if (p.keys && lane == 0) p.keys[t] = 0ull;
  }
  if (!p.route) return;

  // rows of this workgroup that are past T: zero operand lanes (bf16) so the
  // MFMA reads defined values; their logits are never used.
  const int nrows = min(kRows, T - t0);
  if constexpr (sizeof(ST) == 2) {
    if (nrows < kRows) {
      bf16_t* tile = reinterpret_cast<bf16_t*>(smem);
      const int nkt = H / kKStep;
      for (int i = threadIdx.x; i < nkt * kWave; i += kBlock) {
        const int ln = i % kWave;
        if ((ln % 16) >= nrows) *reinterpret_cast<uint4*>(tile + i * 8) = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __syncthreads();

  // ------------------------------------------------------------ phase 2
  if constexpr (sizeof(ST) == 2) {
    if (wave * 16 < d.E) {
      const bf16_t* tile = reinterpret_cast<const bf16_t*>(smem);
      const bf16_t* wr = reinterpret_cast<const bf16_t*>(p.router) +
                         static_cast<int64_t>(wave) * (H / kKStep) * kFragElems;
      f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      const int nkt = H / kKStep;
      int kt = 0;
      for (; kt + 1 < nkt; kt += 2) {
        acc0 = mfma16(load_frag(wr + kt * kFragElems + lane * 8), load_frag(tile + (kt * kWave + lane) * 8), acc0);
        acc1 = mfma16(load_frag(wr + (kt + 1) * kFragElems + lane * 8),
                      load_frag(tile + ((kt + 1) * kWave + lane) * 8), acc1);
      }
      if (kt < nkt)
        acc0 = mfma16(load_frag(wr + kt * kFragElems + lane * 8), load_frag(tile + (kt * kWave + lane) * 8), acc0);
      // lane holds z[expert 16*wave + 4*(lane/16) + i][row lane%16]
#pragma unroll
      for (int i = 0; i < 4; ++i) zl[lane % 16][wave * 16 + 4 * (lane / 16) + i] = acc0[i] + acc1[i];
    }
  } else {
    const float* rows = reinterpret_cast<const float*>(smem);
    const float* wr = reinterpret_cast<const float*>(p.router);
    for (int i = threadIdx.x; i < nrows * d.E; i += kBlock) {
      const int n = i / d.E, e = i % d.E;
      const float* xr = rows + n * H;
      const float* w = wr + static_cast<int64_t>(e) * H;
      float acc = 0.0f;
      for (int h = 0; h < H; ++h) acc = __fadd_rn(acc, __fmul_rn(xr[h], w[h]));
      zl[n][e] = acc;
    }
  }
  __syncthreads();

  // ------------------------------------------------------------ phase 3
  for (int n = wave; n < nrows; n += 4) {
    const int t = t0 + n;
    uint64_t key = lane < d.E ? argmax_key(zl[n][lane], static_cast<uint32_t>(lane)) : 0ull;
    int sel_e[kMaxTopK];
    float sel_z[kMaxTopK];
    for (int j = 0; j < k; ++j) {
      const uint64_t best = wave_max_u64(key);
      const int e = static_cast<int>(argmax_key_index(best));
      sel_e[j] = e;
      sel_z[j] = zl[n][e];
      if (lane == e) key = 0ull;
    }
    float ex[kMaxTopK];
    float den = 0.0f;
    for (int j = 0; j < k; ++j) {
      ex[j] = expf(sel_z[j] - sel_z[0]);
      den = __fadd_rn(den, ex[j]);
    }
    if (lane < k) {
      float wj = 0.0f;
      int ej = 0;
      for (int j = 0; j < k; ++j)
        if (j == lane) {
          wj = ex[j] / den;
          ej = sel_e[j];
        }
      p.idx_out[t * k + lane] = ej;
      p.w_out[t * k + lane] = wj;
    }
  }
}

}  // namespace

hipError_t launch_norm_router(const Dims& d, const NormRouterParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  const dim3 grid((p.T + kRows - 1) / kRows);
  if (d.bf16) {
    const size_t smem = p.route ? static_cast<size_t>(d.H) * 32 : 0;  // 16 rows x H bf16
    hipLaunchKernelGGL(k_norm_router<bf16_t>, grid, dim3(kBlock), smem, s, d, p);
  } else {
    const size_t smem = p.route ? static_cast<size_t>(d.H) * kRows * sizeof(float) : 0;
    hipLaunchKernelGGL(k_norm_router<float>, grid, dim3(kBlock), smem, s, d, p);
  }
  return hipGetLastError();
}

}  // namespace moe
