// LM head + greedy arg-max + longest-prefix acceptance.
//
// The vocabulary matrix is streamed from HBM exactly once per step; logits are
// never written.  bfloat16: each workgroup owns 64*R vocabulary rows (R row
// tiles of 16 per wavefront); the K loop runs over chunks of KC 32-wide
// k-steps.  Weight tiles go straight to registers (pre-tiled, coalesced 1 KiB
// per wavefront per tile, one chunk prefetched ahead); the final-norm
// activations of all tokens for the chunk are staged in LDS in operand order
// (double-buffered) and shared by the four wavefronts.  16x16x32 MFMAs
// accumulate [rows x tokens] in registers.  The epilogue reduces each token's
// best (logit, lowest id) over the workgroup's rows and folds it into a 64-bit
// key with one atomicMax per token; the last workgroup to finish (completion
// counter) decodes the keys into the greedy picks and runs the acceptance:
// the longest prefix of drafts equal to the picks, plus the verifier's next
// pick (page "Jina AI releases lightweight OCR model with built-in speculative
// decoding", section "Speculative decoding without accuracy loss").
#include "kernels.h"

namespace moe {

namespace {

__device__ void finish_step(const LmHeadParams& p, unsigned int n_blocks) {
  __shared__ int is_last;
  __threadfence();  // this thread's key atomics complete before the count below
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int prev = __hip_atomic_fetch_add(p.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == n_blocks - 1);
  }
  __syncthreads();
  if (!is_last) return;
  const int K1 = p.K + 1;
  for (int t = threadIdx.x; t < p.T; t += kBlock) {
    if (p.tstar) {
      const uint64_t key = __hip_atomic_load(p.keys + t, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
      p.tstar[t] = static_cast<int>(argmax_key_index(key));
    }
  }
  for (int b = threadIdx.x; b < p.B; b += kBlock) {
    int pick[8];
    for (int j = 0; j < K1; ++j) {
      const uint64_t key = __hip_atomic_load(p.keys + b * K1 + j, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
      pick[j] = static_cast<int>(argmax_key_index(key));
    }
    int a = 0;
    while (a < p.K && p.drafts[b * p.K + a] == pick[a]) ++a;
    for (int j = 0; j < K1; ++j) p.committed[b * K1 + j] = j <= a ? pick[j] : -1;
    p.counts[b] = a + 1;
  }
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(p.done, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- bf16 ----

template <int NT, int R, int KC>
__global__ __launch_bounds__(kBlock) void k_lmhead_mfma(Dims d, LmHeadParams p) {
  // B operand chunks: [2 buffers][NT token tiles][KC k-steps][64 lanes][8]
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* bl = reinterpret_cast<bf16_t*>(smem);
  __shared__ uint64_t wbest[4][kTile];

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int H = d.H, KT = H / kKStep, nchunks = KT / KC;
  const int tok0 = blockIdx.y * NT * kTile;      // token group of this workgroup
  const int vt0 = (blockIdx.x * 4 + wave) * R;   // first row tile of this wavefront
  const bf16_t* lm = reinterpret_cast<const bf16_t*>(p.lm);
  const bf16_t* xf = reinterpret_cast<const bf16_t*>(p.xf);
  constexpr int kStage = NT * KC * kWave;        // fragments per chunk
  constexpr int kPer = (kStage + kBlock - 1) / kBlock;

  auto a_ptr = [&](int r, int kt) {
    return lm + (static_cast<int64_t>(vt0 + r) * KT + kt) * kFragElems + lane * 8;
  };
  auto stage_load = [&](int c, bf16x8_t (&st)[kPer]) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int f = threadIdx.x + q * kBlock;
      st[q] = zero_frag();
      if (f < kStage) {
        const int ln = f % kWave, kk = (f / kWave) % KC, nt = f / (kWave * KC);
        const int tok = tok0 + nt * kTile + ln % kTile;
        if (tok < p.T)
          st[q] = load_frag(xf + static_cast<int64_t>(tok) * H + (c * KC + kk) * kKStep + (ln / kTile) * 8);
      }
    }
  };
  auto stage_store = [&](int buf, const bf16x8_t (&st)[kPer]) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int f = threadIdx.x + q * kBlock;
      if (f < kStage) *reinterpret_cast<bf16x8_t*>(bl + (buf * kStage + f) * 8) = st[q];
    }
  };

  f32x4_t acc[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[r][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  bf16x8_t a_cur[R][KC], a_nxt[R][KC];
  bf16x8_t st[kPer];
  stage_load(0, st);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) a_cur[r][kk] = load_frag(a_ptr(r, kk));
  stage_store(0, st);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) {
      stage_load(c + 1, st);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) a_nxt[r][kk] = load_frag(a_ptr(r, (c + 1) * KC + kk));
    }
    const bf16_t* bb = bl + (c & 1) * kStage * 8;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(bb + ((nt * KC + kk) * kWave + lane) * 8);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][nt] = mfma16(a_cur[r][kk], b, acc[r][nt]);
      }
    if (more) stage_store((c + 1) & 1, st);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) a_cur[r][kk] = a_nxt[r][kk];
    }
  }

  // arg-max epilogue: lane holds rows 4*(lane/16)+i of each row tile, token lane%16
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    uint64_t best = 0ull;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = (vt0 + r) * kTile + 4 * (lane / kTile) + i;
        if (v < d.V) {
          const uint64_t key = argmax_key(acc[r][nt][i], static_cast<uint32_t>(v));
          best = key > best ? key : best;
        }
      }
    uint64_t o = __shfl_xor(best, 16, kWave);
    best = o > best ? o : best;
    o = __shfl_xor(best, 32, kWave);
    best = o > best ? o : best;
    if (lane < kTile) wbest[wave][lane] = best;
    __syncthreads();
    if (threadIdx.x < kTile) {
      uint64_t b = wbest[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < 4; ++w) b = wbest[w][threadIdx.x] > b ? wbest[w][threadIdx.x] : b;
      const int tok = tok0 + nt * kTile + threadIdx.x;
      if (tok < p.T && b != 0ull) atomicMax(p.keys + tok, static_cast<unsigned long long>(b));
    }
    __syncthreads();
  }
  finish_step(p, gridDim.x * gridDim.y);
}

// ------------------------------------------------------------- float32 ----
// One thread per vocabulary row, loop over tokens; float32 storage only.

__global__ __launch_bounds__(kBlock) void k_lmhead_f32(Dims d, LmHeadParams p) {
  __shared__ uint64_t wbest[4];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int v = blockIdx.x * kBlock + threadIdx.x;
  const float* lm = reinterpret_cast<const float*>(p.lm);
  const float* xf = reinterpret_cast<const float*>(p.xf);
  for (int t = 0; t < p.T; ++t) {
    uint64_t key = 0ull;
    if (v < d.V) {
      const float* w = lm + static_cast<int64_t>(v) * d.H;
      const float* x = xf + static_cast<int64_t>(t) * d.H;
      float acc = 0.f;
      for (int h = 0; h < d.H; ++h) acc = __fadd_rn(acc, __fmul_rn(w[h], x[h]));
      key = argmax_key(acc, static_cast<uint32_t>(v));
    }
    key = wave_max_u64(key);
    if (lane == 0) wbest[wave] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t b = wbest[0];
      for (int w = 1; w < 4; ++w) b = wbest[w] > b ? wbest[w] : b;
      if (b != 0ull) atomicMax(p.keys + t, static_cast<unsigned long long>(b));
    }
    __syncthreads();
  }
  finish_step(p, gridDim.x);
}

template <int NT>
hipError_t lm_nt(const Dims& d, const LmHeadParams& p, hipStream_t s) {
  constexpr int R = 4, KC = 2;
  const int groups = (p.T + NT * kTile - 1) / (NT * kTile);
  const dim3 grid(d.Vpad / (64 * R), groups);
  const size_t smem = 2ull * NT * KC * kWave * 16;
  hipLaunchKernelGGL((k_lmhead_mfma<NT, R, KC>), grid, dim3(kBlock), smem, s, d, p);
  return hipGetLastError();
}

}  // namespace

// Rows of the tiled LM head must be padded to a multiple of this.
int lmhead_row_multiple() { return 256; }

hipError_t launch_lmhead(const Dims& d, const LmHeadParams& p, hipStream_t s) {
  if (!d.bf16) {
    hipLaunchKernelGGL(k_lmhead_f32, dim3((d.V + kBlock - 1) / kBlock), dim3(kBlock), 0, s, d, p);
    return hipGetLastError();
  }
  if ((d.H / kKStep) % 2 != 0) return hipErrorInvalidValue;
  const int nt = (p.T + kTile - 1) / kTile;
  if (nt <= 1) return lm_nt<1>(d, p, s);
  if (nt <= 2) return lm_nt<2>(d, p, s);
  if (nt <= 4) return lm_nt<4>(d, p, s);
  return lm_nt<8>(d, p, s);
}

}  // namespace moe
