// LM head + greedy arg-max + longest-prefix acceptance.
//
// The vocabulary matrix is streamed from HBM exactly once per step; logits are
// never written.  Two bfloat16 kernels:
//  * up to 16 tokens (decode): one workgroup per 16*RPW vocabulary rows; its
//    four wavefronts split the reduction dimension in four, each issues all of
//    its weight-tile loads at once straight into registers (pre-tiled,
//    coalesced 1 KiB per tile) together with the matching activation
//    fragments, runs the 16x16x32 MFMAs and the partial sums meet in LDS;
//  * more tokens: each workgroup owns 64*R rows; the K loop runs over chunks
//    whose activation fragments for all tokens are staged in LDS (double
//    buffered) and shared by the four wavefronts, weights again straight to
//    registers one chunk ahead.
// The epilogue reduces each token's best (logit, lowest id) over the
// workgroup's rows into a 64-bit key and folds it with one atomicMax into one
// of kKeySlots copies of the token's key (spreading same-address atomics).
// A one-workgroup kernel then reduces the copies into the greedy picks and
// runs the acceptance: the longest prefix of drafts equal to the picks, plus
// the verifier's next pick (page "Jina AI releases lightweight OCR model with
// built-in speculative decoding", section "Speculative decoding without
// accuracy loss").
#include "kernels.h"

namespace moe {

namespace {

// Greedy picks from the key copies and the prefix acceptance: one small
// workgroup after the LM-head kernel (the kernel boundary makes every key
// atomic visible, so the head kernels need no fences or completion counter).
__global__ __launch_bounds__(kBlock) void k_accept(LmHeadParams p) {
  const int K1 = p.K + 1;
  auto pick_of = [&](int t) {
    uint64_t best = 0ull;
    for (int q = 0; q < kKeySlots; ++q) {
      const uint64_t key = p.keys[static_cast<int64_t>(q) * p.key_stride + t];
      best = key > best ? key : best;
    }
    return static_cast<int>(argmax_key_index(best));
  };
  if (p.tstar)
    for (int t = threadIdx.x; t < p.T; t += kBlock) p.tstar[t] = pick_of(t);
  for (int b = threadIdx.x; b < p.B; b += kBlock) {
    int pick[8];
    for (int j = 0; j < K1; ++j) pick[j] = pick_of(b * K1 + j);
    int a = 0;
    while (a < p.K && p.drafts[b * p.K + a] == pick[a]) ++a;
    for (int j = 0; j < K1; ++j) p.committed[b * K1 + j] = j <= a ? pick[j] : -1;
    p.counts[b] = a + 1;
  }
  __syncthreads();
  // leave every key copy at zero for the next step
  for (int i = threadIdx.x; i < kKeySlots * p.T; i += kBlock)
    p.keys[static_cast<int64_t>(i / p.T) * p.key_stride + i % p.T] = 0ull;
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
      if (tok < p.T && b != 0ull)
        atomicMax(p.keys + static_cast<int64_t>(blockIdx.x % kKeySlots) * p.key_stride + tok,
                  static_cast<unsigned long long>(b));
    }
    __syncthreads();
  }
}

// K-split kernel for up to 16 tokens.  KQ = H/128 k-steps per wavefront,
// RPW row tiles of 16 vocabulary rows per workgroup.
template <int KQ, int RPW>
__global__ __launch_bounds__(kBlock) void k_lmhead_ksplit(Dims d, LmHeadParams p) {
  __shared__ float red[4][RPW][kWave][4];
  __shared__ uint64_t kbest[RPW * 16][kTile];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int KT = d.H / kKStep, kt0 = wave * KQ;
  const int rt0 = blockIdx.x * RPW;
  const bf16_t* lm = reinterpret_cast<const bf16_t*>(p.lm);
  const bf16_t* xf = reinterpret_cast<const bf16_t*>(p.xf);

  bf16x8_t a[RPW][KQ];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const bf16_t* w = lm + (static_cast<int64_t>(rt0 + r) * KT + kt0) * kFragElems + lane * 8;
#pragma unroll
    for (int i = 0; i < KQ; ++i) a[r][i] = load_frag(w + i * kFragElems);
  }
  const int tok = lane % kTile;
  bf16x8_t b[KQ];
  const bf16_t* xr = xf + static_cast<int64_t>(tok) * d.H + kt0 * kKStep + (lane / kTile) * 8;
#pragma unroll
  for (int i = 0; i < KQ; ++i) b[i] = tok < p.T ? load_frag(xr + i * kKStep) : zero_frag();
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KQ; ++i) c = mfma16(a[r][i], b[i], c);
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][r][lane][i] = c[i];
  }
  __syncthreads();
  // logits of (row, token): sum the four reduction quarters in a fixed order
  for (int q = threadIdx.x; q < RPW * kWave * 4; q += kBlock) {
    const int r = q / (kWave * 4), L = (q / 4) % kWave, i = q % 4;
    const float v = ((red[0][r][L][i] + red[1][r][L][i]) + red[2][r][L][i]) + red[3][r][L][i];
    const int rl = r * 16 + 4 * (L / kTile) + i;  // row within the workgroup
    const int row = rt0 * kTile + rl;
    kbest[rl][L % kTile] = row < d.V ? argmax_key(v, static_cast<uint32_t>(row)) : 0ull;
  }
  __syncthreads();
  if (threadIdx.x < kTile && static_cast<int>(threadIdx.x) < p.T) {
    uint64_t best = 0ull;
    for (int rl = 0; rl < RPW * 16; ++rl) best = kbest[rl][threadIdx.x] > best ? kbest[rl][threadIdx.x] : best;
    if (best != 0ull)
      atomicMax(p.keys + static_cast<int64_t>(blockIdx.x % kKeySlots) * p.key_stride + threadIdx.x,
                static_cast<unsigned long long>(best));
  }
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
      if (b != 0ull)
        atomicMax(p.keys + static_cast<int64_t>(blockIdx.x % kKeySlots) * p.key_stride + t,
                  static_cast<unsigned long long>(b));
    }
    __syncthreads();
  }
}


// ------------------------------------------------- fused decode head ----
// Up to 16 tokens.  Workgroups 0..T-1 first produce one normalised row each
// (finish the last block: m = shared + gate-weighted routed outputs in
// ascending expert order, x = round(x + m), RMSNorm with the final gain), and
// publish it with agent-scope stores and a counter; every workgroup issues
// its weight loads before waiting for the T rows, so the final norm overlaps
// the head's weight stream.  The workgroup that finishes last (counter) turns
// the key copies into the greedy picks and runs the acceptance.  Counters are
// monotonic across steps (the host passes the epoch), waits are bounded (on a
// timeout *err is set and the step's outputs are invalid).
constexpr unsigned kSpinLimit = 1u << 22;

__device__ __forceinline__ void store_u64_agent(void* p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_u64_agent(const void* p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int CPB>  // 4-element chunks per thread: ceil(H / 1024)
__device__ void produce_final_row(const Dims& d, const LmHeadParams& p, int t, float* red) {
  const int H = d.H, k = d.k, T = p.T, tid = threadIdx.x;
  const int nchunks = H / 4;
  const bf16_t* xin = reinterpret_cast<const bf16_t*>(p.x_in) + static_cast<int64_t>(t) * H;
  float x[CPB][4];
#pragma unroll
  for (int c = 0; c < CPB; ++c) {
    const int ch = tid + c * kBlock;
    if (ch < nchunks) {
      const uint2 v = *reinterpret_cast<const uint2*>(xin + 4 * ch);
      x[c][0] = __uint_as_float(v.x << 16);
      x[c][1] = __uint_as_float(v.x & 0xffff0000u);
      x[c][2] = __uint_as_float(v.y << 16);
      x[c][3] = __uint_as_float(v.y & 0xffff0000u);
    }
  }
  // rows in the combine order: shared experts, then routed by ascending expert
  int ids[kMaxTopK], js[kMaxTopK];
  float ws[kMaxTopK];
  for (int j = 0; j < k; ++j) {
    ids[j] = p.prev_idx[t * k + j];
    ws[j] = p.prev_w[t * k + j];
    js[j] = j;
  }
  for (int a = 1; a < k; ++a) {
    const int ia = ids[a], ja = js[a];
    const float wa = ws[a];
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
  const int nrows = d.S + k;
  constexpr int kRowsMax = 4 + kMaxTopK;
  float4 v[kRowsMax][CPB];
  float g[kRowsMax];
#pragma unroll
  for (int r = 0; r < kRowsMax; ++r) {
    if (r < nrows) {
      int64_t row;
      if (r < d.S) {
        row = static_cast<int64_t>(T) * k + r * T + t;
        g[r] = 1.0f;  // shared expert: weight 1 (1*y == y exactly)
      } else {
        row = static_cast<int64_t>(t) * k + js[r - d.S];
        g[r] = ws[r - d.S];
      }
      const float* yr = p.y + row * H;
#pragma unroll
      for (int c = 0; c < CPB; ++c) {
        const int ch = tid + c * kBlock;
        if (ch < nchunks) v[r][c] = *reinterpret_cast<const float4*>(yr + 4 * ch);
      }
    }
  }
  float m[CPB][4];
#pragma unroll
  for (int c = 0; c < CPB; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) m[c][i] = 0.0f;
#pragma unroll
  for (int r = 0; r < kRowsMax; ++r) {
    if (r < nrows) {
#pragma unroll
      for (int c = 0; c < CPB; ++c) {
        m[c][0] = __fadd_rn(m[c][0], __fmul_rn(g[r], v[r][c].x));
        m[c][1] = __fadd_rn(m[c][1], __fmul_rn(g[r], v[r][c].y));
        m[c][2] = __fadd_rn(m[c][2], __fmul_rn(g[r], v[r][c].z));
        m[c][3] = __fadd_rn(m[c][3], __fmul_rn(g[r], v[r][c].w));
      }
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < CPB; ++c) {
    const int ch = tid + c * kBlock;
    if (ch < nchunks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[c][i] = bf16_to_f32(f32_to_bf16(__fadd_rn(x[c][i], m[c][i])));
        ss = __fadd_rn(ss, __fmul_rn(x[c][i], x[c][i]));
      }
      if (p.x_out) {
        ushort4 o;
        o.x = f32_to_bf16(x[c][0]);
        o.y = f32_to_bf16(x[c][1]);
        o.z = f32_to_bf16(x[c][2]);
        o.w = f32_to_bf16(x[c][3]);
        *reinterpret_cast<ushort4*>(reinterpret_cast<bf16_t*>(p.x_out) + static_cast<int64_t>(t) * H + 4 * ch) = o;
      }
      if (p.m_out)
        *reinterpret_cast<float4*>(p.m_out + static_cast<int64_t>(t) * H + 4 * ch) =
            make_float4(m[c][0], m[c][1], m[c][2], m[c][3]);
    }
  }
  ss = wave_sum(ss);
  if (tid % kWave == 0) red[tid / kWave] = ss;
  __syncthreads();
  ss = ((red[0] + red[1]) + red[2]) + red[3];
  const float rms = sqrtf(ss / static_cast<float>(H) + d.eps);
  const bf16_t* gam = reinterpret_cast<const bf16_t*>(p.gamma);
  bf16_t* xf = reinterpret_cast<bf16_t*>(p.xf_out) + static_cast<int64_t>(t) * H;
#pragma unroll
  for (int c = 0; c < CPB; ++c) {
    const int ch = tid + c * kBlock;
    if (ch < nchunks) {
      const uint2 gv = *reinterpret_cast<const uint2*>(gam + 4 * ch);
      const float gg[4] = {__uint_as_float(gv.x << 16), __uint_as_float(gv.x & 0xffff0000u),
                           __uint_as_float(gv.y << 16), __uint_as_float(gv.y & 0xffff0000u)};
      uint64_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        packed |= static_cast<uint64_t>(f32_to_bf16(__fmul_rn(x[c][i] / rms, gg[i]))) << (16 * i);
      store_u64_agent(xf + 4 * ch, packed);
    }
  }
}

template <int KQ, int RPW, int CPB>
__global__ __launch_bounds__(kBlock, 2) void k_lmhead_fused(Dims d, LmHeadParams p) {
  __shared__ float red[4][RPW][kWave][4];
  __shared__ uint64_t kbest[RPW * 16][kTile];
  __shared__ uint64_t run_best[kTile];
  __shared__ float sred[4];
  __shared__ int is_last;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int KT = d.H / kKStep, kt0 = wave * KQ;
  const int n_units = d.Vpad / (kTile * RPW);   // units of RPW row tiles
  const bf16_t* lm = reinterpret_cast<const bf16_t*>(p.lm);
  auto load_unit = [&](int u, bf16x8_t (&a)[RPW][KQ]) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const bf16_t* w = lm + (static_cast<int64_t>(u * RPW + r) * KT + kt0) * kFragElems + lane * 8;
#pragma unroll
      for (int i = 0; i < KQ; ++i) a[r][i] = load_frag(w + i * kFragElems);
    }
  };

  // 1. the first unit's weight tiles, in flight before anything else
  bf16x8_t a0[RPW][KQ], a1[RPW][KQ];
  int u = blockIdx.x;
  if (u < n_units) load_unit(u, a0);
  if (threadIdx.x < kTile) run_best[threadIdx.x] = 0ull;
  // 2. workgroups 0..T-1 produce the normalised rows
  if (static_cast<int>(blockIdx.x) < p.T) {
    produce_final_row<CPB>(d, p, blockIdx.x, sred);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's row stores are done
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(p.norm_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // 3. wait for all T rows (bounded)
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (static_cast<int>(__hip_atomic_load(p.norm_count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                            p.norm_target) < 0) {
      if (++spins > kSpinLimit) {
        *p.err = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  // 4. activation fragments, read once and kept in registers; read coherently
  //    (the rows were just written on other CUs; this CU's L2 may hold an
  //    older copy of those lines)
  const int tok = lane % kTile;
  bf16x8_t b[KQ];
  const bf16_t* xr = reinterpret_cast<const bf16_t*>(p.xf_out) + static_cast<int64_t>(tok) * d.H + kt0 * kKStep +
                     (lane / kTile) * 8;
#pragma unroll
  for (int i = 0; i < KQ; ++i) {
    if (tok < p.T) {
      uint4 w;
      const uint64_t lo = load_u64_agent(xr + i * kKStep), hi = load_u64_agent(xr + i * kKStep + 4);
      w.x = static_cast<uint32_t>(lo);
      w.y = static_cast<uint32_t>(lo >> 32);
      w.z = static_cast<uint32_t>(hi);
      w.w = static_cast<uint32_t>(hi >> 32);
      b[i] = __builtin_bit_cast(bf16x8_t, w);
    } else {
      b[i] = zero_frag();
    }
  }
  // 5. stream this workgroup's units, the next unit's tiles one unit ahead
  auto do_unit = [&](int uu, const bf16x8_t (&a)[RPW][KQ]) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KQ; ++i) c = mfma16(a[r][i], b[i], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][r][lane][i] = c[i];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < RPW * kWave * 4; q += kBlock) {
      const int r = q / (kWave * 4), L = (q / 4) % kWave, i = q % 4;
      const float v = ((red[0][r][L][i] + red[1][r][L][i]) + red[2][r][L][i]) + red[3][r][L][i];
      const int rl = r * 16 + 4 * (L / kTile) + i;
      const int row = uu * RPW * kTile + rl;
      kbest[rl][L % kTile] = row < d.V ? argmax_key(v, static_cast<uint32_t>(row)) : 0ull;
    }
    __syncthreads();
    if (threadIdx.x < kTile) {
      uint64_t best = run_best[threadIdx.x];
      for (int rl = 0; rl < RPW * 16; ++rl) best = kbest[rl][threadIdx.x] > best ? kbest[rl][threadIdx.x] : best;
      run_best[threadIdx.x] = best;
    }
  };
  while (u < n_units) {
    const int un = u + gridDim.x;
    if (un < n_units) load_unit(un, a1);
    do_unit(u, a0);
    u = un;
    if (u >= n_units) break;
    const int un2 = u + gridDim.x;
    if (un2 < n_units) load_unit(un2, a0);
    do_unit(u, a1);
    u = un2;
  }
  __syncthreads();
  if (threadIdx.x < kTile && static_cast<int>(threadIdx.x) < p.T && run_best[threadIdx.x] != 0ull)
    __hip_atomic_fetch_max(p.keys + static_cast<int64_t>(blockIdx.x % kKeySlots) * p.key_stride + threadIdx.x,
                           static_cast<unsigned long long>(run_best[threadIdx.x]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  // 6. the last workgroup to finish runs the acceptance
  __builtin_amdgcn_s_waitcnt(0);  // this thread's key atomic is performed
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(p.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (old - p.done_base) == gridDim.x - 1;
  }
  __syncthreads();
  if (!is_last) return;
  const int K1 = p.K + 1;
  auto pick_of = [&](int t) {
    uint64_t best = 0ull;
    for (int q = 0; q < kKeySlots; ++q) {
      const uint64_t key = load_u64_agent(p.keys + static_cast<int64_t>(q) * p.key_stride + t);
      best = key > best ? key : best;
    }
    return static_cast<int>(argmax_key_index(best));
  };
  if (p.tstar)
    for (int t = threadIdx.x; t < p.T; t += kBlock) p.tstar[t] = pick_of(t);
  for (int bq = threadIdx.x; bq < p.B; bq += kBlock) {
    int pick[8];
    for (int j = 0; j < K1; ++j) pick[j] = pick_of(bq * K1 + j);
    int acc = 0;
    while (acc < p.K && p.drafts[bq * p.K + acc] == pick[acc]) ++acc;
    for (int j = 0; j < K1; ++j) p.committed[bq * K1 + j] = j <= acc ? pick[j] : -1;
    p.counts[bq] = acc + 1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kKeySlots * p.T; i += kBlock)
    store_u64_agent(p.keys + static_cast<int64_t>(i / p.T) * p.key_stride + i % p.T, 0ull);
}

template <int KQ>
hipError_t lm_fused_kq(const Dims& d, const LmHeadParams& p, hipStream_t s, unsigned int* blocks) {
  constexpr int RPW = 2;
  constexpr int CPB = (KQ * 32 + kBlock - 1) / kBlock;  // ceil((H/4) / 256)
  // persistent: two workgroups per CU stream the vocabulary units in turn
  const unsigned units = d.Vpad / (kTile * RPW);
  const unsigned grid = units < 512u ? units : 512u;
  *blocks = grid;
  hipLaunchKernelGGL((k_lmhead_fused<KQ, RPW, CPB>), dim3(grid), dim3(kBlock), 0, s, d, p);
  return hipGetLastError();
}

template <int KQ>
hipError_t lm_ksplit(const Dims& d, const LmHeadParams& p, hipStream_t s) {
  constexpr int RPW = 2;
  hipLaunchKernelGGL((k_lmhead_ksplit<KQ, RPW>), dim3(d.Vpad / (kTile * RPW)), dim3(kBlock), 0, s, d, p);
  return hipGetLastError();
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

hipError_t launch_lmhead_fused(const Dims& d, const LmHeadParams& p, hipStream_t s, unsigned int* blocks) {
  if (!d.bf16 || p.T > kTile || p.T < 1) return hipErrorInvalidValue;
  switch (d.H / 128) {
    case 1: return lm_fused_kq<1>(d, p, s, blocks);   case 2: return lm_fused_kq<2>(d, p, s, blocks);
    case 3: return lm_fused_kq<3>(d, p, s, blocks);   case 4: return lm_fused_kq<4>(d, p, s, blocks);
    case 5: return lm_fused_kq<5>(d, p, s, blocks);   case 6: return lm_fused_kq<6>(d, p, s, blocks);
    case 7: return lm_fused_kq<7>(d, p, s, blocks);   case 8: return lm_fused_kq<8>(d, p, s, blocks);
    case 9: return lm_fused_kq<9>(d, p, s, blocks);   case 10: return lm_fused_kq<10>(d, p, s, blocks);
    case 11: return lm_fused_kq<11>(d, p, s, blocks); case 12: return lm_fused_kq<12>(d, p, s, blocks);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_accept(const LmHeadParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_accept, dim3(1), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_lmhead(const Dims& d, const LmHeadParams& p, hipStream_t s) {
  if (!d.bf16) {
    hipLaunchKernelGGL(k_lmhead_f32, dim3((d.V + kBlock - 1) / kBlock), dim3(kBlock), 0, s, d, p);
    return hipGetLastError();
  }
  if ((d.H / kKStep) % 2 != 0) return hipErrorInvalidValue;
  const int nt = (p.T + kTile - 1) / kTile;
  if (nt <= 1) {
    switch (d.H / 128) {
      case 1: return lm_ksplit<1>(d, p, s);   case 2: return lm_ksplit<2>(d, p, s);
      case 3: return lm_ksplit<3>(d, p, s);   case 4: return lm_ksplit<4>(d, p, s);
      case 5: return lm_ksplit<5>(d, p, s);   case 6: return lm_ksplit<6>(d, p, s);
      case 7: return lm_ksplit<7>(d, p, s);   case 8: return lm_ksplit<8>(d, p, s);
      case 9: return lm_ksplit<9>(d, p, s);   case 10: return lm_ksplit<10>(d, p, s);
      case 11: return lm_ksplit<11>(d, p, s); case 12: return lm_ksplit<12>(d, p, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (nt <= 2) return lm_nt<2>(d, p, s);
  if (nt <= 4) return lm_nt<4>(d, p, s);
  return lm_nt<8>(d, p, s);
}

}  // namespace moe
