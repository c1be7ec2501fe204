// Final norm, LM head + greedy arg-max, longest-prefix acceptance.
//
// Three launches, back to back on the step's stream:
//  1. k_final_norm: one workgroup per token row finishes the last block
//     (shared + gate-weighted routed expert outputs in a fixed order, the
//     residual add and its rounding) and applies the final RMSNorm;
//  2. an LM-head kernel streams the vocabulary matrix from HBM exactly once
//     (non-temporal loads: read once, it should not evict the activation
//     fragments and keys the workgroups keep re-reading from L2)
//     and folds each token's best (logit, lowest id) into one of kKeySlots
//     64-bit keys with an atomicMax (logits are never written):
//       * up to 16 tokens: k_lmhead_stream, persistent, two 256-thread
//         workgroups per CU; the four wavefronts split the reduction and the
//         next unit's weight tiles are loaded while the current one is reduced;
//       * 17..128 tokens: k_lmhead_wide, persistent, one 512-thread workgroup
//         per CU with a register ring of weight fragments and the activation
//         fragments staged in LDS four k-steps at a time;
//       * more: k_lmhead_mfma, activation fragments staged in LDS;
//  3. k_accept reduces the key copies into the greedy picks, leaves them at
//     zero for the next step and runs the acceptance: the longest prefix of
//     drafts equal to the picks, plus the verifier's next pick (page "Jina AI
//     releases lightweight OCR model with built-in speculative decoding",
//     section "Speculative decoding without accuracy loss").
// Separate launches beat in-kernel hand-offs here: a cross-workgroup signal
// through memory costs a store and a poll round trip (several microseconds
// across XCDs), while consecutive launches on one queue start within about a
// microsecond and the kernel boundary orders the memory.
#include "kernels.h"

namespace moe {

namespace {

// ------------------------------------------------------------ acceptance ----
// One workgroup per kAcceptSeqs sequences: every key copy of its tokens is
// read once (all loads in flight together) and cleared, the copies are folded
// per token in LDS, then one thread per sequence runs the acceptance on its
// drafts, which it loaded with the keys (not one dependent load per draft).
constexpr int kAcceptSeqs = 8;
constexpr int kAcceptTok = kAcceptSeqs * 8;  // K + 1 <= 8 tokens per sequence

__global__ __launch_bounds__(kBlock) void k_accept(LmHeadParams p) {
  __shared__ unsigned long long best[kAcceptTok];
  const int K1 = p.K + 1;
  const int b0 = blockIdx.x * kAcceptSeqs;
  const int nb = min(kAcceptSeqs, p.B - b0);
  const int t0 = b0 * K1, nt = nb * K1;
  int dr[7];  // drafts of sequence b0 + threadIdx.x (K <= 7); -1 never matches a pick
#pragma unroll
  for (int j = 0; j < 7; ++j)
    dr[j] = static_cast<int>(threadIdx.x) < nb && j < p.K ? p.drafts[(b0 + threadIdx.x) * p.K + j] : -1;
  for (int t = threadIdx.x; t < nt; t += kBlock) best[t] = 0ull;
  __syncthreads();
  constexpr int kPer = kKeySlots * kAcceptTok / kBlock;
  unsigned long long kv[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = threadIdx.x + q * kBlock;  // copy i / nt of token i % nt
    kv[q] = i < kKeySlots * nt ? p.keys[static_cast<int64_t>(i / nt) * p.key_stride + t0 + i % nt] : 0ull;
  }
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = threadIdx.x + q * kBlock;
    if (i < kKeySlots * nt) {
      p.keys[static_cast<int64_t>(i / nt) * p.key_stride + t0 + i % nt] = 0ull;
      atomicMax(best + i % nt, kv[q]);
    }
  }
  __syncthreads();
  if (p.tstar)
    for (int t = threadIdx.x; t < nt; t += kBlock) p.tstar[t0 + t] = static_cast<int>(argmax_key_index(best[t]));
  if (static_cast<int>(threadIdx.x) < nb) {
    const int b = b0 + threadIdx.x;
    const unsigned long long* pk = best + threadIdx.x * K1;
    int a = 0;
    bool run = true;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      run = run && j < p.K && dr[j] == static_cast<int>(argmax_key_index(pk[j]));
      a += run ? 1 : 0;
    }
    for (int j = 0; j < K1; ++j)
      p.committed[b * K1 + j] = j <= a ? static_cast<int>(argmax_key_index(pk[j])) : -1;
    p.counts[b] = a + 1;
  }
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
    for (int kk = 0; kk < KC; ++kk) a_cur[r][kk] = load_frag_stream(a_ptr(r, kk));
  stage_store(0, st);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) {
      stage_load(c + 1, st);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) a_nxt[r][kk] = load_frag_stream(a_ptr(r, (c + 1) * KC + kk));
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



// One normalised row t, computed by a whole workgroup of NTHR threads: finish
// the last block (m = shared + gate-weighted routed outputs, x = round(x + m))
// and apply the final RMSNorm.  red holds NTHR / 64 floats, stage
// kMaxTopK * NTHR * CPB float4 of LDS.  Every
// load (the row, the gain, the row's expert ids and gate weights, all shared-
// and routed-expert output rows in slot order) is issued before any is used,
// so the row costs about one memory latency.  The combine order -- shared
// experts, then routed experts by ascending id -- is applied through LDS: the
// product w_j * y_j of routed slot j is stored at the slot's rank among the
// row's ids and the products are added back in rank order (the same rounded
// operations in the same order as adding w * y expert by expert).
template <int NTHR, int CPB>  // CPB 4-element chunks per thread: ceil(H / (4 * NTHR))
__device__ __forceinline__ void produce_final_row(const Dims& d, const LmHeadParams& p, int t, float* red,
                                                  float4* stage) {
  const int H = d.H, k = d.k, S = d.S, T = p.T, tid = threadIdx.x;
  const int nchunks = H / 4;
  const bf16_t* xin = reinterpret_cast<const bf16_t*>(p.x_in) + static_cast<int64_t>(t) * H;
  const bf16_t* gam = reinterpret_cast<const bf16_t*>(p.gamma);
  int idv[kMaxTopK];
  float wv[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {  // indices clamped to the row's k entries
    idv[j] = p.prev_idx[t * k + min(j, k - 1)];
    wv[j] = p.prev_w[t * k + min(j, k - 1)];
  }
  uint2 xv[CPB], gv[CPB];
  float4 vs[4][CPB], vr[kMaxTopK][CPB];  // shared-expert rows; routed rows by slot
#pragma unroll
  for (int c = 0; c < CPB; ++c) {
    const int ch = tid + c * NTHR;
    if (ch < nchunks) {
      xv[c] = *reinterpret_cast<const uint2*>(xin + 4 * ch);
      gv[c] = *reinterpret_cast<const uint2*>(gam + 4 * ch);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {  // shared expert r: row T*k + r*T + t
    const float* yr = p.y + (static_cast<int64_t>(T) * k + r * T + t) * H;
#pragma unroll
    for (int c = 0; c < CPB; ++c) {
      const int ch = tid + c * NTHR;
      if (r < S && ch < nchunks) vs[r][c] = *reinterpret_cast<const float4*>(yr + 4 * ch);
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {  // routed slot j: row t*k + j
    const float* yr = p.y + (static_cast<int64_t>(t) * k + j) * H;
#pragma unroll
    for (int c = 0; c < CPB; ++c) {
      const int ch = tid + c * NTHR;
      if (j < k && ch < nchunks) vr[j][c] = *reinterpret_cast<const float4*>(yr + 4 * ch);
    }
  }
  // rank of each slot among the row's (distinct) ids: uniform scalars
  int ids[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) ids[j] = __builtin_amdgcn_readfirstlane(idv[j]);
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      int rank = 0;
#pragma unroll
      for (int q = 0; q < kMaxTopK; ++q) rank += (q < k && ids[q] < ids[j]) ? 1 : 0;
#pragma unroll
      for (int c = 0; c < CPB; ++c) {
        const int ch = tid + c * NTHR;
        if (ch < nchunks)
          stage[(rank * CPB + c) * NTHR + tid] =
              make_float4(__fmul_rn(wv[j], vr[j][c].x), __fmul_rn(wv[j], vr[j][c].y),
                          __fmul_rn(wv[j], vr[j][c].z), __fmul_rn(wv[j], vr[j][c].w));
      }
    }
  }
  float x[CPB][4], m[CPB][4];
#pragma unroll
  for (int c = 0; c < CPB; ++c) {
    x[c][0] = __uint_as_float(xv[c].x << 16);
    x[c][1] = __uint_as_float(xv[c].x & 0xffff0000u);
    x[c][2] = __uint_as_float(xv[c].y << 16);
    x[c][3] = __uint_as_float(xv[c].y & 0xffff0000u);
#pragma unroll
    for (int i = 0; i < 4; ++i) m[c][i] = 0.0f;
  }
  // shared experts: weight 1 (1 * y == y exactly)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r < S) {
#pragma unroll
      for (int c = 0; c < CPB; ++c) {
        m[c][0] = __fadd_rn(m[c][0], vs[r][c].x);
        m[c][1] = __fadd_rn(m[c][1], vs[r][c].y);
        m[c][2] = __fadd_rn(m[c][2], vs[r][c].z);
        m[c][3] = __fadd_rn(m[c][3], vs[r][c].w);
      }
    }
  }
  // routed experts by ascending id (this thread's own LDS slots: no barrier)
#pragma unroll
  for (int q = 0; q < kMaxTopK; ++q) {
    if (q < k) {
#pragma unroll
      for (int c = 0; c < CPB; ++c) {
        const int ch = tid + c * NTHR;
        if (ch < nchunks) {
          const float4 y = stage[(q * CPB + c) * NTHR + tid];
          m[c][0] = __fadd_rn(m[c][0], y.x);
          m[c][1] = __fadd_rn(m[c][1], y.y);
          m[c][2] = __fadd_rn(m[c][2], y.z);
          m[c][3] = __fadd_rn(m[c][3], y.w);
        }
      }
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < CPB; ++c) {
    const int ch = tid + c * NTHR;
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
  ss = red[0];
#pragma unroll
  for (int w = 1; w < NTHR / kWave; ++w) ss += red[w];
  const float rms = sqrtf(ss / static_cast<float>(H) + d.eps);
  bf16_t* xf = reinterpret_cast<bf16_t*>(p.xf_out) + static_cast<int64_t>(t) * H;
#pragma unroll
  for (int c = 0; c < CPB; ++c) {
    const int ch = tid + c * NTHR;
    if (ch < nchunks) {
      const float gg[4] = {__uint_as_float(gv[c].x << 16), __uint_as_float(gv[c].x & 0xffff0000u),
                           __uint_as_float(gv[c].y << 16), __uint_as_float(gv[c].y & 0xffff0000u)};
      uint64_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        packed |= static_cast<uint64_t>(f32_to_bf16(__fmul_rn(x[c][i] / rms, gg[i]))) << (16 * i);
      *reinterpret_cast<uint64_t*>(xf + 4 * ch) = packed;
    }
  }
}


template <int CPB>
__global__ __launch_bounds__(kBlock) void k_final_norm(Dims d, LmHeadParams p) {
  __shared__ float sred[kBlock / kWave];
  __shared__ float4 ystage[kMaxTopK * kBlock * CPB];
  produce_final_row<kBlock, CPB>(d, p, blockIdx.x, sred, ystage);
}

// --------------------------------------------------- up to 16 tokens ----
// Persistent (two 256-thread workgroups per CU) over units of RPW row tiles.
// The four wavefronts split the reduction (KQ = H/128 k-steps each), hold
// their activation fragments in registers for the whole kernel, and load the
// next unit's weight tiles (RPW * KQ fragments, coalesced 1 KiB each) while
// the current unit's partial sums meet in LDS.
template <int KQ, int RPW>
__global__ __launch_bounds__(kBlock, 2) void k_lmhead_stream(Dims d, LmHeadParams p) {
  __shared__ float red[4][RPW][kWave][4];
  __shared__ uint64_t kbest[RPW * 16][kTile];
  __shared__ uint64_t run_best[kTile];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int KT = d.H / kKStep, kt0 = wave * KQ;
  const int n_units = d.Vpad / (kTile * RPW);   // units of RPW row tiles
  const bf16_t* lm = reinterpret_cast<const bf16_t*>(p.lm);
  auto load_unit = [&](int u, bf16x8_t (&a)[RPW][KQ]) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const bf16_t* w = lm + (static_cast<int64_t>(u * RPW + r) * KT + kt0) * kFragElems + lane * 8;
#pragma unroll
      for (int i = 0; i < KQ; ++i) a[r][i] = load_frag_stream(w + i * kFragElems);
    }
  };

  if (threadIdx.x < kTile) run_best[threadIdx.x] = 0ull;
  // activation fragments (token lane % 16; rows past T repeat row T - 1, their
  // results are never used), read once and kept in registers, issued first
  const int tok = min(lane % kTile, p.T - 1);
  bf16x8_t b[KQ];
  const bf16_t* xr = reinterpret_cast<const bf16_t*>(p.xf) + static_cast<int64_t>(tok) * d.H + kt0 * kKStep +
                     (lane / kTile) * 8;
#pragma unroll
  for (int i = 0; i < KQ; ++i) b[i] = load_frag(xr + i * kKStep);
  bf16x8_t a0[RPW][KQ], a1[RPW][KQ];
  int u = blockIdx.x;  // < n_units (grid <= units)
  load_unit(u, a0);

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
    // logits of (row, token): the four reduction quarters summed in a fixed order
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
  // steady state: both units of a pair exist, every load is unconditional
  // (the compiler's wait before a unit's MFMAs then leaves the next unit's
  // loads in flight)
  const int g = gridDim.x;
  for (; u + 2 * g < n_units; u += 2 * g) {
    load_unit(u + g, a1);
    do_unit(u, a0);
    load_unit(u + 2 * g, a0);
    do_unit(u + g, a1);
  }
  if (u + g < n_units) {
    load_unit(u + g, a1);
    do_unit(u, a0);
    do_unit(u + g, a1);
  } else {
    do_unit(u, a0);
  }
  __syncthreads();
  if (threadIdx.x < kTile && static_cast<int>(threadIdx.x) < p.T && run_best[threadIdx.x] != 0ull)
    atomicMax(p.keys + static_cast<int64_t>(blockIdx.x % kKeySlots) * p.key_stride + threadIdx.x,
              static_cast<unsigned long long>(run_best[threadIdx.x]));
}

// ------------------------------------------------- 17..128 tokens ----
// One 512-thread workgroup per CU, persistent over units of 8R row tiles
// (R = 2: with R = 4 the accumulators and rings of 8 token tiles spill);
// wavefront w owns the unit's row tiles Rw..Rw+R-1 over the whole
// reduction, so its accumulators (R row tiles x NT token tiles) never leave
// registers.  The k-steps go in groups of four:
//  * weight fragments go straight to registers from a ring of four steps
//    per wavefront (8 KiB, 64 KiB per CU), each slot refilled with the next
//    group's step as soon as it is used (a ring of eight steps measured no
//    better);
//  * the activation fragments of all NT token tiles for the group's four
//    steps (4 x NT KiB, shared by the 8 wavefronts) come from a
//    double-buffered LDS stage; wavefront w loads token tile w % NT of the
//    four steps of group q + 2 at the start of group q and writes them to
//    the stage during group q + 1.  One barrier per group: with one per step
//    (the previous design) a late weight fragment of one wavefront held the
//    other seven back every step, and the B = 32 head took 70.5 against
//    64.9 us.
// Every load is unconditional (rows past the matrix clamped, activation
// steps wrapping) and the loop is entered in the state it leaves, so the
// compiler's own wait counts are exact.
constexpr int kWideThreads = 512;
constexpr int kWideWaves = kWideThreads / kWave;
constexpr int kWideStageBytes = kWideWaves * 1024;  // one fragment slot per wavefront
constexpr int kWideGroupBytes = 4 * kWideStageBytes;  // four steps of fragment slots (one LDS stage)

template <int NT, int R>
__global__ __launch_bounds__(kWideThreads, 1) void k_lmhead_wide(Dims d, LmHeadParams p) {
  static_assert(NT >= 1 && NT <= kWideWaves, "one activation fragment per wavefront and step");
  constexpr int kUnitTiles = kWideWaves * R;
  __shared__ __align__(16) unsigned char bring[2 * kWideGroupBytes];
  __shared__ uint64_t wbest[kWideWaves][NT * kTile];
  const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int H = d.H, KT = H / kKStep;
  const int n_tiles = d.Vpad / kTile;
  const int n_units = (n_tiles + kUnitTiles - 1) / kUnitTiles;
  const int groups = ((n_units - 1 - static_cast<int>(blockIdx.x)) / static_cast<int>(gridDim.x) + 1) * KT / 4;
  const bf16_t* lm = reinterpret_cast<const bf16_t*>(p.lm);

  int a_u = blockIdx.x, a_kt = 0;
  auto load_a_next = [&](bf16x8_t (&a)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int vt = min(a_u * kUnitTiles + wave * R + r, n_tiles - 1);
      a[r] = load_frag_stream(lm + (static_cast<int64_t>(vt) * KT + a_kt) * kFragElems + lane * 8);
    }
    if (++a_kt == KT) {
      a_kt = 0;
      a_u += gridDim.x;
    }
  };
  const int btok = min((wave % NT) * kTile + lane % kTile, p.T - 1);
  const bf16_t* bsrc = reinterpret_cast<const bf16_t*>(p.xf) + static_cast<int64_t>(btok) * H + (lane / kTile) * 8;
  int b_kt = 0;
  auto load_b_group = [&](bf16x8_t (&pb)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pb[j] = load_frag(bsrc + b_kt * kKStep);
      if (++b_kt == KT) b_kt = 0;
    }
  };
  auto put_b_group = [&](int q, const bf16x8_t (&pb)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<bf16x8_t*>(bring + (q & 1) * kWideGroupBytes + j * kWideStageBytes + wave * 1024 + lane * 16) =
          pb[j];
  };

  f32x4_t acc[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[r][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint64_t lbest[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) lbest[nt] = 0ull;
  int cur_u = blockIdx.x;
  auto fold_unit = [&](auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    const int row0 = (cur_u * kUnitTiles + wave * R) * kTile + 4 * (lane / kTile);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float bv = acc[0][nt][0];
      int bj = 0;
      if (kMasked && row0 >= d.V) bv = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (r == 0 && i == 0) continue;
          const int j = r * kTile + i;
          float v = acc[r][nt][i];
          if (kMasked && row0 + j >= d.V) v = -__builtin_inff();
          bj = v > bv ? j : bj;
          bv = v > bv ? v : bv;
        }
      uint64_t key = argmax_key(bv, static_cast<uint32_t>(row0 + bj));
      if (kMasked && row0 + bj >= d.V) key = 0ull;
      lbest[nt] = key > lbest[nt] ? key : lbest[nt];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  // prologue in the loop's steady order: group 0's activations (written to
  // stage 0 now), group 1's (written during group 0), then the weights of
  // group 0's four steps
  bf16x8_t pb[4], a[4][R];
  load_b_group(pb);
  bf16x8_t pn[4];
  load_b_group(pn);
#pragma unroll
  for (int j = 0; j < 4; ++j) load_a_next(a[j]);
  put_b_group(0, pb);
#pragma unroll
  for (int j = 0; j < 4; ++j) pb[j] = pn[j];
  lds_barrier();

  for (int q = 0; q < groups; ++q) {
    // group q + 1's activations to the other stage (read by nobody since the
    // last barrier), then group q + 2's requested
    put_b_group(q + 1, pb);
    load_b_group(pb);
    const unsigned char* st = bring + (q & 1) * kWideGroupBytes + lane * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8_t b_ = *reinterpret_cast<const bf16x8_t*>(st + j * kWideStageBytes + nt * 1024);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][nt] = mfma16(a[j][r], b_, acc[r][nt]);
      }
      load_a_next(a[j]);  // the next group's step j (clamped past the end)
    }
    if (((q + 1) * 4) % KT == 0) {
      if ((cur_u + 1) * kUnitTiles * kTile > d.V)
        fold_unit(std::true_type{});
      else
        fold_unit(std::false_type{});
      cur_u += gridDim.x;
    }
    lds_barrier();
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    uint64_t best = lbest[nt];
    uint64_t o = __shfl_xor(best, 16, kWave);
    best = o > best ? o : best;
    o = __shfl_xor(best, 32, kWave);
    best = o > best ? o : best;
    if (lane < kTile) wbest[wave][nt * kTile + lane] = best;
  }
  lds_barrier();
  const int t = threadIdx.x;
  if (t < NT * kTile && t < p.T) {
    uint64_t b = 0ull;
#pragma unroll
    for (int w = 0; w < kWideWaves; ++w) b = wbest[w][t] > b ? wbest[w][t] : b;
    if (b != 0ull)
      __hip_atomic_fetch_max(p.keys + static_cast<int64_t>(blockIdx.x % kKeySlots) * p.key_stride + t,
                             static_cast<unsigned long long>(b), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int NT, int R>
hipError_t lm_wide_nt(const Dims& d, const LmHeadParams& p, hipStream_t s) {
  constexpr int kUnitTiles = kWideWaves * R;
  const unsigned units = (d.Vpad / kTile + kUnitTiles - 1) / kUnitTiles;
  const unsigned grid = units < static_cast<unsigned>(d.n_cu) ? units : static_cast<unsigned>(d.n_cu);
  hipLaunchKernelGGL((k_lmhead_wide<NT, R>), dim3(grid), dim3(kWideThreads), 0, s, d, p);
  return hipGetLastError();
}

template <int KQ>
hipError_t lm_stream_kq(const Dims& d, const LmHeadParams& p, hipStream_t s) {
  constexpr int RPW = 2;
  // persistent: two workgroups per CU stream the vocabulary units in turn
  const unsigned units = d.Vpad / (kTile * RPW);
  const unsigned cap = 2u * static_cast<unsigned>(d.n_cu);
  const unsigned grid = units < cap ? units : cap;
  hipLaunchKernelGGL((k_lmhead_stream<KQ, RPW>), dim3(grid), dim3(kBlock), 0, s, d, p);
  return hipGetLastError();
}

template <int NT, int R, int KC>
hipError_t lm_nt(const Dims& d, const LmHeadParams& p, hipStream_t s) {
  const int groups = (p.T + NT * kTile - 1) / (NT * kTile);
  const dim3 grid(d.Vpad / (64 * R), groups);
  const size_t smem = 2ull * NT * KC * kWave * 16;
  hipLaunchKernelGGL((k_lmhead_mfma<NT, R, KC>), grid, dim3(kBlock), smem, s, d, p);
  return hipGetLastError();
}

}  // namespace

// Rows of the tiled LM head must be padded to a multiple of this.
int lmhead_row_multiple() { return 256; }

hipError_t launch_final_norm(const Dims& d, const LmHeadParams& p, hipStream_t s) {
  if (!d.bf16 || p.T < 1) return hipErrorInvalidValue;
  const int chunks = d.H / 4;  // 4-element chunks per row
  if (chunks <= kBlock) {
    hipLaunchKernelGGL((k_final_norm<1>), dim3(p.T), dim3(kBlock), 0, s, d, p);
  } else if (chunks <= 2 * kBlock) {
    hipLaunchKernelGGL((k_final_norm<2>), dim3(p.T), dim3(kBlock), 0, s, d, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_accept(const LmHeadParams& p, hipStream_t s) {
  if (p.K + 1 > 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_accept, dim3((p.B + kAcceptSeqs - 1) / kAcceptSeqs), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_lmhead(const Dims& d, const LmHeadParams& p, hipStream_t s) {
  if (!d.bf16) {
    hipLaunchKernelGGL(k_lmhead_f32, dim3((d.V + kBlock - 1) / kBlock), dim3(kBlock), 0, s, d, p);
    return hipGetLastError();
  }
  if (d.H % 128 != 0) return hipErrorInvalidValue;
  if (p.T <= kTile) {
    switch (d.H / 128) {
      case 1: return lm_stream_kq<1>(d, p, s);   case 2: return lm_stream_kq<2>(d, p, s);
      case 3: return lm_stream_kq<3>(d, p, s);   case 4: return lm_stream_kq<4>(d, p, s);
      case 5: return lm_stream_kq<5>(d, p, s);   case 6: return lm_stream_kq<6>(d, p, s);
      case 7: return lm_stream_kq<7>(d, p, s);   case 8: return lm_stream_kq<8>(d, p, s);
      case 9: return lm_stream_kq<9>(d, p, s);   case 10: return lm_stream_kq<10>(d, p, s);
      case 11: return lm_stream_kq<11>(d, p, s); case 12: return lm_stream_kq<12>(d, p, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int nt = (p.T + kTile - 1) / kTile;
  if (nt <= 2) return lm_wide_nt<2, 2>(d, p, s);
  if (nt <= 4) return lm_wide_nt<4, 2>(d, p, s);
  if (nt <= 8) return lm_wide_nt<8, 2>(d, p, s);
  return lm_nt<8, 4, 2>(d, p, s);
}

}  // namespace moe
