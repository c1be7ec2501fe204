// Combine + RMSNorm + top-k softmax router (+ counting sort for small steps),
// one 1024-thread workgroup (16 wavefronts) per 16 token rows; steps of
// 17..256 rows take one row per workgroup (bfloat16, the split phase 1 below)
// or four, to spread the combine reads over more CUs.
//
// Phase 1 (wavefront w owns row w): optionally finish the previous block
//   (m = shared outputs + gate-weighted routed outputs in ascending expert
//   order, x' = round(x + m)), then RMSNorm xh = round(x / sqrt(mean(x^2)+eps) * gamma).
//   All loads of a row are issued before they are consumed, so the phase costs
//   a few memory latencies, not one per expert row.
// Phase 2: router logits z = W_r xh.  bfloat16 storage uses 16x16x32 MFMA:
//   wavefront w computes expert tile w%4 over reduction quarter w/4 (its
//   router fragments are loaded at kernel start), the rows' xh sit in LDS in
//   operand layout, the four quarters are summed in a fixed order.  float32
//   storage uses plain FMAs.
// Phase 3 (one wavefront per row, one lane per expert): each expert's rank by
//   (logit desc, lower expert first) from all-pairs comparisons of broadcast
//   keys; the k best, in rank order, get the softmax over the selected logits.
// Tail (steps of at most 16 tokens, one workgroup): the stable counting sort
//   of all T*k (token, slot) pairs by expert in LDS (ballot ranks within a
//   wavefront, per-wavefront counts, prefix over wavefronts), so the expert
//   kernels that follow know each expert's tokens without another launch.
//   Larger steps sort in a separate launch: a cross-workgroup hand-off inside
//   the kernel (release fence, counter, acquire fence) costs more here.
// The mixture of 64 routed experts with top-6 routing is the decoder of the
// page "Jina AI releases lightweight OCR model with built-in speculative
// decoding", section "Lean architecture with a compressed encoder"; the norm,
// softmax-over-selection and combine order are this library's reading.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kThreads = 1024;   // 16 wavefronts
constexpr int kWaves = kThreads / kWave;
constexpr int kRows = 16;        // token rows a workgroup can hold (MFMA tile columns)
constexpr int kRouterHelpers = 64;  // workgroups that only bring the router matrix into L2
constexpr int kGroup = 2;        // expert rows loaded together in the combine
constexpr int kSplitShared = 2;  // most shared experts on the split path
constexpr int kSplitRouted = 6;  // most routed experts per token on the split path

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

// Stable counting sort of P pairs by expert, by one 1024-thread workgroup.
// scratch: >= kWaves*64 + 2*64 ints of LDS.  The expert ids are read from
// `ids` (LDS) when given, else from s.idx.
__device__ void counting_sort_block(const Dims& d, const SortParams& s, int P, int* scratch, const int* ids) {
  int* hist = scratch;                 // [64]
  int* base = scratch + 64;            // [64]
  int* wcnt = scratch + 128;           // [kWaves][64]
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int E = d.E;
  if (tid < 64) hist[tid] = 0;
  __syncthreads();
  for (int i = tid; i < P; i += kThreads) atomicAdd(&hist[ids ? ids[i] : s.idx[i]], 1);
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
    base[lane] = incl - c;
    // active experts in ascending order (at most 16 tokens: every expert has
    // about the same load, so no busiest-first ordering)
    if (lane < E) {
      s.cnt[lane] = c;
      s.off[lane] = incl - c;
      const unsigned long long below = (1ull << lane) - 1ull;
      const unsigned long long inact = ~act & (E == 64 ? ~0ull : ((1ull << E) - 1ull));
      if (c > 0) {
        const int r = __popcll(act & below);
        s.active[r] = lane;
        s.desc[r] = make_int4(lane, c, incl - c, 0);
      } else {
        s.desc[__popcll(act) + __popcll(inact & below)] = make_int4(-1, 0, 0, 0);
      }
    }
    if (lane == kWave - 1) {
      s.off[E] = incl;
      *s.n_active = static_cast<int>(__popcll(act));
    }
  }
  for (int c0 = 0; c0 < P; c0 += kThreads) {
    for (int i = tid; i < kWaves * 64; i += kThreads) wcnt[i] = 0;
    __syncthreads();
    const int pidx = c0 + tid;
    const bool valid = pidx < P;
    const int e = valid ? (ids ? ids[pidx] : s.idx[pidx]) : -1;
    // lanes of this wavefront holding the same expert
    unsigned long long match = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 6; ++b) {
      const unsigned long long bit = __ballot(valid && ((e >> b) & 1));
      match &= ((e >> b) & 1) ? bit : ~bit;
    }
    const int rank = __popcll(match & ((1ull << lane) - 1ull));
    if (valid && rank == 0) wcnt[wave * 64 + e] = __popcll(match);
    __syncthreads();
    if (valid) {
      int pos = base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w * 64 + e];
      s.perm[pos] = pidx;
    }
    __syncthreads();
    if (tid < 64) {
      int tot = 0;
      for (int w = 0; w < kWaves; ++w) tot += wcnt[w * 64 + tid];
      base[tid] += tot;
    }
    __syncthreads();
  }
}

// EARLY: no combine in this launch (the first block of a step, or the MoE
// block after an attention sublayer), so phase 1 is light and the router
// fragments are requested at kernel start, their latency overlapping the row
// loads; with a combine they are requested after phase 1 (to keep phase 1
// within 128 registers).
// SPLIT (bf16, steps of 17..256 rows): one row per workgroup (so the row
// reads spread over as many CUs as there are rows) and eight wavefronts per
// row in phase 1, wavefront c of a row owning the row's
// 4-element chunks c*64 + lane -- the chunks one wavefront holds in slot c
// otherwise -- so that every row of the combine is requested at once (one
// memory round trip, not one per pair of expert rows) and the router
// fragments can be requested at kernel start.  The per-lane partial sums of
// squares of the slots are added in slot order through LDS before the same
// wavefront reduction, so the normalised rows are bit-identical to the
// one-wavefront-per-row path (a sequence gives the same rows at any batch).
template <typename ST, int KQ, bool EARLY, bool SPLIT>  // KQ = H / 128: router k-steps per wavefront (bf16)
__global__ __launch_bounds__(kThreads) void k_norm_router(Dims d, NormRouterParams p, int rows) {
  // dynamic LDS: [0, 16 KiB) router partials zp[4][16][64] (reused by the sort);
  // then bf16 xh operand tiles [H/32][64 lanes][8] or f32 xh rows [16][H]
  extern __shared__ __align__(16) unsigned char smem[];
  float* zp = reinterpret_cast<float*>(smem);
  unsigned char* xs = smem + 4 * kRows * 64 * sizeof(float);
  __shared__ int sel[kRows * kMaxTopK];  // this workgroup's selections (single-workgroup sort)

  const int H = d.H, k = d.k, T = p.T;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * rows;  // rows <= kRows token rows per workgroup
  const int nchunks = H / 4;
  constexpr int CPL = (KQ + 1) / 2;  // 4-element chunks per lane: ceil(H / 256)

  const int et = wave % 4, kq = wave / 4;

  // Helper workgroups (after the rows' workgroups): one CU takes ~5 us to pull
  // the 160 KiB router matrix (its misses in flight are few), so 64 helpers
  // each load one eighth of it and exit.  Workgroups go to the eight XCDs in
  // turn, so every XCD gets eight helpers covering the whole matrix, and the
  // row workgroups' requests find it in their XCD's L2.
  if (static_cast<int>(blockIdx.x) >= (T + rows - 1) / rows) {
    if constexpr (sizeof(ST) == 2) {
      const int h = static_cast<int>(blockIdx.x) - (T + rows - 1) / rows;
      const int frags = 4 * (H / kKStep), per = (frags + 7) / 8;  // 1 KiB fragments: [64 / 16][H / 32]
      const int f0 = ((h / 8) % 8) * per;
      const bf16_t* wr = reinterpret_cast<const bf16_t*>(p.router);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int f = f0 + wave + q * kWaves;
        if (wave + q * kWaves < per && f < frags) {
          const bf16x8_t v = load_frag(wr + static_cast<int64_t>(f) * kFragElems + lane * 8);
          asm volatile("" ::"v"(v));
        }
      }
    }
    return;
  }

  // router fragments of this wavefront, requested after phase 1 (to keep
  // phase 1 within 128 registers)
  bf16x8_t ra[KQ];
  const int n = wave;
  const int t = t0 + n;
  const bool has_row = n < rows && t < T;
  auto load_router = [&]() {
    if constexpr (sizeof(ST) == 2) {
      if (p.route && et * 16 < d.E) {
        const bf16_t* wr = reinterpret_cast<const bf16_t*>(p.router) +
                           (static_cast<int64_t>(et) * (H / kKStep) + kq * KQ) * kFragElems + lane * 8;
#pragma unroll
        for (int i = 0; i < KQ; ++i) ra[i] = load_frag(wr + i * kFragElems);
      }
    }
  };

  // ------------------------------------------------------------ phase 1
  if constexpr (SPLIT) {
    static_assert(sizeof(ST) == 2, "the split phase 1 is for bfloat16 storage");
    const int n1 = wave / 8, c1 = wave % 8;   // row, chunk slot
    const int t1 = t0 + n1;
    const int ch = lane + c1 * kWave;
    const bool mine = n1 < rows && t1 < T && c1 < CPL && ch < nchunks;
    float xv[4];
    Vec4<ST> gv;
    if (mine) {
      load4<ST>(reinterpret_cast<const ST*>(p.x_in) + static_cast<int64_t>(t1) * H + 4 * ch, xv);
      if (p.norm) gv = *reinterpret_cast<const Vec4<ST>*>(reinterpret_cast<const ST*>(p.gamma) + 4 * ch);
    }
    // the router fragments after the row loads (loads complete in order)
    load_router();
    if (mine && p.combine) {
      // every row is requested at once, by slot (row r < S: shared expert r;
      // r >= S: routed slot r - S, pair t*k + r - S), before the selection
      // that orders them is known; the routed rows are then added by
      // ascending expert (the rank of each slot's expert among the token's)
      int ids[kSplitRouted];
      float ws[kSplitRouted];
#pragma unroll
      for (int j = 0; j < kSplitRouted; ++j) {
        ids[j] = j < k ? p.prev_idx[t1 * k + j] : 0x7fffffff;
        ws[j] = j < k ? p.prev_w[t1 * k + j] : 0.0f;
      }
      const int P = T * k;
      float4 vs[kSplitShared], vr[kSplitRouted];
#pragma unroll
      for (int r = 0; r < kSplitShared; ++r)
        if (r < d.S) vs[r] = *reinterpret_cast<const float4*>(p.y + (static_cast<int64_t>(P) + r * T + t1) * H + 4 * ch);
#pragma unroll
      for (int j = 0; j < kSplitRouted; ++j)
        if (j < k) vr[j] = *reinterpret_cast<const float4*>(p.y + (static_cast<int64_t>(t1) * k + j) * H + 4 * ch);
      int rank[kSplitRouted];
#pragma unroll
      for (int j = 0; j < kSplitRouted; ++j) {
        rank[j] = 0;
#pragma unroll
        for (int jj = 0; jj < kSplitRouted; ++jj)
          if (jj < k) rank[j] += ids[jj] < ids[j] ? 1 : 0;
      }
      float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      auto add = [&](float g, const float4& y) {
        m[0] = __fadd_rn(m[0], __fmul_rn(g, y.x));
        m[1] = __fadd_rn(m[1], __fmul_rn(g, y.y));
        m[2] = __fadd_rn(m[2], __fmul_rn(g, y.z));
        m[3] = __fadd_rn(m[3], __fmul_rn(g, y.w));
      };
#pragma unroll
      for (int r = 0; r < kSplitShared; ++r)
        if (r < d.S) add(1.0f, vs[r]);  // shared expert: weight 1 (1*y == y exactly)
#pragma unroll
      for (int q = 0; q < kSplitRouted; ++q) {
        if (q < k) {
          // the routed slot whose expert is the q-th smallest of the token's
          float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
          float g = 0.0f;
#pragma unroll
          for (int j = 0; j < kSplitRouted; ++j)
            if (j < k && rank[j] == q) {
              y = vr[j];
              g = ws[j];
            }
          add(g, y);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = Storage<ST>::round(__fadd_rn(xv[i], m[i]));
      store4<ST>(reinterpret_cast<ST*>(p.x_out) + static_cast<int64_t>(t1) * H + 4 * ch, xv);
      if (p.m_out)
        *reinterpret_cast<float4*>(p.m_out + static_cast<int64_t>(t1) * H + 4 * ch) = make_float4(m[0], m[1], m[2], m[3]);
    }
    if (p.norm) {
      // per-lane partial of this slot, added to the others in slot order
      float* sq = zp;  // [2][8][64], free until phase 2
      float part = 0.0f;
      if (mine)
#pragma unroll
        for (int i = 0; i < 4; ++i) part = __fadd_rn(part, __fmul_rn(xv[i], xv[i]));
      sq[(n1 * 8 + c1) * kWave + lane] = part;
      __syncthreads();
      if (n1 < rows && t1 < T && c1 < CPL) {
        float ss = 0.0f;
        for (int c = 0; c < CPL; ++c) ss = __fadd_rn(ss, sq[(n1 * 8 + c) * kWave + lane]);
        ss = wave_sum(ss);
        const float rms = sqrtf(ss / static_cast<float>(H) + d.eps);
        if (ch < nchunks) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = Storage<ST>::round(__fmul_rn(xv[i] / rms, Storage<ST>::load(gv.v, i)));
          store4<ST>(reinterpret_cast<ST*>(p.xhat) + static_cast<int64_t>(t1) * H + 4 * ch, v);
          if (p.route) {
            const int h = 4 * ch;
            bf16_t* tile = reinterpret_cast<bf16_t*>(xs);
            const int kt = h / 32, ln = n1 + 16 * ((h % 32) / 8);
            store4<bf16_t>(tile + (kt * kWave + ln) * 8 + (h % 8), v);
          }
        }
      }
      __syncthreads();  // sq is reused as the router partials
    }
  } else {
  float x[CPL][4];
  Vec4<ST> gg[CPL];  // the gain, loaded with the row, converted when used
  const ST* xin = reinterpret_cast<const ST*>(p.x_in) + static_cast<int64_t>(t) * H;
  const ST* gam = reinterpret_cast<const ST*>(p.gamma);
  if (has_row) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + c * kWave;
      if (ch < nchunks) {
        load4<ST>(xin + 4 * ch, x[c]);
        if (p.norm) gg[c] = *reinterpret_cast<const Vec4<ST>*>(gam + 4 * ch);
      }
    }
  }
  // EARLY: the router fragments are requested right after the row loads (a
  // wavefront's loads complete in order, so requested first they would hold
  // up the rows by the whole matrix pull)
  if constexpr (EARLY) load_router();
  if (has_row) {
    if (!EARLY && p.combine) {
      // rows to add, in order: shared experts, then routed by ascending expert
      const int nrows = d.S + k;
      int ids[kMaxTopK];
      float ws[kMaxTopK];
      int js[kMaxTopK];
      for (int j = 0; j < k; ++j) {
        ids[j] = p.prev_idx[t * k + j];
        ws[j] = p.prev_w[t * k + j];
        js[j] = j;
      }
      for (int a = 1; a < k; ++a) {  // insertion sort by expert id
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
      const int P = T * k;
      float m[CPL][4];
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) m[c][i] = 0.0f;
      for (int r0 = 0; r0 < nrows; r0 += kGroup) {
        float4 v[kGroup][CPL];
        float g[kGroup];
#pragma unroll
        for (int q = 0; q < kGroup; ++q) {
          const int r = r0 + q;
          if (r < nrows) {
            int64_t row;
            if (r < d.S) {
              row = P + r * T + t;
              g[q] = 1.0f;  // shared expert: weight 1 (1*y == y exactly)
            } else {
              row = static_cast<int64_t>(t) * k + js[r - d.S];
              g[q] = ws[r - d.S];
            }
            const float* yr = p.y + row * H;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              const int ch = lane + c * kWave;
              if (ch < nchunks) v[q][c] = *reinterpret_cast<const float4*>(yr + 4 * ch);
            }
          }
        }
#pragma unroll
        for (int q = 0; q < kGroup; ++q) {
          if (r0 + q < nrows) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              m[c][0] = __fadd_rn(m[c][0], __fmul_rn(g[q], v[q][c].x));
              m[c][1] = __fadd_rn(m[c][1], __fmul_rn(g[q], v[q][c].y));
              m[c][2] = __fadd_rn(m[c][2], __fmul_rn(g[q], v[q][c].z));
              m[c][3] = __fadd_rn(m[c][3], __fmul_rn(g[q], v[q][c].w));
            }
          }
        }
      }
      ST* xout = reinterpret_cast<ST*>(p.x_out) + static_cast<int64_t>(t) * H;
      float* mo = p.m_out ? p.m_out + static_cast<int64_t>(t) * H : nullptr;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ch = lane + c * kWave;
        if (ch < nchunks) {
#pragma unroll
          for (int i = 0; i < 4; ++i) x[c][i] = Storage<ST>::round(__fadd_rn(x[c][i], m[c][i]));
          store4<ST>(xout + 4 * ch, x[c]);
          if (mo) *reinterpret_cast<float4*>(mo + 4 * ch) = make_float4(m[c][0], m[c][1], m[c][2], m[c][3]);
        }
      }
    }
    if (p.norm) {
      // per-lane partial of each chunk slot, added in slot order (the split
      // path adds the same partials in the same order)
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ch = lane + c * kWave;
        float part = 0.0f;
        if (ch < nchunks)
#pragma unroll
          for (int i = 0; i < 4; ++i) part = __fadd_rn(part, __fmul_rn(x[c][i], x[c][i]));
        ss = __fadd_rn(ss, part);
      }
      ss = wave_sum(ss);
      const float rms = sqrtf(ss / static_cast<float>(H) + d.eps);
      ST* xh = reinterpret_cast<ST*>(p.xhat) + static_cast<int64_t>(t) * H;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ch = lane + c * kWave;
        if (ch < nchunks) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = Storage<ST>::round(__fmul_rn(x[c][i] / rms, Storage<ST>::load(gg[c].v, i)));
          store4<ST>(xh + 4 * ch, v);
          if (p.route) {
            const int h = 4 * ch;
            if constexpr (sizeof(ST) == 2) {
              // operand tile kt = h/32; lane n + 16*((h%32)/8); element h%8
              bf16_t* tile = reinterpret_cast<bf16_t*>(xs);
              const int kt = h / 32, ln = n + 16 * ((h % 32) / 8);
              store4<bf16_t>(tile + (kt * kWave + ln) * 8 + (h % 8), v);
            } else {
              float* rows = reinterpret_cast<float*>(xs);
              *reinterpret_cast<float4*>(rows + n * H + h) = make_float4(v[0], v[1], v[2], v[3]);
            }
          }
        }
      }
    }
  }
  }  // SPLIT
  if (!p.route) return;
  if constexpr (!EARLY && !SPLIT) load_router();
  const int nrows = min(rows, T - t0);
  if constexpr (sizeof(ST) == 2) {
    // rows of this workgroup past T: zero operand lanes so MFMA reads defined values
    if (nrows < kRows) {
      bf16_t* tile = reinterpret_cast<bf16_t*>(xs);
      const int nkt = H / kKStep;
      for (int i = threadIdx.x; i < nkt * kWave; i += kThreads) {
        const int ln = i % kWave;
        if ((ln % 16) >= nrows) *reinterpret_cast<uint4*>(tile + i * 8) = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __syncthreads();

  // ------------------------------------------------------------ phase 2
  int nq;
  if constexpr (sizeof(ST) == 2) {
    nq = 4;
    if (et * 16 < d.E) {
      const bf16_t* tile = reinterpret_cast<const bf16_t*>(xs);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KQ; ++i) acc = mfma16(ra[i], load_frag(tile + ((kq * KQ + i) * kWave + lane) * 8), acc);
      // lane holds z[expert 16*et + 4*(lane/16) + i][row lane%16] over quarter kq
#pragma unroll
      for (int i = 0; i < 4; ++i) zp[(kq * kRows + lane % 16) * 64 + et * 16 + 4 * (lane / 16) + i] = acc[i];
    }
  } else {
    nq = 1;
    const float* rows = reinterpret_cast<const float*>(xs);
    const float* wr = reinterpret_cast<const float*>(p.router);
    for (int i = threadIdx.x; i < nrows * d.E; i += kThreads) {
      const int rn = i / d.E, e = i % d.E;
      const float* xr = rows + rn * H;
      const float* w = wr + static_cast<int64_t>(e) * H;
      float acc = 0.0f;
      for (int h = 0; h < H; ++h) acc = __fadd_rn(acc, __fmul_rn(xr[h], w[h]));
      zp[rn * 64 + e] = acc;
    }
  }
  __syncthreads();

  // ------------------------------------------------------------ phase 3
  if (n < nrows) {
    float z = 0.0f;
    if (lane < d.E) {
      z = zp[n * 64 + lane];
      for (int q = 1; q < nq; ++q) z = __fadd_rn(z, zp[(q * kRows + n) * 64 + lane]);
    }
    // rank of each expert (lane) among the row's logits, by (logit desc,
    // expert asc): the number of experts with a larger key.  Every key is
    // broadcast from its lane (scalar reads, no dependent shuffle chain).
    const uint64_t key = lane < d.E ? argmax_key(z, static_cast<uint32_t>(lane)) : 0ull;
    const uint32_t klo = static_cast<uint32_t>(key), khi = static_cast<uint32_t>(key >> 32);
    int rank = 0;
#pragma unroll
    for (int e = 0; e < kMaxExperts; ++e) {
      // (readlane returns int: go through uint32_t, never sign-extend)
      const uint64_t ke = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(khi, e))) << 32) |
                          static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(klo, e)));
      rank += ke > key ? 1 : 0;
    }
    const bool chosen = lane < d.E && rank < k;
    // softmax over the selection, max-subtracted, denominator summed in
    // selection order (rank 0, 1, ...)
    const unsigned long long first = __ballot(chosen && rank == 0);
    const float z0 = __shfl(z, __ffsll(static_cast<long long>(first)) - 1, kWave);
    const float ex = chosen ? expf(z - z0) : 0.0f;
    float den = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        const unsigned long long m = __ballot(chosen && rank == j);
        den = __fadd_rn(den, __shfl(ex, __ffsll(static_cast<long long>(m)) - 1, kWave));
      }
    }
    if (chosen) {
      p.idx_out[t * k + rank] = lane;
      p.w_out[t * k + rank] = ex / den;
      sel[n * k + rank] = lane;
    }
  }
  if (!p.sort.fused) return;

  // ------------------------------------------------------------ sort tail
  // one workgroup holds every selection: sort from LDS, no cross-CU sync
  __syncthreads();
  counting_sort_block(d, p.sort, T * k, reinterpret_cast<int*>(smem), sel);
}

// Prefill-sized steps (bf16, more than 256 rows, no combine): RMSNorm and
// top-k routing of 16 rows per 256-thread workgroup, several workgroups per
// CU (the 1024-thread kernel above fits one per CU, so its rows' memory
// round trips and reductions ran back to back).  Wavefront w normalises rows
// w, w + 4, w + 8, w + 12 (all four rows' loads issued first) and then
// computes the logits of expert tile w over the whole reduction, quarter by
// quarter with the next quarter's router fragments in flight; the quarters
// are added in the same fixed order as above, so the logits, selections and
// gate weights are bit-identical to the 1024-thread kernel's.  Logits meet
// through LDS, and each wavefront ranks its four rows' experts as above.
constexpr int kPfThreads = 256;
constexpr int kPfWaves = kPfThreads / kWave;
constexpr int kPfRowsPerWave = kRows / kPfWaves;

template <int KQ>  // H / 128: k-steps per reduction quarter
__global__ __launch_bounds__(kPfThreads) void k_router_rows(Dims d, NormRouterParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* zs = reinterpret_cast<float*>(smem);                     // [16 rows][64 experts]
  bf16_t* tile = reinterpret_cast<bf16_t*>(smem + kRows * 64 * sizeof(float));  // [H/32][64 lanes][8]
  const int H = d.H, k = d.k, T = p.T;
  const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t0 = blockIdx.x * kRows;
  const int nchunks = H / 4;
  constexpr int CPL = (KQ + 1) / 2;  // 4-element chunks per lane: ceil(H / 256)

  // this wavefront's rows and the gain, then its expert tile's first quarter
  // of router fragments (loads complete in order: the rows arrive first)
  Vec4<bf16_t> xv[kPfRowsPerWave][CPL], gv[CPL];
#pragma unroll
  for (int q = 0; q < kPfRowsPerWave; ++q) {
    const int t = min(t0 + wave + q * kPfWaves, T - 1);
    const bf16_t* xin = reinterpret_cast<const bf16_t*>(p.x_in) + static_cast<int64_t>(t) * H;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = min(lane + c * kWave, nchunks - 1);
      xv[q][c] = *reinterpret_cast<const Vec4<bf16_t>*>(xin + 4 * ch);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = min(lane + c * kWave, nchunks - 1);
    gv[c] = *reinterpret_cast<const Vec4<bf16_t>*>(reinterpret_cast<const bf16_t*>(p.gamma) + 4 * ch);
  }
  const int et = wave;  // expert tile of this wavefront (E <= 64)
  const bool has_tile = et * 16 < d.E;
  const bf16_t* wr = reinterpret_cast<const bf16_t*>(p.router) + static_cast<int64_t>(et) * (H / kKStep) * kFragElems +
                     lane * 8;
  bf16x8_t ra[2][KQ];
#pragma unroll
  for (int i = 0; i < KQ; ++i) ra[0][i] = load_frag(wr + i * kFragElems);

  // ------------------------------------------------------------ phase 1
#pragma unroll
  for (int q = 0; q < kPfRowsPerWave; ++q) {
    const int n = wave + q * kPfWaves, t = t0 + n;
    float x[CPL][4];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + c * kWave;
      float part = 0.0f;
      if (ch < nchunks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[c][i] = bf16_to_f32(xv[q][c].v[i]);
          part = __fadd_rn(part, __fmul_rn(x[c][i], x[c][i]));
        }
      }
      ss = __fadd_rn(ss, part);
    }
    ss = wave_sum(ss);
    const float rms = sqrtf(ss / static_cast<float>(H) + d.eps);
    bf16_t* xh = reinterpret_cast<bf16_t*>(p.xhat) + static_cast<int64_t>(t) * H;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + c * kWave;
      if (ch < nchunks) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = Storage<bf16_t>::round(__fmul_rn(x[c][i] / rms, bf16_to_f32(gv[c].v[i])));
        if (t < T) store4<bf16_t>(xh + 4 * ch, v);
        // operand tile kt = h/32; lane n + 16*((h%32)/8); element h%8 (rows
        // past T are zero: their logits are never used)
        const int h = 4 * ch, kt = h / 32, ln = n + 16 * ((h % 32) / 8);
        if (t >= T) v[0] = v[1] = v[2] = v[3] = 0.0f;
        store4<bf16_t>(tile + (kt * kWave + ln) * 8 + (h % 8), v);
      }
    }
  }
  __syncthreads();

  // ------------------------------------------------------------ phase 2
  // quarter kq of the reduction on ring slot kq & 1, the next quarter's
  // fragments requested before this quarter's MFMAs; the quarter sums are
  // added in quarter order as the 1024-thread kernel adds its four waves'
  f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) {
    if (kq + 1 < 4) {
#pragma unroll
      for (int i = 0; i < KQ; ++i) ra[(kq + 1) & 1][i] = load_frag(wr + ((kq + 1) * KQ + i) * kFragElems);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KQ; ++i) acc = mfma16(ra[kq & 1][i], load_frag(tile + ((kq * KQ + i) * kWave + lane) * 8), acc);
    if (kq == 0) {
      z = acc;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = __fadd_rn(z[i], acc[i]);
    }
  }
  // lane holds z[expert 16*et + 4*(lane/16) + i][row lane%16]
  if (has_tile) {
#pragma unroll
    for (int i = 0; i < 4; ++i) zs[(lane % 16) * 64 + et * 16 + 4 * (lane / 16) + i] = z[i];
  }
  __syncthreads();

  // ------------------------------------------------------------ phase 3
#pragma unroll 1
  for (int q = 0; q < kPfRowsPerWave; ++q) {
    const int n = wave + q * kPfWaves, t = t0 + n;
    if (t >= T) break;
    const float zl = lane < d.E ? zs[n * 64 + lane] : 0.0f;
    // rank of each expert (lane) by (logit desc, expert asc), as above
    const uint64_t key = lane < d.E ? argmax_key(zl, static_cast<uint32_t>(lane)) : 0ull;
    const uint32_t klo = static_cast<uint32_t>(key), khi = static_cast<uint32_t>(key >> 32);
    int rank = 0;
#pragma unroll
    for (int e = 0; e < kMaxExperts; ++e) {
      const uint64_t ke = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(khi, e))) << 32) |
                          static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(klo, e)));
      rank += ke > key ? 1 : 0;
    }
    const bool chosen = lane < d.E && rank < k;
    const unsigned long long first = __ballot(chosen && rank == 0);
    const float z0 = __shfl(zl, __ffsll(static_cast<long long>(first)) - 1, kWave);
    const float ex = chosen ? expf(zl - z0) : 0.0f;
    float den = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        const unsigned long long m = __ballot(chosen && rank == j);
        den = __fadd_rn(den, __shfl(ex, __ffsll(static_cast<long long>(m)) - 1, kWave));
      }
    }
    if (chosen) {
      p.idx_out[t * k + rank] = lane;
      p.w_out[t * k + rank] = ex / den;
    }
  }
}

template <typename ST, int KQ>
hipError_t launch_kq(const Dims& d, const NormRouterParams& p, hipStream_t s) {
  if constexpr (sizeof(ST) == 2) {
    if (p.T > 256 && !p.combine && p.norm && p.route && !p.sort.fused && d.E <= kMaxExperts) {
      const size_t smem = kRows * 64 * sizeof(float) + static_cast<size_t>(d.H) * 32;
      hipLaunchKernelGGL(k_router_rows<KQ>, dim3((p.T + kRows - 1) / kRows), dim3(kPfThreads), smem, s, d, p);
      return hipGetLastError();
    }
  }
  // 16 rows per workgroup when one workgroup takes the whole step (fused sort)
  // or the step is prefill-sized; otherwise one (split path, eight wavefronts
  // per row) or four, so that a verify step of a few hundred rows spreads its
  // combine reads over more CUs
  const bool split = sizeof(ST) == 2 && p.T > kRows && p.T <= 256 && !p.sort.fused && d.S <= kSplitShared && d.k <= kSplitRouted;
  const int rows = split ? 1 : (p.T <= kRows || p.T > 256) ? kRows : 4;
  // the rows' workgroups, then the router-matrix helpers (bf16 routing only)
  const dim3 grid((p.T + rows - 1) / rows + (p.route && sizeof(ST) == 2 ? kRouterHelpers : 0));
  const size_t xs = p.route ? (sizeof(ST) == 2 ? static_cast<size_t>(d.H) * 32 : static_cast<size_t>(d.H) * kRows * 4) : 0;
  const size_t smem = 4 * kRows * 64 * sizeof(float) + xs;
  if constexpr (sizeof(ST) == 2) {
    if (split) {
      hipLaunchKernelGGL((k_norm_router<ST, KQ, false, true>), grid, dim3(kThreads), smem, s, d, p, rows);
      return hipGetLastError();
    }
  }
  if (!p.combine && p.route && sizeof(ST) == 2)
    hipLaunchKernelGGL((k_norm_router<ST, KQ, true, false>), grid, dim3(kThreads), smem, s, d, p, rows);
  else
    hipLaunchKernelGGL((k_norm_router<ST, KQ, false, false>), grid, dim3(kThreads), smem, s, d, p, rows);
  return hipGetLastError();
}

template <typename ST>
hipError_t launch_st(const Dims& d, const NormRouterParams& p, hipStream_t s) {
  switch (d.H / 128) {
    case 1: return launch_kq<ST, 1>(d, p, s);
    case 2: return launch_kq<ST, 2>(d, p, s);
    case 3: return launch_kq<ST, 3>(d, p, s);
    case 4: return launch_kq<ST, 4>(d, p, s);
    case 5: return launch_kq<ST, 5>(d, p, s);
    case 6: return launch_kq<ST, 6>(d, p, s);
    case 7: return launch_kq<ST, 7>(d, p, s);
    case 8: return launch_kq<ST, 8>(d, p, s);
    case 9: return launch_kq<ST, 9>(d, p, s);
    case 10: return launch_kq<ST, 10>(d, p, s);
    case 11: return launch_kq<ST, 11>(d, p, s);
    case 12: return launch_kq<ST, 12>(d, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t norm_router_lds_bytes(const Dims& d) {
  return 4 * kRows * 64 * sizeof(float) + (d.bf16 ? static_cast<size_t>(d.H) * 32 : static_cast<size_t>(d.H) * kRows * 4);
}

int norm_router_sort_limit() { return kRows; }

hipError_t launch_norm_router(const Dims& d, const NormRouterParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  return d.bf16 ? launch_st<bf16_t>(d, p, s) : launch_st<float>(d, p, s);
}

}  // namespace moe
