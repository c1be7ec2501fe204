// Launch interface between the C ABI (api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

// Model dimensions (H hidden, E routed, k top-k, S shared, I SwiGLU width,
// V vocabulary, Vpad padded vocabulary rows of the tiled LM head).
struct Dims {
  int H, E, k, S, I, V, Vpad, L;
  float eps;
  int bf16;  // 1: bfloat16 storage and MFMA kernels; 0: float32 storage
  int n_cu;  // compute units of the device (sizes persistent grids)
};

// Stable counting sort of the T*k (token, slot) pairs by expert.
struct SortParams {
  const int* idx;        // [P] expert of pair p = t*k + j
  int* cnt;              // [E]
  int* off;              // [E+1]
  int* perm;             // [P]
  int* active;           // [E] experts with cnt > 0, ascending
  int* n_active;         // [1]
  int4* desc;            // [E] slot descriptors (see PermuteParams)
  int fused;             // 1: the (single) norm/router workgroup sorts in LDS
};

// Combine (previous block) + RMSNorm + router/top-k over T token rows.
struct NormRouterParams {
  const void* x_in;        // [T][H] storage: residual stream entering the kernel
  void* x_out;             // [T][H] storage: x_in + m (combine only; may equal x_in)
  const float* y;          // [T*k + S*T][H] previous block's expert outputs (combine)
  const int* prev_idx;     // [T][k] previous block's selection (combine)
  const float* prev_w;     // [T][k] previous block's gate weights (combine)
  float* m_out;            // [T][H] previous block's MoE output, optional (combine)
  const void* gamma;       // [H] storage, RMSNorm gain (norm)
  const void* router;      // bf16: tiled [64/16][H/32][512]; f32: [E][H] (route)
  void* xhat;              // [T][H] storage out (norm)
  int* idx_out;            // [T][k] (route)
  float* w_out;            // [T][k] (route)
  SortParams sort;           // fused counting sort (sort.fused: single-workgroup steps only)
  int T;
  int combine, norm, route;
};
hipError_t launch_norm_router(const Dims& d, const NormRouterParams& p, hipStream_t s);
size_t norm_router_lds_bytes(const Dims& d);
int norm_router_sort_limit();  // largest T the fused single-workgroup sort handles

// Stable counting sort of the T*k (token, slot) pairs by expert.
struct PermuteParams {
  const int* idx;  // [P] expert of pair p = t*k + j
  int P;
  int* cnt;        // [E]
  int* off;        // [E+1]
  int* perm;       // [P]
  int* active;     // [E] experts with cnt > 0, busiest first; entries past n_active unused
  int* n_active;   // [1]
  int4* desc;      // [E] routed slot i: (expert, tokens, first pair in perm, 0) of active[i];
                   //     (-1, 0, 0, 0) past n_active -- one read tells an expert workgroup its work
  // grouped-GEMM tile table, optional (see kGemmTokens): written by the
  // first workgroup from the same histogram when `tiles` is set
  int4* tiles;
  int* n_tiles;
  int tile_T;      // tokens of the block (the shared experts' rows)
  int n_shared;    // shared experts (slots of the tile table before the routed ones)
};
hipError_t launch_permute(const Dims& d, const PermuteParams& p, hipStream_t s);

// Expert SwiGLU on the decode path.  Expert slots: 0..S-1 are the shared
// experts (every token), then the active routed experts in the order of the
// active list (busiest first when the permutation kernel built it).
// Activation / output rows: pair p = t*k + j for routed, T*k + s*T + t for shared.
struct ExpertParams {
  const void* xhat;      // [T][H] storage
  const int* cnt;        // [E]
  const int* off;        // [E+1]
  const int* perm;       // [T*k]
  const int* active;     // [E]
  const int* n_active;   // [1]
  const int4* desc;      // [E] routed slot descriptors (null when there are no routed experts)
  const void* w_gate;    // this layer: bf16 tiled [E+S][I/16][H/32][512]; f32 [E+S][I][H]
  const void* w_up;      // same layout as w_gate
  const void* w_down;    // bf16 tiled [E+S][H/16][I/32][512]; f32 [E+S][H][I]
  void* act;             // [T*k + S*T][I] storage
  float* y;              // [T*k + S*T][H] float32
  int T;
};
hipError_t launch_expert_up(const Dims& d, const ExpertParams& p, hipStream_t s);
hipError_t launch_expert_down(const Dims& d, const ExpertParams& p, hipStream_t s);

// Attention projections on the down kernel (d: E = 0, k = 0, I = H; bf16).
constexpr int kHeadDim = 128;
struct EpiParams {
  // q/k/v (d.S = 3: slot 0 q, 1 k, 2 v, all reading act rows 0..T-1; token
  // n = b*K1 + j sits at position positions[b] + j)
  const int* positions;   // [B]
  int K1, P, nh;
  const float* inv_freq;  // [kHeadDim / 2] rotary inverse frequencies
  bf16_t* q;              // [T][H] rotated queries
  bf16_t* kc;             // this layer's key cache [seqs][nh][P][kHeadDim]
  bf16_t* vc;             // value cache, same layout
  // residual (d.S = 1): x_out = round(x_in + W act)
  const bf16_t* x_in;     // [T][H]
  bf16_t* x_out;          // [T][H]
};
hipError_t launch_linear_qkv(const Dims& d, const ExpertParams& p, const EpiParams& e, hipStream_t s);
hipError_t launch_linear_resid(const Dims& d, const ExpertParams& p, const EpiParams& e, hipStream_t s);

// First cache position of sequence b's verify step: positions[b] clamped into
// [0, P - K1], so every row the step writes or reads stays inside the cache.
// The q/k/v projection (rotary angle, cache rows written) and the attention
// (rows attended) both take it from here, so a position outside the range
// behaves exactly like the nearest one inside it.
__device__ __forceinline__ int step_position(const int* positions, int b, int P, int K1) {
  return min(max(positions[b], 0), P - K1);
}

// Decode attention of the verify step: K1 query rows per sequence against
// positions 0..positions[b]+j of the cache (keys / values [seqs][nh][P][128]).
struct AttnParams {
  const bf16_t* q;        // [T][H], T = B*K1
  const bf16_t* kc;
  const bf16_t* vc;
  const int* positions;   // [B]
  int B, K1, nh, P, G;    // G position groups per (sequence, head)
  float* part;            // [B][nh][G][K1][2 + kHeadDim]: running max, sum, weighted values
  bf16_t* ctx;            // [T][H] attention output (combine)
};
int attn_groups(const Dims& d, int B, int nh);
size_t attn_part_floats(int T, int nh, int G);
hipError_t launch_attention(const Dims& d, const AttnParams& p, hipStream_t s);          // split + combine
hipError_t launch_attention_split(const Dims& d, const AttnParams& p, hipStream_t s);
hipError_t launch_attention_combine(const AttnParams& p, hipStream_t s);

// Grouped GEMM for prefill-sized token counts (MFMA, LDS-staged tiles).
// Grouped-GEMM tile table: one entry per (slot, token tile of kGemmTokens),
// shared slots first, then the routed experts in ascending order; entry =
// (expert weight index, shared slot or -1 - offset into perm, first token,
// tokens).  Built by the permutation kernel.
constexpr int kGemmTokens = 256;
struct GemmParams {
  const void* xhat;      // [T][H] bf16
  const void* w_gate;    // tiled, this layer (see ExpertParams)
  const void* w_up;
  const void* w_down;
  const int* perm;       // [T*k]
  const int4* tiles;
  const int* n_tiles;
  void* act;             // SwiGLU activations in operand-tile order, gemm_act_rows rows of I
  float* y;              // [T*k + S*T][H] float32 (down, when yb is null)
  bf16_t* yb;            // [T*k + S*T][H] bf16 gate-weighted rows (down), or null
  const float* gate_w;   // [T][k] gate weights (down with yb)
  int T;
  int xhat_zero_row;     // an all-zero row of xhat (padding tokens read it)
};
int gemm_max_tiles(const Dims& d, int T);
int64_t gemm_act_rows(const Dims& d, int T);  // rows of the tiled activation buffer
size_t gemm_lds_bytes();
hipError_t launch_grouped_gemm(const Dims& d, const GemmParams& p, int up, hipStream_t s);

// Combine of a block whose expert rows are bf16 and already gate-weighted:
// m = shared rows + routed rows by ascending expert (fp32), x_out = round(x_in + m).
struct CombineParams {
  const void* x_in;      // [T][H] bf16
  void* x_out;           // [T][H] bf16
  const bf16_t* yb;      // [T*k + S*T][H] bf16
  const int* idx;        // [T][k] the block's selection
  float* m_out;          // [T][H] float32, optional
  int T;
};
hipError_t launch_combine_bf16(const Dims& d, const CombineParams& p, hipStream_t s);

// LM head + greedy arg-max + prefix acceptance.
constexpr int kKeySlots = 32;  // arg-max keys are spread over this many copies
struct LmHeadParams {
  const void* xf;            // [T][H] storage (final-norm activations)
  const void* lm;            // bf16 tiled [Vpad/16][H/32][512]; f32 [V][H]
  int T;
  unsigned long long* keys;  // [kKeySlots][key_stride], zero between steps
  int key_stride;
  const int* drafts;         // [B][K]
  int B, K;
  int* committed;            // [B][K+1]
  int* counts;               // [B]
  int* tstar;                // [T], optional
  // Final combine + RMSNorm (launch_final_norm), writing xf_out:
  const void* x_in;          // [T][H] storage: residual entering the last block
  const float* y;            // last block's expert outputs (see NormRouterParams)
  const int* prev_idx;       // [T][k]
  const float* prev_w;       // [T][k]
  const void* gamma;         // [H] final RMSNorm gain
  void* x_out;               // [T][H] storage: final residual, optional
  float* m_out;              // [T][H] last block's MoE output, optional
  void* xf_out;              // [T][H] bf16 normalised rows
};
// bf16: one workgroup per row finishes the last block and normalises it.
hipError_t launch_final_norm(const Dims& d, const LmHeadParams& p, hipStream_t s);
hipError_t launch_lmhead(const Dims& d, const LmHeadParams& p, hipStream_t s);  // keys only
hipError_t launch_accept(const LmHeadParams& p, hipStream_t s);  // picks + acceptance, keys cleared

// Draft head row kernels (one 256-thread workgroup per sequence; d.H <= 2048).
// Row layouts: x holds [2][B][H] (normalised state rows, then normalised
// token-embedding rows: the projection's two slots), yp [2][B][H] their
// projections, y [Sf][B][H] the FFN slots' outputs.
struct DraftParams {
  int B, R, V, Vd, K;
  int step;                    // 0-based step of this launch
  int last;                    // 1: the final step (no next-step inputs are written)
  int Sf;                      // FFN slots
  const bf16_t* hidden;        // [B][R][H] (k_draft_in)
  const int* committed;        // [B][R] (k_draft_in)
  const int* counts;           // [B] or null (k_draft_in)
  const bf16_t* embed;         // [V][H]
  const bf16_t* gamma_h;
  const bf16_t* gamma_e;
  const bf16_t* gamma_f;
  const bf16_t* gamma_o;
  bf16_t* x;                   // [2][B][H]
  const float* yp;             // [2][B][H]
  bf16_t* u;                   // [B][H]
  bf16_t* uh;                  // [B][H] FFN input
  const float* y;              // [Sf][B][H]
  bf16_t* xf;                  // [B][H] head input
  bf16_t* states;              // [K][B][H] or null
  unsigned long long* keys;    // [kKeySlots][key_stride]
  int key_stride;
  const int* head_ids;         // [Vd] or null (row = token)
  int* drafts;                 // [B][K]
};
hipError_t launch_draft_in(const Dims& d, const DraftParams& p, hipStream_t s);
hipError_t launch_draft_mid(const Dims& d, const DraftParams& p, hipStream_t s);
hipError_t launch_draft_out(const Dims& d, const DraftParams& p, hipStream_t s);
hipError_t launch_draft_pick(const Dims& d, const DraftParams& p, hipStream_t s);

// Weight repacking.  Tiled layout of an [R][C] bf16 matrix (R padded to Rpad
// with zero rows): tile (rt, kt) of 16 rows x 32 columns is 512 contiguous
// elements in which lane l of a wavefront owns the 8 elements of row
// rt*16 + l%16, columns kt*32 + (l/16)*8 .. +8 -- the operand layout of one
// 16x16x32 MFMA, so a wavefront loads a tile with one coalesced 1 KiB read.
hipError_t launch_tile_bf16(const bf16_t* src, int64_t src_mat_stride, bf16_t* dst,
                            int64_t n_mats, int R, int C, int Rpad, hipStream_t s);
// The same for matrices whose rows are `ld` elements apart (column slices of a
// wider matrix); ld and src_mat_stride are multiples of 8.
hipError_t launch_tile_bf16_ld(const bf16_t* src, int64_t src_mat_stride, int64_t ld, bf16_t* dst,
                               int64_t n_mats, int R, int C, int Rpad, hipStream_t s);

}  // namespace moe
