/*
 * moe_draft.h -- C ABI of the FastMTP-style draft head of the MI355X (gfx950)
 * MoE speculative decoding library: K draft tokens per sequence from one
 * dense block applied recursively.
 *
 * What a draft call computes.  For each of B sequences it starts from a
 * hidden state h (the verifier's residual stream after its last block) and a
 * token t, and applies the same block K times; step j outputs a state v_j and
 * a token d_j, and step j+1 continues from (v_j, d_j):
 *   a = RMSNorm(h; gamma_h)          e = RMSNorm(E[t]; gamma_e)
 *   u = W_proj [a; e]                (W_proj: H x 2H)
 *   v = u + W_down (silu(W_gate RMSNorm(u; gamma_f)) * (W_up RMSNorm(u; gamma_f)))
 *   d = arg-max over the draft head's rows of head . RMSNorm(v; gamma_o)
 * Sources:
 *   - page "Jina AI releases lightweight OCR model with built-in speculative
 *     decoding", section "Speculative decoding without accuracy loss": one
 *     compressed draft block executed recursively for K = 3 steps, with draft
 *     parameters that do not grow with the depth;
 *   - page "jina-ocr-v1 : Analyse de documents plus rapide sur des GPU a
 *     budget limite", section "Modele et entrainement" (one dense block applied
 *     recursively for K = 3 steps) and section "Pour commencer" (the head is
 *     trained with recursive hidden-state feedback: each step continues from
 *     the previous step's output instead of being reset onto the verifier).
 * The pages give no internals of the block; the projection of the normalised
 * state and token embedding, the dense SwiGLU FFN with residual, the output
 * norm and the shared LM head are this library's reading, and the block has
 * no attention (the verify step has an attention variant, moe_verify_step_kv
 * in moe_verify.h; the draft block does not).
 *
 * Numerics.  bfloat16 storage, float32 arithmetic; values are rounded to
 * bfloat16 (nearest, ties to even) at: every normalised activation (a, e,
 * the FFN input, the head input), the SwiGLU activation, u and v.  Arg-max
 * ties go to the lower head row.  A token id outside [0, V) embeds as zeros.
 *
 * Layouts, streams, ownership and errors are as in moe_verify.h: dense
 * row-major tensors, weights [out][in]; calls enqueue on `hip_stream` and
 * return without synchronising; 0 or a negative MOE_E* code, with the message
 * from moe_verify_last_error().  A draft context uses its verifier's LM head
 * and must be destroyed before that verifier.  Calls on one draft context
 * must not overlap.
 */
#ifndef MOE_DRAFT_H
#define MOE_DRAFT_H

#include <stdint.h>

#include "moe_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_draft_ctx moe_draft_ctx;

/*
 *   inter      Id, the dense SwiGLU width: a multiple of 128, 128..16384
 *   head_rows  Vd: 0 = the verifier's whole LM head (all V rows, shared, not
 *              copied); otherwise 1..V rows given in weights.head/head_ids
 *   max_batch  largest B, 1..1024
 *   k_max      largest K, 1..7
 * H, V, the RMSNorm epsilon and the storage type are the verifier's, which
 * must have bfloat16 storage and an LM head.
 */
typedef struct moe_draft_config {
  int32_t inter;
  int32_t head_rows;
  int32_t max_batch;
  int32_t k_max;
} moe_draft_config;

/*
 * Device pointers, 16-byte aligned, bfloat16 unless stated:
 *   embed     [V][H]   token embedding
 *   gamma_h, gamma_e, gamma_f, gamma_o   [H] RMSNorm gains (state, token,
 *             FFN input, head input)
 *   w_proj    [H][2H]  columns 0..H-1 act on the normalised state, H..2H-1
 *             on the normalised token embedding
 *   w_gate, w_up [Id][H]     w_down [H][Id]
 *   head      [Vd][H]  draft head rows (NULL when head_rows == 0)
 *   head_ids  int32 [Vd] token id of each head row (NULL when head_rows == 0)
 * moe_draft_init copies them (repacked); no pointer is kept afterwards.
 */
typedef struct moe_draft_weights {
  const void* embed;
  const void* gamma_h;
  const void* gamma_e;
  const void* w_proj;
  const void* gamma_f;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* gamma_o;
  const void* head;
  const int32_t* head_ids;
} moe_draft_weights;

/*
 * Create a draft context bound to `verifier`, copying and repacking the
 * weights on `hip_stream`, then synchronising it.  *out is NULL on failure.
 * Errors: MOE_EINVAL (NULL or misaligned pointers, sizes out of range),
 * MOE_EUNSUPPORTED (verifier without LM head or with float32 storage),
 * MOE_ENOMEM, MOE_EHIP.
 */
int moe_draft_init(moe_verify_ctx* verifier, const moe_draft_config* cfg, const moe_draft_weights* weights,
                   void* hip_stream, moe_draft_ctx** out);

/*
 * K recursive draft steps for B sequences.
 *   hidden    device, [B][R][H]: R states per sequence (a verify step's
 *             hidden_out has R = K'+1 rows per sequence)
 *   committed device, int32 [B][R]: the token at each of those rows
 *             (a verify step's committed output)
 *   counts    device, int32 [B] or NULL: sequence b starts from row
 *             counts[b]-1 (clamped into [0, R-1]) -- with a verify step's
 *             counts, the position whose greedy pick was its last committed
 *             token; NULL: row R-1
 *   drafts    device out, int32 [B][K]: d_1..d_K of each sequence, ready to
 *             be the next verify step's drafts
 *   states    device out, [K][B][H] or NULL: the step outputs v_1..v_K
 * Requires 1 <= R <= 8, 1 <= B <= max_batch, 1 <= K <= k_max.
 * Asynchronous; allocates nothing.
 */
int moe_draft_step(moe_draft_ctx* ctx, const void* hidden, const int32_t* committed, const int32_t* counts,
                   int32_t R, int32_t B, int32_t K, int32_t* drafts, void* states, void* hip_stream);

/*
 * One moe_draft_step(ctx, hidden, committed, counts, R, B, K, drafts, states)
 * enqueued on `hip_stream` captured into an executable graph, run with
 * moe_verify_graph_launch and freed with moe_verify_graph_destroy (the same
 * handle type as a captured verify step; semantics and errors as
 * moe_verify_graph_create: the buffers are fixed, their contents may change
 * between launches; destroy the graph before the context).  The draft call is
 * K * 7 + 1 launches, so it is the call whose fixed launch cost a graph
 * replay would save, if any (page "jina-ocr-v1 : Analyse de documents plus
 * rapide sur des GPU a budget limite", section "Decodage speculatif sur un
 * L4", on graphs against eager execution).
 */
int moe_draft_graph_create(moe_draft_ctx* ctx, const void* hidden, const int32_t* committed, const int32_t* counts,
                           int32_t R, int32_t B, int32_t K, int32_t* drafts, void* states, void* hip_stream,
                           moe_verify_graph** out);

/*
 * Timing hook of the next moe_draft_step on `ctx` (as
 * moe_verify_set_stage_events): MOE_STAGE_LMHEAD brackets the first step's
 * head kernel, MOE_STAGE_EXPERT_UP / MOE_STAGE_EXPERT_DOWN the first step's
 * FFN kernels, MOE_STAGE_ALL the whole call.
 */
int moe_draft_set_stage_events(moe_draft_ctx* ctx, int32_t stage, void* before, void* after);

/* Free everything the draft context owns.  NULL is accepted. */
void moe_draft_destroy(moe_draft_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DRAFT_H */
