/*
 * moe_verify.h -- C ABI of the MI355X (gfx950) library that runs one
 * speculative verification step of a mixture-of-experts decoder.
 *
 * What the step computes.  B sequences each carry K+1 positions: the last
 * committed token and K drafts.  For every position the library runs L
 * pre-norm MoE-FFN blocks (RMSNorm, a softmax router that keeps the top k of
 * E routed experts, k routed SwiGLU experts plus S always-on shared experts,
 * a gate-weighted combine and the residual add), a final RMSNorm, the LM
 * head and a greedy arg-max; then, per sequence, it accepts the longest
 * prefix of drafts that agree with those greedy picks and commits one more
 * token of the verifier's own.  The committed tokens therefore equal plain
 * greedy decoding.  Sources:
 *   - page "Jina AI releases lightweight OCR model with built-in speculative
 *     decoding", section "Lean architecture with a compressed encoder"
 *     (64 routed + 2 shared experts, top-6 routing, 12 layers) and section
 *     "Speculative decoding without accuracy loss" (greedy verification,
 *     longest agreeing prefix plus one extra token, bonus when all drafts
 *     match, output identical to greedy decoding);
 *   - page "jina-ocr-v1 : Analyse de documents plus rapide sur des GPU a
 *     budget limite", section "Modele et entrainement" (K = 3 drafts checked
 *     greedily, committed sequence equals the verifier's greedy sequence).
 * The pages give no layer internals: RMSNorm, SwiGLU, softmax-over-selected
 * gates, combine order and the bf16 rounding points below are this library's
 * plain reading of them.
 *
 * Numerics.  Storage type is float32 or bfloat16 (config.dtype).  All
 * arithmetic is float32.  With bfloat16 storage, values are rounded to
 * bfloat16 (nearest, ties to even) at exactly three points: the normalised
 * activations (router/expert input and LM-head input), the SwiGLU activation
 * silu(Wg x)*(Wu x), and each block's output x + m.  Top-k ties go to the
 * lower expert index; arg-max ties to the lower token id.
 *
 * Layouts.  Every tensor is dense row-major; weights are [out][in] as in a
 * linear layer.  T = B*(K+1) token rows, ordered sequence-major
 * (row b*(K+1)+j is position j of sequence b).
 *
 * Streams and ownership.  Every entry point that takes `hip_stream` (a
 * hipStream_t, NULL = the default stream) enqueues its work on that stream
 * and returns without synchronising.  Outputs are valid once the stream has
 * completed the work.  The caller owns every buffer it passes in.  A context
 * owns repacked copies of the weights and its own workspace: calls on one
 * context must not overlap (use one stream per context, or synchronise).
 *
 * Errors.  0 on success, otherwise a negative MOE_E* code; the message for
 * the last failure on the calling thread is returned by
 * moe_verify_last_error().  Argument errors are detected before any HIP
 * runtime call is made.  No C++ exception crosses this interface.
 */
#ifndef MOE_VERIFY_H
#define MOE_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)       /* null/misaligned pointer, bad size or count */
#define MOE_EUNSUPPORTED (-2) /* a shape or dtype the kernels do not cover  */
#define MOE_ENOMEM (-3)       /* device allocation failed                   */
#define MOE_EHIP (-4)         /* a HIP runtime or launch error              */

#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1

/* Opaque context: repacked weights, workspace, launch plan. */
typedef struct moe_verify_ctx moe_verify_ctx;

/*
 * Model and capacity description.
 *   hidden     H, a multiple of 128, at most 1536 (bf16) / 768 (f32)
 *   n_routed   E routed experts, 1..64 (one router lane per expert)
 *   top_k      k experts per token, 1..min(E, 8)
 *   n_shared   S always-on shared experts, 0..4
 *   inter      I SwiGLU width, a multiple of 128, at most 2048
 *   vocab      V LM-head rows, >= 1 (ignored without an LM head)
 *   n_layers   L blocks, 1..64
 *   max_tokens          largest T = B*(K+1) a verify step may use, 1..65536
 *   max_prefill_tokens  largest T for moe_block_forward, 0..65536 (0: max_tokens)
 *   k_max      largest K a verify step may use, 0..7
 *   rms_eps    RMSNorm epsilon, > 0
 *   dtype      MOE_DTYPE_F32 or MOE_DTYPE_BF16 (storage of every tensor)
 *   has_lm_head 1: verify steps available; 0: only moe_block_forward
 *   n_heads    0: the blocks are MoE-FFN only (moe_verify_step); otherwise
 *              every layer is attention then MoE (moe_verify_step_kv) with
 *              n_heads heads of 128 (hidden == 128 * n_heads), bf16 only
 *   max_positions  KV-cache positions per sequence, 8..32768 (attention only)
 *   max_seqs   KV-cache sequences, 1..1024 (attention only)
 *   rope_theta rotary base, > 0 (attention only)
 */
typedef struct moe_verify_config {
  int32_t hidden;
  int32_t n_routed;
  int32_t top_k;
  int32_t n_shared;
  int32_t inter;
  int32_t vocab;
  int32_t n_layers;
  int32_t max_tokens;
  int32_t max_prefill_tokens;
  int32_t k_max;
  float rms_eps;
  int32_t dtype;
  int32_t has_lm_head;
  int32_t n_heads;
  int32_t max_positions;
  int32_t max_seqs;
  float rope_theta;
} moe_verify_config;

/*
 * Device pointers to the weights, each 16-byte aligned, in the storage type.
 *   router      [L][E][H]
 *   w_gate      [L][E][I][H]      w_up   [L][E][I][H]     w_down [L][E][H][I]
 *   s_gate      [L][S][I][H]      s_up   [L][S][I][H]     s_down [L][S][H][I]
 *               (may be NULL when S == 0)
 *   norm_gamma  [L][H]   pre-block RMSNorm gains
 *   final_gamma [H]      final RMSNorm gain (NULL when has_lm_head == 0)
 *   lm_head     [V][H]   (NULL when has_lm_head == 0)
 *   attn_gamma  [L][H]   pre-attention RMSNorm gains        (NULL when n_heads == 0)
 *   w_q, w_k, w_v, w_o   [L][H][H] attention projections    (NULL when n_heads == 0)
 * moe_verify_init copies them (repacked); no pointer is kept afterwards.
 */
typedef struct moe_verify_weights {
  const void* router;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* s_gate;
  const void* s_up;
  const void* s_down;
  const void* norm_gamma;
  const void* final_gamma;
  const void* lm_head;
  const void* attn_gamma;
  const void* w_q;
  const void* w_k;
  const void* w_v;
  const void* w_o;
} moe_verify_weights;

/*
 * Optional device outputs for inspection and parity checks (any field may be
 * NULL; every non-NULL pointer must be 16-byte aligned).  T is the step's
 * token count; l indexes the layer.
 *   topk_idx      int32 [L][T][k]  selected experts, descending router logit
 *   topk_w        float [L][T][k]  gate weights (softmax over the selection)
 *   expert_count  int32 [L][E]     tokens routed to each expert
 *   expert_offset int32 [L][E+1]   exclusive prefix sum of expert_count
 *   perm          int32 [L][T*k]   pair ids t*k+j grouped by expert, stable
 *   moe_out       float [L][T][H]  block output before the residual add
 *   hidden_out    storage [T][H]   residual stream after the last block
 *   tstar         int32 [T]        greedy pick after each position
 *   attn_out      storage [L][T][H] each layer's attention-sublayer output
 *                 x + W_o attn (moe_verify_step_kv only)
 */
typedef struct moe_verify_aux {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* expert_count;
  int32_t* expert_offset;
  int32_t* perm;
  float* moe_out;
  void* hidden_out;
  int32_t* tstar;
  void* attn_out;
} moe_verify_aux;

/*
 * The decoder whose blocks these are has 64 routed experts, two shared
 * experts, top-6 routing and 12 layers (page "Jina AI releases lightweight OCR
 * model with built-in speculative decoding", section "Lean architecture with a
 * compressed encoder"); the config carries those counts, and the widths the
 * pages leave open.
 * Validate `cfg`, allocate the context and repack the weights into it on
 * `hip_stream`, then synchronise that stream (so the caller may free its
 * weight tensors as soon as this returns).  On success *out receives the
 * context; on failure *out is set to NULL and nothing is leaked.
 * Errors: MOE_EINVAL (NULL cfg/weights/out, a NULL or misaligned required
 * weight pointer, a size out of the ranges above), MOE_EUNSUPPORTED,
 * MOE_ENOMEM, MOE_EHIP.
 */
int moe_verify_init(const moe_verify_config* cfg, const moe_verify_weights* weights,
                    void* hip_stream, moe_verify_ctx** out);

/*
 * One verification step (the pages' greedy verify of K drafts per sequence).
 *   hidden    device, storage [B][K+1][H]: residual stream entering block 0
 *   drafts    device, int32 [B][K]: draft j of sequence b proposes the token
 *             at position j+1 and is compared with the pick after position j;
 *             an id outside [0, V) simply never matches.  May be NULL if K == 0.
 *   committed device out, int32 [B][K+1]: accepted picks, then -1 padding
 *   counts    device out, int32 [B]: tokens committed, 1..K+1 (K+1 means all
 *             drafts matched and the last token is the bonus)
 * Requires has_lm_head and n_heads == 0; 1 <= B; 0 <= K <= k_max;
 * B*(K+1) <= max_tokens.  Asynchronous; allocates nothing.
 */
int moe_verify_step(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts,
                    int32_t B, int32_t K, int32_t* committed, int32_t* counts,
                    void* hip_stream);

/*
 * The verify step of a context with attention (n_heads > 0): every layer is
 * x <- x + W_o Attn(RMSNorm(x; attn_gamma)) then the MoE block.  Attention is
 * multi-head (heads of 128) with the rotary embedding of dimension pairs
 * (2i, 2i+1) by pos * rope_theta^(-2i/128) and a KV cache: sequence b uses
 * cache slot b; its K+1 positions sit at positions[b] .. positions[b]+K, their
 * keys and values are written there, and position j attends to cache entries
 * 0 .. positions[b]+j (scores q.k / sqrt(128), softmax in float32).  After
 * the step the caller advances positions[b] by counts[b]: the entries of the
 * accepted tokens stay valid and those of rejected drafts are overwritten by
 * the next step.  The pages give no attention internals; this is the
 * library's reading of the decoder on the page "Jina AI releases lightweight
 * OCR model with built-in speculative decoding", section "Lean architecture
 * with a compressed encoder" (12 layers, 32,768 positions).
 *   positions device, int32 [B]: 0 <= positions[b] <= max_positions - (K+1);
 *             a value outside that range is clamped to it (the step then
 *             behaves exactly as at the clamped position, for the rotary
 *             angles, the cache rows written and the rows attended alike)
 * Other arguments as moe_verify_step_ex; requires B <= max_seqs and
 * K+1 <= max_positions.  Asynchronous; allocates nothing.
 */
int moe_verify_step_kv(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts,
                       const int32_t* positions, int32_t B, int32_t K, int32_t* committed,
                       int32_t* counts, const moe_verify_aux* aux, void* hip_stream);

/*
 * The context's KV cache (n_heads > 0): *k_cache and *v_cache receive device
 * pointers to bfloat16 [L][max_seqs][n_heads][max_positions][128] arrays
 * (rotated keys; values), zero after init.  The caller may write the entries
 * of earlier positions (a prompt's keys and values) with ordinary copies on
 * the context's stream.  Errors: MOE_EINVAL (NULL arguments, no attention).
 */
int moe_verify_kv_cache(moe_verify_ctx* ctx, void** k_cache, void** v_cache);

/* moe_verify_step plus the optional outputs in `aux` (aux may be NULL). */
int moe_verify_step_ex(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts,
                       int32_t B, int32_t K, int32_t* committed, int32_t* counts,
                       const moe_verify_aux* aux, void* hip_stream);

/*
 * One MoE-FFN block of layer `layer` over T token rows (the prefill path: a
 * page enters the decoder as at most 1,156 visual tokens, 256 global plus up
 * to nine local tiles of 100, page "Jina AI releases lightweight OCR model
 * with built-in speculative decoding", section "Lean architecture with a
 * compressed encoder"; several pages and their prompts make thousands of rows):
 *   x  device, storage [T][H] in;  y  device, storage [T][H] out = x + MoE(RMSNorm(x)).
 * x and y may not overlap.  aux (may be NULL) receives layer-0-indexed
 * topk_idx/topk_w/expert_count/expert_offset/perm/moe_out for this block;
 * hidden_out and tstar are ignored.  Requires 1 <= T <= max_prefill_tokens
 * (or <= max_tokens when max_prefill_tokens is 0).  Asynchronous.
 */
int moe_block_forward(moe_verify_ctx* ctx, int32_t layer, const void* x, int32_t T, void* y,
                      const moe_verify_aux* aux, void* hip_stream);

/*
 * The verify step replayed through a HIP graph.  The page "jina-ocr-v1 :
 * Analyse de documents plus rapide sur des GPU a budget limite", section
 * "Decodage speculatif sur un L4", finds that the verify step's fixed
 * overhead decides the best K (CUDA graphs against eager execution); these
 * calls let a caller run and time the step both ways.
 * moe_verify_graph_create captures one moe_verify_step(ctx, hidden, drafts,
 * B, K, committed, counts) enqueued on `hip_stream` into an executable graph
 * (nothing runs; the stream may not be NULL, as the default stream cannot be
 * captured).  Every moe_verify_graph_launch, on any stream, then runs that
 * step on those same buffers -- their contents may change between launches,
 * the pointers may not -- with moe_verify_step's results.  A graph belongs to
 * its context: destroy it first, and do not let its launches overlap other
 * calls on the context.  Timing hooks must be clear when capturing.
 * Errors (create): those of moe_verify_step, MOE_EINVAL for a NULL `out` or
 * stream or a timing hook that is set, MOE_ENOMEM, MOE_EHIP (capture or
 * instantiation failed); *out is NULL on failure.  Launch: MOE_EINVAL for a
 * NULL graph, MOE_EHIP.  Destroy accepts NULL.
 */
typedef struct moe_verify_graph moe_verify_graph;
int moe_verify_graph_create(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts,
                            int32_t B, int32_t K, int32_t* committed, int32_t* counts,
                            void* hip_stream, moe_verify_graph** out);
/* The same for moe_verify_step_kv (a context with attention): the captured
 * step reads `positions` at every launch, so the caller may advance them
 * between launches. */
int moe_verify_graph_create_kv(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts,
                               const int32_t* positions, int32_t B, int32_t K, int32_t* committed,
                               int32_t* counts, void* hip_stream, moe_verify_graph** out);
int moe_verify_graph_launch(moe_verify_graph* graph, void* hip_stream);
void moe_verify_graph_destroy(moe_verify_graph* graph);

/* Stages that can be bracketed by timing events. */
#define MOE_STAGE_LMHEAD 0      /* LM head + arg-max + acceptance kernel of a verify step   */
#define MOE_STAGE_EXPERT_UP 1   /* expert gate/up kernel of the first block of a call        */
#define MOE_STAGE_EXPERT_DOWN 2 /* expert down kernel of the first block of a call           */
#define MOE_STAGE_ALL 3         /* the whole call, first kernel to last                      */
#define MOE_STAGE_ATTENTION 4   /* decode-attention kernel of the first layer (step_kv)      */
#define MOE_STAGE_COUNT 5

/*
 * Timing hook for profiling.  `before` and `after` are hipEvent_t handles
 * created by the caller (or NULL to clear).  The next moe_verify_step /
 * moe_verify_step_ex / moe_block_forward call on `ctx` records `before` on
 * its stream right before it launches stage `stage` and `after` right after,
 * then forgets the pair (one call only), so a caller times N calls with N
 * event pairs.  The events add two stream records to that call.
 * Errors: MOE_EINVAL for a NULL ctx or a stage outside [0, MOE_STAGE_COUNT).
 */
int moe_verify_set_stage_events(moe_verify_ctx* ctx, int32_t stage, void* before, void* after);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the verify
 * step of moe_verify_step with its workspace -- residual and normalised rows,
 * selections, permutation, SwiGLU activations, expert outputs, arg-max keys
 * -- in a file-scope device array of MOE_STATIC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends, instead of
 * the context's own workspace.  The call allocates nothing; the caller
 * passes inputs and outputs exactly as for moe_verify_step, with the same
 * results.  Limits: B*(K+1) <= MOE_STATIC_MAX_TOKENS (and <= max_tokens),
 * a context without attention, the context's device current.  Every call on
 * one GPU uses that GPU's one array: calls that overlap on one GPU (on
 * different streams, or from several threads or contexts) race, and must be
 * serialised by the caller.  Errors: those of moe_verify_step; MOE_EINVAL
 * for a step larger than the limits or a workspace that would not fit.
 */
#define MOE_STATIC_SCRATCH_BYTES (16u << 20)
#define MOE_STATIC_MAX_TOKENS 128
int moe_verify_step_static(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts,
                           int32_t B, int32_t K, int32_t* committed, int32_t* counts,
                           void* hip_stream);

/* Free everything the context owns.  NULL is accepted.  Synchronises the
 * device work the context may still have in flight. */
void moe_verify_destroy(moe_verify_ctx* ctx);

/* Message of the last failure on the calling thread ("" if none). */
const char* moe_verify_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_VERIFY_H */
