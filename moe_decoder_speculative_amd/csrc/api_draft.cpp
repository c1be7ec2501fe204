// C ABI of the draft head (declared in include/moe_draft.h): context creation
// with weight repacking, and the launch sequence of K recursive draft steps.
// The projection and the dense FFN run on the decode expert kernels as
// shared-only expert slots; the head is the verifier's LM-head kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <new>
#include <string>
#include <vector>

#include "api_internal.h"
#include "kernels.h"
#include "moe_draft.h"

using moe::bf16_t;
using moe::api::check_ptr;
using moe::api::fail;
using moe::api::mark;

namespace moe {
int lmhead_row_multiple();
}

struct moe_draft_ctx {
  moe_verify_ctx* verifier = nullptr;
  moe_draft_config cfg{};
  int device = 0;
  std::vector<void*> allocs;
  moe::Dims dp{}, df{}, dh{};  // projection slots, FFN slots, head
  int If = 0, Sf = 0;          // FFN slot width and count

  // weights
  char* embed = nullptr;       // [V][H]
  char* gammas = nullptr;      // [4][H]: h, e, f, o
  char* proj = nullptr;        // tiled [2][H/16][H/32][512]
  char* gate = nullptr;        // tiled [Sf][If/16][H/32][512]
  char* up = nullptr;
  char* down = nullptr;        // tiled [Sf][H/16][If/32][512]
  const char* head = nullptr;  // tiled [Vpad/16][H/32][512] (own copy or the verifier's)
  int* head_ids = nullptr;     // [Vd] or null

  // workspace (B = max_batch rows)
  char* x = nullptr;           // [2][B][H]
  float* yp = nullptr;         // [2][B][H]
  char* u = nullptr;           // [B][H]
  char* uh = nullptr;          // [B][H]
  char* act = nullptr;         // [Sf][B][If]
  float* y = nullptr;          // [Sf][B][H]
  char* xf = nullptr;          // [B][H]
  unsigned long long* keys = nullptr;  // [kKeySlots][B], zero between uses
  int* zero = nullptr;         // a device 0: no routed experts are active

  hipEvent_t ev_before[MOE_STAGE_COUNT] = {};
  hipEvent_t ev_after[MOE_STAGE_COUNT] = {};
};

namespace {

void draft_free(moe_draft_ctx* c) {
  if (!c) return;
  moe::api::dev_free_all(c->allocs, c->device);
  delete c;
}

int alloc(moe_draft_ctx* c, size_t bytes, char** out) { return moe::api::dev_alloc(c->allocs, bytes, out); }
template <typename P>
int alloc_t(moe_draft_ctx* c, size_t bytes, P** out) {
  char* p = nullptr;
  const int r = alloc(c, bytes, &p);
  *out = reinterpret_cast<P*>(p);
  return r;
}

// Widest slot (a multiple of 128, at most 1024) that divides the dense width.
int slot_width(int Id) {
  for (int m = 8; m >= 1; --m)
    if ((Id / 128) % m == 0) return 128 * m;
  return 128;
}

int create(moe_verify_ctx* v, const moe_draft_config& g, const moe_draft_weights& w, hipStream_t s,
           moe_draft_ctx* c) {
  c->verifier = v;
  c->cfg = g;
  c->device = v->device;
  const moe::Dims& vd = v->d;
  const int64_t H = vd.H, V = vd.V, Id = g.inter, Bm = g.max_batch;
  c->If = slot_width(g.inter);
  c->Sf = g.inter / c->If;
  moe::Dims base = vd;
  base.E = 0;
  base.k = 0;
  base.L = 1;
  c->dp = base;
  c->dp.S = 2;
  c->dp.I = vd.H;
  c->df = base;
  c->df.S = c->Sf;
  c->df.I = c->If;
  c->dh = vd;
  if (g.head_rows > 0) {
    const int mult = moe::lmhead_row_multiple();
    c->dh.V = g.head_rows;
    c->dh.Vpad = (g.head_rows + mult - 1) / mult * mult;
  }

  int r;
  if ((r = alloc(c, V * H * 2, &c->embed))) return r;
  if ((r = alloc(c, 4 * H * 2, &c->gammas))) return r;
  if ((r = alloc(c, 2 * H * H * 2, &c->proj))) return r;
  if ((r = alloc(c, Id * H * 2, &c->gate))) return r;
  if ((r = alloc(c, Id * H * 2, &c->up))) return r;
  if ((r = alloc(c, H * Id * 2, &c->down))) return r;
  if (g.head_rows > 0) {
    char* h = nullptr;
    if ((r = alloc(c, static_cast<size_t>(c->dh.Vpad) * H * 2, &h))) return r;
    c->head = h;
    if ((r = alloc_t(c, static_cast<size_t>(g.head_rows) * sizeof(int), &c->head_ids))) return r;
  } else {
    c->head = v->lm;
  }
  if ((r = alloc(c, 2 * Bm * H * 2, &c->x))) return r;
  if ((r = alloc_t(c, 2 * Bm * H * sizeof(float), &c->yp))) return r;
  if ((r = alloc(c, Bm * H * 2, &c->u))) return r;
  if ((r = alloc(c, Bm * H * 2, &c->uh))) return r;
  if ((r = alloc(c, Bm * Id * 2, &c->act))) return r;
  if ((r = alloc_t(c, static_cast<size_t>(c->Sf) * Bm * H * sizeof(float), &c->y))) return r;
  if ((r = alloc(c, Bm * H * 2, &c->xf))) return r;
  if ((r = alloc_t(c, moe::kKeySlots * Bm * sizeof(unsigned long long), &c->keys))) return r;
  if ((r = alloc_t(c, 16, &c->zero))) return r;
  MOE_HIP(hipMemsetAsync(c->keys, 0, moe::kKeySlots * Bm * sizeof(unsigned long long), s));
  MOE_HIP(hipMemsetAsync(c->zero, 0, 16, s));

  // repack: projection halves and FFN column blocks become expert slots
  MOE_HIP(hipMemcpyAsync(c->embed, w.embed, V * H * 2, hipMemcpyDeviceToDevice, s));
  const void* gs[4] = {w.gamma_h, w.gamma_e, w.gamma_f, w.gamma_o};
  for (int i = 0; i < 4; ++i)
    MOE_HIP(hipMemcpyAsync(c->gammas + i * H * 2, gs[i], H * 2, hipMemcpyDeviceToDevice, s));
  const int Hi = static_cast<int>(H), If = c->If;
  MOE_HIP(moe::launch_tile_bf16_ld(static_cast<const bf16_t*>(w.w_proj), H, 2 * H,
                                   reinterpret_cast<bf16_t*>(c->proj), 2, Hi, Hi, Hi, s));
  MOE_HIP(moe::launch_tile_bf16(static_cast<const bf16_t*>(w.w_gate), static_cast<int64_t>(If) * H,
                                reinterpret_cast<bf16_t*>(c->gate), c->Sf, If, Hi, If, s));
  MOE_HIP(moe::launch_tile_bf16(static_cast<const bf16_t*>(w.w_up), static_cast<int64_t>(If) * H,
                                reinterpret_cast<bf16_t*>(c->up), c->Sf, If, Hi, If, s));
  MOE_HIP(moe::launch_tile_bf16_ld(static_cast<const bf16_t*>(w.w_down), If, Id,
                                   reinterpret_cast<bf16_t*>(c->down), c->Sf, Hi, If, Hi, s));
  if (g.head_rows > 0) {
    MOE_HIP(moe::launch_tile_bf16(static_cast<const bf16_t*>(w.head), 0,
                                  reinterpret_cast<bf16_t*>(const_cast<char*>(c->head)), 1, g.head_rows, Hi,
                                  c->dh.Vpad, s));
    MOE_HIP(hipMemcpyAsync(c->head_ids, w.head_ids, static_cast<size_t>(g.head_rows) * sizeof(int),
                           hipMemcpyDeviceToDevice, s));
  }
  MOE_HIP(hipStreamSynchronize(s));
  return MOE_OK;
}

int validate(moe_verify_ctx* v, const moe_draft_config& g, const moe_draft_weights& w) {
  const moe_verify_config& vc = v->cfg;
  if (!vc.has_lm_head) return fail(MOE_EUNSUPPORTED, "the verifier has no LM head to share");
  if (vc.dtype != MOE_DTYPE_BF16) return fail(MOE_EUNSUPPORTED, "the draft head needs bfloat16 storage");
  auto bad = [](const std::string& m) { return fail(MOE_EINVAL, "draft config: " + m); };
  if (g.inter < 128 || g.inter > 16384 || g.inter % 128 != 0) return bad("inter must be a multiple of 128 in [128, 16384]");
  if (g.head_rows < 0 || g.head_rows > vc.vocab) return bad("head_rows must be in [0, vocab]");
  if (g.max_batch < 1 || g.max_batch > 1024) return bad("max_batch must be in [1, 1024]");
  if (g.k_max < 1 || g.k_max > 7) return bad("k_max must be in [1, 7]");
  struct Item { const void* p; const char* name; bool required; };
  const Item items[] = {
      {w.embed, "embed", true},     {w.gamma_h, "gamma_h", true}, {w.gamma_e, "gamma_e", true},
      {w.w_proj, "w_proj", true},   {w.gamma_f, "gamma_f", true}, {w.w_gate, "w_gate", true},
      {w.w_up, "w_up", true},       {w.w_down, "w_down", true},   {w.gamma_o, "gamma_o", true},
      {w.head, "head", g.head_rows > 0}, {w.head_ids, "head_ids", g.head_rows > 0},
  };
  for (const Item& it : items) {
    int r;
    if ((r = check_ptr(it.p, (std::string("draft weights: ") + it.name).c_str(), it.required))) return r;
  }
  return MOE_OK;
}

int step_impl(moe_draft_ctx* c, const void* hidden, const int32_t* committed, const int32_t* counts, int32_t R,
              int32_t B, int32_t K, int32_t* drafts, void* states, void* stream) {
  if (!c) return fail(MOE_EINVAL, "draft ctx is NULL");
  if (R < 1 || R > 8) return fail(MOE_EINVAL, "R must be in [1, 8]");
  if (B < 1 || B > c->cfg.max_batch) return fail(MOE_EINVAL, "B must be in [1, max_batch]");
  if (K < 1 || K > c->cfg.k_max) return fail(MOE_EINVAL, "K must be in [1, k_max]");
  int r;
  if ((r = check_ptr(hidden, "hidden", true))) return r;
  if ((r = check_ptr(committed, "committed", true))) return r;
  if ((r = check_ptr(counts, "counts", false))) return r;
  if ((r = check_ptr(drafts, "drafts", true))) return r;
  if ((r = check_ptr(states, "states", false))) return r;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t H = c->dh.H;

  moe::DraftParams p{};
  p.B = B;
  p.R = R;
  p.V = c->verifier->d.V;
  p.Vd = c->dh.V;
  p.K = K;
  p.Sf = c->Sf;
  p.hidden = static_cast<const bf16_t*>(hidden);
  p.committed = committed;
  p.counts = counts;
  p.embed = reinterpret_cast<const bf16_t*>(c->embed);
  p.gamma_h = reinterpret_cast<const bf16_t*>(c->gammas);
  p.gamma_e = reinterpret_cast<const bf16_t*>(c->gammas + H * 2);
  p.gamma_f = reinterpret_cast<const bf16_t*>(c->gammas + 2 * H * 2);
  p.gamma_o = reinterpret_cast<const bf16_t*>(c->gammas + 3 * H * 2);
  p.x = reinterpret_cast<bf16_t*>(c->x);
  p.yp = c->yp;
  p.u = reinterpret_cast<bf16_t*>(c->u);
  p.uh = reinterpret_cast<bf16_t*>(c->uh);
  p.y = c->y;
  p.xf = reinterpret_cast<bf16_t*>(c->xf);
  p.states = static_cast<bf16_t*>(states);
  p.keys = c->keys;
  p.key_stride = c->cfg.max_batch;
  p.head_ids = c->head_ids;
  p.drafts = drafts;

  moe::ExpertParams pe{};  // projection: slot s reads x rows s*B + b
  pe.n_active = c->zero;
  pe.w_down = c->proj;
  pe.act = c->x;
  pe.y = c->yp;
  pe.T = B;
  moe::ExpertParams fe{};  // dense FFN: Sf shared slots
  fe.n_active = c->zero;
  fe.xhat = c->uh;
  fe.w_gate = c->gate;
  fe.w_up = c->up;
  fe.w_down = c->down;
  fe.act = c->act;
  fe.y = c->y;
  fe.T = B;
  moe::LmHeadParams lp{};
  lp.xf = c->xf;
  lp.lm = c->head;
  lp.T = B;
  lp.keys = c->keys;
  lp.key_stride = c->cfg.max_batch;

  MOE_HIP(mark(c->ev_before[MOE_STAGE_ALL], s));
  MOE_HIP(moe::launch_draft_in(c->dh, p, s));
  for (int j = 0; j < K; ++j) {
    p.step = j;
    p.last = j == K - 1;
    MOE_HIP(moe::launch_expert_down(c->dp, pe, s));
    MOE_HIP(moe::launch_draft_mid(c->dh, p, s));
    if (j == 0) MOE_HIP(mark(c->ev_before[MOE_STAGE_EXPERT_UP], s));
    MOE_HIP(moe::launch_expert_up(c->df, fe, s));
    if (j == 0) MOE_HIP(mark(c->ev_after[MOE_STAGE_EXPERT_UP], s));
    if (j == 0) MOE_HIP(mark(c->ev_before[MOE_STAGE_EXPERT_DOWN], s));
    MOE_HIP(moe::launch_expert_down(c->df, fe, s));
    if (j == 0) MOE_HIP(mark(c->ev_after[MOE_STAGE_EXPERT_DOWN], s));
    MOE_HIP(moe::launch_draft_out(c->dh, p, s));
    if (j == 0) MOE_HIP(mark(c->ev_before[MOE_STAGE_LMHEAD], s));
    MOE_HIP(moe::launch_lmhead(c->dh, lp, s));
    if (j == 0) MOE_HIP(mark(c->ev_after[MOE_STAGE_LMHEAD], s));
    MOE_HIP(moe::launch_draft_pick(c->dh, p, s));
  }
  MOE_HIP(mark(c->ev_after[MOE_STAGE_ALL], s));
  return MOE_OK;
}

void clear_hooks(moe_draft_ctx* c) {
  for (int i = 0; i < MOE_STAGE_COUNT; ++i) c->ev_before[i] = c->ev_after[i] = nullptr;
}

}  // namespace

extern "C" {

int moe_draft_init(moe_verify_ctx* verifier, const moe_draft_config* cfg, const moe_draft_weights* weights,
                   void* hip_stream, moe_draft_ctx** out) {
  if (out) *out = nullptr;
  if (!verifier || !cfg || !weights || !out) return fail(MOE_EINVAL, "verifier, cfg, weights and out must be non-NULL");
  int r;
  if ((r = validate(verifier, *cfg, *weights))) return r;
  moe_draft_ctx* c = new (std::nothrow) moe_draft_ctx();
  if (!c) return fail(MOE_ENOMEM, "host allocation failed");
  int cur = 0;
  const bool switched = hipGetDevice(&cur) == hipSuccess && cur != verifier->device;
  if (switched) (void)hipSetDevice(verifier->device);
  try {
    r = create(verifier, *cfg, *weights, static_cast<hipStream_t>(hip_stream), c);
  } catch (...) {
    r = fail(MOE_ENOMEM, "host exception during init");
  }
  if (switched) (void)hipSetDevice(cur);
  if (r != MOE_OK) {
    const std::string keep = moe::api::last_error();
    draft_free(c);
    fail(r, keep);
    return r;
  }
  *out = c;
  moe::api::clear_error();
  return MOE_OK;
}

int moe_draft_step(moe_draft_ctx* ctx, const void* hidden, const int32_t* committed, const int32_t* counts,
                   int32_t R, int32_t B, int32_t K, int32_t* drafts, void* states, void* hip_stream) {
  const int r = step_impl(ctx, hidden, committed, counts, R, B, K, drafts, states, hip_stream);
  if (ctx) clear_hooks(ctx);
  return r;
}

int moe_draft_graph_create(moe_draft_ctx* ctx, const void* hidden, const int32_t* committed, const int32_t* counts,
                           int32_t R, int32_t B, int32_t K, int32_t* drafts, void* states, void* hip_stream,
                           moe_verify_graph** out) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  if (!ctx) return fail(MOE_EINVAL, "draft ctx is NULL");
  for (int i = 0; i < MOE_STAGE_COUNT; ++i)
    if (ctx->ev_before[i] || ctx->ev_after[i]) return fail(MOE_EINVAL, "a timing hook is set; clear it first");
  return moe::api::capture_graph(
      hip_stream,
      [&]() { return step_impl(ctx, hidden, committed, counts, R, B, K, drafts, states, hip_stream); }, out);
}

int moe_draft_set_stage_events(moe_draft_ctx* ctx, int32_t stage, void* before, void* after) {
  if (!ctx) return fail(MOE_EINVAL, "draft ctx is NULL");
  if (stage < 0 || stage >= MOE_STAGE_COUNT) return fail(MOE_EINVAL, "stage out of range");
  ctx->ev_before[stage] = static_cast<hipEvent_t>(before);
  ctx->ev_after[stage] = static_cast<hipEvent_t>(after);
  return MOE_OK;
}

void moe_draft_destroy(moe_draft_ctx* ctx) { draft_free(ctx); }

}  // extern "C"
