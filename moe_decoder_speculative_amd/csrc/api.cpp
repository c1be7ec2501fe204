// C ABI of the MoE speculative verification library (declared in
// include/moe_verify.h): argument validation, context creation with weight
// repacking, workspace, and the launch sequence of one verification step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <new>
#include <string>
#include <vector>

#include "api_internal.h"
#include "kernels.h"
#include "moe_verify.h"

using moe::bf16_t;

namespace moe {
int lmhead_row_multiple();
}

namespace moe {
namespace api {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

void clear_error() { g_last_error.clear(); }
const char* last_error() { return g_last_error.c_str(); }

int check_ptr(const void* p, const char* name, bool required) {
  if (!p) return required ? fail(MOE_EINVAL, std::string(name) + " is NULL") : MOE_OK;
  if (!aligned16(p)) return fail(MOE_EINVAL, std::string(name) + " is not 16-byte aligned");
  return MOE_OK;
}

int dev_alloc(std::vector<void*>& allocs, size_t bytes, char** out) {
  void* p = nullptr;
  if (bytes == 0) bytes = 16;
  if (std::getenv("MOE_VERIFY_FAULT") && std::strcmp(std::getenv("MOE_VERIFY_FAULT"), "alloc") == 0)
    return fail(MOE_ENOMEM, "device allocation failed (injected by MOE_VERIFY_FAULT=alloc)");
  const hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ENOMEM, "hipMalloc of " + std::to_string(bytes) + " bytes failed: " + hipGetErrorString(e));
  }
  allocs.push_back(p);
  *out = static_cast<char*>(p);
  return MOE_OK;
}

int capture_graph(void* hip_stream, const std::function<int()>& enqueue, moe_verify_graph** out) {
  *out = nullptr;
  if (!hip_stream) return fail(MOE_EINVAL, "capture needs a stream other than the default stream");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const hipError_t eb = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (eb != hipSuccess) return fail(MOE_EHIP, std::string("hipStreamBeginCapture: ") + hipGetErrorString(eb));
  const int r = enqueue();
  hipGraph_t graph = nullptr;
  const hipError_t e = hipStreamEndCapture(s, &graph);
  if (r != MOE_OK || e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return r != MOE_OK ? r : fail(MOE_EHIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (ei != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return fail(MOE_EHIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(ei));
  }
  moe_verify_graph* g = new (std::nothrow) moe_verify_graph;
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return fail(MOE_ENOMEM, "graph handle");
  }
  g->graph = graph;
  g->exec = exec;
  *out = g;
  return MOE_OK;
}

void dev_free_all(std::vector<void*>& allocs, int device) {
  if (allocs.empty()) return;
  int cur = 0;
  if (hipGetDevice(&cur) == hipSuccess && cur != device) (void)hipSetDevice(device);
  (void)hipDeviceSynchronize();
  for (void* p : allocs) (void)hipFree(p);
  allocs.clear();
  if (cur != device) (void)hipSetDevice(cur);
}

}  // namespace api
}  // namespace moe

namespace {

using moe::api::aligned16;
using moe::api::check_ptr;
using moe::api::fail;
using moe::api::mark;

// Token rows from which a block's experts run as grouped GEMMs on LDS-staged
// MFMA tiles instead of the weight-streaming decode kernels.
constexpr int kGemmMinTokens = 512;

void clear_hooks(moe_verify_ctx* c) {
  for (int i = 0; i < MOE_STAGE_COUNT; ++i) c->ev_before[i] = c->ev_after[i] = nullptr;
}

int validate_config(const moe_verify_config& c) {
  auto bad = [](const std::string& m) { return fail(MOE_EINVAL, "config: " + m); };
  if (c.dtype != MOE_DTYPE_F32 && c.dtype != MOE_DTYPE_BF16) return bad("dtype must be 0 (f32) or 1 (bf16)");
  if (c.hidden < 128 || c.hidden % 128 != 0) return bad("hidden must be a multiple of 128");
  if (c.dtype == MOE_DTYPE_BF16 && c.hidden > 1536) return bad("hidden must be at most 1536 for bf16");
  if (c.dtype == MOE_DTYPE_F32 && c.hidden > 768) return bad("hidden must be at most 768 for f32");
  if (c.inter < 128 || c.inter > 2048 || c.inter % 128 != 0) return bad("inter must be a multiple of 128 in [128, 2048]");
  if (c.n_routed < 1 || c.n_routed > 64) return bad("n_routed must be in [1, 64]");
  if (c.top_k < 1 || c.top_k > 8 || c.top_k > c.n_routed) return bad("top_k must be in [1, min(n_routed, 8)]");
  if (c.n_shared < 0 || c.n_shared > 4) return bad("n_shared must be in [0, 4]");
  if (c.n_layers < 1 || c.n_layers > 64) return bad("n_layers must be in [1, 64]");
  if (c.max_tokens < 1 || c.max_tokens > 65536) return bad("max_tokens must be in [1, 65536]");
  if (c.max_prefill_tokens < 0 || c.max_prefill_tokens > 65536) return bad("max_prefill_tokens must be in [0, 65536]");
  if (c.k_max < 0 || c.k_max > 7) return bad("k_max must be in [0, 7]");
  if (!(c.rms_eps > 0.0f) || !std::isfinite(c.rms_eps)) return bad("rms_eps must be a positive finite number");
  if (c.has_lm_head != 0 && c.has_lm_head != 1) return bad("has_lm_head must be 0 or 1");
  if (c.has_lm_head && (c.vocab < 1 || c.vocab > (1 << 24))) return bad("vocab must be in [1, 2^24]");
  if (c.n_heads < 0) return bad("n_heads must be >= 0");
  if (c.n_heads > 0) {
    if (c.dtype != MOE_DTYPE_BF16) return fail(MOE_EUNSUPPORTED, "config: attention needs bfloat16 storage");
    if (c.hidden != c.n_heads * moe::kHeadDim) return bad("hidden must be 128 * n_heads");
    if (c.max_positions < 8 || c.max_positions > 32768) return bad("max_positions must be in [8, 32768]");
    if (c.max_seqs < 1 || c.max_seqs > 1024) return bad("max_seqs must be in [1, 1024]");
    if (!(c.rope_theta > 0.0f) || !std::isfinite(c.rope_theta)) return bad("rope_theta must be a positive finite number");
  }
  return MOE_OK;
}

int validate_weights(const moe_verify_config& c, const moe_verify_weights& w) {
  struct Item { const void* p; const char* name; bool required; };
  const Item items[] = {
      {w.router, "router", true},      {w.w_gate, "w_gate", true},    {w.w_up, "w_up", true},
      {w.w_down, "w_down", true},      {w.s_gate, "s_gate", c.n_shared > 0},
      {w.s_up, "s_up", c.n_shared > 0}, {w.s_down, "s_down", c.n_shared > 0},
      {w.norm_gamma, "norm_gamma", true}, {w.final_gamma, "final_gamma", c.has_lm_head != 0},
      {w.lm_head, "lm_head", c.has_lm_head != 0},
      {w.attn_gamma, "attn_gamma", c.n_heads > 0}, {w.w_q, "w_q", c.n_heads > 0},
      {w.w_k, "w_k", c.n_heads > 0},   {w.w_v, "w_v", c.n_heads > 0}, {w.w_o, "w_o", c.n_heads > 0},
  };
  for (const Item& it : items) {
    if (!it.required) continue;
    if (!it.p) return fail(MOE_EINVAL, std::string("weights: ") + it.name + " is NULL");
    if (!aligned16(it.p)) return fail(MOE_EINVAL, std::string("weights: ") + it.name + " is not 16-byte aligned");
  }
  return MOE_OK;
}

int check_aux(const moe_verify_aux* a) {
  if (!a) return MOE_OK;
  int r;
  if ((r = check_ptr(a->topk_idx, "aux.topk_idx", false))) return r;
  if ((r = check_ptr(a->topk_w, "aux.topk_w", false))) return r;
  if ((r = check_ptr(a->expert_count, "aux.expert_count", false))) return r;
  if ((r = check_ptr(a->expert_offset, "aux.expert_offset", false))) return r;
  if ((r = check_ptr(a->perm, "aux.perm", false))) return r;
  if ((r = check_ptr(a->moe_out, "aux.moe_out", false))) return r;
  if ((r = check_ptr(a->hidden_out, "aux.hidden_out", false))) return r;
  if ((r = check_ptr(a->tstar, "aux.tstar", false))) return r;
  if ((r = check_ptr(a->attn_out, "aux.attn_out", false))) return r;
  return MOE_OK;
}

int ctx_alloc(moe_verify_ctx* c, size_t bytes, char** out) { return moe::api::dev_alloc(c->allocs, bytes, out); }

template <typename P>
int ctx_alloc_t(moe_verify_ctx* c, size_t bytes, P** out) {
  char* p = nullptr;
  const int r = ctx_alloc(c, bytes, &p);
  *out = reinterpret_cast<P*>(p);
  return r;
}

void ctx_free(moe_verify_ctx* c) {
  if (!c) return;
  moe::api::dev_free_all(c->allocs, c->device);
  delete c;
}

// Repack the weights into the context.
int repack(moe_verify_ctx* c, const moe_verify_weights& w, hipStream_t s) {
  const moe_verify_config& g = c->cfg;
  const int64_t L = g.n_layers, E = g.n_routed, S = g.n_shared, H = g.hidden, I = g.inter;
  const size_t es = c->esize;
  if (g.dtype == MOE_DTYPE_BF16) {
    for (int64_t l = 0; l < L; ++l) {
      const bf16_t* r = static_cast<const bf16_t*>(w.router) + l * E * H;
      MOE_HIP(moe::launch_tile_bf16(r, 0, reinterpret_cast<bf16_t*>(c->router + l * c->router_layer), 1, (int)E, (int)H, 64, s));
      struct Pair { const void* routed; const void* shared; char* dst; size_t layer; int R, C; };
      const Pair ps[] = {{w.w_gate, w.s_gate, c->gate, c->gate_layer, (int)I, (int)H},
                         {w.w_up, w.s_up, c->up, c->gate_layer, (int)I, (int)H},
                         {w.w_down, w.s_down, c->down, c->down_layer, (int)H, (int)I}};
      for (const Pair& p : ps) {
        const int64_t mat = static_cast<int64_t>(p.R) * p.C;
        bf16_t* dst = reinterpret_cast<bf16_t*>(p.dst + l * p.layer);
        MOE_HIP(moe::launch_tile_bf16(static_cast<const bf16_t*>(p.routed) + l * E * mat, mat, dst, E, p.R, p.C, p.R, s));
        if (S > 0)
          MOE_HIP(moe::launch_tile_bf16(static_cast<const bf16_t*>(p.shared) + l * S * mat, mat, dst + E * mat, S, p.R,
                                        p.C, p.R, s));
      }
    }
    if (g.has_lm_head)
      MOE_HIP(moe::launch_tile_bf16(static_cast<const bf16_t*>(w.lm_head), 0, reinterpret_cast<bf16_t*>(c->lm), 1,
                                    g.vocab, (int)H, c->d.Vpad, s));
  } else {
    MOE_HIP(hipMemcpyAsync(c->router, w.router, L * E * H * es, hipMemcpyDeviceToDevice, s));
    struct Pair { const void* routed; const void* shared; char* dst; int64_t mat; };
    const Pair ps[] = {{w.w_gate, w.s_gate, c->gate, I * H}, {w.w_up, w.s_up, c->up, I * H},
                       {w.w_down, w.s_down, c->down, H * I}};
    for (const Pair& p : ps)
      for (int64_t l = 0; l < L; ++l) {
        char* dst = p.dst + l * (E + S) * p.mat * es;
        MOE_HIP(hipMemcpyAsync(dst, static_cast<const char*>(p.routed) + l * E * p.mat * es, E * p.mat * es,
                               hipMemcpyDeviceToDevice, s));
        if (S > 0)
          MOE_HIP(hipMemcpyAsync(dst + E * p.mat * es, static_cast<const char*>(p.shared) + l * S * p.mat * es,
                                 S * p.mat * es, hipMemcpyDeviceToDevice, s));
      }
    if (g.has_lm_head)
      MOE_HIP(hipMemcpyAsync(c->lm, w.lm_head, static_cast<size_t>(g.vocab) * H * es, hipMemcpyDeviceToDevice, s));
  }
  MOE_HIP(hipMemcpyAsync(c->gamma, w.norm_gamma, L * H * es, hipMemcpyDeviceToDevice, s));
  if (g.has_lm_head) MOE_HIP(hipMemcpyAsync(c->final_gamma, w.final_gamma, H * es, hipMemcpyDeviceToDevice, s));
  if (g.n_heads > 0) {
    MOE_HIP(hipMemcpyAsync(c->attn_gamma, w.attn_gamma, L * H * es, hipMemcpyDeviceToDevice, s));
    const void* qkv[3] = {w.w_q, w.w_k, w.w_v};
    for (int64_t l = 0; l < L; ++l) {
      for (int m = 0; m < 3; ++m)
        MOE_HIP(moe::launch_tile_bf16(static_cast<const bf16_t*>(qkv[m]) + l * H * H, 0,
                                      reinterpret_cast<bf16_t*>(c->wqkv) + (l * 3 + m) * H * H, 1, (int)H, (int)H,
                                      (int)H, s));
      MOE_HIP(moe::launch_tile_bf16(static_cast<const bf16_t*>(w.w_o) + l * H * H, 0,
                                    reinterpret_cast<bf16_t*>(c->wo) + l * H * H, 1, (int)H, (int)H, (int)H, s));
    }
    float inv[moe::kHeadDim / 2];
    for (int i = 0; i < moe::kHeadDim / 2; ++i)
      inv[i] = static_cast<float>(std::pow(static_cast<double>(g.rope_theta), -2.0 * i / moe::kHeadDim));
    MOE_HIP(hipMemcpyAsync(c->inv_freq, inv, sizeof(inv), hipMemcpyHostToDevice, s));
    MOE_HIP(hipStreamSynchronize(s));  // `inv` is a host stack array
  }
  return MOE_OK;
}

int create(const moe_verify_config& g, const moe_verify_weights& w, hipStream_t s, moe_verify_ctx* c) {
  c->cfg = g;
  c->esize = g.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  moe::Dims& d = c->d;
  d.H = g.hidden; d.E = g.n_routed; d.k = g.top_k; d.S = g.n_shared; d.I = g.inter;
  d.V = g.has_lm_head ? g.vocab : 0; d.L = g.n_layers; d.eps = g.rms_eps; d.bf16 = g.dtype == MOE_DTYPE_BF16;
  const int mult = moe::lmhead_row_multiple();
  d.Vpad = g.has_lm_head ? (d.bf16 ? (d.V + mult - 1) / mult * mult : d.V) : 0;
  MOE_HIP(hipGetDevice(&c->device));
  int lds = 0;
  MOE_HIP(hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, c->device));
  MOE_HIP(hipDeviceGetAttribute(&d.n_cu, hipDeviceAttributeMultiprocessorCount, c->device));
  if (d.n_cu < 1) d.n_cu = 1;
  c->gemm_ok = d.bf16 && d.H % 256 == 0 && static_cast<size_t>(lds) >= moe::gemm_lds_bytes();
  if (static_cast<size_t>(lds) < moe::norm_router_lds_bytes(d) + 256)
    return fail(MOE_EUNSUPPORTED, "hidden size needs " + std::to_string(moe::norm_router_lds_bytes(d)) +
                                      " bytes of LDS per workgroup; the device offers " + std::to_string(lds));

  const int64_t L = g.n_layers, E = g.n_routed, S = g.n_shared, H = g.hidden, I = g.inter;
  const size_t es = c->esize;
  c->router_layer = (d.bf16 ? 64 : E) * H * es;
  c->gate_layer = (E + S) * I * H * es;
  c->down_layer = (E + S) * H * I * es;
  int r;
  if ((r = ctx_alloc(c, L * c->router_layer, &c->router))) return r;
  if ((r = ctx_alloc(c, L * c->gate_layer, &c->gate))) return r;
  if ((r = ctx_alloc(c, L * c->gate_layer, &c->up))) return r;
  if ((r = ctx_alloc(c, L * c->down_layer, &c->down))) return r;
  if ((r = ctx_alloc(c, L * H * es, &c->gamma))) return r;
  if (g.has_lm_head) {
    if ((r = ctx_alloc(c, H * es, &c->final_gamma))) return r;
    if ((r = ctx_alloc(c, static_cast<size_t>(d.Vpad) * H * es, &c->lm))) return r;
    if (d.bf16) MOE_HIP(hipMemsetAsync(c->lm, 0, static_cast<size_t>(d.Vpad) * H * es, s));
  }

  const int64_t tw = std::max<int64_t>(g.max_tokens, g.max_prefill_tokens);
  c->ws.tw = tw;
  const int64_t rows = tw * (g.top_k + S);
  if ((r = ctx_alloc(c, tw * H * es, &c->ws.xres))) return r;
  // one extra all-zero row past the end of xhat and act: padding lanes of the
  // grouped GEMM read it instead of branching
  if ((r = ctx_alloc(c, (tw + 1) * H * es, &c->ws.xhat))) return r;
  MOE_HIP(hipMemsetAsync(c->ws.xhat + tw * H * es, 0, H * es, s));
  for (int i = 0; i < 2; ++i) {
    if ((r = ctx_alloc_t(c, tw * g.top_k * sizeof(int), &c->ws.idx[i]))) return r;
    if ((r = ctx_alloc_t(c, tw * g.top_k * sizeof(float), &c->ws.w[i]))) return r;
  }
  if ((r = ctx_alloc_t(c, E * sizeof(int), &c->ws.cnt))) return r;
  if ((r = ctx_alloc_t(c, (E + 1) * sizeof(int), &c->ws.off))) return r;
  if ((r = ctx_alloc_t(c, tw * g.top_k * sizeof(int), &c->ws.perm))) return r;
  if ((r = ctx_alloc_t(c, E * sizeof(int), &c->ws.active))) return r;
  if ((r = ctx_alloc_t(c, 16, &c->ws.n_active))) return r;
  if ((r = ctx_alloc_t(c, E * sizeof(int4), &c->ws.desc))) return r;
  // pair rows (decode kernels) plus an all-zero row, or the grouped GEMM's
  // tiled rows, whichever is larger
  const int64_t act_rows = std::max<int64_t>(rows + 1, c->gemm_ok ? moe::gemm_act_rows(d, static_cast<int>(tw)) : 0);
  if ((r = ctx_alloc(c, act_rows * I * es, &c->ws.act))) return r;
  MOE_HIP(hipMemsetAsync(c->ws.act + rows * I * es, 0, I * es, s));
  if ((r = ctx_alloc_t(c, rows * H * sizeof(float), &c->ws.y))) return r;
  if ((r = ctx_alloc_t(c, moe::kKeySlots * tw * sizeof(unsigned long long), &c->ws.keys))) return r;
  if ((r = ctx_alloc_t(c, static_cast<size_t>(moe::gemm_max_tiles(d, static_cast<int>(tw))) * sizeof(int4), &c->ws.tiles)))
    return r;
  if ((r = ctx_alloc_t(c, 16, &c->ws.n_tiles))) return r;

  if (g.n_heads > 0) {
    d.L = g.n_layers;
    c->dq = d;
    c->dq.E = 0;
    c->dq.k = 0;
    c->dq.S = 3;
    c->dq.I = g.hidden;
    c->dout = c->dq;
    c->dout.S = 1;
    const size_t cache = static_cast<size_t>(L) * g.max_seqs * g.n_heads * g.max_positions * moe::kHeadDim * 2;
    const int G = 64;
    if ((r = ctx_alloc(c, L * H * es, &c->attn_gamma))) return r;
    if ((r = ctx_alloc(c, L * 3 * H * H * es, &c->wqkv))) return r;
    if ((r = ctx_alloc(c, L * H * H * es, &c->wo))) return r;
    if ((r = ctx_alloc_t(c, 64 * sizeof(float), &c->inv_freq))) return r;
    if ((r = ctx_alloc(c, cache, &c->kcache))) return r;
    if ((r = ctx_alloc(c, cache, &c->vcache))) return r;
    MOE_HIP(hipMemsetAsync(c->kcache, 0, cache, s));
    MOE_HIP(hipMemsetAsync(c->vcache, 0, cache, s));
    if ((r = ctx_alloc(c, g.max_tokens * H * es, &c->xattn))) return r;
    if ((r = ctx_alloc(c, g.max_tokens * H * es, &c->qbuf))) return r;
    if ((r = ctx_alloc(c, g.max_tokens * H * es, &c->actx))) return r;
    if ((r = ctx_alloc_t(c, moe::attn_part_floats(g.max_tokens, g.n_heads, G) * sizeof(float), &c->apart))) return r;
    if ((r = ctx_alloc_t(c, 16, &c->zero))) return r;
    MOE_HIP(hipMemsetAsync(c->zero, 0, 16, s));
  }

  // arg-max keys are zero between steps (the acceptance clears them after use)
  MOE_HIP(hipMemsetAsync(c->ws.keys, 0, moe::kKeySlots * tw * sizeof(unsigned long long), s));

  if ((r = repack(c, w, s))) return r;
  MOE_HIP(hipStreamSynchronize(s));
  return MOE_OK;
}

// The blocks of a step: for layer l, norm+router (with the combine of layer
// l-1 when l > 0), permutation, expert up, expert down.
// The attention sublayer of layer l (verify steps of a context with
// attention): pre-attention RMSNorm (after the combine of the previous
// layer's MoE block when li > 0), q/k/v projection with the rotary embedding
// and the cache writes, decode attention, output projection with the
// residual add into xattn.
int run_attention(moe_verify_ctx* c, const moe::api::Workspace& W, const void* x_prev, int li, int l, int T, int B, int K1, const int* positions,
                  const moe_verify_aux* aux, hipStream_t s) {
  const moe::Dims& d = c->d;
  const moe_verify_config& g = c->cfg;
  const int64_t H = g.hidden, k = g.top_k;
  const size_t es = c->esize;
  moe::NormRouterParams an{};
  an.x_in = x_prev;
  if (li > 0) {  // finish the previous layer's MoE block into xres
    an.x_out = W.xres;
    an.y = W.y;
    an.prev_idx = aux && aux->topk_idx ? aux->topk_idx + (li - 1) * T * k : W.idx[(li - 1) & 1];
    an.prev_w = aux && aux->topk_w ? aux->topk_w + (li - 1) * T * k : W.w[(li - 1) & 1];
    an.m_out = aux && aux->moe_out ? aux->moe_out + (li - 1) * T * H : nullptr;
    an.combine = 1;
  }
  an.gamma = c->attn_gamma + l * H * es;
  an.xhat = W.xhat;
  an.T = T;
  an.norm = 1;
  an.route = 0;
  MOE_HIP(moe::launch_norm_router(d, an, s));
  const void* x_res = li > 0 ? W.xres : x_prev;

  const size_t cache_layer = static_cast<size_t>(g.max_seqs) * g.n_heads * g.max_positions * moe::kHeadDim;
  bf16_t* kc = reinterpret_cast<bf16_t*>(c->kcache) + l * cache_layer;
  bf16_t* vc = reinterpret_cast<bf16_t*>(c->vcache) + l * cache_layer;
  moe::ExpertParams qe{};
  qe.n_active = c->zero;
  qe.w_down = c->wqkv + l * 3 * H * H * es;
  qe.act = W.xhat;
  qe.T = T;
  moe::EpiParams qp{};
  qp.positions = positions;
  qp.K1 = K1;
  qp.P = g.max_positions;
  qp.nh = g.n_heads;
  qp.inv_freq = c->inv_freq;
  qp.q = reinterpret_cast<bf16_t*>(c->qbuf);
  qp.kc = kc;
  qp.vc = vc;
  MOE_HIP(moe::launch_linear_qkv(c->dq, qe, qp, s));

  moe::AttnParams ap{};
  ap.q = reinterpret_cast<const bf16_t*>(c->qbuf);
  ap.kc = kc;
  ap.vc = vc;
  ap.positions = positions;
  ap.B = B;
  ap.K1 = K1;
  ap.nh = g.n_heads;
  ap.P = g.max_positions;
  ap.G = moe::attn_groups(d, B, g.n_heads);
  ap.part = c->apart;
  ap.ctx = reinterpret_cast<bf16_t*>(c->actx);
  if (li == 0) MOE_HIP(mark(c->ev_before[MOE_STAGE_ATTENTION], s));
  MOE_HIP(moe::launch_attention_split(d, ap, s));
  if (li == 0) MOE_HIP(mark(c->ev_after[MOE_STAGE_ATTENTION], s));
  MOE_HIP(moe::launch_attention_combine(ap, s));

  moe::ExpertParams oe{};
  oe.n_active = c->zero;
  oe.w_down = c->wo + l * H * H * es;
  oe.act = c->actx;
  oe.T = T;
  moe::EpiParams op{};
  op.x_in = static_cast<const bf16_t*>(x_res);
  op.x_out = aux && aux->attn_out ? static_cast<bf16_t*>(aux->attn_out) + li * T * H
                                  : reinterpret_cast<bf16_t*>(c->xattn);
  MOE_HIP(moe::launch_linear_resid(c->dout, oe, op, s));
  return MOE_OK;
}

// True when a block over T rows runs its experts as grouped GEMMs.
bool use_gemm(const moe_verify_ctx* c, int T) { return c->gemm_ok && T >= kGemmMinTokens; }

// bf16_rows: the grouped GEMM writes bf16 gate-weighted expert rows (a
// prefill block, combined by launch_combine_bf16) instead of fp32 rows.
int run_blocks(moe_verify_ctx* c, const moe::api::Workspace& W, const void* hidden, int T, const moe_verify_aux* aux, int layer0, int nlayers,
               hipStream_t s, const void** x_last, const int* positions = nullptr, int B = 0, int K1 = 0,
               bool bf16_rows = false) {
  const moe::Dims& d = c->d;
  const moe_verify_config& g = c->cfg;
  const int64_t H = g.hidden, k = g.top_k, E = g.n_routed;
  const bool attn = positions != nullptr;
  const void* x_prev = hidden;  // residual stream entering the previous block
  for (int li = 0; li < nlayers; ++li) {
    const int l = layer0 + li;
    int* idx = aux && aux->topk_idx ? aux->topk_idx + li * T * k : W.idx[li & 1];
    float* wg = aux && aux->topk_w ? aux->topk_w + li * T * k : W.w[li & 1];
    moe::NormRouterParams nr{};
    if (attn) {
      int r;
      if ((r = run_attention(c, W, x_prev, li, l, T, B, K1, positions, aux, s))) return r;
      // the MoE block takes the attention sublayer's output
      x_prev = aux && aux->attn_out ? static_cast<const char*>(aux->attn_out) + li * T * H * c->esize
                                    : static_cast<const char*>(c->xattn);
      nr.x_in = x_prev;
    } else if (li == 0) {
      nr.x_in = hidden;
    } else {
      nr.x_in = x_prev;
      nr.x_out = W.xres;
      nr.y = W.y;
      nr.prev_idx = aux && aux->topk_idx ? aux->topk_idx + (li - 1) * T * k : W.idx[(li - 1) & 1];
      nr.prev_w = aux && aux->topk_w ? aux->topk_w + (li - 1) * T * k : W.w[(li - 1) & 1];
      nr.m_out = aux && aux->moe_out ? aux->moe_out + (li - 1) * T * H : nullptr;
      nr.combine = 1;
      x_prev = W.xres;
    }
    nr.gamma = c->gamma + l * H * c->esize;
    nr.router = c->router + l * c->router_layer;
    nr.xhat = W.xhat;
    nr.idx_out = idx;
    nr.w_out = wg;
    nr.T = T;
    nr.norm = 1;
    nr.route = 1;
    moe::PermuteParams pp{};
    pp.idx = idx;
    pp.P = T * static_cast<int>(k);
    pp.cnt = aux && aux->expert_count ? aux->expert_count + li * E : W.cnt;
    pp.off = aux && aux->expert_offset ? aux->expert_offset + li * (E + 1) : W.off;
    pp.perm = aux && aux->perm ? aux->perm + li * T * k : W.perm;
    pp.active = W.active;
    pp.n_active = W.n_active;
    pp.desc = W.desc;
    const bool fused_sort = T <= moe::norm_router_sort_limit();
    if (fused_sort) {
      // the (single) norm/router workgroup sorts the pairs
      nr.sort = moe::SortParams{idx, pp.cnt, pp.off, pp.perm, pp.active, pp.n_active, pp.desc, 1};
    }
    MOE_HIP(moe::launch_norm_router(d, nr, s));
    if (use_gemm(c, T)) {
      // the permutation kernel also builds the grouped GEMM's tile table
      pp.tiles = W.tiles;
      pp.n_tiles = W.n_tiles;
      pp.tile_T = T;
      pp.n_shared = static_cast<int>(g.n_shared);
    }
    if (!fused_sort) MOE_HIP(moe::launch_permute(d, pp, s));

    moe::ExpertParams ep{};
    ep.xhat = W.xhat;
    ep.cnt = pp.cnt;
    ep.off = pp.off;
    ep.perm = pp.perm;
    ep.active = W.active;
    ep.n_active = W.n_active;
    ep.desc = W.desc;
    ep.w_gate = c->gate + l * c->gate_layer;
    ep.w_up = c->up + l * c->gate_layer;
    ep.w_down = c->down + l * c->down_layer;
    ep.act = W.act;
    ep.y = W.y;
    ep.T = T;
    if (use_gemm(c, T)) {
      // prefill-sized: grouped GEMM over (slot, feature tile, token tile) items
      moe::GemmParams gp{};
      gp.xhat = W.xhat;
      gp.w_gate = ep.w_gate;
      gp.w_up = ep.w_up;
      gp.w_down = ep.w_down;
      gp.perm = pp.perm;
      gp.tiles = W.tiles;
      gp.n_tiles = W.n_tiles;
      gp.act = W.act;
      gp.y = W.y;
      gp.T = T;
      gp.xhat_zero_row = static_cast<int>(W.tw);
      gp.yb = bf16_rows ? reinterpret_cast<bf16_t*>(W.y) : nullptr;
      gp.gate_w = wg;
      if (li == 0) MOE_HIP(mark(c->ev_before[MOE_STAGE_EXPERT_UP], s));
      MOE_HIP(moe::launch_grouped_gemm(d, gp, 1, s));
      if (li == 0) MOE_HIP(mark(c->ev_after[MOE_STAGE_EXPERT_UP], s));
      if (li == 0) MOE_HIP(mark(c->ev_before[MOE_STAGE_EXPERT_DOWN], s));
      MOE_HIP(moe::launch_grouped_gemm(d, gp, 0, s));
      if (li == 0) MOE_HIP(mark(c->ev_after[MOE_STAGE_EXPERT_DOWN], s));
      continue;
    }
    if (li == 0) MOE_HIP(mark(c->ev_before[MOE_STAGE_EXPERT_UP], s));
    MOE_HIP(moe::launch_expert_up(d, ep, s));
    if (li == 0) MOE_HIP(mark(c->ev_after[MOE_STAGE_EXPERT_UP], s));
    if (li == 0) MOE_HIP(mark(c->ev_before[MOE_STAGE_EXPERT_DOWN], s));
    MOE_HIP(moe::launch_expert_down(d, ep, s));
    if (li == 0) MOE_HIP(mark(c->ev_after[MOE_STAGE_EXPERT_DOWN], s));
  }
  *x_last = x_prev;
  return MOE_OK;
}

// The context's own workspace (an empty one for a NULL context, which
// step_impl rejects before using it).
const moe::api::Workspace& ws_of(const moe_verify_ctx* c) {
  static const moe::api::Workspace none{};
  return c ? c->ws : none;
}

int step_impl(moe_verify_ctx* c, const moe::api::Workspace& W, const void* hidden, const int32_t* drafts, const int32_t* positions, int32_t B,
              int32_t K, int32_t* committed, int32_t* counts, const moe_verify_aux* aux, void* stream) {
  if (!c) return fail(MOE_EINVAL, "ctx is NULL");
  const moe_verify_config& g = c->cfg;
  if (!g.has_lm_head) return fail(MOE_EINVAL, "context was created without an LM head");
  if (g.n_heads > 0 && !positions) return fail(MOE_EINVAL, "context has attention: use moe_verify_step_kv");
  if (g.n_heads == 0 && positions) return fail(MOE_EINVAL, "context has no attention: use moe_verify_step");
  if (B < 1) return fail(MOE_EINVAL, "B must be >= 1");
  if (K < 0 || K > g.k_max) return fail(MOE_EINVAL, "K must be in [0, k_max]");
  const int64_t T64 = static_cast<int64_t>(B) * (K + 1);
  if (T64 > g.max_tokens) return fail(MOE_EINVAL, "B*(K+1) exceeds max_tokens");
  if (positions && B > g.max_seqs) return fail(MOE_EINVAL, "B exceeds max_seqs");
  if (positions && K + 1 > g.max_positions) return fail(MOE_EINVAL, "K+1 exceeds max_positions");
  int r;
  if ((r = check_ptr(positions, "positions", false))) return r;
  if ((r = check_ptr(hidden, "hidden", true))) return r;
  if ((r = check_ptr(drafts, "drafts", K > 0))) return r;
  if ((r = check_ptr(committed, "committed", true))) return r;
  if ((r = check_ptr(counts, "counts", true))) return r;
  if ((r = check_aux(aux))) return r;
  const int T = static_cast<int>(T64);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe::Dims& d = c->d;

  const void* x_last = nullptr;
  MOE_HIP(mark(c->ev_before[MOE_STAGE_ALL], s));
  if ((r = run_blocks(c, W, hidden, T, aux, 0, g.n_layers, s, &x_last, positions, B, K + 1))) return r;

  const int64_t H = g.hidden, k = g.top_k;
  const int li = g.n_layers - 1;
  moe::LmHeadParams lp{};
  lp.xf = W.xhat;
  lp.lm = c->lm;
  lp.T = T;
  lp.keys = W.keys;
  lp.key_stride = static_cast<int>(W.tw);
  lp.drafts = drafts;
  lp.B = B;
  lp.K = K;
  lp.committed = committed;
  lp.counts = counts;
  lp.tstar = aux ? aux->tstar : nullptr;
  if (d.bf16) {
    // final combine + norm: one workgroup per row
    lp.x_in = x_last;
    lp.y = W.y;
    lp.prev_idx = aux && aux->topk_idx ? aux->topk_idx + li * T * k : W.idx[li & 1];
    lp.prev_w = aux && aux->topk_w ? aux->topk_w + li * T * k : W.w[li & 1];
    lp.gamma = c->final_gamma;
    lp.x_out = aux ? aux->hidden_out : nullptr;
    lp.m_out = aux && aux->moe_out ? aux->moe_out + li * T * H : nullptr;
    lp.xf_out = W.xhat;
    MOE_HIP(moe::launch_final_norm(d, lp, s));
  } else {
    moe::NormRouterParams nr{};
    nr.x_in = x_last;
    nr.x_out = aux && aux->hidden_out ? aux->hidden_out : W.xres;
    nr.y = W.y;
    nr.prev_idx = aux && aux->topk_idx ? aux->topk_idx + li * T * k : W.idx[li & 1];
    nr.prev_w = aux && aux->topk_w ? aux->topk_w + li * T * k : W.w[li & 1];
    nr.m_out = aux && aux->moe_out ? aux->moe_out + li * T * H : nullptr;
    nr.gamma = c->final_gamma;
    nr.xhat = W.xhat;
    nr.T = T;
    nr.combine = 1;
    nr.norm = 1;
    nr.route = 0;
    MOE_HIP(moe::launch_norm_router(d, nr, s));
  }
  MOE_HIP(mark(c->ev_before[MOE_STAGE_LMHEAD], s));
  MOE_HIP(moe::launch_lmhead(d, lp, s));
  MOE_HIP(mark(c->ev_after[MOE_STAGE_LMHEAD], s));
  MOE_HIP(moe::launch_accept(lp, s));
  MOE_HIP(mark(c->ev_after[MOE_STAGE_ALL], s));
  return MOE_OK;
}

}  // namespace

namespace moe {
namespace api {
int verify_step_with(moe_verify_ctx* c, const Workspace& W, const void* hidden, const int32_t* drafts, int32_t B,
                     int32_t K, int32_t* committed, int32_t* counts, void* stream) {
  return step_impl(c, W, hidden, drafts, nullptr, B, K, committed, counts, nullptr, stream);
}
}  // namespace api
}  // namespace moe

extern "C" {

int moe_verify_init(const moe_verify_config* cfg, const moe_verify_weights* weights, void* hip_stream,
                    moe_verify_ctx** out) {
  if (out) *out = nullptr;
  if (!cfg || !weights || !out) return fail(MOE_EINVAL, "cfg, weights and out must be non-NULL");
  int r;
  if ((r = validate_config(*cfg))) return r;
  if ((r = validate_weights(*cfg, *weights))) return r;
  moe_verify_ctx* c = new (std::nothrow) moe_verify_ctx();
  if (!c) return fail(MOE_ENOMEM, "host allocation failed");
  try {
    r = create(*cfg, *weights, static_cast<hipStream_t>(hip_stream), c);
  } catch (...) {
    r = fail(MOE_ENOMEM, "host exception during init");
  }
  // the static scratch of moe_verify_step_static on this device (the
  // context's device is current here)
  if (r == MOE_OK) r = moe::api::static_scratch_setup(c->device);
  if (r != MOE_OK) {
    const std::string keep = moe::api::last_error();
    ctx_free(c);
    fail(r, keep);
    return r;
  }
  *out = c;
  moe::api::clear_error();
  return MOE_OK;
}

int moe_verify_step(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts, int32_t B, int32_t K,
                    int32_t* committed, int32_t* counts, void* hip_stream) {
  const int r = step_impl(ctx, ws_of(ctx), hidden, drafts, nullptr, B, K, committed, counts, nullptr, hip_stream);
  if (ctx) clear_hooks(ctx);
  return r;
}

int moe_verify_step_ex(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts, int32_t B, int32_t K,
                       int32_t* committed, int32_t* counts, const moe_verify_aux* aux, void* hip_stream) {
  const int r = step_impl(ctx, ws_of(ctx), hidden, drafts, nullptr, B, K, committed, counts, aux, hip_stream);
  if (ctx) clear_hooks(ctx);
  return r;
}

int moe_verify_step_kv(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts, const int32_t* positions,
                       int32_t B, int32_t K, int32_t* committed, int32_t* counts, const moe_verify_aux* aux,
                       void* hip_stream) {
  if (!positions) {
    if (ctx) clear_hooks(ctx);
    return fail(MOE_EINVAL, "positions is NULL");
  }
  const int r = step_impl(ctx, ws_of(ctx), hidden, drafts, positions, B, K, committed, counts, aux, hip_stream);
  if (ctx) clear_hooks(ctx);
  return r;
}

int moe_verify_kv_cache(moe_verify_ctx* ctx, void** k_cache, void** v_cache) {
  if (!ctx || !k_cache || !v_cache) return fail(MOE_EINVAL, "ctx, k_cache and v_cache must be non-NULL");
  if (ctx->cfg.n_heads == 0) return fail(MOE_EINVAL, "context has no attention");
  *k_cache = ctx->kcache;
  *v_cache = ctx->vcache;
  return MOE_OK;
}

int moe_verify_graph_create(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts, int32_t B,
                            int32_t K, int32_t* committed, int32_t* counts, void* hip_stream,
                            moe_verify_graph** out) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  if (!ctx) return fail(MOE_EINVAL, "ctx is NULL");
  for (int i = 0; i < MOE_STAGE_COUNT; ++i)
    if (ctx->ev_before[i] || ctx->ev_after[i]) return fail(MOE_EINVAL, "a timing hook is set; clear it first");
  return moe::api::capture_graph(
      hip_stream,
      [&]() { return step_impl(ctx, ws_of(ctx), hidden, drafts, nullptr, B, K, committed, counts, nullptr, hip_stream); },
      out);
}

int moe_verify_graph_create_kv(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts,
                               const int32_t* positions, int32_t B, int32_t K, int32_t* committed, int32_t* counts,
                               void* hip_stream, moe_verify_graph** out) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  if (!ctx) return fail(MOE_EINVAL, "ctx is NULL");
  if (!positions) return fail(MOE_EINVAL, "positions is NULL");
  for (int i = 0; i < MOE_STAGE_COUNT; ++i)
    if (ctx->ev_before[i] || ctx->ev_after[i]) return fail(MOE_EINVAL, "a timing hook is set; clear it first");
  return moe::api::capture_graph(
      hip_stream,
      [&]() { return step_impl(ctx, ws_of(ctx), hidden, drafts, positions, B, K, committed, counts, nullptr, hip_stream); },
      out);
}

int moe_verify_graph_launch(moe_verify_graph* graph, void* hip_stream) {
  if (!graph) return fail(MOE_EINVAL, "graph is NULL");
  MOE_HIP(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(hip_stream)));
  return MOE_OK;
}

void moe_verify_graph_destroy(moe_verify_graph* graph) {
  if (!graph) return;
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipGraphDestroy(graph->graph);
  delete graph;
}

namespace {
int block_impl(moe_verify_ctx* ctx, int32_t layer, const void* x, int32_t T, void* y,
               const moe_verify_aux* aux, void* hip_stream) {
  if (!ctx) return fail(MOE_EINVAL, "ctx is NULL");
  const moe_verify_config& g = ctx->cfg;
  if (layer < 0 || layer >= g.n_layers) return fail(MOE_EINVAL, "layer out of range");
  const int cap = g.max_prefill_tokens > 0 ? g.max_prefill_tokens : g.max_tokens;
  if (T < 1 || T > cap) return fail(MOE_EINVAL, "T must be in [1, max_prefill_tokens]");
  int r;
  if ((r = check_ptr(x, "x", true))) return r;
  if ((r = check_ptr(y, "y", true))) return r;
  if ((r = check_aux(aux))) return r;
  const size_t bytes = static_cast<size_t>(T) * g.hidden * ctx->esize;
  const char* xb = static_cast<const char*>(x);
  const char* yb = static_cast<const char*>(y);
  if (xb < yb + bytes && yb < xb + bytes) return fail(MOE_EINVAL, "x and y overlap");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const void* x_last = nullptr;
  MOE_HIP(mark(ctx->ev_before[MOE_STAGE_ALL], s));
  const bool bf16_rows = use_gemm(ctx, T);
  if ((r = run_blocks(ctx, ctx->ws, x, T, aux, layer, 1, s, &x_last, nullptr, 0, 0, bf16_rows))) return r;
  if (bf16_rows) {
    moe::CombineParams cp{};
    cp.x_in = x;
    cp.x_out = y;
    cp.yb = reinterpret_cast<const bf16_t*>(ctx->ws.y);
    cp.idx = aux && aux->topk_idx ? aux->topk_idx : ctx->ws.idx[0];
    cp.m_out = aux ? aux->moe_out : nullptr;
    cp.T = T;
    MOE_HIP(moe::launch_combine_bf16(ctx->d, cp, s));
    MOE_HIP(mark(ctx->ev_after[MOE_STAGE_ALL], s));
    return MOE_OK;
  }
  moe::NormRouterParams nr{};
  nr.x_in = x;
  nr.x_out = y;
  nr.y = ctx->ws.y;
  nr.prev_idx = aux && aux->topk_idx ? aux->topk_idx : ctx->ws.idx[0];
  nr.prev_w = aux && aux->topk_w ? aux->topk_w : ctx->ws.w[0];
  nr.m_out = aux ? aux->moe_out : nullptr;
  nr.T = T;
  nr.combine = 1;
  MOE_HIP(moe::launch_norm_router(ctx->d, nr, s));
  MOE_HIP(mark(ctx->ev_after[MOE_STAGE_ALL], s));
  return MOE_OK;
}
}  // namespace

int moe_block_forward(moe_verify_ctx* ctx, int32_t layer, const void* x, int32_t T, void* y,
                      const moe_verify_aux* aux, void* hip_stream) {
  const int r = block_impl(ctx, layer, x, T, y, aux, hip_stream);
  if (ctx) clear_hooks(ctx);
  return r;
}

int moe_verify_set_stage_events(moe_verify_ctx* ctx, int32_t stage, void* before, void* after) {
  if (!ctx) return fail(MOE_EINVAL, "ctx is NULL");
  if (stage < 0 || stage >= MOE_STAGE_COUNT) return fail(MOE_EINVAL, "stage out of range");
  ctx->ev_before[stage] = static_cast<hipEvent_t>(before);
  ctx->ev_after[stage] = static_cast<hipEvent_t>(after);
  return MOE_OK;
}

void moe_verify_destroy(moe_verify_ctx* ctx) { ctx_free(ctx); }

const char* moe_verify_last_error(void) { return moe::api::last_error(); }

}  // extern "C"
