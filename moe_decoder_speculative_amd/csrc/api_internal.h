// Internals shared by the C ABI sources (api.cpp: verify step; api_draft.cpp:
// draft head): the verify context, error reporting and argument checks.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <functional>
#include <string>
#include <vector>

#include "kernels.h"
#include "moe_verify.h"

namespace moe {
namespace api {

// Device workspace of a verify step or block: the context's own (allocated
// by moe_verify_init for max(max_tokens, max_prefill_tokens) rows), or one
// carved out of the library's static scratch array for a call that may not
// allocate.
struct Workspace {
  int64_t tw = 0;           // token capacity
  char* xres = nullptr;     // [tw][H] storage
  char* xhat = nullptr;     // [tw+1][H] storage (row tw all zero)
  int* idx[2] = {nullptr, nullptr};   // [tw][k]
  float* w[2] = {nullptr, nullptr};   // [tw][k]
  int* cnt = nullptr;       // [E]
  int* off = nullptr;       // [E+1]
  int* perm = nullptr;      // [tw*k]
  int* active = nullptr;    // [E]
  int* n_active = nullptr;  // [1]
  int4* desc = nullptr;     // [E] routed slot descriptors
  char* act = nullptr;      // [tw*(k+S)+1][I] storage (last row all zero)
  float* y = nullptr;       // [tw*(k+S)][H]
  unsigned long long* keys = nullptr;  // [kKeySlots][tw], zero between steps
  int4* tiles = nullptr;    // grouped-GEMM tile table (contexts with the GEMM path)
  int* n_tiles = nullptr;
};

}  // namespace api
}  // namespace moe

struct moe_verify_ctx {
  moe_verify_config cfg;
  moe::Dims d;
  int device = 0;
  size_t esize = 0;         // bytes per stored element
  std::vector<void*> allocs;

  // repacked weights
  char* router = nullptr;   // bf16 tiled [L][64/16][H/32][512]; f32 [L][E][H]
  char* gate = nullptr;     // [L][E+S] experts (tiled or row-major)
  char* up = nullptr;
  char* down = nullptr;
  char* gamma = nullptr;    // [L][H] storage
  char* final_gamma = nullptr;
  char* lm = nullptr;       // bf16 tiled [Vpad/16][H/32][512]; f32 [V][H]
  size_t router_layer = 0, gate_layer = 0, down_layer = 0;

  moe::api::Workspace ws;   // workspace of moe_verify_step and friends

  // attention (cfg.n_heads > 0)
  moe::Dims dq{}, dout{};              // q/k/v projection (3 slots), output projection (1 slot)
  char* attn_gamma = nullptr;          // [L][H]
  char* wqkv = nullptr;                // tiled [L][3][H/16][H/32][512]
  char* wo = nullptr;                  // tiled [L][1][H/16][H/32][512]
  float* inv_freq = nullptr;           // [64]
  char* kcache = nullptr;              // [L][max_seqs][nh][P][128]
  char* vcache = nullptr;
  char* xattn = nullptr;               // [tw][H] attention sublayer output
  char* qbuf = nullptr;                // [tw][H] rotated queries
  char* actx = nullptr;                // [tw][H] attention output before W_o
  float* apart = nullptr;              // attention partials
  int* zero = nullptr;                 // a device 0 (no routed experts in the projections)

  bool gemm_ok = false;                // LDS allows the prefill grouped GEMM

  // one-call timing hooks (moe_verify_set_stage_events)
  hipEvent_t ev_before[MOE_STAGE_COUNT] = {};
  hipEvent_t ev_after[MOE_STAGE_COUNT] = {};
};

// An instantiated HIP graph of one captured call (verify step or draft call).
struct moe_verify_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

namespace moe {
namespace api {

// Record `msg` as the calling thread's last error and return `code`.
int fail(int code, const std::string& msg);
void clear_error();
const char* last_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// NULL (an error when required) or 16-byte aligned.
int check_ptr(const void* p, const char* name, bool required);

inline hipError_t mark(hipEvent_t ev, hipStream_t s) { return ev ? hipEventRecord(ev, s) : hipSuccess; }

// hipMalloc recorded in `allocs` (freed by the owner); MOE_ENOMEM on failure.
int dev_alloc(std::vector<void*>& allocs, size_t bytes, char** out);

// Capture what `enqueue` launches on `hip_stream` (not the default stream)
// into an instantiated graph; *out is NULL on failure.
int capture_graph(void* hip_stream, const std::function<int()>& enqueue, moe_verify_graph** out);

// Synchronise `device` and free every allocation in `allocs`.
void dev_free_all(std::vector<void*>& allocs, int device);

// A verify step (no attention, no aux outputs) on workspace W.
int verify_step_with(moe_verify_ctx* c, const Workspace& W, const void* hidden, const int32_t* drafts, int32_t B,
                     int32_t K, int32_t* committed, int32_t* counts, void* stream);

// Look up, once per device, the device address of the static scratch array
// behind moe_verify_step_static; `device` must be current.
int static_scratch_setup(int device);

}  // namespace api
}  // namespace moe

#define MOE_HIP(expr)                                                                                  \
  do {                                                                                                 \
    hipError_t e_ = (expr);                                                                            \
    if (e_ != hipSuccess) return ::moe::api::fail(MOE_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)
