// moe_verify_step_static (include/moe_verify.h): the verify step with its
// workspace in a file-scope device array instead of the context's own
// allocation, for callers that cannot allocate device memory.
//
// Every GPU the library runs on holds one copy of `scratch` until the process
// ends.  In host code the array's name is only a host-side handle: its device
// address comes from hipGetSymbolAddress, looked up once per device with that
// device current (moe_verify_init does it for the context's device) and kept
// in g_scratch; kernels get that address, never the name.  All calls on one
// device share the array, so calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "api_internal.h"
#include "kernels.h"
#include "moe_verify.h"

namespace {

constexpr size_t kScratchBytes = size_t{MOE_STATIC_SCRATCH_BYTES};
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
char* g_scratch[kMaxDevices] = {};

// The arg-max keys of a step start at zero: a previous call on this device
// may have left any bytes there (another context lays the array out for its
// own sizes).  A kernel, not a memset, so the call can be captured in a graph.
__global__ __launch_bounds__(256) void k_zero_u64(unsigned long long* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

size_t align_up(size_t v) { return (v + 255) & ~size_t{255}; }

// Carve a step's workspace for T rows out of the array at `base`; returns the
// bytes it needs (nothing is written when that exceeds the array).
size_t carve(const moe_verify_ctx* c, int64_t T, char* base, moe::api::Workspace* W) {
  const moe_verify_config& g = c->cfg;
  const int64_t H = g.hidden, I = g.inter, k = g.top_k, S = g.n_shared, E = g.n_routed;
  const size_t es = c->esize;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    char* p = base + at;
    at = align_up(at + bytes);
    return p;
  };
  W->tw = T;
  W->keys = reinterpret_cast<unsigned long long*>(take(moe::kKeySlots * T * sizeof(unsigned long long)));
  W->xres = take(T * H * es);
  W->xhat = take((T + 1) * H * es);
  for (int i = 0; i < 2; ++i) {
    W->idx[i] = reinterpret_cast<int*>(take(T * k * sizeof(int)));
    W->w[i] = reinterpret_cast<float*>(take(T * k * sizeof(float)));
  }
  W->cnt = reinterpret_cast<int*>(take(E * sizeof(int)));
  W->off = reinterpret_cast<int*>(take((E + 1) * sizeof(int)));
  W->perm = reinterpret_cast<int*>(take(T * k * sizeof(int)));
  W->active = reinterpret_cast<int*>(take(E * sizeof(int)));
  W->n_active = reinterpret_cast<int*>(take(16));
  W->desc = reinterpret_cast<int4*>(take(E * sizeof(int4)));
  W->act = take((T * (k + S) + 1) * I * es);
  W->y = reinterpret_cast<float*>(take(T * (k + S) * H * sizeof(float)));
  W->tiles = nullptr;  // the grouped-GEMM path is not taken at these sizes
  W->n_tiles = nullptr;
  return at;
}

}  // namespace

namespace moe {
namespace api {

int static_scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return fail(MOE_EUNSUPPORTED, "device index beyond the static scratch table");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[device]) return MOE_OK;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    (void)hipGetLastError();
    return fail(MOE_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  }
  g_scratch[device] = static_cast<char*>(ptr);
  return MOE_OK;
}

}  // namespace api
}  // namespace moe

extern "C" int moe_verify_step_static(moe_verify_ctx* ctx, const void* hidden, const int32_t* drafts, int32_t B,
                                      int32_t K, int32_t* committed, int32_t* counts, void* hip_stream) {
  using moe::api::fail;
  if (!ctx) return fail(MOE_EINVAL, "ctx is NULL");
  if (ctx->cfg.n_heads > 0) return fail(MOE_EINVAL, "context has attention: moe_verify_step_static has no KV cache");
  if (B < 1) return fail(MOE_EINVAL, "B must be >= 1");
  if (K < 0 || K > ctx->cfg.k_max) return fail(MOE_EINVAL, "K must be in [0, k_max]");
  const int64_t T = static_cast<int64_t>(B) * (K + 1);
  if (T > MOE_STATIC_MAX_TOKENS) return fail(MOE_EINVAL, "B*(K+1) exceeds MOE_STATIC_MAX_TOKENS");
  moe::api::Workspace W;
  const size_t need = carve(ctx, T, nullptr, &W);
  if (need > kScratchBytes)
    return fail(MOE_EINVAL, "the step needs " + std::to_string(need) + " bytes of workspace; the static scratch holds " +
                                std::to_string(kScratchBytes));
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != ctx->device)
    return fail(MOE_EINVAL, "the context's device must be current");
  int r = moe::api::static_scratch_setup(ctx->device);
  if (r != MOE_OK) return r;
  carve(ctx, T, g_scratch[ctx->device], &W);
  // validate every argument before the first launch
  if ((r = moe::api::check_ptr(hidden, "hidden", true))) return r;
  if ((r = moe::api::check_ptr(drafts, "drafts", K > 0))) return r;
  if ((r = moe::api::check_ptr(committed, "committed", true))) return r;
  if ((r = moe::api::check_ptr(counts, "counts", true))) return r;
  if (T > ctx->cfg.max_tokens) return fail(MOE_EINVAL, "B*(K+1) exceeds max_tokens");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int nkeys = static_cast<int>(moe::kKeySlots * T);
  hipLaunchKernelGGL(k_zero_u64, dim3((nkeys + 255) / 256), dim3(256), 0, s, W.keys, nkeys);
  MOE_HIP(hipGetLastError());
  r = moe::api::verify_step_with(ctx, W, hidden, drafts, B, K, committed, counts, hip_stream);
  for (int i = 0; i < MOE_STAGE_COUNT; ++i) ctx->ev_before[i] = ctx->ev_after[i] = nullptr;
  return r;
}
