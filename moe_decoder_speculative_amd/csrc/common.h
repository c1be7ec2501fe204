// Device helpers shared by the gfx950 kernels of the MoE verification step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;                                           // bfloat16 bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));       // MFMA operand
typedef float f32x4_t __attribute__((ext_vector_type(4)));         // 16x16 MFMA acc

constexpr int kWave = 64;
constexpr int kBlock = 256;       // 4 wavefronts
constexpr int kMaxExperts = 64;   // one router lane per routed expert
constexpr int kMaxTopK = 8;
constexpr int kTile = 16;         // MFMA 16x16x32: rows / tokens per tile
constexpr int kKStep = 32;        // MFMA 16x16x32: reduction per instruction
constexpr int kFragElems = 512;   // bf16 elements of one 16x32 operand tile

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float32 -> bfloat16 on gfx950's conversion instruction: round to nearest,
// ties to even; a NaN stays a (quiet) NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two floats -> two bfloat16 in one 32-bit word (a in the low half), rounded
// as f32_to_bf16 does, in a single conversion instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Storage-type traits: load one element as float, round a float to storage.
template <typename ST> struct Storage;
template <> struct Storage<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ float round(float v) { return v; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Storage<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
  static __device__ __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// 16-byte operand fragment loads (8 bf16).
__device__ __forceinline__ bf16x8_t load_frag(const bf16_t* p) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8_t, v);
}
// The same 16-byte loads with the non-temporal hint, for data a step reads
// once in whole lines (decode expert weights, LM-head rows): streamed through
// the caches at low priority, they no longer push out what the step reads
// again and again (activation rows, pair lists, the router matrix).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t load_frag_stream(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}
__device__ __forceinline__ bf16x8_t zero_frag() {
  return __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]).  waitcnt_vm(n): at most n vector-memory operations
// of this wavefront outstanding; waitcnt_lgkm0: all LDS / scalar operations done.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int waitcnt_lgkm0 = 15 | (3 << 14) | (7 << 4);

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also waits for
// every outstanding global load, which would drain a prefetch pipeline; this
// one waits for this wavefront's LDS operations and keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA: lane L supplies row (A) / column (B) L%32, reduction
// elements 8(L/32) .. +8; it receives, of the 32 x 32 result, column L%32 and
// rows 8g + 4(L/32) + r as element 4g + r (g, r in 0..3).
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

// Order-preserving map of float32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t orderable(float f) {
  // negative: all bits flipped; otherwise the sign bit set (branch-free)
  const uint32_t u = __float_as_uint(f);
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

// Arg-max key: the larger value wins; on equal values the lower index wins.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t index) {
  return (static_cast<uint64_t>(orderable(v)) << 32) | static_cast<uint64_t>(0xffffffffu - index);
}
__device__ __forceinline__ uint32_t argmax_key_index(uint64_t key) {
  return 0xffffffffu - static_cast<uint32_t>(key & 0xffffffffu);
}

// SwiGLU gate: silu(g) * u = g * u / (1 + e^-g), with e^-g = 2^(-g log2 e) on
// the hardware exp2 and the quotient on the hardware reciprocal (about one ulp
// each, far below the bfloat16 rounding that follows).  For very negative g,
// e^-g overflows to inf and the result is a signed zero, the correct limit.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896341f));
}

}  // namespace moe
