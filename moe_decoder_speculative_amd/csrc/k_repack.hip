// Weight repacking at context creation: row-major [R][C] bfloat16 matrices
// into the MFMA operand-tile order the streaming kernels read (see kernels.h).
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(kBlock) void k_tile_bf16(const bf16_t* src, int64_t src_mat_stride, int64_t ld,
                                                     bf16_t* dst, int64_t n_frags, int R, int C, int Rpad) {
  const int64_t f = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (f >= n_frags) return;
  const int lane = static_cast<int>(f % kWave);
  const int64_t tile = f / kWave;
  const int KT = C / kKStep;
  const int kt = static_cast<int>(tile % KT);
  const int64_t rest = tile / KT;
  const int rt = static_cast<int>(rest % (Rpad / kTile));
  const int64_t m = rest / (Rpad / kTile);
  const int r = rt * kTile + lane % kTile;
  const int c = kt * kKStep + (lane / kTile) * 8;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (r < R) v = *reinterpret_cast<const uint4*>(src + m * src_mat_stride + static_cast<int64_t>(r) * ld + c);
  *reinterpret_cast<uint4*>(dst + f * 8) = v;
}

}  // namespace

hipError_t launch_tile_bf16_ld(const bf16_t* src, int64_t src_mat_stride, int64_t ld, bf16_t* dst, int64_t n_mats,
                               int R, int C, int Rpad, hipStream_t s) {
  if (C % kKStep != 0 || Rpad % kTile != 0 || Rpad < R || ld < C || ld % 8 != 0 || src_mat_stride % 8 != 0)
    return hipErrorInvalidValue;
  const int64_t n_frags = n_mats * (Rpad / kTile) * (C / kKStep) * kWave;
  if (n_frags == 0) return hipSuccess;
  const int64_t blocks = (n_frags + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(k_tile_bf16, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, src, src_mat_stride, ld,
                     dst, n_frags, R, C, Rpad);
  return hipGetLastError();
}

hipError_t launch_tile_bf16(const bf16_t* src, int64_t src_mat_stride, bf16_t* dst, int64_t n_mats, int R, int C,
                            int Rpad, hipStream_t s) {
  return launch_tile_bf16_ld(src, src_mat_stride, C, dst, n_mats, R, C, Rpad, s);
}

}  // namespace moe
