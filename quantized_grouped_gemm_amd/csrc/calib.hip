// calib.hip -- measured MFMA ceiling of the GPU (measurement only; not part of
// the method): every SIMD issues independent 32x32x16 bf16 MFMAs back to back,
// the instruction the tall-block grouped GEMM runs, so their rate is the
// matrix-core throughput that kernel can reach on this chip at its clock.
#include "common.h"

namespace moeq4 {

constexpr int kCalibWaves = 4;   // one wave per SIMD of a CU
constexpr int kCalibAcc = 8;     // independent accumulators per wave

__global__ __launch_bounds__(kCalibWaves * 64) void k_mfma_ceiling(int iters, float* __restrict__ out) {
  f32x16 acc[kCalibAcc];
#pragma unroll
  for (int i = 0; i < kCalibAcc; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)((float)(threadIdx.x & 7) * 0.125f + (float)j);
    b[j] = (__bf16)((float)j * 0.5f);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kCalibAcc; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kCalibAcc; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  out[(size_t)blockIdx.x * kCalibWaves * 64 + threadIdx.x] = s;
}

hipError_t calib_mfma_launch(int workgroups, int iters, float* out, hipStream_t stream) {
  return launch("k_mfma_ceiling", (const void*)&k_mfma_ceiling, dim3(workgroups), dim3(kCalibWaves * 64), 0, stream,
                iters, out);
}

}  // namespace moeq4
