// prepack.hip -- one-time re-tiling of group-wise affine 4-bit weights into the
// layout the grouped GEMM streams (see moe_prepack_q4 in moeq4.h).  The codes
// stay packed 4-bit and the byte count is unchanged; only the order moves, so
// that a wave's load of one MFMA weight fragment is 1 KB of contiguous memory.
#include "common.h"

namespace moeq4 {

// one thread per (matrix row, chunk, K quarter): 8 + 8 bytes of codes
__global__ __launch_bounds__(256) void k_prepack_codes(const uint8_t* __restrict__ codes, int rows_total,
                                                       int K, uint8_t* __restrict__ codes_t) {
  const int G = K / kGroup, C = (G + 1) / 2;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)rows_total * C * 4;
  if (idx >= total) return;
  const int q = (int)(idx & 3);
  const int c = (int)((idx >> 2) % C);
  const long long row = (idx >> 2) / C;  // e*N + n
  const long long tile = row >> 4;       // e*NT + t
  const int r = (int)(row & 15);
  const int l = 16 * q + r;
  const uint8_t* src = codes + row * (K / 2) + c * 64 + q * 8;
  const bool full = 2 * c + 1 < G;
  uint8_t* blk = codes_t + tile * 8LL * K + (long long)c * 1024;
  if (full) {
    *(uint2*)(blk + 16 * l) = *(const uint2*)src;
    *(uint2*)(blk + 16 * l + 8) = *(const uint2*)(src + 32);
  } else {
    *(uint2*)(blk + 8 * l) = *(const uint2*)src;
  }
}

// one thread per (matrix row, group): scale and bias
__global__ __launch_bounds__(256) void k_prepack_scales(const uint16_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ biases,
                                                        int rows_total, int K,
                                                        uint16_t* __restrict__ scales_t,
                                                        uint16_t* __restrict__ biases_t) {
  const int G = K / kGroup;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)rows_total * G) return;
  const int g = (int)(idx % G);
  const long long row = idx / G;
  const long long tile = row >> 4;
  const int r = (int)(row & 15);
  const int c = g >> 1;
  const bool full = 2 * c + 1 < G;
  const long long dst = tile * 16LL * G + 32LL * c + (full ? 2 * r + (g & 1) : r);
  scales_t[dst] = scales[idx];
  biases_t[dst] = biases[idx];
}

hipError_t prepack_launch(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases,
                          int E, int N, int K, uint8_t* codes_t, uint16_t* scales_t,
                          uint16_t* biases_t, hipStream_t stream) {
  const long long rows = (long long)E * N;
  const int G = K / kGroup, C = (G + 1) / 2;
  const long long n1 = rows * C * 4, n2 = rows * G;
  hipError_t err = launch("k_prepack_codes", (const void*)&k_prepack_codes,
                          dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, stream, codes, (int)rows,
                          K, codes_t);
  if (err != hipSuccess) return err;
  return launch("k_prepack_scales", (const void*)&k_prepack_scales,
                dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, stream, scales, biases, (int)rows,
                K, scales_t, biases_t);
}

}  // namespace moeq4
