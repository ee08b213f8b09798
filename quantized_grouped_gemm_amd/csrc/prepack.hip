// prepack.hip -- one-time re-tiling of group-wise affine 4-bit weights into the
// layout the grouped GEMM streams (see moe_prepack_q4 in moeq4.h).  The codes
// stay packed 4-bit and the byte count is unchanged; only the order moves, so
// that a wave's load of one MFMA weight fragment is 1 KB of contiguous memory.
#include "common.h"

namespace moeq4 {

// Row-major bytes hold codes (2i, 2i+1) in (low, high) nibble of byte i.  The
// tiled dword of 8 codes c0..c7 holds c0,c2,c4,c6,c1,c3,c5,c7 in nibbles 0..7.
__device__ __forceinline__ uint32_t tile_nibbles(uint32_t x) {
  const uint32_t lo = x & 0x0F0F0F0Fu;         // bytes: c0, c2, c4, c6
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;  // bytes: c1, c3, c5, c7
  const uint32_t nlo = (lo & 0xFu) | ((lo >> 4) & 0xF0u) | ((lo >> 8) & 0xF00u) | ((lo >> 12) & 0xF000u);
  const uint32_t nhi = (hi & 0xFu) | ((hi >> 4) & 0xF0u) | ((hi >> 8) & 0xF00u) | ((hi >> 12) & 0xF000u);
  return nlo | (nhi << 16);
}

__device__ __forceinline__ uint2 tile_nibbles2(uint2 v) {
  return make_uint2(tile_nibbles(v.x), tile_nibbles(v.y));
}

// one thread per (matrix row, chunk, K quarter): 8 + 8 bytes of codes
__global__ __launch_bounds__(256) void k_prepack_codes(const uint8_t* __restrict__ codes, int rows_total,
                                                       int N, int K, uint8_t* __restrict__ codes_t) {
  const int G = K / kGroup, C = (G + 1) / 2;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)rows_total * C * 4;
  if (idx >= total) return;
  const int q = (int)(idx & 3);
  const int c = (int)((idx >> 2) % C);
  const long long row = (idx >> 2) / C;  // e*N + n
  const int NT = N / 16;
  const long long e = row / N;
  const int t = (int)((row % N) >> 4);
  const int r = (int)(row & 15);
  const int l = 16 * q + r;
  const uint8_t* src = codes + row * (K / 2) + c * 64 + q * 8;
  const bool full = 2 * c + 1 < G;
  // chunk-major: the NT tiles of one (expert, chunk) are adjacent
  uint8_t* blk = codes_t + e * (long long)N * (K / 2) + (long long)c * NT * 1024 + (long long)t * (full ? 1024 : 512);
  if (full) {
    *(uint2*)(blk + 16 * l) = tile_nibbles2(*(const uint2*)src);
    *(uint2*)(blk + 16 * l + 8) = tile_nibbles2(*(const uint2*)(src + 32));
  } else {
    *(uint2*)(blk + 8 * l) = tile_nibbles2(*(const uint2*)src);
  }
}

// one thread per (matrix row, group): scale and bias
__global__ __launch_bounds__(256) void k_prepack_scales(const uint16_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ biases,
                                                        int rows_total, int N, int K,
                                                        uint16_t* __restrict__ scales_t,
                                                        uint16_t* __restrict__ biases_t) {
  const int G = K / kGroup;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)rows_total * G) return;
  const int g = (int)(idx % G);
  const long long row = idx / G;
  const int NT = N / 16;
  const long long e = row / N;
  const int t = (int)((row % N) >> 4);
  const int r = (int)(row & 15);
  const int c = g >> 1;
  const bool full = 2 * c + 1 < G;
  const long long dst = e * (long long)N * G + 32LL * c * NT + (full ? 32LL * t + 2 * r + (g & 1) : 16LL * t + r);
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
                          N, K, codes_t);
  if (err != hipSuccess) return err;
  return launch("k_prepack_scales", (const void*)&k_prepack_scales,
                dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, stream, scales, biases, (int)rows,
                N, K, scales_t, biases_t);
}

// ----------------------------------------------------------------------------
// Dequantization into memory (moe_dequant_q4): every weight rebuilt exactly as
// bf16(scale*code + bias) from the tiled layout into a row-major bf16 [E][N][K]
// array.  One thread per (expert, chunk, 16-row tile, lane): the lane's 16 (or,
// in the half-size last chunk, 8) code bytes become 32 (16) bf16 weights of one
// row, written as 16-byte stores.
__global__ __launch_bounds__(256) void k_dequant_q4(const uint8_t* __restrict__ codes_t,
                                                    const uint16_t* __restrict__ scales_t,
                                                    const uint16_t* __restrict__ biases_t, int E, int N, int K,
                                                    uint16_t* __restrict__ out) {
  const int G = K / kGroup, C = (G + 1) / 2, NT = N / 16;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)E * C * NT * 64) return;
  const int l = (int)(idx & 63);
  const int t = (int)((idx >> 6) % NT);
  const int c = (int)((idx >> 6) / NT % C);
  const long long e = (idx >> 6) / NT / C;
  const int r = l & 15, q = l >> 4;
  const int n = 16 * t + r;
  const uint8_t* cq = codes_t + e * (long long)N * (K / 2) + (long long)c * NT * 1024;
  const uint16_t* sq = scales_t + e * (long long)N * G;
  const uint16_t* bq = biases_t + e * (long long)N * G;
  uint16_t* row = out + (e * N + n) * (long long)K + 128 * c + 16 * q;
  auto put16 = [&](uint16_t* dst, uint2 w, uint16_t sb, uint16_t bb) {
    const float sv = bf16_bits_to_f32(sb), bv = bf16_bits_to_f32(bb);
    *(uint4*)dst = rebuild_words(w.x, sv, bv);        // K +0..7
    *(uint4*)(dst + 8) = rebuild_words(w.y, sv, bv);  // K +8..15
  };
  if (2 * c + 1 < G) {
    const uint4 w = *(const uint4*)(cq + (long long)t * 1024 + 16 * l);
    const long long g = ((long long)c * NT + t) * 32 + 2 * r;
    put16(row, make_uint2(w.x, w.y), sq[g], bq[g]);
    put16(row + 64, make_uint2(w.z, w.w), sq[g + 1], bq[g + 1]);
  } else {
    const uint2 w = *(const uint2*)(cq + (long long)t * 512 + 8 * l);
    const long long g = (long long)c * NT * 32 + 16 * t + r;
    put16(row, w, sq[g], bq[g]);
  }
}

hipError_t dequant_launch(const uint8_t* codes_t, const uint16_t* scales_t, const uint16_t* biases_t, int E, int N,
                          int K, uint16_t* out, hipStream_t stream) {
  const int G = K / kGroup, C = (G + 1) / 2;
  const long long threads = (long long)E * C * (N / 16) * 64;
  if (threads == 0) return hipSuccess;
  return launch("k_dequant_q4", (const void*)&k_dequant_q4, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                stream, codes_t, scales_t, biases_t, E, N, K, out);
}

}  // namespace moeq4
