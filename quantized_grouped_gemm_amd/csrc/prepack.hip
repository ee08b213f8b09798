// prepack.hip -- one-time re-tiling of group-wise affine 4-bit weights into the
// layout the grouped GEMM streams (see moe_prepack_q4 in moeq4.h).  The codes
// stay packed 4-bit and the byte count is unchanged; only the order moves, so
// that a wave's load of one MFMA weight fragment is 1 KB of contiguous memory.
#include "common.h"

namespace moeq4 {

constexpr int kKCodes = 128;  // K values per chunk of the tiled layout

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
// array.  One 256-thread workgroup per (expert, 16-row tile, span of up to
// kDqChunks chunks = 512 K values): its code blocks are read whole (1 KB per
// chunk, coalesced), rebuilt into LDS as 16 rows of the span, and written out
// row by row, so every store instruction writes contiguous row memory.
constexpr int kDqChunks = 4;
constexpr int kDqThreads = 256;

__global__ __launch_bounds__(kDqThreads) void k_dequant_q4(const uint8_t* __restrict__ codes_t,
                                                           const uint16_t* __restrict__ scales_t,
                                                           const uint16_t* __restrict__ biases_t, int E, int N,
                                                           int K, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t tile_s[16][kDqChunks * kKCodes];
  const int G = K / kGroup, C = (G + 1) / 2, NT = N / 16;
  const int spans = (C + kDqChunks - 1) / kDqChunks;
  const long long wg = blockIdx.x;
  const int sp = (int)(wg % spans);
  const int t = (int)(wg / spans % NT);
  const long long e = wg / spans / NT;
  const int c0 = sp * kDqChunks, c1 = min(C, c0 + kDqChunks);
  const uint8_t* cq = codes_t + e * (long long)N * (K / 2);
  const uint16_t* sq = scales_t + e * (long long)N * G;
  const uint16_t* bq = biases_t + e * (long long)N * G;
  // rebuild: thread (chunk slot cs = tid / 64, lane l = tid % 64) takes lane l of chunk c0 + cs
  {
    const int cs = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 15, q = l >> 4;
    const int c = c0 + cs;
    if (c < c1) {
      uint16_t* dst = &tile_s[r][cs * kKCodes + 16 * q];
      auto put16 = [&](uint16_t* d, uint2 w, uint16_t sb, uint16_t bb) {
        const float sv = bf16_bits_to_f32(sb), bv = bf16_bits_to_f32(bb);
        *(uint4*)d = rebuild_words(w.x, sv, bv);        // K +0..7
        *(uint4*)(d + 8) = rebuild_words(w.y, sv, bv);  // K +8..15
      };
      if (2 * c + 1 < G) {
        const uint4 w = *(const uint4*)(cq + ((long long)c * NT + t) * 1024 + 16 * l);
        const long long g = ((long long)c * NT + t) * 32 + 2 * r;
        put16(dst, make_uint2(w.x, w.y), sq[g], bq[g]);
        put16(dst + 64, make_uint2(w.z, w.w), sq[g + 1], bq[g + 1]);
      } else {
        const uint2 w = *(const uint2*)(cq + (long long)c * NT * 1024 + (long long)t * 512 + 8 * l);
        const long long g = (long long)c * NT * 32 + 16 * t + r;
        put16(dst, w, sq[g], bq[g]);
      }
    }
  }
  __syncthreads();
  // write: the span's K range of the 16 rows, 16 bytes per thread per step
  const int k_lo = 128 * c0, k_hi = min(K, 128 * c1);
  const int pieces = (k_hi - k_lo) / 8;  // 16-byte pieces per row
  for (int i = threadIdx.x; i < 16 * pieces; i += kDqThreads) {
    const int r = i / pieces, pc = i % pieces;
    *(uint4*)(out + (e * N + 16 * t + r) * (long long)K + k_lo + 8 * pc) = *(const uint4*)&tile_s[r][8 * pc];
  }
}

hipError_t dequant_launch(const uint8_t* codes_t, const uint16_t* scales_t, const uint16_t* biases_t, int E, int N,
                          int K, uint16_t* out, hipStream_t stream) {
  const int G = K / kGroup, C = (G + 1) / 2;
  const long long wgs = (long long)E * (N / 16) * ((C + kDqChunks - 1) / kDqChunks);
  if (wgs == 0) return hipSuccess;
  return launch("k_dequant_q4", (const void*)&k_dequant_q4, dim3((unsigned)wgs), dim3(kDqThreads), 0, stream,
                codes_t, scales_t, biases_t, E, N, K, out);
}

}  // namespace moeq4
