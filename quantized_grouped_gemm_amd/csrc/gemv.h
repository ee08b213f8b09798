// gemv.h -- matrix-vector building blocks over the tiled 4-bit layout, shared
// by the one-token decode step (decode.hip) and the few-token step (small.hip).
//
// Perplexity Engineering, "Optimizing on-device inference for Apple Silicon",
// section "Optimize the single-row weight path": a row-parallel GEMV for one
// activation row; section "Apple silicon provides different paths for
// different workloads": with little weight reuse it is bound by memory
// bandwidth; section "Dequantize weights during matrix multiplication":
// weights are rebuilt on chip, never stored.
//
// A wave reads one 1 KB block of the tiled layout (16 rows x 128 K values;
// lane 16q+r holds 32 codes of row r, K quarters q), rebuilds each weight
// exactly as bf16(scale * code + bias) (rebuild_words) and multiplies the
// rebuilt pairs with bf16 activation pairs from LDS by v_dot2c_f32_bf16,
// accumulating in fp32.  The rebuild can be done once and the rebuilt block
// applied to several activation vectors (Rebuilt, gemv_rebuilt).
#pragma once
#include "common.h"

namespace moeq4 {

typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16v2, a), __builtin_bit_cast(bf16v2, b), c,
                                         false);
}

// sum over 16 K of x * w for rebuilt weight pairs w0 (K +0..7), w1 (K +8..15)
// and x pairs xa (K +0..7), xb (K +8..15): two interleaved fp32 chains
__device__ __forceinline__ float dot16_rebuilt(uint4 w0, uint4 w1, uint4 xa, uint4 xb) {
  float p = 0.f, q = 0.f;
  p = dot2(w0.x, xa.x, p);  // c0, c1
  q = dot2(w0.y, xa.y, q);  // c2, c3
  p = dot2(w0.z, xa.z, p);  // c4, c5
  q = dot2(w0.w, xa.w, q);  // c6, c7
  p = dot2(w1.x, xb.x, p);
  q = dot2(w1.y, xb.y, q);
  p = dot2(w1.z, xb.z, p);
  q = dot2(w1.w, xb.w, q);
  return p + q;
}

// sum over 16 K of x * bf16(s*q + b): codes in tiled dwords d0 (K +0..7) and
// d1 (K +8..15)
__device__ __forceinline__ float dot16(uint32_t d0, uint32_t d1, uint4 xa, uint4 xb, float s, float b) {
  return dot16_rebuilt(rebuild_words(d0, s, b), rebuild_words(d1, s, b), xa, xb);
}

// One matrix [N][K] of the tiled layout, seen by one GEMV.
struct TiledMat {
  const uint8_t* q;    // codes of this matrix
  const uint16_t* s;   // scales
  const uint16_t* b;   // biases
  int NT;              // N / 16
};

// A lane's part of one full block (chunk c of 128 K values, 16-row tile):
// 32 codes and the scale / bias of its row's two groups.
struct FullBlock {
  uint4 codes;
  uint32_t s2, b2;  // bf16 scale / bias of groups 2c (low half) and 2c+1 (high half)
};

__device__ __forceinline__ FullBlock load_full(const TiledMat& m, int tile, int c, int lane) {
  FullBlock f;
  f.codes = *(const uint4*)(m.q + ((size_t)c * m.NT + tile) * 1024 + 16 * lane);
  const size_t g = 32 * ((size_t)c * m.NT + tile) + 2 * (lane & 15);
  f.s2 = *(const uint32_t*)(m.s + g);
  f.b2 = *(const uint32_t*)(m.b + g);
  return f;
}

// Partial GEMV of row r = lane % 16 of the block's tile over chunk c, with x
// (bf16) in LDS.
__device__ __forceinline__ float gemv_full(const FullBlock& f, int c, int lane, const uint4* xl) {
  const int k0 = 128 * c + 16 * (lane >> 4);  // first K value of the lane's first 16
  const float s0 = bf16_bits_to_f32(f.s2 & 0xFFFFu), s1 = bf16_bits_to_f32(f.s2 >> 16);
  const float b0 = bf16_bits_to_f32(f.b2 & 0xFFFFu), b1 = bf16_bits_to_f32(f.b2 >> 16);
  return dot16(f.codes.x, f.codes.y, xl[k0 / 8], xl[k0 / 8 + 1], s0, b0) +
         dot16(f.codes.z, f.codes.w, xl[(k0 + 64) / 8], xl[(k0 + 64) / 8 + 1], s1, b1);
}

// the half-size last chunk of an odd group count: lane 16q+r holds 16 codes
__device__ __forceinline__ float gemv_tail(const TiledMat& m, int tile, int c, int lane, const uint4* xl) {
  const uint2 cd = *(const uint2*)(m.q + (size_t)c * m.NT * 1024 + (size_t)tile * 512 + 8 * lane);
  const size_t g = 32 * (size_t)c * m.NT + 16 * (size_t)tile + (lane & 15);
  const float s0 = bf16_bits_to_f32(m.s[g]), b0 = bf16_bits_to_f32(m.b[g]);
  const int k0 = 128 * c + 16 * (lane >> 4);
  return dot16(cd.x, cd.y, xl[k0 / 8], xl[k0 / 8 + 1], s0, b0);
}

// A lane's rebuilt weights of one block, to be applied to several vectors:
// w[0], w[1] the 16 K values of group 2c, w[2], w[3] those of group 2c+1 (a
// tail block fills w[0], w[1] only).  Same arithmetic and order as gemv_full
// and gemv_tail.
struct Rebuilt {
  uint4 w[4];
};

__device__ __forceinline__ Rebuilt rebuild_full(const FullBlock& f) {
  const float s0 = bf16_bits_to_f32(f.s2 & 0xFFFFu), s1 = bf16_bits_to_f32(f.s2 >> 16);
  const float b0 = bf16_bits_to_f32(f.b2 & 0xFFFFu), b1 = bf16_bits_to_f32(f.b2 >> 16);
  Rebuilt r;
  r.w[0] = rebuild_words(f.codes.x, s0, b0);
  r.w[1] = rebuild_words(f.codes.y, s0, b0);
  r.w[2] = rebuild_words(f.codes.z, s1, b1);
  r.w[3] = rebuild_words(f.codes.w, s1, b1);
  return r;
}

__device__ __forceinline__ float gemv_rebuilt(const Rebuilt& r, int c, int lane, const uint4* xl) {
  const int k0 = 128 * c + 16 * (lane >> 4);
  return dot16_rebuilt(r.w[0], r.w[1], xl[k0 / 8], xl[k0 / 8 + 1]) +
         dot16_rebuilt(r.w[2], r.w[3], xl[(k0 + 64) / 8], xl[(k0 + 64) / 8 + 1]);
}

__device__ __forceinline__ Rebuilt rebuild_tail(const TiledMat& m, int tile, int c, int lane) {
  const uint2 cd = *(const uint2*)(m.q + (size_t)c * m.NT * 1024 + (size_t)tile * 512 + 8 * lane);
  const size_t g = 32 * (size_t)c * m.NT + 16 * (size_t)tile + (lane & 15);
  const float s0 = bf16_bits_to_f32(m.s[g]), b0 = bf16_bits_to_f32(m.b[g]);
  Rebuilt r;
  r.w[0] = rebuild_words(cd.x, s0, b0);
  r.w[1] = rebuild_words(cd.y, s0, b0);
  r.w[2] = r.w[3] = uint4{0u, 0u, 0u, 0u};
  return r;
}

__device__ __forceinline__ float gemv_tail_rebuilt(const Rebuilt& r, int c, int lane, const uint4* xl) {
  const int k0 = 128 * c + 16 * (lane >> 4);
  return dot16_rebuilt(r.w[0], r.w[1], xl[k0 / 8], xl[k0 / 8 + 1]);
}

// sum of the partials of lanes r, r+16, r+32, r+48 (the four K quarters)
__device__ __forceinline__ float sum_quarters(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Staging of bf16 vectors in LDS, npieces 16-byte pieces in all.  Each thread
// loads its P pieces into registers (stage_load, indices clamped so the loads
// are unconditional) before the weight loads are issued, so that the wait for
// them does not also wait for the weights (loads complete in issue order);
// stage_store then writes them to LDS.  The host keeps npieces <= P * threads.
template <int P>
struct Staged {
  uint4 v[P];
};

template <int P>
__device__ __forceinline__ Staged<P> stage_load(const uint16_t* __restrict__ src, int npieces) {
  Staged<P> st;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int p = min((int)(threadIdx.x + i * blockDim.x), npieces - 1);
    st.v[i] = *(const uint4*)(src + 8 * (size_t)p);
  }
  return st;
}

template <int P>
__device__ __forceinline__ void stage_store(const Staged<P>& st, int npieces, uint4* xl) {
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int p = threadIdx.x + i * blockDim.x;
    if (p < npieces) xl[p] = st.v[i];
  }
}

}  // namespace moeq4
