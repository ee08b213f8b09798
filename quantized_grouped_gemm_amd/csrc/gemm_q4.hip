// gemm_q4.hip -- grouped GEMM over group-wise affine 4-bit expert weights, gfx950.
//
// Perplexity Engineering, "Optimizing on-device inference for Apple Silicon",
// section "Dequantize weights during matrix multiplication": the 4-bit codes
// are rebuilt on chip a small tile at a time, just long enough to be multiplied
// by the routed activation rows, with fp32 accumulation and bf16 output; the
// expanded weight matrix never exists in memory.  Section "Match tile size to
// expert load": each output tile of an expert maps to one workgroup, and the
// tile height follows the rows per expert.
//
// One workgroup = one block-map entry (<= BM routed rows of one expert) x one
// N tile of 4*NF*16 columns.  Its 4 waves split the N tile; each wave owns NF
// 16-column fragments and every row of the block, so a rebuilt weight is used
// by all rows of the block without leaving the wave's registers.
//
// Data flow per pipeline stage (128 K values = two scale groups):
//   * codes: weights are in the tiled layout of moe_prepack_q4, so one
//     fragment's codes for a stage are 1 KB of contiguous memory, read with one
//     16-byte buffer load per lane (scalar offsets, no per-lane address math);
//   * activations: rows are gathered through perm (token = perm[p] / k);
//   * both go into a ring of S register stages, S-1 stages ahead of use; the
//     activations pass through an LDS double buffer (rows padded to 272 B, so
//     the 16-byte fragment reads are conflict free);
//   * bf16 MFMA 16x16x32 with fp32 accumulation; empty 16-row sub-tiles of a
//     partial block are skipped.
//
// Two ways to feed the rebuilt weights to the MFMA (chosen by block height):
//   DQ (blocks of 64/128 rows): each weight is rebuilt exactly as
//      bf16(scale*code + bias) (fp32 fma, then v_cvt_pk_bf16_f32) and used as
//      the B operand; one rebuild serves BM rows.
//   CQ (blocks of 16/32 rows): the codes themselves go to the MFMA as the
//      exact bf16 values 128+code (one v_and_or per two codes), and the affine
//      part is applied once per 64-K group in fp32:
//        sum_k x_k (s q_k + b) = s * sum_k x_k (128 + q_k) + (b - 128 s) * sum_k x_k,
//      with the per-row group sums of the activations taken while staging
//      them.  Rebuilding costs ~1 VALU op per weight instead of ~3, which is
//      what a 16-row block needs to keep up with HBM.  The weight is used
//      unrounded (s*q + b exactly), not rounded to bf16.
//
// K slot mapping inside one MFMA: lane quarter q (lanes 16q..16q+15) supplies
// K indices g*64 + q*16 + j*8 + [0, 8) for K-step j of group g, for A and B
// alike (in CQ mode both operands carry the slots in the order 0,4,1,5,2,6,3,7).
// The grid is sized from the host bound max_blocks; workgroups past the
// device-side *num_blocks exit at once, so no count goes to the host.
#include <stdlib.h>
#include <string.h>

#include "common.h"

namespace moeq4 {

constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int kKC = 128;           // K values per pipeline stage
constexpr int kXRow = kKC + 8;     // staged activation row: 128 bf16 + 16 B pad
constexpr int kBufFlags = 0x00020000;  // raw buffer descriptor word 3 (32-bit data format)

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

// exact rebuild of 8 codes: bf16(s*q + b), natural K order
__device__ __forceinline__ bf16x8 rebuild_dq(uint32_t wd, float s, float b) {
  const uint32_t lo = wd & 0x0F0F0F0Fu;         // codes 0,2,4,6
  const uint32_t hi = (wd >> 4) & 0x0F0F0F0Fu;  // codes 1,3,5,7
  bf16x8 v;
  v[0] = (__bf16)__builtin_fmaf((float)(lo & 0xFF), s, b);
  v[1] = (__bf16)__builtin_fmaf((float)(hi & 0xFF), s, b);
  v[2] = (__bf16)__builtin_fmaf((float)((lo >> 8) & 0xFF), s, b);
  v[3] = (__bf16)__builtin_fmaf((float)((hi >> 8) & 0xFF), s, b);
  v[4] = (__bf16)__builtin_fmaf((float)((lo >> 16) & 0xFF), s, b);
  v[5] = (__bf16)__builtin_fmaf((float)((hi >> 16) & 0xFF), s, b);
  v[6] = (__bf16)__builtin_fmaf((float)(lo >> 24), s, b);
  v[7] = (__bf16)__builtin_fmaf((float)(hi >> 24), s, b);
  return v;
}

// 8 codes as the exact bf16 values 128+q, slot order 0,4,1,5,2,6,3,7
__device__ __forceinline__ bf16x8 rebuild_cq(uint32_t wd) {
  const uint32_t m = 0x000F000Fu, one28 = 0x43004300u;
  return as_bf16x8((wd & m) | one28, ((wd >> 4) & m) | one28, ((wd >> 8) & m) | one28,
                   ((wd >> 12) & m) | one28);
}

// 8 activations in natural order -> slot order 0,4,1,5,2,6,3,7
__device__ __forceinline__ uint4 to_cq_order(uint4 v) {
  return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                    __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                    __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                    __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
}

__device__ __forceinline__ float sum8_bf16(uint4 v) {
  const float a = __uint_as_float(v.x << 16) + __uint_as_float(v.x & 0xFFFF0000u);
  const float b = __uint_as_float(v.y << 16) + __uint_as_float(v.y & 0xFFFF0000u);
  const float c = __uint_as_float(v.z << 16) + __uint_as_float(v.z & 0xFFFF0000u);
  const float d = __uint_as_float(v.w << 16) + __uint_as_float(v.w & 0xFFFF0000u);
  return (a + b) + (c + d);
}

template <int NF, int XP>
struct Stage {
  u32x4 w[NF];      // codes: dwords 0,1 = group 2c, dwords 2,3 = group 2c+1
  uint32_t s[NF];   // scales of groups 2c (low half) and 2c+1 (high half)
  uint32_t b[NF];   // biases, same packing
  uint4 x[XP];      // activation pieces
};

template <int BM, int NF, bool CQ, int S>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_q4(
    const uint16_t* __restrict__ X, int T, int K, int N, int E, int A, int k,
    const uint8_t* __restrict__ Wt, const uint16_t* __restrict__ St,
    const uint16_t* __restrict__ Bt, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ num_blocks,
    uint16_t* __restrict__ Y) {
  constexpr int MF = BM / 16;
  constexpr int XP = BM * (kKC / 8) / kGemmThreads;  // 16-B activation pieces per thread per stage
  static_assert(XP >= 1 && BM * (kKC / 8) % kGemmThreads == 0, "tile");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kXRow];
  __shared__ __attribute__((aligned(16))) float xsum[CQ ? 2 : 1][2][BM];

  const int blk = blockIdx.x;
  if (blk >= *num_blocks) return;
  const int e = blocks[4 * blk + 0];
  const int row0 = blocks[4 * blk + 1];
  const int rows = min(blocks[4 * blk + 2], BM);
  if (e < 0 || e >= E || row0 < 0 || rows <= 0 || row0 + rows > A) return;  // malformed entry

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int quarter = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_wave = blockIdx.y * (kGemmWaves * NF * 16) + wave * NF * 16;
  const int G = K / kGroup;
  const int nch = (G + 1) >> 1;
  const bool odd_tail = (G & 1) != 0;  // last chunk holds one group only
  const int mfa = (rows + 15) >> 4;
  const int NT = N / 16;

  // ---- buffer resources: one expert's weights; the activation matrix
  const size_t tile_bytes = (size_t)8 * K;  // codes of 16 rows
  const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Wt + (size_t)e * NT * tile_bytes), (short)0, (int)(NT * tile_bytes), kBufFlags);
  const __amdgpu_buffer_rsrc_t ssrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(St + (size_t)e * NT * 16 * G), (short)0, NT * 16 * G * 2, kBufFlags);
  const __amdgpu_buffer_rsrc_t bsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Bt + (size_t)e * NT * 16 * G), (short)0, NT * 16 * G * 2, kBufFlags);
  const __amdgpu_buffer_rsrc_t xsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, T * K * 2, kBufFlags);

  // fragments past N load nothing (their MFMAs and stores are skipped)
  const int nf_live = min(NF, max(0, (N - n_wave) / 16));
  const int t0 = n_wave / 16;

  // per-thread activation pieces: row offset in bytes, or -1 for rows past the block
  int xoff[XP];
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int p = tid + i * kGemmThreads;
    const int r = p >> 4, col = p & 15;
    xoff[i] = (r < rows) ? (perm[row0 + r] / k) * K * 2 + col * 16 : -1;
  }

  Stage<NF, XP> st[S];
  auto load = [&](Stage<NF, XP>& s, int c) {
    const bool half = odd_tail && c == nch - 1;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f >= nf_live) break;
      const int soff = (t0 + f) * (int)tile_bytes + c * 1024;
      const int goff = ((t0 + f) * 16 * G + 32 * c) * 2;
      if (!half) {
        s.w[f] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, lane * 16, soff, 0);
        s.s[f] = __builtin_amdgcn_raw_buffer_load_b32(ssrc, (lane & 15) * 4, goff, 0);
        s.b[f] = __builtin_amdgcn_raw_buffer_load_b32(bsrc, (lane & 15) * 4, goff, 0);
      } else {
        typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wsrc, lane * 8, soff, 0);
        s.w[f] = u32x4{v[0], v[1], 0u, 0u};
        s.s[f] = __builtin_amdgcn_raw_buffer_load_b16(ssrc, (lane & 15) * 2, goff, 0);
        s.b[f] = __builtin_amdgcn_raw_buffer_load_b16(bsrc, (lane & 15) * 2, goff, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int col = (tid + i * kGemmThreads) & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (xoff[i] >= 0 && (!half || col < 8)) {
        const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(xsrc, xoff[i], c * kKC * 2, 0);
        v = make_uint4(r[0], r[1], r[2], r[3]);
      }
      s.x[i] = v;
    }
  };
  auto store_x = [&](const Stage<NF, XP>& s, int buf) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = tid + i * kGemmThreads;
      const int r = p >> 4, col = p & 15;
      uint4 v = s.x[i];
      if constexpr (CQ) {
        // group sums: the 8 pieces of (row, group) sit in 8 consecutive lanes
        float sm = sum8_bf16(v);
        sm += __shfl_xor(sm, 1);
        sm += __shfl_xor(sm, 2);
        sm += __shfl_xor(sm, 4);
        if ((col & 7) == 0) xsum[buf][col >> 3][r] = sm;
        v = to_cq_order(v);
      }
      *(uint4*)(&xs[buf][r * kXRow + col * 8]) = v;
    }
  };

  f32x4 acc[MF][NF];
#pragma unroll
  for (int r = 0; r < MF; ++r)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[r][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, const Stage<NF, XP>& s, bool two_groups) {
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      if (gi == 1 && !two_groups) break;
      bf16x8 bfr[NF][2];
      float sc[NF], cc[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f >= nf_live) break;
        const float sv = gi ? __uint_as_float(s.s[f] & 0xFFFF0000u) : __uint_as_float(s.s[f] << 16);
        const float bv = gi ? __uint_as_float(s.b[f] & 0xFFFF0000u) : __uint_as_float(s.b[f] << 16);
        const uint32_t w0 = s.w[f][2 * gi], w1 = s.w[f][2 * gi + 1];
        if constexpr (CQ) {
          sc[f] = sv;
          cc[f] = __builtin_fmaf(-128.f, sv, bv);
          bfr[f][0] = rebuild_cq(w0);
          bfr[f][1] = rebuild_cq(w1);
        } else {
          bfr[f][0] = rebuild_dq(w0, sv, bv);
          bfr[f][1] = rebuild_dq(w1, sv, bv);
        }
      }
      const uint16_t* xb = &xs[buf][(lane & 15) * kXRow + gi * 64 + quarter * 16];
#pragma unroll
      for (int r = 0; r < MF; ++r) {
        if (r >= mfa) break;
        const bf16x8 a0 = *(const bf16x8*)(xb + r * 16 * kXRow);
        const bf16x8 a1 = *(const bf16x8*)(xb + r * 16 * kXRow + 8);
        if constexpr (CQ) {
          const float4 xsv = *(const float4*)(&xsum[buf][gi][r * 16 + quarter * 4]);
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            if (f >= nf_live) break;
            f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bfr[f][0], zero, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bfr[f][1], p, 0, 0, 0);
            f32x4 t = acc[r][f];
            t[0] = __builtin_fmaf(xsv.x, cc[f], __builtin_fmaf(p[0], sc[f], t[0]));
            t[1] = __builtin_fmaf(xsv.y, cc[f], __builtin_fmaf(p[1], sc[f], t[1]));
            t[2] = __builtin_fmaf(xsv.z, cc[f], __builtin_fmaf(p[2], sc[f], t[2]));
            t[3] = __builtin_fmaf(xsv.w, cc[f], __builtin_fmaf(p[3], sc[f], t[3]));
            acc[r][f] = t;
          }
        } else {
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            if (f >= nf_live) break;
            acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bfr[f][0], acc[r][f], 0, 0, 0);
          }
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            if (f >= nf_live) break;
            acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bfr[f][1], acc[r][f], 0, 0, 0);
          }
        }
      }
    }
  };

  // ---- pipeline.  Chunk c is loaded into register stage c % S at iteration
  // c - (S-1); its activations go to LDS buffer c & 1 at iteration c - 1 and
  // its MFMAs run at iteration c.  Loads complete in issue order, so the
  // activation wait at iteration c - 1 only covers loads issued S-2
  // iterations earlier, never the newer prefetches.
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nch) load(st[s], s);
  store_x(st[0], 0);
  __syncthreads();

  for (int c0 = 0; c0 < nch; c0 += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int c = c0 + u;
      if (c >= nch) break;
      if (c + S - 1 < nch) load(st[(u + S - 1) % S], c + S - 1);
      if (c + 1 < nch) store_x(st[(u + 1) % S], (c + 1) & 1);
      compute(c & 1, st[u], !(odd_tail && c == nch - 1));
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds rows 4*quarter + i of column lane&15 of each fragment
#pragma unroll
  for (int r = 0; r < MF; ++r) {
    if (r >= mfa) break;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f >= nf_live) break;
      const int n = n_wave + f * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r * 16 + quarter * 4 + i;
        if (row < rows) Y[(size_t)(row0 + row) * N + n] = f32_to_bf16_bits(acc[r][f][i]);
      }
    }
  }
}

namespace {

struct GemmVariant {
  const char* name;
  int bm, nf;
  const void* fn;
};

#define MOEQ4_GEMM_VARIANT(BM, NF, CQ, S) \
  {"bm" #BM "_nf" #NF "_" #CQ "_s" #S, BM, NF, (const void*)&k_gemm_q4<BM, NF, CQ, S>}

// The first entry of each block height is its default.
const GemmVariant kVariants[] = {
    MOEQ4_GEMM_VARIANT(16, 2, true, 4),
    MOEQ4_GEMM_VARIANT(32, 2, true, 4),
    MOEQ4_GEMM_VARIANT(64, 4, false, 3),
    MOEQ4_GEMM_VARIANT(128, 4, false, 2),
    MOEQ4_GEMM_VARIANT(16, 4, true, 4),
    MOEQ4_GEMM_VARIANT(16, 1, true, 4),
    MOEQ4_GEMM_VARIANT(32, 4, true, 3),
    MOEQ4_GEMM_VARIANT(32, 4, true, 4),
    MOEQ4_GEMM_VARIANT(32, 1, true, 4),
    MOEQ4_GEMM_VARIANT(32, 2, true, 3),
    MOEQ4_GEMM_VARIANT(32, 2, false, 4),
    MOEQ4_GEMM_VARIANT(64, 2, true, 3),
    MOEQ4_GEMM_VARIANT(64, 4, false, 2),
    MOEQ4_GEMM_VARIANT(128, 4, false, 3),
    MOEQ4_GEMM_VARIANT(128, 2, false, 3),
};
#undef MOEQ4_GEMM_VARIANT

// Tile choice by block height; MOEQ4_GEMM_VARIANT=<name> (same block height)
// overrides it for tuning sweeps.
const GemmVariant* pick_variant(int bm) {
  static const char* forced = getenv("MOEQ4_GEMM_VARIANT");
  if (forced)
    for (const GemmVariant& v : kVariants)
      if (v.bm == bm && strcmp(v.name, forced) == 0) return &v;
  for (const GemmVariant& v : kVariants)
    if (v.bm == bm) return &v;
  return nullptr;
}

}  // namespace

hipError_t gemm_q4_launch(const uint16_t* X, int T, int K, int N, int E, int k, const uint8_t* Wt,
                          const uint16_t* St, const uint16_t* Bt, const int32_t* perm,
                          const int32_t* blocks, const int32_t* num_blocks, int max_blocks,
                          int BM, uint16_t* Y, hipStream_t stream) {
  if (max_blocks <= 0) return hipSuccess;
  const GemmVariant* v = pick_variant(BM);
  if (!v) return hipErrorInvalidValue;
  const int ntile = kGemmWaves * v->nf * 16;
  const dim3 grid(max_blocks, (N + ntile - 1) / ntile);
  return launch("k_gemm_q4", v->fn, grid, dim3(kGemmThreads), 0, stream, X, T, K, N, E, T * k, k,
                Wt, St, Bt, perm, blocks, num_blocks, Y);
}

}  // namespace moeq4
