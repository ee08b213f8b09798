// gemm_q4.hip -- grouped GEMM over group-wise affine 4-bit expert weights, gfx950.
//
// Perplexity Engineering, "Optimizing on-device inference for Apple Silicon",
// section "Dequantize weights during matrix multiplication": the 4-bit codes
// are rebuilt into bf16 a small tile at a time on chip, just long enough to be
// multiplied by the routed activation rows, with fp32 accumulation and bf16
// output; the expanded weight matrix never exists in memory.  Section "Match
// tile size to expert load": each output tile of an expert maps to one
// workgroup, and the tile height follows the rows per expert.
//
// MI355X design (one workgroup = one block-map entry x one N tile):
//   * 4 waves split the N tile; each wave owns NF 16-column fragments and all
//     BM rows of the block, so every rebuilt weight is used by every row of
//     the block without leaving the wave's registers.
//   * Packed codes are read straight from HBM into VGPRs (8 bytes per lane =
//     16 codes of one weight row), rebuilt as s*q + b in fp32 and rounded to
//     bf16 (v_cvt_pk_bf16_f32), which is exactly the B operand layout of
//     v_mfma_f32_16x16x32_bf16: lane l holds 8 K values of column l%16.
//   * Activation rows are gathered through perm (token = perm[p] / k), staged
//     64 K values at a time in LDS (double buffered, rows padded to 144 B so
//     the 16-B fragment reads are conflict free), and read as A fragments.
//   * Empty 16-row sub-tiles of a partial block are skipped.
//   * The grid is sized from the host bound max_blocks; workgroups past the
//     device-side *num_blocks exit at once, so no count goes to the host.
// K slots inside one MFMA: lane quarter q (lanes 16q..16q+15) supplies K
// indices c*64 + q*16 + j*8 + [0, 8) for K-step j of chunk c, for both A and B.
#include "common.h"

namespace moeq4 {

constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int kLdsRow = 64 + 8;  // bf16 per staged row: 64 K values + 16 B pad

template <int BM, int NF>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_q4(
    const uint16_t* __restrict__ X, int K, int N, int E, int A, int k, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ S, const uint16_t* __restrict__ Bias,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blocks,
    const int32_t* __restrict__ num_blocks, uint16_t* __restrict__ Y) {
  constexpr int MF = BM / 16;
  constexpr int XP = (BM * 8 + kGemmThreads - 1) / kGemmThreads;  // 16-B pieces per thread
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kLdsRow];
  __shared__ int tok_s[BM];

  const int blk = blockIdx.x;
  if (blk >= *num_blocks) return;
  const int e = blocks[4 * blk + 0];
  const int row0 = blocks[4 * blk + 1];
  const int rows = min(blocks[4 * blk + 2], BM);
  if (e < 0 || e >= E || row0 < 0 || rows <= 0 || row0 + rows > A) return;  // malformed entry

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n_wave = blockIdx.y * (kGemmWaves * NF * 16) + wv * NF * 16;
  const int G = K / kGroup;
  const int mfa = (rows + 15) >> 4;

  for (int r = tid; r < BM; r += kGemmThreads) tok_s[r] = (r < rows) ? perm[row0 + r] / k : -1;
  __syncthreads();

  // ---- activation staging
  uint4 xr[XP];
  auto load_x = [&](int c) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int piece = tid + i * kGemmThreads;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (piece < BM * 8) {
        const int t = tok_s[piece >> 3];
        if (t >= 0) v = *(const uint4*)(X + (size_t)t * K + c * 64 + (piece & 7) * 8);
      }
      xr[i] = v;
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int piece = tid + i * kGemmThreads;
      if (piece < BM * 8) *(uint4*)(&xs[buf][(piece >> 3) * kLdsRow + (piece & 7) * 8]) = xr[i];
    }
  };

  // ---- weights: lane -> column n = n_wave + f*16 + (lane & 15), K quarter q = lane >> 4
  uint2 wr[NF];
  uint32_t sb[NF];
  size_t wrow[NF];
  bool nf_ok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    nf_ok[f] = (n_wave + f * 16) < N;
    wrow[f] = (size_t)e * N + (nf_ok[f] ? n_wave + f * 16 + (lane & 15) : 0);
  }
  auto load_w = [&](int c) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (nf_ok[f]) {
        wr[f] = *(const uint2*)(Wq + wrow[f] * (K / 2) + c * 32 + (lane >> 4) * 8);
        sb[f] = (uint32_t)S[wrow[f] * G + c] | ((uint32_t)Bias[wrow[f] * G + c] << 16);
      }
    }
  };
  bf16x8 bfr[NF][2];
  auto dequant = [&]() {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (!nf_ok[f]) continue;
      const float s = bf16_bits_to_f32(sb[f] & 0xFFFFu);
      const float b = bf16_bits_to_f32(sb[f] >> 16);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t wd = j ? wr[f].y : wr[f].x;
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
        bfr[f][j] = v;
      }
    }
  };

  f32x4 acc[MF][NF];
#pragma unroll
  for (int r = 0; r < MF; ++r)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[r][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int r = 0; r < MF; ++r) {
        if (r < mfa) {
          const bf16x8 a = *(const bf16x8*)(&xs[buf][(r * 16 + (lane & 15)) * kLdsRow +
                                                     (lane >> 4) * 16 + j * 8]);
#pragma unroll
          for (int f = 0; f < NF; ++f)
            if (nf_ok[f])
              acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bfr[f][j], acc[r][f], 0, 0, 0);
        }
      }
    }
  };

  load_x(0);
  load_w(0);
  store_x(0);
  dequant();
  __syncthreads();
  for (int c = 0; c < G; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < G;
    if (more) {
      load_x(c + 1);
      load_w(c + 1);
    }
    compute(buf);
    if (more) {
      store_x(buf ^ 1);
      dequant();
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*(lane>>4) + i of column lane&15 of each fragment
#pragma unroll
  for (int r = 0; r < MF; ++r) {
    if (r >= mfa) continue;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (!nf_ok[f]) continue;
      const int n = n_wave + f * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r * 16 + (lane >> 4) * 4 + i;
        if (row < rows) Y[(size_t)(row0 + row) * N + n] = f32_to_bf16_bits(acc[r][f][i]);
      }
    }
  }
}

hipError_t gemm_q4_launch(const uint16_t* X, int T, int K, int N, int E, int k, const uint8_t* Wq,
                          const uint16_t* S, const uint16_t* B, const int32_t* perm,
                          const int32_t* blocks, const int32_t* num_blocks, int max_blocks,
                          int BM, uint16_t* Y, hipStream_t stream) {
  if (max_blocks <= 0) return hipSuccess;
  constexpr int NF = 4;
  const int ntile = kGemmWaves * NF * 16;
  const dim3 grid(max_blocks, (N + ntile - 1) / ntile);
  const void* fn;
  switch (BM) {
    case 16: fn = (const void*)&k_gemm_q4<16, NF>; break;
    case 32: fn = (const void*)&k_gemm_q4<32, NF>; break;
    case 64: fn = (const void*)&k_gemm_q4<64, NF>; break;
    default: fn = (const void*)&k_gemm_q4<128, NF>; break;
  }
  return launch("k_gemm_q4", fn, grid, dim3(kGemmThreads), 0, stream, X, K, N, E, T * k, k, Wq, S, B, perm,
                blocks, num_blocks, Y);
}

}  // namespace moeq4
