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
// With the routing's top-k done, the 64-row kernel can also rank the rows
// itself (k_gemm_q4_w32 with FR, route_gemm_q4_launch): the routing's
// histogram, scan and scatter then need no launches of their own.
//
// Blocks of up to 32 rows (k_gemm_q4): one workgroup = one block-map entry
// (<= BM routed rows of one expert) x one N tile of WAVES*NF*16 columns.  Its
// waves split the N tile; each wave owns NF 16-column fragments and every row
// of the block, so a rebuilt weight is used by all rows of the block without
// leaving the wave's registers.  Taller blocks: k_gemm_q4_w32 and
// k_gemm_q4_kres below.
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
// Every weight is rebuilt exactly as bf16(scale*code + bias) (one fp32 fma,
// then v_cvt_pk_bf16_f32) and used as the B operand; one rebuild serves every
// row of the block.
//
// K slot mapping inside one MFMA: lane quarter q (lanes 16q..16q+15) supplies
// K indices g*64 + q*16 + j*8 + [0, 8) for K-step j of group g, in natural
// order, for A and B alike.
// The grid is sized from the host bound max_blocks; workgroups past the
// device-side *num_blocks exit at once, so no count goes to the host.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"

namespace moeq4 {

constexpr int kKC = 128;           // K values per pipeline stage
constexpr int kXRow = kKC + 8;     // staged activation row: 128 bf16 + 16 B pad
constexpr int kBufFlags = 0x00020000;  // raw buffer descriptor word 3 (32-bit data format)

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

// A dword of the tiled layout holds 8 consecutive codes c0..c7 with nibble p
// (bits 4p..4p+3) holding c0,c2,c4,c6,c1,c3,c5,c7 for p = 0..7, so that
// (dword >> 4i) & 0x000F000F is the pair (c_2i, c_2i+1) in the two 16-bit halves.

// exact rebuild of 8 codes as bf16 MFMA operand, natural K order (see rebuild_words)
__device__ __forceinline__ bf16x8 rebuild_dq(uint32_t wd, float s, float b) {
  const uint4 w = rebuild_words(wd, s, b);
  return as_bf16x8(w.x, w.y, w.z, w.w);
}

template <int NF, int XP>
struct Stage {
  u32x4 w[NF];      // codes: dwords 0,1 = group 2c, dwords 2,3 = group 2c+1
  uint32_t s[NF];   // scales of groups 2c (low half) and 2c+1 (high half)
  uint32_t b[NF];   // biases, same packing
  uint4 x[XP];      // activation pieces
};

constexpr int kXcds = 8;  // MI355X: workgroup i of a launch runs on XCD i % 8

// Decoded block-map entry of one workgroup; false for a malformed entry.
__device__ __forceinline__ bool gemm_block(const GemmArgs& a, int BM, int blk, int& e, int& row0, int& rows) {
  if (a.blocks) {
    e = a.blocks[4 * blk + 0];
    row0 = a.blocks[4 * blk + 1];
    rows = min(a.blocks[4 * blk + 2], BM);
  } else {  // dense: BM-row blocks over all A rows of expert 0
    e = 0;
    row0 = blk * BM;
    rows = min(BM, a.A - row0);
  }
  return !(e < 0 || e >= a.E || row0 < 0 || rows <= 0 || row0 + rows > a.A);
}

__device__ __forceinline__ int gemm_nblocks(const GemmArgs& a, int BM) {
  return a.blocks ? *a.num_blocks : (a.A + BM - 1) / BM;
}

// gemm_task + gemm_block in one: the task slot does not depend on the routed
// block count, so the count and the block-map entry (at a clamped index) are
// read together instead of one after the other.  Returns false when the
// workgroup has no task or the entry is malformed.
__device__ __forceinline__ bool gemm_task_entry(const GemmArgs& a0, int BM, int ntiles, bool& dense, int& blk,
                                                int& ntile, int& e, int& row0, int& rows) {
  const int dblocks = (a0.d_rows + BM - 1) / BM;
  gemm_task(dblocks, 0x7FFFFFFF, ntiles, dense, blk, ntile);
  int nb, A = a0.A, E = a0.E;
  if (dense || !a0.blocks) {
    A = dense ? a0.d_rows : a0.A;
    E = dense ? 1 : a0.E;
    nb = dense ? dblocks : (A + BM - 1) / BM;
    e = 0;
    row0 = blk * BM;
    rows = min(BM, A - row0);
  } else {
    const int cap = max(a0.max_blocks, 1) - 1;
    int cb = min(blk, cap);
    nb = *a0.num_blocks;
    if (a0.order) cb = min(max(a0.order[cb], 0), cap);  // past the count: unwritten, never used
    e = a0.blocks[4 * cb + 0];
    row0 = a0.blocks[4 * cb + 1];
    rows = min(a0.blocks[4 * cb + 2], BM);
  }
  if (blk >= nb) return false;
  return !(e < 0 || e >= E || row0 < 0 || rows <= 0 || row0 + rows > A);
}

// byte offset of sorted row p's activations in X
__device__ __forceinline__ int gemm_xrow(const GemmArgs& a, int p) {
  return (a.gather ? a.gather[p] / a.k : p) * a.K * 2;
}

// Byte offsets in X of block rows r[i] (clamped into the block: rows past it
// get their offset replaced by the caller) for the N rows a thread stages.  The
// gather branch is outside the loop, so the N index loads go out back to back
// and are waited for once (a load inside a per-row branch is waited for before
// the branch rejoins).
template <int N>
__device__ __forceinline__ void gemm_xrows(const GemmArgs& a, int row0, int rows, const int (&r)[N], int (&g)[N]) {
  if (a.gather) {
    int v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = a.gather[row0 + min(r[i], rows - 1)];
#pragma unroll
    for (int i = 0; i < N; ++i) g[i] = v[i] / a.k * a.K * 2;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) g[i] = (row0 + min(r[i], rows - 1)) * a.K * 2;
  }
}

// Per-workgroup table of the kEpiScale rows: the assignment each sorted row
// goes back to and its routing weight, read once before the main loop (the
// epilogue then needs no dependent global loads between its stores).
struct EpiTab {
  int as[256];
  float w[256];
};

// f(std::integral_constant<int, m>) with m = clamp(mfa, 1, M): the number of
// filled 32-row tiles of a block as a compile-time constant (one copy of the
// caller's loop per value)
template <int M, typename F>
__device__ __forceinline__ void with_mfa(int mfa, F&& f) {
  if constexpr (M <= 1) {
    f(std::integral_constant<int, 1>{});
  } else {
    if (mfa >= M) f(std::integral_constant<int, M>{});
    else with_mfa<M - 1>(mfa, f);
  }
}

template <int EPI>
__device__ __forceinline__ void epi_fill(const GemmArgs& a, int row0, int rows, EpiTab* tab) {
  if constexpr (EPI == kEpiScale) {
    for (int r = threadIdx.x; r < rows; r += blockDim.x) {
      if (!a.perm) {  // dense problem: rows keep their index, weight 1
        tab->as[r] = row0 + r;
        tab->w[r] = 1.f;
        continue;
      }
      const int as = a.perm[row0 + r];
      const bool ok = as >= 0 && as < a.A;  // a malformed permutation writes nothing
      tab->as[r] = ok ? as : -1;
      tab->w[r] = ok ? a.topk_w[as] : 0.f;
    }
  }
}

// elements 4j..4j+3 of a 32x32 MFMA accumulator (j compile-time after unrolling)
__device__ __forceinline__ f32x4 quad(const f32x16& a, int j) {
  return f32x4{a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]};
}

// silu(g) * u = g * u / (1 + e^-g), with the hardware exponential and
// reciprocal (each within a few fp32 ulp; the result is then rounded to bf16).
// g -> -inf: e^-g = inf, reciprocal 0, result -0; g -> +inf: e^-g = 0, result g * u.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

// Epilogue of one output row (row `row` of the block starting at sorted row row0).
template <int EPI>
struct EpiRow {
  uint16_t* y;    // output row (null: not written)
  float w;        // kEpiScale: routing weight of the row's assignment
  __device__ __forceinline__ EpiRow(uint16_t* Y, int ldy, int row0, int row, const EpiTab* tab) {
    if constexpr (EPI == kEpiScale) {
      const int as = tab->as[row];
      y = as >= 0 ? Y + (size_t)as * ldy : nullptr;
      w = tab->w[row];
    } else {
      y = Y + (size_t)(row0 + row) * ldy;
      w = 1.f;
    }
  }
  // value v of output column n (g, u for kEpiSwiglu)
  __device__ __forceinline__ void store(int n, float v, float u = 0.f) const {
    if constexpr (EPI == kEpiScale) {
      if (!y) return;
    }
    if constexpr (EPI == kEpiSwiglu) {
      y[n] = f32_to_bf16_bits(silu_mul(v, u));
    } else if constexpr (EPI == kEpiScale) {
      y[n] = term_bits(w * v);
    } else if constexpr (EPI == kEpiTerm) {
      y[n] = term_bits(v);
    } else {
      y[n] = f32_to_bf16_bits(v);
    }
  }
  // the 16-bit outputs of values v[0..3] (and u[0..3] for kEpiSwiglu), packed
  __device__ __forceinline__ uint2 pack4(f32x4 v, f32x4 u) const {
    uint32_t b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (EPI == kEpiSwiglu) b[q] = f32_to_bf16_bits(silu_mul(v[q], u[q]));
      else if constexpr (EPI == kEpiScale) b[q] = term_bits(w * v[q]);
      else if constexpr (EPI == kEpiTerm) b[q] = term_bits(v[q]);
      else b[q] = f32_to_bf16_bits(v[q]);
    }
    return make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
  }
  // values of output columns n..n+3 (n % 4 == 0), written with one 8-byte store
  __device__ __forceinline__ void store4(int n, f32x4 v, f32x4 u) const {
    if constexpr (EPI == kEpiScale) {
      if (!y) return;
    }
    *(uint2*)(y + n) = pack4(v, u);
  }
  // 8 packed outputs of columns n..n+7 (n % 8 == 0), one 16-byte store
  __device__ __forceinline__ void store8(int n, uint4 bits) const {
    if constexpr (EPI == kEpiScale) {
      if (!y) return;
    }
    *(uint4*)(y + n) = bits;
  }
};

template <int BM, int NF, int S, int WAVES, int EPI>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_q4(const GemmArgs a) {
  static_assert(EPI != kEpiSwiglu || NF % 2 == 0, "SwiGLU pairs gate and up fragments");
  constexpr int MF = BM / 16;
  constexpr int NFO = EPI == kEpiSwiglu ? NF / 2 : NF;  // output fragments per wave
  const int K = a.K, N = a.N;
  const uint8_t* __restrict__ Wt = a.Wt;
  const uint16_t* __restrict__ St = a.St;
  const uint16_t* __restrict__ Bt = a.Bt;
  const int NOUT = EPI == kEpiSwiglu ? N / 2 : N;  // output columns
  constexpr int NTHR = WAVES * 64;
  constexpr int XP = (BM * (kKC / 8) + NTHR - 1) / NTHR;  // 16-B activation pieces per thread per stage
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kXRow];

  // XCD-aware task order (gemm_task): the N tiles of a block, which gather the
  // same activation rows, run on one XCD; blocks go round-robin over the XCDs.
  // Tasks past the device-side block count exit.
  const int ntiles = (NOUT + WAVES * NFO * 16 - 1) / (WAVES * NFO * 16);
  bool dense;
  int blk, ntile;
  if (!gemm_task(0, gemm_nblocks(a, BM), ntiles, dense, blk, ntile)) return;
  int e, row0, rows;
  if (!gemm_block(a, BM, blk, e, row0, rows)) return;  // malformed entry
  static_assert(BM <= 256, "the epilogue table holds 256 rows");
  __shared__ EpiTab ep_tab;
  epi_fill<EPI>(a, row0, rows, &ep_tab);
  uint16_t* const Yout = a.Y;
  const int ldy = a.ldy;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int quarter = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_wave = ntile * (WAVES * NFO * 16) + wave * NFO * 16;  // first output column of the wave
  const int G = K / kGroup;
  const int nfull = G >> 1;            // chunks holding two groups
  const bool odd_tail = (G & 1) != 0;  // one more chunk with a single group
  const int mfa = (rows + 15) >> 4;
  const int NT = N / 16;

  // ---- buffer resources: one expert's weights (chunk-major tiled layout); the activations
  const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Wt + (size_t)e * N * (K / 2)), (short)0, N * (K / 2), kBufFlags);
  const __amdgpu_buffer_rsrc_t ssrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(St + (size_t)e * N * G), (short)0, N * G * 2, kBufFlags);
  const __amdgpu_buffer_rsrc_t bsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Bt + (size_t)e * N * G), (short)0, N * G * 2, kBufFlags);
  const __amdgpu_buffer_rsrc_t xsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.X, (short)0, a.xrows * K * 2, kBufFlags);

  // Fragments past the output columns still load (from the last tile, so every
  // address stays inside the expert's weights) and run their MFMAs, but are not
  // stored.  SwiGLU: fragment f < NF/2 holds gate columns, f + NF/2 the up
  // columns NOUT further on.
  const int nf_live = min(NFO, max(0, (NOUT - n_wave) / 16));
  int tile[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int n = f < NFO ? n_wave + f * 16 : NOUT + n_wave + (f - NFO) * 16;
    tile[f] = min(n / 16, NT - 1);
  }

  // per-thread activation pieces: byte offset of (activation row, 16-B column).
  // Rows past the block get an offset past the buffer: the buffer load returns
  // zeros without touching memory.
  const int x_oob = a.xrows * K * 2;
  int xoff[XP], xr[XP], xg[XP];
#pragma unroll
  for (int i = 0; i < XP; ++i) xr[i] = (tid + i * NTHR) >> 4;
  gemm_xrows(a, row0, rows, xr, xg);
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int p = tid + i * NTHR;
    const int r = p >> 4, col = p & 15;
    xoff[i] = (r < rows && p < BM * 16) ? xg[i] + col * 16 : x_oob;
  }

  Stage<NF, XP> st[S];
  // full chunk c (clamped to the last full chunk): every lane loads, no branches,
  // so the compiler's wait counts stay exact across the ring
  auto load = [&](Stage<NF, XP>& s, int c) __attribute__((always_inline)) {
    const int cl = min(c, nfull - 1);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int soff = (cl * NT + tile[f]) * 1024;
      const int goff = (cl * NT + tile[f]) * 64;
      s.w[f] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, lane * 16, soff, 0);
      s.s[f] = __builtin_amdgcn_raw_buffer_load_b32(ssrc, (lane & 15) * 4, goff, 0);
      s.b[f] = __builtin_amdgcn_raw_buffer_load_b32(bsrc, (lane & 15) * 4, goff, 0);
    }
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(xsrc, xoff[i], cl * kKC * 2, 0);
      s.x[i] = make_uint4(r[0], r[1], r[2], r[3]);
    }
  };
  // the single-group chunk that ends an odd G
  auto load_tail = [&](Stage<NF, XP>& s) __attribute__((always_inline)) {
    const int c = nfull;
    typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int soff = c * NT * 1024 + tile[f] * 512;
      const int goff = (c * NT * 32 + tile[f] * 16) * 2;
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wsrc, lane * 8, soff, 0);
      s.w[f] = u32x4{v[0], v[1], 0u, 0u};
      s.s[f] = __builtin_amdgcn_raw_buffer_load_b16(ssrc, (lane & 15) * 2, goff, 0);
      s.b[f] = __builtin_amdgcn_raw_buffer_load_b16(bsrc, (lane & 15) * 2, goff, 0);
    }
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int col = (tid + i * NTHR) & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < 8) {
        const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(xsrc, xoff[i], c * kKC * 2, 0);
        v = make_uint4(r[0], r[1], r[2], r[3]);
      }
      s.x[i] = v;
    }
  };
  auto store_x = [&](const Stage<NF, XP>& s, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = tid + i * NTHR;
      const int r = p >> 4, col = p & 15;
      if (XP * NTHR == BM * 16 || p < BM * 16) *(uint4*)(&xs[buf][r * kXRow + col * 8]) = s.x[i];
    }
  };

  f32x4 acc[MF][NF];
#pragma unroll
  for (int r = 0; r < MF; ++r)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[r][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MFA > 0: exactly MFA row sub-tiles (straight-line code); MFA == 0: `mfa` at run time
  auto compute = [&](auto mfa_c, int buf, const Stage<NF, XP>& s, int ngroups) __attribute__((always_inline)) {
    constexpr int MFA = decltype(mfa_c)::value;
    constexpr int RMAX = MFA > 0 ? MFA : MF;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      if (gi >= ngroups) break;
      bf16x8 bfr[NF][2];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const float sv = gi ? __uint_as_float(s.s[f] & 0xFFFF0000u) : __uint_as_float(s.s[f] << 16);
        const float bv = gi ? __uint_as_float(s.b[f] & 0xFFFF0000u) : __uint_as_float(s.b[f] << 16);
        bfr[f][0] = rebuild_dq(s.w[f][2 * gi], sv, bv);
        bfr[f][1] = rebuild_dq(s.w[f][2 * gi + 1], sv, bv);
      }
      const uint16_t* xb = &xs[buf][(lane & 15) * kXRow + gi * 64 + quarter * 16];
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        if (MFA == 0 && r >= mfa) break;
        const bf16x8 a0 = *(const bf16x8*)(xb + r * 16 * kXRow);
        const bf16x8 a1 = *(const bf16x8*)(xb + r * 16 * kXRow + 8);
#pragma unroll
        for (int f = 0; f < NF; ++f)
          acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bfr[f][0], acc[r][f], 0, 0, 0);
#pragma unroll
        for (int f = 0; f < NF; ++f)
          acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bfr[f][1], acc[r][f], 0, 0, 0);
      }
    }
  };

  // ---- pipeline over the full chunks.  Chunk c is loaded into register
  // stage c % S at iteration c - (S-1); its activations go to LDS buffer c & 1
  // at iteration c - 1 and its MFMAs run at iteration c.  Loads complete in
  // issue order, so the activation wait at iteration c - 1 only covers loads
  // issued S-2 iterations earlier, never the newer prefetches.  Iterations past
  // the last chunk (when S does not divide it) reload the last chunk and skip
  // the MFMAs.
  auto run = [&](auto mfa_c) __attribute__((always_inline)) {
    if (nfull > 0) {
#pragma unroll
      for (int s = 0; s < S - 1; ++s) load(st[s], s);
      store_x(st[0], 0);
      __syncthreads();
      for (int c0 = 0; c0 < nfull; c0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
          const int c = c0 + u;
          load(st[(u + S - 1) % S], c + S - 1);
          store_x(st[(u + 1) % S], (c + 1) & 1);
          if (c < nfull) compute(mfa_c, c & 1, st[u], 2);
          __syncthreads();
        }
      }
    }
    if (odd_tail) {
      load_tail(st[0]);
      store_x(st[0], 0);
      __syncthreads();
      compute(mfa_c, 0, st[0], 1);
    }
  };
  // blocks of up to 32 rows: one copy of the loop per filled sub-tile count
  if constexpr (MF <= 2) {
    if (mfa == MF) run(std::integral_constant<int, MF>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 0>{});
  }

  // ---- epilogue: lane holds rows 4*quarter + i of column lane&15 of each fragment
#pragma unroll
  for (int r = 0; r < MF; ++r) {
    if (r >= mfa) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r * 16 + quarter * 4 + i;
      if (row >= rows) continue;
      const EpiRow<EPI> er(Yout, ldy, row0, row, &ep_tab);
#pragma unroll
      for (int f = 0; f < NFO; ++f) {
        if (f >= nf_live) break;
        const int n = n_wave + f * 16 + (lane & 15);
        if constexpr (EPI == kEpiSwiglu) er.store(n, acc[r][f][i], acc[r][f + NFO][i]);
        else er.store(n, acc[r][f][i]);
      }
    }
  }
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it
// does not wait for the wave's global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// The routing tables of a launch that routes, by one workgroup of NTHR
// threads: counts, offsets, the block map of BM-row blocks and its count,
// from a histogram of the ids (LDS atomics) and one scan over the experts in
// order (thread t takes experts [t*EPT, t*EPT + EPT)).  lds: at least
// MOEQ4_MAX_EXPERTS + 2 * NTHR / 64 ints.
template <int BM, int NTHR>
__device__ void route_tables(const GemmArgs& a, int* lds) {
  constexpr int NW = NTHR / 64;
  constexpr int EPT = (MOEQ4_MAX_EXPERTS + NTHR - 1) / NTHR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int A = a.A, E = a.E;
  int* const hist = lds;
  int* const part = lds + MOEQ4_MAX_EXPERTS;  // [2][NW] wave totals of rows and blocks
  for (int j = tid; j < E; j += NTHR) hist[j] = 0;
  lds_barrier();
  constexpr int U = 8;  // loads in flight per thread
  for (int i0 = 0; i0 < A; i0 += U * NTHR) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = a.ids[min(i0 + u * NTHR + tid, A - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + u * NTHR + tid < A) atomicAdd(&hist[min(max(v[u], 0), E - 1)], 1);
  }
  lds_barrier();
  int c[EPT], nb[EPT], sc = 0, sb = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid * EPT + j;
    c[j] = e < E ? hist[e] : 0;
    nb[j] = (c[j] + BM - 1) / BM;
    sc += c[j];
    sb += nb[j];
  }
  int ic = sc, ib = sb;  // inclusive scans over the wave's lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int tc = __shfl_up(ic, o), tb = __shfl_up(ib, o);
    if (lane >= o) {
      ic += tc;
      ib += tb;
    }
  }
  if (lane == 63) {
    part[wave] = ic;
    part[NW + wave] = ib;
  }
  lds_barrier();
  int oc = ic - sc, ob = ib - sb, nbt = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) {
      oc += part[w];
      ob += part[NW + w];
    }
    nbt += part[NW + w];
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid * EPT + j;
    if (e < E) {
      a.r_counts[e] = c[j];
      a.r_offsets[e] = oc;
      for (int b = 0; b < nb[j]; ++b)
        *(int4*)&a.r_blocks[4 * (size_t)(ob + b)] = make_int4(e, oc + b * BM, min(BM, c[j] - b * BM), b);
    }
    oc += c[j];
    ob += nb[j];
  }
  if (tid == 0) {
    a.r_offsets[E] = A;
    *a.r_num_blocks = nbt;
  }
}

// ---------------------------------------------------------------------------
// Tall blocks (64/128/256 rows): bf16 MFMA 32x32x16, exact bf16 rebuild (DQ).
//
// One wave covers every row of the block (BM/32 row tiles) and NF32 tiles of
// 32 columns, so each rebuilt weight feeds BM/32 MFMAs, and the 32x32x16 MFMA
// keeps the matrix cores busy with only a few independent accumulators.  With
// SwiGLU and NF32 == 1 the wave's one tile pairs 16 gate columns (tile rows
// 0..15) with their 16 up columns (rows 16..31); in the transposed accumulator
// a lane then holds gate element i and its up partner at i + 8.  The
// weights come from the same tiled layout: for 32-column tile u, lane
// l = 32h + n (h in 0..1, n in 0..31) loads the two 16-byte quarter slices
// q = 2h and 2h+1 of column n%16 of 16-row tile 2u + n/16, i.e. 32 codes of
// K indices 32h + [0,32) in each of the chunk's two groups.  K-step s4 of group
// g then takes K indices g*64 + 32h + 8*s4 + [0,8) from lane half h, for both
// operands, so every K-step stays inside one scale group.
// OCC: workgroups per CU the kernel is sized for (registers and LDS)
// FR: routing in the launch (section "Keep expert routing on the GPU"): the
// tasks are experts instead of block-map entries; a workgroup ranks its
// expert's assignments from the top-k ids (the stable counting sort), writes
// that expert's part of perm and inv_perm, and runs the expert's rows BM at a
// time; the grid's last workgroup writes counts, offsets and the block map
// (route_tables).  The outputs are those of the routing kernels followed by
// the same launch without FR.
template <int BM, int NF32, int S, int WAVES, int EPI, int OCC, bool FR = false>
__global__ __launch_bounds__(WAVES * 64, OCC) void k_gemm_q4_w32(const GemmArgs a0) {
  constexpr bool PAIRED = EPI == kEpiSwiglu && NF32 == 1;  // gate and up in one tile
  static_assert(EPI != kEpiSwiglu || NF32 % 2 == 0 || PAIRED, "SwiGLU pairs gate and up fragments");
  constexpr int MF32 = BM / 32;
  constexpr int NTHR = WAVES * 64;
  constexpr int NFO = EPI == kEpiSwiglu && !PAIRED ? NF32 / 2 : NF32;  // output fragments per wave
  constexpr int OUTF = PAIRED ? 16 : 32;                                // output columns per fragment
  constexpr int TILE_N = WAVES * NFO * OUTF;                            // output columns per workgroup
  // activation buffers in LDS: three (the DMA runs two chunks ahead) for one
  // workgroup per CU of up to 128 rows; two where that would not fit or where
  // two workgroups share a CU (2 x 66 KB for 128 rows)
  constexpr int NBUF = BM <= 128 && OCC == 1 ? 3 : 2;
  // Activations reach LDS by DMA (buffer_load ... lds): each wave instruction
  // fills 1 KB = 4 rows of 256 B.  In row r, 16-byte slot s holds the row's
  // 16-byte column s ^ (r & 15), so that the 32 rows an MFMA operand read
  // touches sit in distinct banks.
  constexpr int IPW = BM * 16 / 64 / WAVES;  // DMA instructions per wave per chunk
  static_assert(IPW * 64 * WAVES == BM * 16, "rows split evenly over the waves");
  (void)NTHR;
  __shared__ __attribute__((aligned(16))) uint16_t xs[NBUF][BM * kKC];
  const int NOUT = EPI == kEpiSwiglu ? a0.N / 2 : a0.N;
  const int ntiles = (NOUT + TILE_N - 1) / TILE_N;
  bool dense;
  int blk, ntile, e, row0, rows;
  if constexpr (FR) {  // one expert per task; its rows come from the routing below
    if (blockIdx.x == gridDim.x - 1) {  // the last workgroup writes the other routing tables
      static_assert(!FR || (MOEQ4_MAX_EXPERTS + 2 * WAVES) * 4 <= (int)sizeof(xs), "table scratch fits");
      route_tables<BM, NTHR>(a0, reinterpret_cast<int*>(&xs[0][0]));
      return;
    }
    if (!gemm_task(0, a0.E, ntiles, dense, blk, ntile)) return;
    e = blk;
    row0 = 0;
    rows = 1;
  } else {
    if (!gemm_task_entry(a0, BM, ntiles, dense, blk, ntile, e, row0, rows)) return;
  }
  const GemmArgs a = dense ? gemm_dense(a0) : a0;
  const int K = a.K, N = a.N;
  const uint8_t* __restrict__ Wt = a.Wt;
  const uint16_t* __restrict__ St = a.St;
  const uint16_t* __restrict__ Bt = a.Bt;
  static_assert(BM <= 256 && BM <= WAVES * 64, "the epilogue table holds 256 rows, one per thread");
  // the epilogue table lives in the last bytes of the activation buffers,
  // written once the main loop is done with them
  EpiTab* const ep_tab = reinterpret_cast<EpiTab*>(reinterpret_cast<char*>(&xs[0][0]) + sizeof(xs) - sizeof(EpiTab));
  uint16_t* const Yout = a.Y;
  const int ldy = a.ldy;

  const int tid = threadIdx.x;
  // kEpiScale: thread tid's row of the epilogue table (assignment and routing
  // weight of block row tid).  The assignment is read first, the weight once
  // the main loop's first loads are out, and the table is written to LDS only
  // before the epilogue, so neither read delays the first MFMAs.
  int ep_as = row0 + tid;
  float ep_w = 1.f;
  const int lane = tid & 63;
  const int half = lane >> 5;   // K half inside a K-step
  const int col = lane & 31;    // column inside a 32-column tile
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_wave = ntile * TILE_N + wave * NFO * OUTF;  // first output column of the wave
  const int G = K / kGroup;
  const int nfull = G >> 1;
  const bool odd_tail = (G & 1) != 0;
  int mfa = (rows + 31) >> 5;  // row tiles holding rows
  const int NT = N / 16;

  const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Wt + (size_t)e * N * (K / 2)), (short)0, N * (K / 2), kBufFlags);
  const __amdgpu_buffer_rsrc_t ssrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(St + (size_t)e * N * G), (short)0, N * G * 2, kBufFlags);
  const __amdgpu_buffer_rsrc_t bsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Bt + (size_t)e * N * G), (short)0, N * G * 2, kBufFlags);
  const __amdgpu_buffer_rsrc_t xsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.X, (short)0, a.xrows * K * 2, kBufFlags);

  // this lane's 16-row tile per 32-column tile (clamped inside the expert: columns
  // past the output load the last tile and are never stored) and its row inside
  // that tile.  SwiGLU: fragment f < NF32/2 holds gate columns, f + NF32/2 the up
  // columns NOUT further on.
  int tile16[NF32];
#pragma unroll
  for (int f = 0; f < NF32; ++f) {
    int n;
    if constexpr (PAIRED) n = col < 16 ? n_wave + col : NOUT + n_wave + (col - 16);
    else n = f < NFO ? n_wave + f * 32 + col : NOUT + n_wave + (f - NFO) * 32 + col;
    tile16[f] = min(n >> 4, NT - 1);
  }
  const int r16 = col & 15;

  const int x_oob = a.xrows * K * 2;  // rows past the block: the load returns zeros, no traffic
  // this lane's DMA source per instruction: row rb + lane/16, 16-byte column
  // (lane & 15) ^ (row & 15) of it
  int xoff[IPW], xr[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) xr[i] = 4 * (wave * IPW + i) + (lane >> 4);
  if constexpr (!FR) {
    int xg[IPW];
    gemm_xrows(a, row0, rows, xr, xg);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = xr[i];
      const int c16 = (lane & 15) ^ (r & 15);
      xoff[i] = r < rows ? xg[i] + c16 * 16 : x_oob;
    }
  }
  if constexpr (EPI == kEpiScale)
    if (a.perm) ep_as = a.perm[row0 + min(tid, rows - 1)];
  // the routing weight of the row, read behind the main loop's first loads
  auto ep_weight = [&]() __attribute__((always_inline)) {
    if constexpr (EPI == kEpiScale) {
      const bool ok = ep_as >= 0 && ep_as < a.A;  // a malformed permutation entry writes nothing
      if (a.perm) ep_w = a.topk_w[ok ? ep_as : 0];
      if (!ok) ep_as = -1;
    }
  };
  typedef __attribute__((address_space(3))) void lds_void;
  // activations of chunk c (K values [128c, 128c + 128)) into LDS buffer buf.
  // The tail chunk of an odd G has only 8 columns: the other slots get the
  // out-of-range offset (the range check covers the vector offset only, so the
  // row must not be overrun through the chunk offset).
  // instruction i (0..IPW-1) of dma_x(c, buf, false) on its own
  auto dma_op = [&](int c, int buf, int i) __attribute__((always_inline)) {
    const int off = xoff[i];  // (passing xoff[i] itself drops the kernel's host-side stub)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrc, (lds_void*)&xs[buf][4 * (wave * IPW + i) * kKC], 16, off,
                                             c * kKC * 2, 0, 0);
  };
  auto dma_x = [&](int c, int buf, bool tail) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = 4 * (wave * IPW + i) + (lane >> 4);
      const int off = (tail && ((lane & 15) ^ (r & 15)) >= 8) ? x_oob : xoff[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrc, (lds_void*)&xs[buf][4 * (wave * IPW + i) * kKC], 16, off,
                                               c * kKC * 2, 0, 0);
    }
  };

  struct St32 {
    u32x4 w[NF32][2];   // quarter slices 2h and 2h+1
    uint32_t s[NF32], b[NF32];
  };
  St32 st[S];
  auto load = [&](St32& s, int c) __attribute__((always_inline)) {
    const int cl = min(c, nfull - 1);
#pragma unroll
    for (int f = 0; f < NF32; ++f) {
      const int base = (cl * NT + tile16[f]) * 1024 + r16 * 16;
      s.w[f][0] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, base + (2 * half) * 256, 0, 0);
      s.w[f][1] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, base + (2 * half + 1) * 256, 0, 0);
      const int gbase = ((cl * NT + tile16[f]) * 32 + 2 * r16) * 2;
      s.s[f] = __builtin_amdgcn_raw_buffer_load_b32(ssrc, gbase, 0, 0);
      s.b[f] = __builtin_amdgcn_raw_buffer_load_b32(bsrc, gbase, 0, 0);
    }
  };
  // instruction j (0..4*NF32-1) of load(s, c) on its own: fragment j/4, part j%4
  auto load_op = [&](St32& s, int c, int j) __attribute__((always_inline)) {
    const int cl = min(c, nfull - 1);
    const int f = j >> 2, part = j & 3;
    const int base = (cl * NT + tile16[f]) * 1024 + r16 * 16;
    const int gbase = ((cl * NT + tile16[f]) * 32 + 2 * r16) * 2;
    if (part < 2) s.w[f][part] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, base + (2 * half + part) * 256, 0, 0);
    else if (part == 2) s.s[f] = __builtin_amdgcn_raw_buffer_load_b32(ssrc, gbase, 0, 0);
    else s.b[f] = __builtin_amdgcn_raw_buffer_load_b32(bsrc, gbase, 0, 0);
  };
  auto load_tail = [&](St32& s) __attribute__((always_inline)) {
    const int c = nfull;
    typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
#pragma unroll
    for (int f = 0; f < NF32; ++f) {
      const int base = c * NT * 1024 + tile16[f] * 512 + r16 * 8;
      const u32x2 v0 = __builtin_amdgcn_raw_buffer_load_b64(wsrc, base + (2 * half) * 128, 0, 0);
      const u32x2 v1 = __builtin_amdgcn_raw_buffer_load_b64(wsrc, base + (2 * half + 1) * 128, 0, 0);
      s.w[f][0] = u32x4{v0[0], v0[1], 0u, 0u};
      s.w[f][1] = u32x4{v1[0], v1[1], 0u, 0u};
      const int gbase = (c * NT * 32 + tile16[f] * 16 + r16) * 2;
      s.s[f] = __builtin_amdgcn_raw_buffer_load_b16(ssrc, gbase, 0, 0);
      s.b[f] = __builtin_amdgcn_raw_buffer_load_b16(bsrc, gbase, 0, 0);
    }
  };

  f32x16 acc[MF32][NF32];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < MF32; ++r)
#pragma unroll
      for (int f = 0; f < NF32; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][f][i] = 0.f;
  };
  if constexpr (!FR) zero_acc();  // (routing in the launch: at the start of each pass)

  // K-step ks (0..7) of a chunk: K indices 64*(ks/4) + 32*half + 8*(ks%4) + [0,8) of the
  // chunk, from lane half `half`, for the activations (LDS, row col + 32 per row
  // tile, swizzled 16-byte column) and the rebuilt weights alike
  auto load_a = [&](auto mfa_c, bf16x8* av, int buf, int ks) __attribute__((always_inline)) {
    constexpr int MFA = decltype(mfa_c)::value;
    const int gi = ks >> 2, s4 = ks & 3;
    const uint16_t* xb = &xs[buf][col * kKC + (((gi * 8 + half * 4 + s4) ^ (col & 15)) * 8)];
#pragma unroll
    for (int r = 0; r < MFA; ++r) av[r] = *(const bf16x8*)(xb + r * 32 * kKC);
  };
  auto rebuild_b = [&](bf16x8* bw, const St32& s, int ks) __attribute__((always_inline)) {
    const int gi = ks >> 2, s4 = ks & 3;
#pragma unroll
    for (int f = 0; f < NF32; ++f) {
      const float sv = gi ? __uint_as_float(s.s[f] & 0xFFFF0000u) : __uint_as_float(s.s[f] << 16);
      const float bv = gi ? __uint_as_float(s.b[f] & 0xFFFF0000u) : __uint_as_float(s.b[f] << 16);
      bw[f] = rebuild_dq(s.w[f][s4 >> 1][2 * gi + (s4 & 1)], sv, bv);
    }
  };
  auto mfma_step = [&](auto mfa_c, const bf16x8* av, const bf16x8* bw) __attribute__((always_inline)) {
    constexpr int MFA = decltype(mfa_c)::value;
#pragma unroll
    for (int r = 0; r < MFA; ++r)
#pragma unroll
      for (int f = 0; f < NF32; ++f)
        acc[r][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[f], av[r], acc[r][f], 0, 0, 0);
  };

  // Pipeline over the full chunks.  With three LDS buffers, iteration c first
  // sends the weight loads of chunk c+S-1 and then the DMA of chunk c+2's
  // activations (into the buffer chunk c-1 used); with two, the DMA of chunk
  // c+1 and then the weight loads.  Then chunk c's MFMAs run, then the wave
  // waits until only the loads that iteration c+1 does not need are still in
  // flight (vector memory operations complete in issue order, so this is a
  // count) and the iteration ends in a barrier, after which every wave's part
  // of chunk c+1 is in LDS.  Inside a chunk the K-steps are software pipelined
  // one step deep: while the MFMAs of a step run, the next step's activation
  // fragments are read from LDS and its weights rebuilt into the other register
  // set; each step ends in a scheduling barrier that keeps this order.  Loads
  // and DMAs past the last chunk re-read it (clamped) and are not used.
  constexpr int kLoadsPerChunk = 4 * NF32;  // vector memory instructions of load()
  constexpr int kAhead = NBUF - 1;           // chunks the DMA runs ahead
  constexpr int kInFlight = (NBUF == 3 ? IPW : 0) + (S > 2 ? kLoadsPerChunk : 0);
  static_assert(kInFlight < 64, "vmcnt range");
  // The next chunks' loads are issued a few per K-step over the first kSpread
  // K-steps, after that step's MFMAs, not all at the top of the chunk: issued
  // together, the workgroup's waves queue behind each other at the vector
  // memory unit and none of them reaches its MFMAs meanwhile.  The order is
  // that of the burst it replaces (three buffers: weights, then DMA; two: DMA,
  // then weights), so the counted wait at the end of the chunk is unchanged.
  constexpr int kOps = IPW + kLoadsPerChunk;
  constexpr int kSpread = 4;
  constexpr int kPer = (kOps + kSpread - 1) / kSpread;
  auto issue_ops = [&](St32& s, int c, int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int j = ks * kPer + t;
      if (j >= kOps) break;
      const int cd = min(c + kAhead, nfull - 1), bd = (c + kAhead) % NBUF;
      if constexpr (NBUF == 3) {
        if (j < kLoadsPerChunk) load_op(s, c + S - 1, j);
        else dma_op(cd, bd, j - kLoadsPerChunk);
      } else {
        if (j < IPW) dma_op(cd, bd, j);
        else load_op(s, c + S - 1, j - IPW);
      }
    }
  };
  // Blocks of more than four row tiles hold one activation fragment at a time
  // (the next row tile's read in flight while this tile's MFMAs run) instead
  // of every row tile's fragments for two K-steps: the accumulators of five
  // row tiles leave no room for the double set.
  constexpr bool LEAN = MF32 > 4 && NF32 > 1;
  // the activation fragment of row tile 0 at K-step ks of buffer buf
  auto lean_first = [&](int buf, int ks) __attribute__((always_inline)) {
    const int gi = ks >> 2, s4 = ks & 3;
    return *(const bf16x8*)&xs[buf][col * kKC + (((gi * 8 + half * 4 + s4) ^ (col & 15)) * 8)];
  };
  // a0 holds row tile 0's fragment of K-step ks on entry and, when ks + 1 < kend,
  // row tile 0's fragment of K-step ks + 1 on return (read during the last row
  // tile's MFMAs, so no K-step starts on an LDS read it has just issued)
  auto lean_step = [&](auto mfa_c, int buf, int ks, int kend, const bf16x8* bw, bf16x8& a0) __attribute__((always_inline)) {
    constexpr int MFA = decltype(mfa_c)::value;
    const int gi = ks >> 2, s4 = ks & 3;
    const uint16_t* xb = &xs[buf][col * kKC + (((gi * 8 + half * 4 + s4) ^ (col & 15)) * 8)];
    bf16x8 a_cur = a0;
#pragma unroll
    for (int r = 0; r < MFA; ++r) {
      bf16x8 a_next = a_cur;
      if (r + 1 < MFA) a_next = *(const bf16x8*)(xb + (r + 1) * 32 * kKC);
      else if (ks + 1 < kend) a_next = lean_first(buf, ks + 1);
#pragma unroll
      for (int f = 0; f < NF32; ++f)
        acc[r][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[f], a_cur, acc[r][f], 0, 0, 0);
      a_cur = a_next;
    }
    a0 = a_cur;
  };
  auto run = [&](auto mfa_c) __attribute__((always_inline)) {
    constexpr int MFA = decltype(mfa_c)::value;
    bf16x8 av[LEAN ? 1 : 2][LEAN ? 1 : MFA];
    bf16x8 bw[2][NF32];
    if (nfull > 0) {
      if constexpr (!FR)  // (routing in the launch: issued before each pass)
#pragma unroll
        for (int s = 0; s < S - 1; ++s) load(st[s], s);
#pragma unroll
      for (int b = 0; b < kAhead; ++b) dma_x(min(b, nfull - 1), b, false);
      ep_weight();
      __syncthreads();
      for (int c0 = 0; c0 < nfull; c0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
          const int c = c0 + u;
          const int buf = c % NBUF;
          St32& nxt = st[(u + S - 1) % S];
          if (c < nfull) {
            if constexpr (LEAN) {
              rebuild_b(bw[0], st[u], 0);
              bf16x8 a0 = lean_first(buf, 0);
#pragma unroll
              for (int ks = 0; ks < 8; ++ks) {
                const int p = ks & 1;
                if (ks < 7) rebuild_b(bw[p ^ 1], st[u], ks + 1);
                lean_step(mfa_c, buf, ks, 8, bw[p], a0);
                if (ks < kSpread) issue_ops(nxt, c, ks);
                __builtin_amdgcn_sched_barrier(0);
              }
            } else {
              load_a(mfa_c, av[0], buf, 0);
              rebuild_b(bw[0], st[u], 0);
#pragma unroll
              for (int ks = 0; ks < 8; ++ks) {
                const int p = ks & 1;
                if (ks < 7) {
                  load_a(mfa_c, av[p ^ 1], buf, ks + 1);
                  rebuild_b(bw[p ^ 1], st[u], ks + 1);
                }
                mfma_step(mfa_c, av[p], bw[p]);
                if (ks < kSpread) issue_ops(nxt, c, ks);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          } else {
#pragma unroll
            for (int ks = 0; ks < kSpread; ++ks) issue_ops(nxt, c, ks);
          }
          // vmcnt <= kInFlight (expcnt and lgkmcnt unconstrained): this wave's DMA
          // of chunk c+1 has landed in LDS, and its LDS reads of this chunk have
          // all returned (their MFMAs used them); the barrier then makes every
          // wave's part of chunk c+1 visible and frees buffer c % NBUF for the
          // next DMA.  A plain s_barrier: a __syncthreads() here would also wait
          // for every DMA in flight (vmcnt(0)).
          __builtin_amdgcn_s_waitcnt((kInFlight & 15) | ((kInFlight >> 4) << 14) | (7 << 4) | (15 << 8));
          __builtin_amdgcn_s_barrier();
        }
      }
      // drain the DMAs of the clamped chunks past the end: no write into this
      // workgroup's LDS may still be in flight when it moves on (or ends)
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    }
    if (nfull == 0) ep_weight();
    if (odd_tail) {
      load_tail(st[0]);
      dma_x(nfull, 0, true);
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        rebuild_b(bw[0], st[0], ks);
        if constexpr (LEAN) {
          bf16x8 a0 = lean_first(0, ks);
          lean_step(mfa_c, 0, ks, ks + 1, bw[0], a0);
        } else {
          load_a(mfa_c, av[0], 0, ks);
          mfma_step(mfa_c, av[0], bw[0]);
        }
      }
    }
  };
  static_assert(MF32 >= 1 && MF32 <= 8, "row tiles per block");
  int r_cnt = 0, r_off = 0;  // routing in the launch: the expert's rows and its first sorted row
  // Routing in the launch keeps its state in registers and in the activation
  // buffers before each pass's first DMA: the launch needs no LDS beyond them
  // (measured: a 64-row launch with even 256 B of LDS past its 32 KB of
  // buffers runs about 10% slower).
  constexpr int RR = FR ? kRouteInLaunchMax / NTHR : 1;  // rounds of 64 assignments per wave
  int v[RR];              // this lane's expert ids, one per round
  int lim = 0, seg0 = 0;  // rounds of valid assignments of this lane; this wave's first rank
  int* const red = reinterpret_cast<int*>(&xs[0][0]);  // [2][WAVES] the waves' counts
  int* const rlp = red + 4 * WAVES;                     // [BM] the pass's rows: their tokens
  // Ranks of this lane's rows of expert e in assignment order (waves, then
  // rounds, then lanes: the stable counting sort), from the wave's ballots;
  // f(i, rank) for each.
  auto for_ranks = [&](auto&& f) __attribute__((always_inline)) {
    const uint64_t ltm = lanemask_lt();
    int run = seg0;
#pragma unroll
    for (int i = 0; i < RR; ++i) {
      const bool eq = (i < lim) & (v[i] == e);
      const uint64_t b = __ballot(eq);
      if (eq) f(i, run + (int)__popcll(b & ltm));
      run += (int)__popcll(b);
    }
  };
  // rlp = the tokens of ranks [pass*BM, pass*BM + BM)
  auto fill_pass_rows = [&](int pass) __attribute__((always_inline)) {
    const int lo = pass * BM;
    for_ranks([&](int i, int rank) {
      if (rank >= lo && rank < lo + BM) rlp[rank - lo] = (wave * RR * 64 + i * 64 + lane) / a0.k;
    });
  };
  if constexpr (FR) {
    // The expert's rows from the ids.  Wave w takes the assignments [w*Q,
    // (w+1)*Q), Q = RR*64, one per lane and round.  The expert's first weight
    // loads need no routing: they go out right behind the ids, so the waits
    // for the ids leave them in flight.  Ballots count the wave's rows of e
    // and its assignments to experts below e; the waves' counts give each
    // wave's first rank, the expert's row count and its offset.  (The ids
    // come from this call's top-k, so they lie in [0, E).)
    static_assert(!FR || (EPI == kEpiPlain && (4 * WAVES + BM) * 4 <= (int)sizeof(xs)), "routing in the launch");
    const int A = a0.A;
    constexpr int Q = RR * 64;
    const int a_w = wave * Q;
#pragma unroll
    for (int i = 0; i < RR; ++i) v[i] = a0.ids[min(a_w + i * 64 + lane, A - 1)];  // clamped: all in flight
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < S - 1; ++s) load(st[s], s);
    __builtin_amdgcn_sched_barrier(0);
    lim = min(RR, max(0, (A - a_w - lane + 63) >> 6));
    int run = 0, lt = 0;
#pragma unroll
    for (int i = 0; i < RR; ++i) {
      const bool valid = i < lim;
      lt += valid & (v[i] < e) ? 1 : 0;
      run += (int)__popcll(__ballot(valid & (v[i] == e)));
    }
    lt = wave_sum_i32(lt);
    if (lane == 0) {
      red[wave] = run;
      red[WAVES + wave] = lt;
    }
    lds_barrier();
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      seg0 += w < wave ? red[w] : 0;
      r_cnt += red[w];
      r_off += red[WAVES + w];
    }
    // this expert's part of perm and inv_perm (the other tables: the last
    // workgroup), and the first pass's rows
    // (r_off + r_cnt <= A holds for ids in [0, E); the check keeps every
    // write inside perm, inv_perm and Y whatever the ids)
    const bool in_range = r_off + r_cnt <= A;
    const bool tab = ntile == 0 && in_range;
    for_ranks([&](int i, int rank) {
      const int as = a_w + i * 64 + lane;
      if (tab) {
        a0.r_perm[r_off + rank] = as;
        a0.r_inv_perm[as] = r_off + rank;
      }
      if (rank < BM) rlp[rank] = as / a0.k;
    });
    if (r_cnt == 0 || !in_range) {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): no load left in flight
      return;
    }
    lds_barrier();
  }

  // One pass per BM rows of the expert when routing in the launch; one pass otherwise.
  for (int pass = 0;; ++pass) {
    if constexpr (FR) {
      row0 = r_off + pass * BM;
      rows = min(BM, r_cnt - pass * BM);
      mfa = (rows + 31) >> 5;
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int r = xr[i];
        const int c16 = (lane & 15) ^ (r & 15);
        const int tok = rlp[min(r, rows - 1)];
        xoff[i] = r < rows ? tok * K * 2 + c16 * 16 : x_oob;
      }
      zero_acc();
      if (pass > 0)
#pragma unroll
        for (int s = 0; s < S - 1; ++s) load(st[s], s);
      lds_barrier();  // every wave has its rows before the DMA overwrites them
    }
    with_mfa<MF32>(mfa, run);

    // epilogue: the MFMAs take the weights as the A operand, so each 32x32
    // accumulator tile is transposed: lane l holds block row r*32 + l%32 and tile
    // rows 8*(i/4) + 4*(l/32) + i%4 (i = 0..15), i.e. four runs of 4 adjacent
    // columns.  Paired SwiGLU: runs 0 and 1 are gate columns whose up partners
    // are runs 2 and 3.  Each wave converts its outputs of one 32-row tile into
    // its own staging rows in LDS (the activation buffers, free after the
    // loop), then reads them back row-wise: a lane stores 16 contiguous bytes
    // and WCOLS/8 lanes one contiguous row segment, so a store instruction
    // covers 64*8/WCOLS rows instead of 32 rows of 16 bytes each.  Only this
    // wave touches its staging rows, and a wave's LDS operations complete in
    // order, so the waits between writes and reads are the wave's own.
    constexpr int WCOLS = NFO * OUTF;  // output columns of a wave
    constexpr int SROW = WCOLS + 8;    // staged row, 16-byte pad
    constexpr int LPR = WCOLS / 8;     // lanes per staged row
    constexpr int RPI = 64 / LPR;      // rows per store instruction
    static_assert(WAVES * 32 * SROW * 2 + (int)sizeof(EpiTab) <= (int)sizeof(xs),
                  "staging and the epilogue table fit in the activation buffers");
    if constexpr (EPI == kEpiScale) {
      __syncthreads();  // every wave is done with the activation buffers
      if (tid < rows) {
        ep_tab->as[tid] = ep_as;
        ep_tab->w[tid] = ep_as >= 0 ? ep_w : 0.f;
      }
    }
    __syncthreads();  // every wave is done with the activation buffers; the table is written
    uint16_t* const stg = &xs[0][0] + wave * 32 * SROW;
#pragma unroll
    for (int r = 0; r < MF32; ++r) {
      if (r >= mfa) break;
      {
        const EpiRow<EPI> er(Yout, ldy, row0, min(r * 32 + col, rows - 1), ep_tab);
        if constexpr (PAIRED) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            *(uint2*)&stg[col * SROW + 8 * j + 4 * half] = er.pack4(quad(acc[r][0], j), quad(acc[r][0], j + 2));
        } else {
#pragma unroll
          for (int f = 0; f < NFO; ++f)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const f32x4 v = quad(acc[r][f], j);
              f32x4 u = v;
              if constexpr (EPI == kEpiSwiglu) u = quad(acc[r][f + NFO], j);
              *(uint2*)&stg[col * SROW + f * 32 + 8 * j + 4 * half] = er.pack4(v, u);
            }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int rr = i * RPI + lane / LPR, cq = lane % LPR;
        const int row = r * 32 + rr, n = n_wave + 8 * cq;
        const uint4 bits = *(const uint4*)&stg[rr * SROW + 8 * cq];
        if (row < rows && n < NOUT) EpiRow<EPI>(Yout, ldy, row0, row, ep_tab).store8(n, bits);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads back before the next tile's writes
    }
    if constexpr (!FR) {
      break;
    } else {
      if ((pass + 1) * BM >= r_cnt) break;
      __syncthreads();  // every wave's staging reads are done before the next pass's rows
      fill_pass_rows(pass + 1);
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// Short K (K <= 512, K % 128 == 0; the FFN's down projections): the block's
// activations for the whole of K stay in LDS (BM x K bf16, swizzled as in
// k_gemm_q4_w32, loaded once by DMA), and each wave then streams the weights of
// its columns through an S-stage register ring across all the N tiles of the
// workgroup's range, with no barrier in the loop.  A workgroup covers one
// block and NR output columns, so every weight of that range is rebuilt once
// per block and the activations are read once.
constexpr int kKResMax = 512;

template <int BM, int NF32, int NCH, int S, int WAVES, int EPI>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_q4_kres(const GemmArgs a0, int NR) {
  // NCH = K / 128 chunks; the register ring has S stages, S dividing NCH, so
  // that the stage of step (N tile nt, chunk c) is c % S: a compile-time index
  // in the unrolled loop
  static_assert(NCH % S == 0 && S >= 2, "ring stages divide the chunks");
  static_assert(EPI != kEpiSwiglu, "gate/up pairs columns across the whole N: not this kernel");
  constexpr int MF32 = BM / 32;
  constexpr int TILE_N = WAVES * NF32 * 32;
  constexpr int IPW = BM * 16 / 64 / WAVES;  // DMA instructions per wave per chunk
  static_assert(IPW * 64 * WAVES == BM * 16, "rows split evenly over the waves");
  extern __shared__ __attribute__((aligned(16))) uint16_t xk[];  // [K/128][BM][128]
  const int nsplit = (a0.N + NR - 1) / NR;
  bool dense;
  int blk, split;
  if (!gemm_task((a0.d_rows + BM - 1) / BM, gemm_nblocks(a0, BM), nsplit, dense, blk, split)) return;
  const GemmArgs a = dense ? gemm_dense(a0) : a0;
  const int K = a.K, N = a.N;
  const int n_lo = split * NR;
  const int n_hi = min(N, n_lo + NR);
  int e, row0, rows;
  if (!gemm_block(a, BM, blk, e, row0, rows)) return;  // malformed entry
  static_assert(BM <= 256, "the epilogue table holds 256 rows");
  __shared__ EpiTab ep_tab;
  epi_fill<EPI>(a, row0, rows, &ep_tab);
  uint16_t* const Yout = a.Y;
  const int ldy = a.ldy;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = K / kGroup;
  constexpr int nch = NCH;
  const int NT = N / 16;
  const int mfa = (rows + 31) >> 5;
  const int ntl = (n_hi - n_lo + TILE_N - 1) / TILE_N;  // N tiles of this workgroup
  const int nsteps = ntl * nch;                          // (N tile, chunk) steps, chunk fastest

  const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.Wt + (size_t)e * N * (K / 2)), (short)0, N * (K / 2), kBufFlags);  // rsrcs hold the fields
  const __amdgpu_buffer_rsrc_t ssrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.St + (size_t)e * N * G), (short)0, N * G * 2, kBufFlags);
  const __amdgpu_buffer_rsrc_t bsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.Bt + (size_t)e * N * G), (short)0, N * G * 2, kBufFlags);
  const __amdgpu_buffer_rsrc_t xsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.X, (short)0, a.xrows * K * 2, kBufFlags);

  // ---- the block's activations, all chunks, by DMA (rows past the block: zeros)
  typedef __attribute__((address_space(3))) void lds_void;
  const int x_oob = a.xrows * K * 2;
  int xr[IPW], xg[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) xr[i] = 4 * (wave * IPW + i) + (lane >> 4);
  gemm_xrows(a, row0, rows, xr, xg);
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = xr[i];
    const int c16 = (lane & 15) ^ (r & 15);
    const int off = r < rows ? xg[i] + c16 * 16 : x_oob;
    for (int c = 0; c < nch; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xsrc, (lds_void*)&xk[((size_t)c * BM + 4 * (wave * IPW + i)) * kKC], 16, off, c * kKC * 2, 0, 0);
  }

  struct StK {
    u32x4 w[NF32][2];
    uint32_t s[NF32], b[NF32];
  };
  StK st[S];
  // weights of step j (clamped to the last step: every lane loads, so the
  // compiler's wait counts stay exact)
  auto load = [&](StK& sg, int j) __attribute__((always_inline)) {
    const int jc = min(j, nsteps - 1);
    const int nt = jc / nch, c = jc - nt * nch;
    const int n_wave = n_lo + nt * TILE_N + wave * NF32 * 32;
#pragma unroll
    for (int f = 0; f < NF32; ++f) {
      const int tile16 = min((n_wave + f * 32 + col) >> 4, NT - 1);
      const int r16 = col & 15;
      const int base = (c * NT + tile16) * 1024 + r16 * 16;
      sg.w[f][0] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, base + (2 * half) * 256, 0, 0);
      sg.w[f][1] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, base + (2 * half + 1) * 256, 0, 0);
      const int gbase = ((c * NT + tile16) * 32 + 2 * r16) * 2;
      sg.s[f] = __builtin_amdgcn_raw_buffer_load_b32(ssrc, gbase, 0, 0);
      sg.b[f] = __builtin_amdgcn_raw_buffer_load_b32(bsrc, gbase, 0, 0);
    }
  };

  f32x16 acc[MF32][NF32];
  auto zero = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < MF32; ++r)
#pragma unroll
      for (int f = 0; f < NF32; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][f][i] = 0.f;
  };
  zero();

  // K-step ks (0..7) of chunk c takes K indices 128c + 64*(ks/4) + 32*half + 8*(ks%4) + [0,8)
  // from lane half `half`, for the activations (LDS) and the rebuilt weights alike
  auto load_a = [&](auto mfa_c, bf16x8* av, int c, int ks) __attribute__((always_inline)) {
    constexpr int MFA = decltype(mfa_c)::value;
    const int gi = ks >> 2, s4 = ks & 3;
    const uint16_t* xb = &xk[(size_t)c * BM * kKC] + col * kKC + (((gi * 8 + half * 4 + s4) ^ (col & 15)) * 8);
#pragma unroll
    for (int r = 0; r < MFA; ++r) av[r] = *(const bf16x8*)(xb + r * 32 * kKC);
  };
  auto rebuild_b = [&](bf16x8* bw, const StK& sg, int ks) __attribute__((always_inline)) {
    const int gi = ks >> 2, s4 = ks & 3;
#pragma unroll
    for (int f = 0; f < NF32; ++f) {
      const float sv = gi ? __uint_as_float(sg.s[f] & 0xFFFF0000u) : __uint_as_float(sg.s[f] << 16);
      const float bv = gi ? __uint_as_float(sg.b[f] & 0xFFFF0000u) : __uint_as_float(sg.b[f] << 16);
      bw[f] = rebuild_dq(sg.w[f][s4 >> 1][2 * gi + (s4 & 1)], sv, bv);
    }
  };
  auto mfma_step = [&](auto mfa_c, const bf16x8* av, const bf16x8* bw) __attribute__((always_inline)) {
    constexpr int MFA = decltype(mfa_c)::value;
#pragma unroll
    for (int r = 0; r < MFA; ++r)
#pragma unroll
      for (int f = 0; f < NF32; ++f)
        acc[r][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[f], av[r], acc[r][f], 0, 0, 0);
  };

  // transposed accumulator tiles (weights are the A operand): lane l holds block
  // row r*32 + l%32 and columns 8*(i/4) + 4*(l/32) + i%4 of each 32-column tile
  auto epilogue = [&](int nt) __attribute__((always_inline)) {
    const int n_wave = n_lo + nt * TILE_N + wave * NF32 * 32;
#pragma unroll
    for (int r = 0; r < MF32; ++r) {
      if (r >= mfa) break;
      const int row = r * 32 + col;
      if (row >= rows) continue;
      const EpiRow<EPI> er(Yout, ldy, row0, row, &ep_tab);
#pragma unroll
      for (int f = 0; f < NF32; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n_wave + f * 32 + 8 * j + 4 * half;
          if (n < n_hi) er.store4(n, quad(acc[r][f], j), quad(acc[r][f], j));
        }
    }
  };

  // Software pipeline, one K-step deep: while the MFMAs of step g run, the
  // activation fragments of step g+1 are read from LDS and its weights rebuilt
  // into the other register set.  The last step of a chunk reads the next
  // chunk's activations (or chunk 0's, for the next N tile); it also rebuilds
  // that chunk's first weights when the ring is deep enough (S > 2) for them
  // to have been loaded a chunk earlier -- with S = 2 they were sent at the
  // start of this chunk, and the first rebuild waits for the chunk boundary.
  // Each step ends in a scheduling barrier so that the compiler keeps this
  // order rather than reading LDS just before each MFMA.
  constexpr bool kCrossRebuild = S > 2;
  auto run = [&](auto mfa_c) __attribute__((always_inline)) {
    constexpr int MFA = decltype(mfa_c)::value;
    bf16x8 av[2][MFA > 0 ? MFA : 1];
    bf16x8 bw[2][NF32];
#pragma unroll
    for (int s = 0; s < S - 1; ++s) load(st[s], s);
    __syncthreads();  // the activations are in LDS (the barrier waits for the DMA)
    load_a(mfa_c, av[0], 0, 0);
    if (kCrossRebuild) rebuild_b(bw[0], st[0], 0);
    for (int nt = 0; nt < ntl; ++nt) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        // the load of step j + S - 1 into the stage step j - 1 used
        load(st[(c + S - 1) % S], nt * NCH + c + S - 1);
        asm volatile("" ::: "memory");  // keep the loads ahead of the MFMAs
        if (!kCrossRebuild) rebuild_b(bw[0], st[c % S], 0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int p = ks & 1;  // 8 steps per chunk: the parity restarts with each chunk
          const int cn = ks < 7 ? c : (c + 1) % NCH;
          load_a(mfa_c, av[p ^ 1], cn, (ks + 1) & 7);
          if (ks < 7 || kCrossRebuild) rebuild_b(bw[p ^ 1], st[cn % S], (ks + 1) & 7);
          mfma_step(mfa_c, av[p], bw[p]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      epilogue(nt);
      zero();
    }
  };
  static_assert(MF32 >= 1 && MF32 <= 4, "row tiles per block");
  with_mfa<MF32>(mfa, run);
}

namespace {

// One kernel instance per (block height, epilogue), chosen from sweeps on
// MI355X.  Blocks of 16/32 rows use the 16x16x32 kernel (8 waves, NF
// 16-column fragments per wave, an S-stage register ring), taller ones the
// 32x32x16 kernel (4 waves sized for two workgroups per CU, or 8 waves for
// 256-row blocks and the dense 128-row down projection).
struct GemmVariant {
  int bm;
  int epi;
  int tile_n;  // output columns per workgroup
  int waves;   // waves per workgroup
  const void* fn;
  bool dense;  // runs a dense second problem (GemmArgs::d_rows)
};

#define MOEQ4_GEMM16(BM, NF, S, WAVES, EPI)                                                       \
  {BM, EPI, WAVES * NF * 16 / (EPI == kEpiSwiglu ? 2 : 1), WAVES, (const void*)&k_gemm_q4<BM, NF, S, WAVES, EPI>, \
   false}
#define MOEQ4_GEMM32(BM, NF32, S, WAVES, EPI)                                                     \
  {BM, EPI, WAVES * NF32 * 32 / (EPI == kEpiSwiglu ? 2 : 1), WAVES,                              \
   (const void*)&k_gemm_q4_w32<BM, NF32, S, WAVES, EPI, (WAVES == 4 ? 2 : 1)>, true}

const GemmVariant kVariants[] = {
    MOEQ4_GEMM16(16, 2, 4, 8, kEpiPlain),
    MOEQ4_GEMM16(32, 2, 3, 8, kEpiPlain),
    MOEQ4_GEMM32(64, 2, 2, 4, kEpiPlain),
    MOEQ4_GEMM32(128, 2, 2, 4, kEpiPlain),
    MOEQ4_GEMM32(160, 2, 2, 4, kEpiPlain),
    MOEQ4_GEMM32(256, 1, 2, 8, kEpiPlain),
    // FFN: gate+up with SwiGLU, down scaled by the routing weight, shared down + combine
    MOEQ4_GEMM16(16, 2, 4, 8, kEpiSwiglu),
    MOEQ4_GEMM16(32, 2, 3, 8, kEpiSwiglu),
    MOEQ4_GEMM32(64, 2, 2, 4, kEpiSwiglu),
    MOEQ4_GEMM32(128, 2, 2, 4, kEpiSwiglu),
    MOEQ4_GEMM32(160, 2, 2, 4, kEpiSwiglu),
    MOEQ4_GEMM32(256, 1, 2, 8, kEpiSwiglu),
    MOEQ4_GEMM16(16, 2, 4, 8, kEpiScale),
    MOEQ4_GEMM16(32, 2, 3, 8, kEpiScale),
    MOEQ4_GEMM32(64, 2, 2, 4, kEpiScale),
    MOEQ4_GEMM32(128, 2, 2, 4, kEpiScale),
    MOEQ4_GEMM32(160, 2, 2, 4, kEpiScale),
    MOEQ4_GEMM32(256, 1, 2, 8, kEpiScale),
    MOEQ4_GEMM16(16, 2, 4, 8, kEpiTerm),
    MOEQ4_GEMM16(32, 2, 3, 8, kEpiTerm),
    MOEQ4_GEMM32(64, 2, 2, 4, kEpiTerm),
    MOEQ4_GEMM32(128, 1, 2, 8, kEpiTerm),
    MOEQ4_GEMM32(256, 1, 2, 8, kEpiTerm),
};
#undef MOEQ4_GEMM16
#undef MOEQ4_GEMM32

const GemmVariant* pick_variant(int bm, int epi) {
  for (const GemmVariant& v : kVariants)
    if (v.bm == bm && v.epi == epi) return &v;
  return nullptr;
}

// The short-K kernel for the FFN's down projections, 64-row blocks (for
// 128-row blocks two 4-wave tall-block workgroups per CU measured faster).
struct KresVariant {
  int bm, epi, nch, waves, tile_n;
  const void* fn;
};
#define MOEQ4_KRES(BM, NF32, NCH, S, WAVES, EPI) \
  {BM, EPI, NCH, WAVES, WAVES * NF32 * 32, (const void*)&k_gemm_q4_kres<BM, NF32, NCH, S, WAVES, EPI>}
const KresVariant kKres[] = {
    MOEQ4_KRES(64, 1, 4, 4, 8, kEpiScale),
    MOEQ4_KRES(64, 1, 4, 4, 8, kEpiTerm),
    MOEQ4_KRES(64, 1, 2, 2, 8, kEpiScale),
    MOEQ4_KRES(64, 1, 2, 2, 8, kEpiTerm),
};
#undef MOEQ4_KRES
constexpr int kNumKres = sizeof(kKres) / sizeof(kKres[0]);
static_assert(kNumKres <= 32, "one bit per variant");

int pick_kres(int bm, int epi, int nch) {
  for (int i = 0; i < kNumKres; ++i)
    if (kKres[i].bm == bm && kKres[i].epi == epi && kKres[i].nch == nch) return i;
  return -1;
}

// Per device, one bit per short-K variant whose dynamic-LDS limit has been
// raised.  Two threads may both raise it (the call is idempotent); the bit
// only saves later calls the runtime round trip.
constexpr int kMaxDevices = 64;
std::atomic<uint32_t> g_kres_raised[kMaxDevices];

hipError_t raise_kres_lds(int vi, int bytes) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) {
    note_hip_error(err, "hipGetDevice");
    return err;
  }
  const uint32_t bit = 1u << vi;
  std::atomic<uint32_t>* flag = dev >= 0 && dev < kMaxDevices ? &g_kres_raised[dev] : nullptr;
  if (flag && (flag->load(std::memory_order_acquire) & bit)) return hipSuccess;
  err = hipFuncSetAttribute(kKres[vi].fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (err != hipSuccess) {
    note_hip_error(err, "hipFuncSetAttribute(k_gemm_q4_kres)");
    return err;
  }
  if (flag) flag->fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

}  // namespace

// grid of a launch with dense_blocks dense blocks and at most max_blocks routed
// ones, ntiles N tiles each (the layout gemm_task decodes)
static dim3 task_grid(long long dense_blocks, long long max_blocks, long long ntiles) {
  return dim3((unsigned)(((dense_blocks + kXcds - 1) / kXcds + (max_blocks + kXcds - 1) / kXcds) * ntiles * kXcds));
}

// The most block-map entries any routing of A assignments over E experts can
// produce with BM-row blocks (each expert's last block may be partial).
static long long routed_block_bound(long long A, long long E, int BM) {
  const long long m = A < E ? A : E;
  return (A + m * (BM - 1)) / BM;
}

hipError_t gemm_launch(const GemmArgs& a_in, int epi, int BM, int max_blocks, hipStream_t stream) {
  // The routed grid never needs more than the bound: a larger max_blocks
  // (buffers sized for another T) only adds workgroups that would index past
  // the routing tables of this launch.
  long long mb = max(max_blocks, 0);
  if (a_in.blocks) mb = std::min(mb, routed_block_bound(a_in.A, a_in.E, BM));
  else mb = std::min(mb, (long long)(a_in.A + BM - 1) / BM);
  max_blocks = (int)mb;
  if (max_blocks == 0 && a_in.d_rows <= 0) return hipSuccess;
  GemmArgs a = a_in;
  a.max_blocks = max_blocks;
  const long long dense_blocks = a.d_rows > 0 ? (a.d_rows + BM - 1) / BM : 0;
  const int kv = a.K <= kKResMax && a.K % kKC == 0 ? pick_kres(BM, epi, a.K / kKC) : -1;
  if (kv >= 0) {
    const KresVariant& v = kKres[kv];
    // columns per workgroup: all of N, or fewer when there are too few blocks
    // to fill the GPU (the dense shared expert)
    int nsplit = max(1, min(a.N / v.tile_n, 512 / max(1, max_blocks)));
    const int NR = (a.N / nsplit + v.tile_n - 1) / v.tile_n * v.tile_n;
    nsplit = (a.N + NR - 1) / NR;
    const dim3 grid = task_grid(dense_blocks, max_blocks, nsplit);
    const size_t lds = (size_t)BM * a.K * 2;  // up to 64 KB of the 160 KB a workgroup may use
    const hipError_t err = raise_kres_lds(kv, (int)(BM * kKResMax * 2));
    if (err != hipSuccess) return err;
    return launch("k_gemm_q4_kres", v.fn, grid, dim3(v.waves * 64), lds, stream, a, NR);
  }
  const GemmVariant* v = pick_variant(BM, epi);
  if (!v || (dense_blocks > 0 && !v->dense)) return hipErrorInvalidValue;
  const int nout = epi == kEpiSwiglu ? a.N / 2 : a.N;
  const long long ntiles = (nout + v->tile_n - 1) / v->tile_n;
  return launch("k_gemm_q4", v->fn, task_grid(dense_blocks, max_blocks, ntiles), dim3(v->waves * 64), 0, stream, a);
}

hipError_t gemm_q4_launch(const uint16_t* X, int T, int K, int N, int E, int k, const uint8_t* Wt,
                          const uint16_t* St, const uint16_t* Bt, const int32_t* perm,
                          const int32_t* blocks, const int32_t* num_blocks, int max_blocks,
                          int BM, uint16_t* Y, hipStream_t stream) {
  GemmArgs a{};
  a.X = X;
  a.xrows = T;
  a.K = K;
  a.N = N;
  a.E = E;
  a.A = T * k;
  a.k = k;
  a.Wt = Wt;
  a.St = St;
  a.Bt = Bt;
  a.gather = perm;
  a.blocks = blocks;
  a.num_blocks = num_blocks;
  a.Y = Y;
  a.ldy = N;
  return gemm_launch(a, kEpiPlain, BM, max_blocks, stream);
}

hipError_t route_gemm_q4_launch(const int32_t* ids, const uint16_t* X, int T, int K, int N, int E, int k,
                                const uint8_t* Wt, const uint16_t* St, const uint16_t* Bt, int32_t* counts,
                                int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* blocks,
                                int32_t* num_blocks, uint16_t* Y, hipStream_t stream) {
  if ((long long)T * k > kRouteInLaunchMax || T < 1) return hipErrorInvalidValue;
  GemmArgs a{};
  a.X = X;
  a.xrows = T;
  a.K = K;
  a.N = N;
  a.E = E;
  a.A = T * k;
  a.k = k;
  a.Wt = Wt;
  a.St = St;
  a.Bt = Bt;
  a.Y = Y;
  a.ldy = N;
  a.ids = ids;
  a.r_counts = counts;
  a.r_offsets = offsets;
  a.r_perm = perm;
  a.r_inv_perm = inv_perm;
  a.r_blocks = blocks;
  a.r_num_blocks = num_blocks;
  // the 64-row tall-block kernel: 4 waves x 2 fragments of 32 columns per task
  constexpr int kTileN = 4 * 2 * 32;
  const void* fn = (const void*)&k_gemm_q4_w32<64, 2, 2, 4, kEpiPlain, 2, true>;
  // one more workgroup, the last, for the routing tables
  dim3 grid = task_grid(0, E, (N + kTileN - 1) / kTileN);
  grid.x += 1;
  return launch("k_gemm_q4_w32 (routing)", fn, grid, dim3(4 * 64), 0, stream, a);
}

}  // namespace moeq4
