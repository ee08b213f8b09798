// common.h -- device helpers shared by the HIP kernels of the MoE Q4 library
// (gfx950 / CDNA4, wave64).  Internal: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moeq4.h"

namespace moeq4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kWave = 64;
constexpr int kGroup = 64;  // weights per scale/bias group along K

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // v_cvt_pk_bf16_f32: round to nearest even
}

// two fp32 values as one packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}

// ---- exact rebuild of 4-bit codes: bf16(s*q + b) with s*q + b formed by one
// ---- fp32 fma (exact for bf16 s, b and q < 16 unless the sum needs more than
// ---- 24 bits, in which case it is the correctly rounded fp32 value).
//
// A dword of the tiled weight layout holds 8 consecutive codes with its low
// 16-bit half holding c0,c2,c4,c6 and its high half c1,c3,c5,c7 (nibble 0 = the
// lowest bits).  Masking leaves one code in each half; read as fp16, such a half
// is the subnormal q*2^-24 (code in bits 0..3) or q*2^-20 (bits 4..7), exactly
// (fp16 subnormals are kept: the kernels run with fp16 denormals on), so with
// sc = s*2^24 (or s*2^20) one v_fma_mix_f32 per code forms s*q + b with the
// same single rounding as fma(s, q, b).  Requires s*2^24 finite (|s| < 2^104).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t mix_pair(uint32_t m, float sc, float b) {
  const f16x2 h = __builtin_bit_cast(f16x2, m);
  return pk_bf16(__builtin_fmaf(sc, (float)h[0], b), __builtin_fmaf(sc, (float)h[1], b));
}
// the 8 codes of dword wd as 4 packed bf16 pairs (c0,c1), (c2,c3), (c4,c5), (c6,c7);
// 17 VALU ops
__device__ __forceinline__ uint4 rebuild_words(uint32_t wd, float s, float b) {
  const float s24 = s * 16777216.f, s20 = s * 1048576.f;
  const uint32_t t = wd >> 8;
  return make_uint4(mix_pair(wd & 0x000F000Fu, s24, b), mix_pair(wd & 0x00F000F0u, s20, b),
                    mix_pair(t & 0x000F000Fu, s24, b), mix_pair(t & 0x00F000F0u, s20, b));
}

// The FFN keeps the weighted routed terms between its two projections as fp16
// holding value * 2^-8 (11-bit significand, range to ~1.7e7): the combine then
// adds terms rounded 8x finer than bf16 at the same bytes.
constexpr float kTermScale = 1.f / 256.f;

__device__ __forceinline__ uint16_t term_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)(v * kTermScale));  // round to nearest even
}

__device__ __forceinline__ float term_value(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16) * (1.f / kTermScale);
}

// ---- wave64 reductions through DPP; the full result lands in lane 63 and is
// ---- broadcast with readlane (uniform, lives in an SGPR).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, ROW_MASK, 0xF, false);
}

// wave-wide maximum of a signed int; the result is uniform (SGPR)
__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, dpp_i32<0xB1>(x));        // quad_perm [1,0,3,2]
  x = max(x, dpp_i32<0x4E>(x));        // quad_perm [2,3,0,1]
  x = max(x, dpp_i32<0x141>(x));       // row_half_mirror
  x = max(x, dpp_i32<0x140>(x));       // row_mirror
  x = max(x, dpp_i32<0x142, 0xA>(x));  // row_bcast:15 into rows 1 and 3
  x = max(x, dpp_i32<0x143, 0xC>(x));  // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(x, 63);
}

__device__ __forceinline__ float wave_sum_f32(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  x += dpp_f32<0x142, 0xA>(x);
  x += dpp_f32<0x143, 0xC>(x);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Order-preserving integer image of a float (monotone for non-NaN values;
// -0 is folded into +0 so equal logits get equal keys).  It is an involution on
// the folded bits: applying it again returns the float's bits.
__device__ __forceinline__ int order_key(float v) {
  const int u = __float_as_int(v + 0.0f);  // -0 + 0 = +0
  return u ^ ((u >> 31) & 0x7FFFFFFF);
}

__device__ __forceinline__ float key_value(int key) {
  return __int_as_float(key ^ ((key >> 31) & 0x7FFFFFFF));
}

constexpr int kKeyTaken = (int)0x80000000;  // below every finite logit's key

// Top-k of one token's logits held by one wave: lane l holds the keys of
// experts l*VPT + s (kKeyTaken where there is no expert).  k rounds of a
// wave-wide maximum select the largest key, the lowest expert id among equal
// keys (Perplexity Engineering, "Optimizing on-device inference for Apple
// Silicon", section "Qwen creates three workload shapes": the router keeps the
// best-scoring experts of each token).  Lane j < k receives the j-th selected
// expert id and logit; v0 (uniform) is the largest logit.  Consumes `key`.
template <int VPT>
__device__ __forceinline__ void wave_topk(int (&key)[VPT], int E, int k, int& my_id, float& my_v,
                                          float& v0) {
  const int lane = threadIdx.x & 63;
  my_id = 0;
  my_v = 0.f;
  v0 = 0.f;
  for (int j = 0; j < k; ++j) {
    // best of this lane: larger key, lower slot on ties
    int bk = key[0], bs = 0;
#pragma unroll
    for (int s = 1; s < VPT; ++s) {
      if (key[s] > bk) {
        bk = key[s];
        bs = s;
      }
    }
    const int m = wave_max_i32(bk);  // uniform
    const uint64_t bal = __ballot(bk == m);
    const int wl = __builtin_amdgcn_readfirstlane(bal ? (__ffsll((unsigned long long)bal) - 1) : 0);
    const int ws = __builtin_amdgcn_readlane(bs, wl);
    const float sel_v = key_value(m);
    if (j == 0) v0 = sel_v;
#pragma unroll
    for (int s = 0; s < VPT; ++s)
      if (lane == wl && s == ws) key[s] = kKeyTaken;
    if (lane == j) {
      my_id = min(wl * VPT + ws, E - 1);  // stays in range even for non-finite input
      my_v = sel_v;
    }
  }
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---- host side: launch through hipLaunchKernel so the status is returned.
void note_hip_error(hipError_t err, const char* what);  // api.hip: per-thread detail text

template <typename... Args>
inline hipError_t launch(const char* name, const void* fn, dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  const hipError_t err = hipLaunchKernel(fn, grid, block, argv, shmem, stream);
  if (err != hipSuccess) note_hip_error(err, name);
  return err;
}

// ---- internal entry points implemented in route.hip / gemm_q4.hip / prepack.hip
struct RoutePlan {
  int waves;      // waves per workgroup of the top-k/rank kernel
  int tpc;        // tokens per chunk (one workgroup of the top-k/rank kernel)
  int nchunks;    // ceil(T / tpc)
  int nbits;      // bits that distinguish expert ids: ceil(log2(E))
  size_t ws_chunk_counts;  // byte offset of chunk counts [nchunks][E]
  size_t ws_local_rank;    // byte offset of in-chunk ranks [T*k]
  size_t ws_bytes;         // total workspace
};

RoutePlan route_plan(int T, int E, int k);

// top-k + softmax alone (ids and weights), one wave per token
hipError_t topk_launch(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                       hipStream_t stream);

hipError_t route_launch(const RoutePlan& plan, const float* logits, int T, int E, int k, int block_rows,
                        int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* inv_perm, int32_t* blocks, int32_t* num_blocks,
                        void* workspace, hipStream_t stream);

// One grouped-GEMM launch over tiled group-wise affine 4-bit weights.
enum GemmEpi {
  kEpiPlain = 0,    // Y[p][n] = bf16(acc)                         (sorted row p)
  kEpiSwiglu = 1,   // Y[p][n] = bf16(silu(acc_n) * acc_{n+N/2})    (N/2 output columns)
  kEpiScale = 2,    // Y[perm[p]][n] = term_bits(topk_w[perm[p]] * acc)  (assignment order)
  kEpiTerm = 3,     // Y[p][n] = term_bits(acc)
};

struct GemmArgs {
  const uint16_t* X;  // activations: xrows rows of K bf16
  int xrows;
  int K, N, E, A, k;  // N weight rows per expert; A rows in the block-map space
  const uint8_t* Wt;  // tiled weights of E experts
  const uint16_t* St;
  const uint16_t* Bt;
  const int32_t* gather;      // non-null: row p reads X[gather[p] / k]; null: X[p]
  const int32_t* blocks;      // block map; null: dense BM-row blocks over A rows of expert 0
  const int32_t* num_blocks;  // device count of block-map entries
  int max_blocks;             // entries blocks[] holds (the launch grid's bound)
  const int32_t* order;       // non-null: routed task i takes block-map entry order[i] (a permutation)
  uint16_t* Y;                // output, row stride ldy
  int ldy;
  const int32_t* perm;        // kEpiScale; null: row p goes to row p with weight 1
  const float* topk_w;        // kEpiScale
  // Optional dense second problem run by the same launch (the shared expert
  // next to the routed ones): rows 0..d_rows-1 of dX through one expert's
  // weights dWt/dSt/dBt into dY (same K, N, ldy and epilogue; kEpiScale rows
  // keep their index and weight 1).  d_rows == 0: none.
  const uint16_t* dX;
  int d_rows;
  const uint8_t* dWt;
  const uint16_t* dSt;
  const uint16_t* dBt;
  uint16_t* dY;
  // Routing in the launch (tall-block kernels, no dense problem): non-null ids
  // (the T*k selected experts) make each task one expert x one N tile; the
  // task finds its expert's rows from the ids, writes the routing tables of
  // its expert (N tile 0 only) and runs the expert's rows BM at a time.
  const int32_t* ids;
  int32_t* r_counts;
  int32_t* r_offsets;
  int32_t* r_perm;
  int32_t* r_inv_perm;
  int32_t* r_blocks;
  int32_t* r_num_blocks;
};

// Assignments (T*k) up to which a tall-block GEMM launch can do the routing's
// counting sort itself (one expert per task; each lane keeps one id per 256
// assignments in registers).
constexpr int kRouteInLaunchMax = 4096;

// Workgroup -> (block, N tile) of a launch with dense_blocks dense blocks ahead
// of the routed ones (routed_blocks, counted on the device), ntiles N tiles each.
// Workgroup i runs on XCD i % 8.  Blocks are dealt to the XCDs round-robin
// (block b to XCD b % 8) with all N tiles of a block on one XCD, so those
// tiles, which gather the same activation rows, share an L2, and every XCD gets
// a like share of full and partial blocks however skewed the experts are.  On
// each XCD the dense blocks come first, so they start in the first wave of
// workgroups.  Returns false when the workgroup has no task.
__device__ __forceinline__ bool gemm_task(int dense_blocks, int routed_blocks, int ntiles, bool& dense, int& blk,
                                          int& ntile) {
  constexpr int kX = 8;
  const int xcd = blockIdx.x % kX;
  int slot = blockIdx.x / kX;
  const int dslots = (dense_blocks + kX - 1) / kX * ntiles;
  dense = slot < dslots;
  if (!dense) slot -= dslots;
  blk = slot / ntiles * kX + xcd;
  ntile = slot % ntiles;
  return blk < (dense ? dense_blocks : routed_blocks);
}

// the arguments of the dense problem, as a problem of its own
__device__ __forceinline__ GemmArgs gemm_dense(const GemmArgs& a) {
  GemmArgs d = a;
  d.X = a.dX;
  d.xrows = a.d_rows;
  d.E = 1;
  d.A = a.d_rows;
  d.k = 1;
  d.Wt = a.dWt;
  d.St = a.dSt;
  d.Bt = a.dBt;
  d.gather = nullptr;
  d.blocks = nullptr;
  d.num_blocks = nullptr;
  d.order = nullptr;
  d.Y = a.dY;
  d.perm = nullptr;
  d.topk_w = nullptr;
  d.d_rows = 0;
  return d;
}

hipError_t gemm_launch(const GemmArgs& a, int epi, int block_rows, int max_blocks, hipStream_t stream);

hipError_t gemm_q4_launch(const uint16_t* X, int T, int K, int N, int E, int k, const uint8_t* Wt,
                          const uint16_t* St, const uint16_t* Bt, const int32_t* perm,
                          const int32_t* blocks, const int32_t* num_blocks, int max_blocks,
                          int block_rows, uint16_t* Y, hipStream_t stream);

// Routing's counting sort (counts, offsets, perm, inv_perm, block map of 64-row
// blocks) and the grouped GEMM in one launch, from the top-k ids; T*k <=
// kRouteInLaunchMax.
hipError_t route_gemm_q4_launch(const int32_t* ids, const uint16_t* X, int T, int K, int N, int E, int k,
                                const uint8_t* Wt, const uint16_t* St, const uint16_t* Bt, int32_t* counts,
                                int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* blocks,
                                int32_t* num_blocks, uint16_t* Y, hipStream_t stream);

// prepack.hip: every weight rebuilt exactly into row-major bf16 [E][N][K]
hipError_t dequant_launch(const uint8_t* codes_t, const uint16_t* scales_t, const uint16_t* biases_t, int E, int N,
                          int K, uint16_t* out, hipStream_t stream);

// measured MFMA ceiling (calib.hip): workgroups x 4 waves, each issuing
// iters x 8 independent 32x32x16 bf16 MFMAs; out holds workgroups * 256 floats
hipError_t calib_mfma_launch(int workgroups, int iters, float* out, hipStream_t stream);

struct DecodePlan {
  int J;               // experts per step: k routed + the shared one if given
  size_t ws_ids, ws_w, ws_h, ws_bytes;  // workspace byte offsets / total
  size_t lds_gateup, lds_down;                               // dynamic LDS bytes per kernel
};

DecodePlan decode_plan(int E, int k, int H, int I, bool shared);

// decode.hip: the calling thread's current device's copy of the static scratch
// array that moe_decode_ffn_q4_noalloc uses as its workspace
// (MOEQ4_DECODE_SCRATCH_BYTES; its address is looked up once per device)
hipError_t decode_scratch(void** ptr);

hipError_t decode_launch(const DecodePlan& p, const float* logits, const uint16_t* x, int E, int k, int H, int I,
                         const uint8_t* gu_q, const uint16_t* gu_s, const uint16_t* gu_b, const uint8_t* dn_q,
                         const uint16_t* dn_s, const uint16_t* dn_b, const uint8_t* sh_gu_q,
                         const uint16_t* sh_gu_s, const uint16_t* sh_gu_b, const uint8_t* sh_dn_q,
                         const uint16_t* sh_dn_s, const uint16_t* sh_dn_b, int32_t* ids_out, float* w_out,
                         uint16_t* out, void* workspace, hipStream_t stream);

// small.hip: the layer for 1..MOEQ4_SMALL_MAX_T tokens, every distinct
// selected expert read once for all the tokens that chose it
struct SmallPlan {
  int umax;            // slots for distinct experts: min(E, T*k)
  int nsplit;          // parts the down projection splits the slots into (1 or 2)
  size_t ws_plan;      // int32 [1 + umax]: the distinct-expert count, then the experts in ascending order
  size_t ws_jt;        // uint32 [1 + umax][2]: per slot, byte i = token i's choice (slot umax: shared expert)
  size_t ws_ids, ws_w;  // int32 / fp32 [T][k]: the routing of every token
  size_t ws_h;         // bf16 [T][k+1][I]: SwiGLU output per (token, choice); choice k = shared expert
  size_t ws_part;      // fp32 [nsplit][T][H]: partial sums of the down projection (nsplit > 1)
  size_t ws_bytes;
  size_t lds_gateup, lds_down;  // dynamic LDS bytes per kernel
};

SmallPlan small_plan(int T, int E, int k, int H, int I);
bool small_fits(int T, int E, int k, int H, int I);  // staging and LDS limits of the two kernels

hipError_t small_launch(const SmallPlan& p, const float* logits, const uint16_t* x, int T, int E, int k, int H,
                        int I, const uint8_t* gu_q, const uint16_t* gu_s, const uint16_t* gu_b,
                        const uint8_t* dn_q, const uint16_t* dn_s, const uint16_t* dn_b, const uint8_t* sh_gu_q,
                        const uint16_t* sh_gu_s, const uint16_t* sh_gu_b, const uint8_t* sh_dn_q,
                        const uint16_t* sh_dn_s, const uint16_t* sh_dn_b, int32_t* ids_out, float* w_out,
                        uint16_t* out, void* workspace, hipStream_t stream);

struct FfnPlan {
  // workspace: routed h [T*k][I], shared h [T][I], routed terms [T*k][H], shared term [T][H],
  // task order of the routed blocks [T*k]
  size_t ws_h, ws_hs, ws_dw, ws_dsh, ws_order, ws_bytes;
  int bm_shared;                        // dense block height of the shared expert's gate+up
  int bm_shared_dn;                     // ... and of its down projection
};

FfnPlan ffn_plan(int T, int H, int I, int k, bool shared);

hipError_t ffn_launch(const FfnPlan& p, const uint16_t* X, int T, int H, int I, int E, int k,
                      const uint8_t* gu_q, const uint16_t* gu_s, const uint16_t* gu_b, const uint8_t* dn_q,
                      const uint16_t* dn_s, const uint16_t* dn_b, const uint8_t* sh_gu_q, const uint16_t* sh_gu_s,
                      const uint16_t* sh_gu_b, const uint8_t* sh_dn_q, const uint16_t* sh_dn_s,
                      const uint16_t* sh_dn_b, const float* topk_w, const int32_t* perm, const int32_t* blocks,
                      const int32_t* num_blocks, int max_blocks, int BM, uint16_t* out, void* workspace,
                      hipStream_t stream);

hipError_t prepack_launch(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases,
                          int E, int N, int K, uint8_t* codes_t, uint16_t* scales_t,
                          uint16_t* biases_t, hipStream_t stream);

}  // namespace moeq4
