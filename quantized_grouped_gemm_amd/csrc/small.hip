// small.hip -- the MoE layer for a few tokens at once (1 to MOEQ4_SMALL_MAX_T), gfx950.
//
// Perplexity Engineering, "Optimizing on-device inference for Apple Silicon",
// section "Limits of further optimization": verifying a speculative draft
// hands the layer groups of two to five rows, a shape that suits neither the
// matrix path nor the one-row path, and those rows often select different
// experts, so more expert weights are read.  Here such a group runs as the
// decode design (sections "Decode: minimize bytes moved per token",
// "Optimize the single-row weight path" and "Reduce intermediate and state
// traffic") widened to T tokens, with every distinct
// selected expert read once for all the tokens that chose it.
//
//   k_small_route    one workgroup: wave w routes token w (top-k over the E
//                    logits, softmax over the k), then the ascending list of
//                    the distinct selected experts (a bit set and prefix
//                    popcounts) and, per list entry ("slot"), one 8-byte word
//                    holding each token's choice of that expert.
//   k_small_gateup   workgroup (slot u, 16-row tile of I): gate and up
//                    tiles of the u-th distinct expert (or of the shared
//                    expert, in the last slot) rebuilt once per block and
//                    applied to the x of each token that chose it:
//                    h[tok][j] = bf16(silu(g) * u), j the token's choice (k for
//                    the shared expert).  The grid holds min(E, T*k) routed
//                    slots; those past the distinct-expert count end at once,
//                    so nothing waits on the host.
//   k_small_down     workgroup (16-row tile of H, half of the slots; all of
//                    them below kSbSplitSlots slots): every down block rebuilt
//                    once and applied to the h of each token that chose the
//                    slot's expert, times its routing weight (1 for the shared
//                    expert); with two halves, fp32 partial sums that
//                    k_small_combine adds in a fixed order, so that all CUs
//                    take part and the result is the same run after run.
// The plan a kernel reads (counts, expert ids, choice words, weights) is the
// same for every lane of a wave: it is read with uniform loads into scalar
// registers, and the branches on it are scalar.
#include "gemv.h"

namespace moeq4 {

constexpr int kSbWaves = 8;  // routing and gate/up workgroups; routing wave w takes token w
constexpr int kSbThreads = kSbWaves * 64;
constexpr int kSbBatch = 4;  // weight blocks a gate/up wave keeps in flight
constexpr int kSbDownWaves = 16;
constexpr int kSbDownThreads = kSbDownWaves * 64;
constexpr int kSbDownBatch = 6;  // weight blocks a down wave keeps in flight
constexpr int kSbXPieces = 4;    // 16-byte pieces of x per gate/up thread: T*H <= 8 * 4 * 512
constexpr int kSbHPieces = 6;    // 16-byte pieces of h per down thread: T*(k+1)*I <= 8 * 6 * 1024
constexpr int kSbSplitSlots = 16;       // slots from which the down projection splits them in two
constexpr int kSbMaxT = MOEQ4_SMALL_MAX_T;
constexpr int kSbMaxSlots = kSbMaxT * MOEQ4_MAX_TOPK;
static_assert(kSbMaxT <= kSbWaves, "one routing wave per token");

// The routing of the T tokens, in LDS.
struct SbRoute {
  int ids[kSbMaxT][MOEQ4_MAX_TOPK];
  float w[kSbMaxT][MOEQ4_MAX_TOPK];
  uint32_t bits[MOEQ4_MAX_EXPERTS / 32];  // selected experts
  int uexp[kSbMaxSlots];                  // the distinct ones, ascending
  int U;                                  // how many
};

template <int VPT>
__device__ void sb_route(const float* __restrict__ logits, int T, int E, int k, SbRoute& r) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nw = (E + 31) >> 5;
  for (int i = tid; i < nw; i += blockDim.x) r.bits[i] = 0u;
  if (wv < T) {
    float lg[VPT];
#pragma unroll
    for (int s = 0; s < VPT; ++s) lg[s] = logits[(size_t)wv * E + min(lane * VPT + s, E - 1)];
    int key[VPT];
#pragma unroll
    for (int s = 0; s < VPT; ++s) key[s] = lane * VPT + s < E ? order_key(lg[s]) : kKeyTaken;
    int my_id;
    float my_v, v0;
    wave_topk<VPT>(key, E, k, my_id, my_v, v0);
    const float ex = lane < k ? expf(my_v - v0) : 0.f;
    const float sum = wave_sum_f32(ex);
    if (lane < k) {
      r.ids[wv][lane] = my_id;
      r.w[wv][lane] = ex / sum;
    }
  }
  __syncthreads();
  const int A = T * k;
  for (int a = tid; a < A; a += blockDim.x) {
    const int e = r.ids[a / k][a % k];
    atomicOr(&r.bits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  // the rank of an expert among the selected ones is the number of selected
  // experts below it; equal experts write the same entry with the same value
  for (int a = tid; a < A; a += blockDim.x) {
    const int e = r.ids[a / k][a % k];
    int rank = __popc(r.bits[e >> 5] & ((1u << (e & 31)) - 1u));
    for (int i = 0; i < (e >> 5); ++i) rank += __popc(r.bits[i]);
    r.uexp[rank] = e;
  }
  if (tid == 0) {
    int u = 0;
    for (int i = 0; i < nw; ++i) u += __popc(r.bits[i]);
    r.U = u;
  }
  __syncthreads();
}

// ----------------------------------------------------------------------------
template <int VPT>
__global__ __launch_bounds__(kSbThreads) void k_small_route(
    const float* __restrict__ logits, int T, int E, int k, int umax, int has_shared, int32_t* __restrict__ plan_ws,
    uint2* __restrict__ jt_ws, int32_t* __restrict__ ids_ws, float* __restrict__ w_ws,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  __shared__ SbRoute rt;
  const int tid = threadIdx.x;
  sb_route<VPT>(logits, T, E, k, rt);
  const int U = rt.U;
  for (int a = tid; a < T * k; a += kSbThreads) {
    const int id = rt.ids[a / k][a % k];
    const float w = rt.w[a / k][a % k];
    ids_ws[a] = id;
    w_ws[a] = w;
    if (ids_out) ids_out[a] = id;
    if (w_out) w_out[a] = w;
  }
  // slot u < U: the u-th distinct expert; slot umax: the shared expert.  Byte
  // i of a slot's word: token i's choice of the slot's expert (0xFF: none).
  for (int u = tid; u < U + has_shared; u += kSbThreads) {
    const bool sh = u == U;
    const int e = sh ? -1 : rt.uexp[u];
    uint32_t word[2] = {0xFFFFFFFFu, 0xFFFFFFFFu};
    for (int tok = 0; tok < T; ++tok) {
      int j = sh ? k : -1;
      if (!sh)
        for (int i = 0; i < k; ++i) j = rt.ids[tok][i] == e ? i : j;
      const int b = 8 * (tok & 3);
      word[tok >> 2] = (word[tok >> 2] & ~(0xFFu << b)) | ((uint32_t)(j & 0xFF) << b);
    }
    jt_ws[sh ? umax : u] = uint2{word[0], word[1]};
    if (!sh) plan_ws[1 + u] = e;
  }
  if (tid == 0) plan_ws[0] = U;
}

// token i's choice in a slot's word (uniform: scalar registers), -1 if none
__device__ __forceinline__ int sb_choice(uint32_t w0, uint32_t w1, int i) {
  return (int)(int8_t)(((i < 4 ? w0 : w1) >> (8 * (i & 3))) & 0xFFu);
}

// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kSbThreads) void k_small_gateup(
    const uint16_t* __restrict__ x, int T, int k, int H, int I, int umax,
    const uint8_t* __restrict__ gu_q, const uint16_t* __restrict__ gu_s, const uint16_t* __restrict__ gu_b,
    const uint8_t* __restrict__ sh_q, const uint16_t* __restrict__ sh_s, const uint16_t* __restrict__ sh_b,
    const int32_t* __restrict__ plan_ws, const uint2* __restrict__ jt_ws, uint16_t* __restrict__ h_ws) {
  extern __shared__ uint4 dsm[];
  uint4* xl = dsm;  // x of the T tokens, [T][H] bf16
  __shared__ float red[kSbWaves][kSbMaxT][16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int IT = I / 16;
  const int slot = blockIdx.x / IT, t = blockIdx.x % IT;
  const bool sh_slot = slot == umax;  // the last slot: the shared expert

  // x of every token, in flight while the plan is read (a slot's tokens are
  // known only from the plan)
  const Staged<kSbXPieces> xr = stage_load<kSbXPieces>(x, T * (H / 8));
  const int U = plan_ws[0];
  if (!sh_slot && slot >= U) return;  // no such distinct expert (uniform over the workgroup)
  const int e = sh_slot ? 0 : plan_ws[1 + slot];
  const uint2 jw = jt_ws[slot];
  const uint32_t w0 = __builtin_amdgcn_readfirstlane(jw.x), w1 = __builtin_amdgcn_readfirstlane(jw.y);

  const size_t mat_codes = (size_t)I * H;  // bytes of one [2I][H] code matrix
  const size_t mat_groups = (size_t)2 * I * (H / kGroup);
  TiledMat m;
  m.q = sh_slot ? sh_q : gu_q + (size_t)e * mat_codes;
  m.s = sh_slot ? sh_s : gu_s + (size_t)e * mat_groups;
  m.b = sh_slot ? sh_b : gu_b + (size_t)e * mat_groups;
  m.NT = 2 * IT;
  const int G = H / kGroup, nfull = G / 2;

  // waves 0..3: gate tile t, waves 4..7: up tile t + I/16; wave w & 3 takes
  // chunks w&3, (w&3)+4, ...  Loads are unconditional (chunk index clamped,
  // surplus results unused).
  constexpr int WPT = kSbWaves / 2;
  const int c_first = wv % WPT;
  const int tile = wv < WPT ? t : t + IT;
  FullBlock f[kSbBatch];
  auto load_batch = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kSbBatch; ++i) f[i] = load_full(m, tile, min(c0 + WPT * i, nfull - 1), lane);
  };
  load_batch(c_first);
  stage_store(xr, T * (H / 8), xl);
  __syncthreads();
  float acc[kSbMaxT];
#pragma unroll
  for (int i = 0; i < kSbMaxT; ++i) acc[i] = 0.f;
  auto apply = [&](const Rebuilt& rb, int c, bool tail) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kSbMaxT; ++i)
      if (sb_choice(w0, w1, i) >= 0) {
        const uint4* xt = xl + (size_t)i * (H / 8);
        acc[i] += tail ? gemv_tail_rebuilt(rb, c, lane, xt) : gemv_rebuilt(rb, c, lane, xt);
      }
  };
  for (int c0 = c_first; c0 < nfull; c0 += kSbBatch * WPT) {
    if (c0 != c_first) load_batch(c0);
#pragma unroll
    for (int i = 0; i < kSbBatch; ++i) {
      const int c = c0 + WPT * i;
      if (c < nfull) apply(rebuild_full(f[i]), c, false);
    }
  }
  if ((G & 1) && c_first == nfull % WPT) apply(rebuild_tail(m, tile, nfull, lane), nfull, true);
#pragma unroll
  for (int i = 0; i < kSbMaxT; ++i)
    if (sb_choice(w0, w1, i) >= 0) {
      const float v = sum_quarters(acc[i]);
      if (lane < 16) red[wv][i][lane] = v;
    }
  __syncthreads();
  if (tid < 16 * T) {
    const int tok = tid >> 4, r = tid & 15;
    const int j = (int)(int8_t)((((tok < 4) ? jw.x : jw.y) >> (8 * (tok & 3))) & 0xFFu);
    if (j >= 0) {
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < WPT; ++w) {
        g += red[w][tok][r];
        u += red[WPT + w][tok][r];
      }
      const float silu = g / (1.f + expf(-g));
      h_ws[((size_t)tok * (k + 1) + j) * I + 16 * t + r] = f32_to_bf16_bits(silu * u);
    }
  }
}

// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kSbDownThreads) void k_small_down(
    int T, int k, int H, int I, int umax, int has_shared, int nsplit, const uint8_t* __restrict__ dn_q,
    const uint16_t* __restrict__ dn_s, const uint16_t* __restrict__ dn_b, const uint8_t* __restrict__ sh_q,
    const uint16_t* __restrict__ sh_s, const uint16_t* __restrict__ sh_b, const int32_t* __restrict__ plan_ws,
    const uint2* __restrict__ jt_ws, const float* __restrict__ w_ws, const uint16_t* __restrict__ h_ws,
    float* __restrict__ part_ws, uint16_t* __restrict__ out) {
  extern __shared__ uint4 dsm[];
  uint4* hl = dsm;  // [T][k+1][I] bf16
  __shared__ float red[kSbDownWaves][kSbMaxT][16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = blockIdx.x % (H / 16);  // 16-row tile of the output
  const int sp = blockIdx.x / (H / 16);  // which part of the slots
  const int J1 = k + 1;

  const Staged<kSbHPieces> hr = stage_load<kSbHPieces>(h_ws, T * J1 * (I / 8));
  const int U = plan_ws[0];
  const int nslots = U + has_shared;  // slot U (if any): the shared expert
  const int per = (nslots + nsplit - 1) / nsplit;
  const int s_lo = min(nslots, sp * per), s_hi = min(nslots, s_lo + per);

  const size_t mat_codes = (size_t)H * I / 2;
  const size_t mat_groups = (size_t)H * (I / kGroup);
  const int G = I / kGroup, nfull = G / 2;
  const int nb = (s_hi - s_lo) * nfull;  // full blocks: (slot, chunk); wave w takes w, w+16, ...
  auto mat = [&](int u) {
    TiledMat m1;
    const bool sh = u == U;
    const size_t e = sh ? 0 : (size_t)plan_ws[1 + u];
    m1.q = sh ? sh_q : dn_q + e * mat_codes;
    m1.s = sh ? sh_s : dn_s + e * mat_groups;
    m1.b = sh ? sh_b : dn_b + e * mat_groups;
    m1.NT = H / 16;
    return m1;
  };
  float acc[kSbMaxT];
#pragma unroll
  for (int i = 0; i < kSbMaxT; ++i) acc[i] = 0.f;
  auto apply = [&](const Rebuilt& rb, int u, int c, bool tail) __attribute__((always_inline)) {
    const uint2 jw = jt_ws[u == U ? umax : u];
    const uint32_t w0 = __builtin_amdgcn_readfirstlane(jw.x), w1 = __builtin_amdgcn_readfirstlane(jw.y);
#pragma unroll
    for (int i = 0; i < kSbMaxT; ++i) {
      const int j = sb_choice(w0, w1, i);
      if (j >= 0) {
        const float wt = j < k ? w_ws[i * k + j] : 1.f;
        const uint4* ht = hl + ((size_t)i * J1 + j) * (I / 8);
        acc[i] = __builtin_fmaf(wt, tail ? gemv_tail_rebuilt(rb, c, lane, ht) : gemv_rebuilt(rb, c, lane, ht),
                                acc[i]);
      }
    }
  };
  FullBlock f[kSbDownBatch];
  auto load_batch = [&](int b0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kSbDownBatch; ++i) {
      const int b = min(b0 + kSbDownWaves * i, nb - 1);
      f[i] = load_full(mat(s_lo + b / nfull), t, b % nfull, lane);
    }
  };
  if (nb > 0) load_batch(wv);  // in flight while h is staged
  stage_store(hr, T * J1 * (I / 8), hl);
  __syncthreads();
  for (int b0 = wv; b0 < nb; b0 += kSbDownWaves * kSbDownBatch) {
    if (b0 != wv) load_batch(b0);
#pragma unroll
    for (int i = 0; i < kSbDownBatch; ++i) {
      const int b = b0 + kSbDownWaves * i;
      if (b < nb) apply(rebuild_full(f[i]), s_lo + b / nfull, b % nfull, false);
    }
  }
  if (G & 1)  // half-size last chunk of every slot's matrix
    for (int u = s_lo + wv; u < s_hi; u += kSbDownWaves) apply(rebuild_tail(mat(u), t, nfull, lane), u, nfull, true);
#pragma unroll
  for (int i = 0; i < kSbMaxT; ++i)
    if (i < T) {
      const float v = sum_quarters(acc[i]);
      if (lane < 16) red[wv][i][lane] = v;
    }
  __syncthreads();
  if (tid < 16 * T) {
    const int tok = tid >> 4, r = tid & 15;
    float p = 0.f;
#pragma unroll
    for (int w = 0; w < kSbDownWaves; ++w) p += red[w][tok][r];
    const size_t o = (size_t)tok * H + 16 * t + r;
    if (nsplit == 1) out[o] = f32_to_bf16_bits(p);
    else part_ws[(size_t)sp * T * H + o] = p;
  }
}

// out = bf16(part[0] + part[1] + ...), parts added in order
__global__ __launch_bounds__(256) void k_small_combine(int n, int nsplit, const float* __restrict__ part_ws,
                                                       uint16_t* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float p = part_ws[i];
  for (int s = 1; s < nsplit; ++s) p += part_ws[(size_t)s * n + i];
  out[i] = f32_to_bf16_bits(p);
}

// ----------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SmallPlan small_plan(int T, int E, int k, int H, int I) {
  SmallPlan p{};
  p.umax = (long long)T * k < E ? T * k : E;
  // two halves of the slots per output tile once there are enough of them
  p.nsplit = p.umax + 1 >= kSbSplitSlots ? 2 : 1;
  p.ws_plan = 0;
  p.ws_jt = align256(sizeof(int32_t) * (size_t)(1 + p.umax));
  p.ws_ids = p.ws_jt + align256(sizeof(uint32_t) * 2 * (size_t)(1 + p.umax));
  p.ws_w = p.ws_ids + align256(sizeof(int32_t) * (size_t)T * k);
  p.ws_h = p.ws_w + align256(sizeof(float) * (size_t)T * k);
  p.ws_part = p.ws_h + align256(sizeof(uint16_t) * (size_t)T * (k + 1) * I);
  p.ws_bytes = p.ws_part + (p.nsplit > 1 ? align256(sizeof(float) * (size_t)p.nsplit * T * H) : 0);
  p.lds_gateup = (size_t)T * H * 2;
  p.lds_down = (size_t)T * (k + 1) * I * 2;
  return p;
}

bool small_fits(int T, int E, int k, int H, int I) {
  (void)E;
  const long long xp = (long long)T * (H / 8), hp = (long long)T * (k + 1) * (I / 8);
  return T >= 1 && T <= kSbMaxT && xp <= (long long)kSbXPieces * kSbThreads &&
         hp <= (long long)kSbHPieces * kSbDownThreads;
}

hipError_t small_launch(const SmallPlan& p, const float* logits, const uint16_t* x, int T, int E, int k, int H,
                        int I, const uint8_t* gu_q, const uint16_t* gu_s, const uint16_t* gu_b,
                        const uint8_t* dn_q, const uint16_t* dn_s, const uint16_t* dn_b, const uint8_t* sh_gu_q,
                        const uint16_t* sh_gu_s, const uint16_t* sh_gu_b, const uint8_t* sh_dn_q,
                        const uint16_t* sh_dn_s, const uint16_t* sh_dn_b, int32_t* ids_out, float* w_out,
                        uint16_t* out, void* workspace, hipStream_t stream) {
  char* ws = (char*)workspace;
  int32_t* plan_ws = (int32_t*)(ws + p.ws_plan);
  uint2* jt_ws = (uint2*)(ws + p.ws_jt);
  int32_t* ids_ws = (int32_t*)(ws + p.ws_ids);
  float* w_ws = (float*)(ws + p.ws_w);
  uint16_t* h_ws = (uint16_t*)(ws + p.ws_h);
  float* part_ws = p.nsplit > 1 ? (float*)(ws + p.ws_part) : nullptr;
  const int has_shared = sh_gu_q != nullptr;
  const void* fn;
  if (E <= 64) fn = (const void*)&k_small_route<1>;
  else if (E <= 128) fn = (const void*)&k_small_route<2>;
  else if (E <= 256) fn = (const void*)&k_small_route<4>;
  else if (E <= 512) fn = (const void*)&k_small_route<8>;
  else fn = (const void*)&k_small_route<16>;
  hipError_t err = launch("k_small_route", fn, dim3(1), dim3(kSbThreads), 0, stream, logits, T, E, k, p.umax,
                          has_shared, plan_ws, jt_ws, ids_ws, w_ws, ids_out, w_out);
  if (err != hipSuccess) return err;
  const int slots = p.umax + has_shared, IT = I / 16;
  err = launch("k_small_gateup", (const void*)&k_small_gateup, dim3(slots * IT), dim3(kSbThreads), p.lds_gateup,
               stream, x, T, k, H, I, p.umax, gu_q, gu_s, gu_b, sh_gu_q, sh_gu_s, sh_gu_b, (const int32_t*)plan_ws,
               (const uint2*)jt_ws, h_ws);
  if (err != hipSuccess) return err;
  // the down kernel stages up to kSbHPieces * 16 bytes per thread of h in LDS
  // (96 KB): raise its dynamic LDS limit once
  static const hipError_t lds_err = hipFuncSetAttribute((const void*)&k_small_down,
                                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                                        kSbHPieces * kSbDownThreads * 16);
  if (lds_err != hipSuccess) {
    note_hip_error(lds_err, "hipFuncSetAttribute(k_small_down)");
    return lds_err;
  }
  err = launch("k_small_down", (const void*)&k_small_down, dim3((H / 16) * p.nsplit), dim3(kSbDownThreads),
               p.lds_down, stream, T, k, H, I, p.umax, has_shared, p.nsplit, dn_q, dn_s, dn_b, sh_dn_q, sh_dn_s,
               sh_dn_b, (const int32_t*)plan_ws, (const uint2*)jt_ws, (const float*)w_ws, (const uint16_t*)h_ws,
               part_ws, out);
  if (err != hipSuccess || p.nsplit == 1) return err;
  const int n = T * H;
  return launch("k_small_combine", (const void*)&k_small_combine, dim3((n + 255) / 256), dim3(256), 0, stream, n,
                p.nsplit, (const float*)part_ws, out);
}

}  // namespace moeq4
