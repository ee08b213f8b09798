// ffn.hip -- the routed experts' FFN plus the shared expert over a prefill
// batch, as four grouped-GEMM launches on the caller's stream.
//
// Perplexity Engineering, "Optimizing on-device inference for Apple Silicon":
//   section "Reduce intermediate and state traffic": the two input projections
//   run with their gated activation fused, and the output projection with its
//   routing score and the shared expert's result;
//   section "Qwen creates three workload shapes": the shared expert processes
//   every token next to the routed ones;
//   section "Dequantize weights during matrix multiplication": all four
//   products rebuild the 4-bit weights on chip.
//
// Steps 1 and 2 (and 3 and 4) share one launch when the routed blocks are tall:
// the shared expert is then the launch's dense second problem, whose tasks the
// first workgroups on every XCD take.
//
//   1. routed gate+up   h[p]  = bf16(silu(G x) * (U x))   rows p in expert-sorted order,
//                                                      x = X[perm[p] / k]
//   2. shared gate+up   hs[t] = bf16(silu(Gs x_t) * (Us x_t))   dense, all T tokens
//   3. routed down      Dw[a] = w_a * (D h[p]),  a = perm[p]: rows back in
//                                                      assignment order t*k + j,
//                                                      kept as fp16 of value*2^-8
//   4. shared down      Dsh[t] = Ds hs[t], kept like Dw
//   5. combine          out[t] = bf16(Dsh[t] + sum_j Dw[t*k + j]): 16-byte reads of
//                        every term, added in a fixed order (the shared term,
//                        then j ascending), so the result does not depend on
//                        scheduling.
#include "common.h"

namespace moeq4 {

constexpr int kCombineThreads = 256;

// out[t][n] = bf16(Dsh[t][n] + sum_j Dw[t*k + j][n]) over the stored terms
// (Dsh may be null), 8 columns per thread
__global__ __launch_bounds__(kCombineThreads) void k_combine(const uint16_t* __restrict__ Dw,
                                                             const uint16_t* __restrict__ Dsh, int T, int H, int k,
                                                             uint16_t* __restrict__ out) {
  const long long i = (long long)blockIdx.x * kCombineThreads + threadIdx.x;  // 8-column piece
  const int pieces = H / 8;
  if (i >= (long long)T * pieces) return;
  const int t = (int)(i / pieces), c8 = (int)(i % pieces) * 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint16_t* src) {
    const uint4 v = *(const uint4*)src;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[2 * q] += term_value(w[q] & 0xFFFFu);
      s[2 * q + 1] += term_value(w[q] >> 16);
    }
  };
  if (Dsh) add(Dsh + (size_t)t * H + c8);
  for (int j = 0; j < k; ++j) add(Dw + ((size_t)t * k + j) * H + c8);
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = (uint32_t)f32_to_bf16_bits(s[2 * q]) | ((uint32_t)f32_to_bf16_bits(s[2 * q + 1]) << 16);
  *(uint4*)(out + (size_t)t * H + c8) = make_uint4(o[0], o[1], o[2], o[3]);
}

// Task order of the routed blocks for the tall-block kernels: taller blocks
// (more filled 32-row tiles) first, so that the last workgroups a launch
// dispatches are the short tail blocks and the GPU does not idle behind a few
// full-length ones.  Blocks are independent, so any order gives the same
// outputs; inside a class the order comes from LDS atomics.
constexpr int kOrderThreads = 1024;
constexpr int kOrderClasses = 9;  // 8 - (filled 32-row tiles) for 1..8 tiles; 8: malformed entries

__global__ __launch_bounds__(kOrderThreads) void k_block_order(const int32_t* __restrict__ blocks,
                                                               const int32_t* __restrict__ num_blocks, int max_blocks,
                                                               int32_t* __restrict__ order) {
  __shared__ int cnt[kOrderClasses], base[kOrderClasses];
  const int tid = threadIdx.x;
  const int nb = min(*num_blocks, max_blocks);
  if (tid < kOrderClasses) cnt[tid] = 0;
  __syncthreads();
  auto cls = [&](int b) {
    const int rows = blocks[4 * b + 2];
    return rows >= 1 ? 8 - min(8, (rows + 31) >> 5) : 8;
  };
  for (int b = tid; b < nb; b += kOrderThreads) atomicAdd(&cnt[cls(b)], 1);
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int c = 0; c < kOrderClasses; ++c) {
      base[c] = run;
      run += cnt[c];
    }
  }
  __syncthreads();
  for (int b = tid; b < nb; b += kOrderThreads) order[atomicAdd(&base[cls(b)], 1)] = b;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

FfnPlan ffn_plan(int T, int H, int I, int k, bool shared) {
  FfnPlan p{};
  const size_t A = (size_t)T * k;
  p.ws_h = 0;
  p.ws_hs = align256(A * I * 2);
  p.ws_dw = p.ws_hs + (shared ? align256((size_t)T * I * 2) : 0);
  p.ws_dsh = p.ws_dw + align256(A * H * 2);
  p.ws_order = p.ws_dsh + (shared ? align256((size_t)T * H * 2) : 0);
  p.ws_bytes = p.ws_order + align256((2 * A + 1) * 4);  // >= moe_max_blocks for any block height
  // dense block height of the shared expert: as for one expert holding all T rows
  int bm = 16;
  while (bm < 128 && bm < (5LL * T + 3) / 4) bm <<= 1;
  p.bm_shared = bm;
  p.bm_shared_dn = bm < 64 ? bm : 64;  // the short-K down kernel keeps 64 rows' activations resident
  return p;
}

hipError_t ffn_launch(const FfnPlan& p, const uint16_t* X, int T, int H, int I, int E, int k,
                      const uint8_t* gu_q, const uint16_t* gu_s, const uint16_t* gu_b, const uint8_t* dn_q,
                      const uint16_t* dn_s, const uint16_t* dn_b, const uint8_t* sh_gu_q, const uint16_t* sh_gu_s,
                      const uint16_t* sh_gu_b, const uint8_t* sh_dn_q, const uint16_t* sh_dn_s,
                      const uint16_t* sh_dn_b, const float* topk_w, const int32_t* perm, const int32_t* blocks,
                      const int32_t* num_blocks, int max_blocks, int BM, uint16_t* out, void* workspace,
                      hipStream_t stream) {
  const bool shared = sh_gu_q != nullptr;
  const int A = T * k;
  char* ws = (char*)workspace;
  uint16_t* h = (uint16_t*)(ws + p.ws_h);
  uint16_t* hs = (uint16_t*)(ws + p.ws_hs);
  uint16_t* Dw = (uint16_t*)(ws + p.ws_dw);
  uint16_t* Dsh = shared ? (uint16_t*)(ws + p.ws_dsh) : nullptr;
  const int sh_blocks = (T + p.bm_shared - 1) / p.bm_shared;

  // The shared expert's two projections join the routed launches as their
  // dense second problem when the routed blocks are tall (64 rows and up: the
  // tall-block kernels take one); otherwise they are launches of their own.
  const bool fuse = shared && BM >= 64;

  // 0. tall-block launches take the routed blocks tallest first
  int32_t* order = nullptr;
  if (BM >= 64 && max_blocks > 0) {
    order = (int32_t*)(ws + p.ws_order);
    hipError_t oerr = launch("k_block_order", (const void*)&k_block_order, dim3(1), dim3(kOrderThreads), 0, stream,
                             blocks, num_blocks, max_blocks, order);
    if (oerr != hipSuccess) return oerr;
  }

  // 1. routed gate+up with SwiGLU (+ shared gate+up)
  GemmArgs g{};
  g.X = X;
  g.xrows = T;
  g.K = H;
  g.N = 2 * I;
  g.E = E;
  g.A = A;
  g.k = k;
  g.Wt = gu_q;
  g.St = gu_s;
  g.Bt = gu_b;
  g.gather = perm;
  g.blocks = blocks;
  g.num_blocks = num_blocks;
  g.order = order;
  g.Y = h;
  g.ldy = I;
  if (fuse) {
    g.dX = X;
    g.d_rows = T;
    g.dWt = sh_gu_q;
    g.dSt = sh_gu_s;
    g.dBt = sh_gu_b;
    g.dY = hs;
  }
  hipError_t err = gemm_launch(g, kEpiSwiglu, BM, max_blocks, stream);
  if (err != hipSuccess) return err;

  // 2. shared gate+up, dense over the tokens
  if (shared && !fuse) {
    GemmArgs s = g;
    s.E = 1;
    s.A = T;
    s.k = 1;
    s.Wt = sh_gu_q;
    s.St = sh_gu_s;
    s.Bt = sh_gu_b;
    s.gather = nullptr;
    s.blocks = nullptr;
    s.num_blocks = nullptr;
    s.order = nullptr;
    s.Y = hs;
    err = gemm_launch(s, kEpiSwiglu, p.bm_shared, sh_blocks, stream);
    if (err != hipSuccess) return err;
  }

  // 3. routed down, scaled by the routing weight, rows back in assignment order
  GemmArgs d{};
  d.X = h;
  d.xrows = A;
  d.K = I;
  d.N = H;
  d.E = E;
  d.A = A;
  d.k = k;
  d.Wt = dn_q;
  d.St = dn_s;
  d.Bt = dn_b;
  d.gather = nullptr;
  d.blocks = blocks;
  d.num_blocks = num_blocks;
  d.order = order;
  d.Y = Dw;
  d.ldy = H;
  d.perm = perm;
  d.topk_w = topk_w;
  if (fuse) {  // the shared rows keep their index and weight 1: Dsh[t] = term_bits(Ds hs[t])
    d.dX = hs;
    d.d_rows = T;
    d.dWt = sh_dn_q;
    d.dSt = sh_dn_s;
    d.dBt = sh_dn_b;
    d.dY = Dsh;
  }
  err = gemm_launch(d, kEpiScale, BM, max_blocks, stream);
  if (err != hipSuccess) return err;

  // 4. shared down, dense over the tokens
  if (shared && !fuse) {
    GemmArgs s{};
    s.X = hs;
    s.xrows = T;
    s.K = I;
    s.N = H;
    s.E = 1;
    s.A = T;
    s.k = 1;
    s.Wt = sh_dn_q;
    s.St = sh_dn_s;
    s.Bt = sh_dn_b;
    s.Y = Dsh;
    s.ldy = H;
    err = gemm_launch(s, kEpiTerm, p.bm_shared_dn, (T + p.bm_shared_dn - 1) / p.bm_shared_dn, stream);
    if (err != hipSuccess) return err;
  }

  // 5. combine
  const long long pieces = (long long)T * (H / 8);
  return launch("k_combine", (const void*)&k_combine, dim3((unsigned)((pieces + kCombineThreads - 1) / kCombineThreads)),
                dim3(kCombineThreads), 0, stream, (const uint16_t*)Dw, (const uint16_t*)Dsh, T, H, k, out);
}

}  // namespace moeq4
