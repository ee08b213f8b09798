// decode.hip -- batch-1 decode step of the MoE layer (one token), gfx950.
//
// Perplexity Engineering, "Optimizing on-device inference for Apple Silicon":
//   section "Decode: minimize bytes moved per token": with one token per step
//   there is almost no weight reuse, so the step is bound by the bytes it
//   moves; section "Apple silicon provides different paths for different
//   workloads": a matrix-vector product is limited mainly by memory bandwidth;
//   section "Optimize the single-row weight path": a row-parallel GEMV in which
//   a group of lanes shares each output while reading different parts of the
//   weight matrix;
//   section "Reduce intermediate and state traffic": the two input projections
//   run together with their gated activation, and the output projection
//   together with the routing score and the shared expert's result;
//   section "Qwen creates three workload shapes": 8 of 256 experts per token
//   plus one shared expert that sees every token.
//
// Two kernels on the caller's stream, reading the same tiled weights as the
// grouped GEMM (moe_prepack_q4), so one copy of the weights serves both:
//   k_decode_gateup  one workgroup per (selected expert j, 16-row tile t of the
//                    intermediate dimension I).  Each workgroup routes the
//                    token itself (wave_topk over the E logits: no separate
//                    routing launch, no host round trip), reads gate tile t and
//                    up tile t + I/16 of expert e_j and writes
//                    h_j[16t..16t+16) = bf16(silu(g) * u).  Workgroup 0 also
//                    writes the k ids and softmax weights.
//   k_decode_down    one 16-wave workgroup per 8 rows of H (half a 16-row
//                    tile, so the H / 8 workgroups cover every CU): the sum over
//                    all selected experts of w_j * (Wd[e_j] h_j), with w = 1 for
//                    the shared expert, reduced in a fixed order, so the result
//                    is the same run after run.
//
// GEMV inner loop: a wave reads one 1 KB block of the tiled layout (16 rows x
// 128 K values; lane 16q+r holds 32 codes of row r) and rebuilds every weight
// exactly as bf16(scale * code + bias) (section "Dequantize weights during
// matrix multiplication": bf16 weights are rebuilt on chip before the
// multiply); v_dot2c_f32_bf16 multiplies the rebuilt pairs with bf16
// activation pairs from LDS and accumulates in fp32.  All of a lane's block
// loads are issued before any math, behind the activation loads, so the waits
// are exact (loads complete in issue order).
#include <atomic>
#include <mutex>

#include "gemv.h"

namespace moeq4 {

constexpr int kDecWaves = 8;          // gate/up workgroup
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecBatch = 4;          // weight blocks a gate/up wave keeps in flight
constexpr int kDownWaves = 16;        // down workgroup
constexpr int kDownThreads = kDownWaves * 64;
constexpr int kDownBatch = 2;         // item pairs a down wave keeps in flight

// Sum over the chunks c = c_first, c_first + c_step, ... of the full chunks
// (nfull of them), batched so that a wave keeps kDecBatch block loads in flight.
__device__ __forceinline__ float gemv_chunks(const TiledMat& m, int tile, int nfull, int c_first, int c_step,
                                             int lane, const uint4* xl) {
  float acc = 0.f;
  for (int c0 = c_first; c0 < nfull; c0 += kDecBatch * c_step) {
    FullBlock f[kDecBatch];
#pragma unroll
    for (int i = 0; i < kDecBatch; ++i) f[i] = load_full(m, tile, min(c0 + i * c_step, nfull - 1), lane);
#pragma unroll
    for (int i = 0; i < kDecBatch; ++i) {
      const int c = c0 + i * c_step;
      if (c < nfull) acc += gemv_full(f[i], c, lane, xl);
    }
  }
  return acc;
}

constexpr int kGateupPieces = 2;  // H <= 2 * 8 * kDecThreads
constexpr int kDownPieces = 4;    // J * I <= 4 * 8 * kDownThreads

// ----------------------------------------------------------------------------
template <int VPT>
__global__ __launch_bounds__(kDecThreads) void k_decode_gateup(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int E, int k, int H, int I,
    const uint8_t* __restrict__ gu_q, const uint16_t* __restrict__ gu_s, const uint16_t* __restrict__ gu_b,
    const uint8_t* __restrict__ sh_q, const uint16_t* __restrict__ sh_s, const uint16_t* __restrict__ sh_b,
    int32_t* __restrict__ ids_ws, float* __restrict__ w_ws, uint16_t* __restrict__ h_ws,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  extern __shared__ uint4 dsm[];
  uint4* xl = dsm;  // x as bf16, H values
  __shared__ float red[kDecWaves][16];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int IT = I / 16;
  const int j = blockIdx.x / IT, t = blockIdx.x % IT;

  const Staged<kGateupPieces> xr = stage_load<kGateupPieces>(x, H / 8);  // needed by every workgroup: first
  // ---- which expert: the token's j-th choice (every wave selects on its own)
  int e = 0;
  if (j < k) {
    float lg[VPT];
#pragma unroll
    for (int s = 0; s < VPT; ++s) lg[s] = logits[min(lane * VPT + s, E - 1)];
    int key[VPT];
#pragma unroll
    for (int s = 0; s < VPT; ++s) key[s] = lane * VPT + s < E ? order_key(lg[s]) : kKeyTaken;
    int my_id;
    float my_v, v0;
    wave_topk<VPT>(key, E, k, my_id, my_v, v0);
    e = __builtin_amdgcn_readlane(my_id, j);
    if (blockIdx.x == 0 && wv == 0) {
      const float ex = (lane < k) ? expf(my_v - v0) : 0.f;
      const float sum = wave_sum_f32(ex);
      if (lane < k) {
        ids_ws[lane] = my_id;
        w_ws[lane] = ex / sum;
        if (ids_out) ids_out[lane] = my_id;
        if (w_out) w_out[lane] = ex / sum;
      }
    }
  }

  const size_t mat_codes = (size_t)I * H;  // bytes of one [2I][H] code matrix
  const size_t mat_groups = (size_t)2 * I * (H / kGroup);
  TiledMat m;
  m.q = j < k ? gu_q + e * mat_codes : sh_q;
  m.s = j < k ? gu_s + e * mat_groups : sh_s;
  m.b = j < k ? gu_b + e * mat_groups : sh_b;
  m.NT = 2 * IT;
  const int G = H / kGroup, nfull = G / 2;

  // waves 0..3: gate tile t, waves 4..7: up tile t + I/16; wave w & 3 takes
  // chunks w&3, (w&3)+4, ...  Loads are unconditional (chunk index clamped,
  // surplus results unused) so the wait for x below is exact.
  constexpr int WPT = kDecWaves / 2;  // waves per tile
  const int tile = (wv < WPT) ? t : t + IT;
  const int c_first = wv % WPT;
  FullBlock f[kDecBatch];
#pragma unroll
  for (int i = 0; i < kDecBatch; ++i) f[i] = load_full(m, tile, min(c_first + WPT * i, nfull - 1), lane);
  stage_store(xr, H / 8, xl);
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kDecBatch; ++i) {
    const int c = c_first + WPT * i;
    if (c < nfull) acc += gemv_full(f[i], c, lane, xl);
  }
  acc += gemv_chunks(m, tile, nfull, c_first + WPT * kDecBatch, WPT, lane, xl);
  if ((G & 1) && c_first == nfull % WPT) acc += gemv_tail(m, tile, nfull, lane, xl);
  acc = sum_quarters(acc);
  if (lane < 16) red[wv][lane] = acc;
  __syncthreads();
  if (threadIdx.x < 16) {
    const int r = threadIdx.x;
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      g += red[w][r];
      u += red[WPT + w][r];
    }
    const float silu = g / (1.f + expf(-g));
    h_ws[(size_t)j * I + 16 * t + r] = f32_to_bf16_bits(silu * u);
  }
}

// ----------------------------------------------------------------------------
// Down projection over half tiles: workgroup u covers output rows [8u, 8u + 8),
// half h = u & 1 of 16-row tile u / 2, so H / 8 workgroups spread the step's
// weight reads and rebuilds over all CUs.  The work items are the blocks
// (selected expert j, chunk c) of that tile, full chunks first, then the
// half-size last chunks of an odd group count.  A wave takes two items at a
// time: lane 16q + r reads K quarter q of row 8h + (r & 7) of item 2p + (r >> 3),
// so all 64 lanes load and rebuild.  Partial sums meet in a fixed order (the
// four K quarters, then the two items of a pair, then the waves), so the result
// is the same run after run.
struct DownItem {
  int j, c;   // selected expert slot (k = shared expert) and chunk
  bool tail;  // the half-size last chunk of an odd group count
};

__device__ __forceinline__ DownItem down_item(int it, int nfull, int J) {
  DownItem d;
  const int nf = J * nfull;
  if (it < nf) {
    d.j = it / nfull;
    d.c = it % nfull;
    d.tail = false;
  } else {
    d.j = it - nf;
    d.c = nfull;
    d.tail = true;
  }
  return d;
}

// a lane's share of one item: 32 codes of a full chunk (16 of a tail chunk)
// and the scale / bias of its row's groups
struct DownLoad {
  uint4 codes;
  uint32_t s2, b2;
  float w;  // routing weight of the item's expert (1 for the shared expert)
};

__global__ __launch_bounds__(kDownThreads) void k_decode_down(
    int k, int H, int I, int J, const uint8_t* __restrict__ dn_q, const uint16_t* __restrict__ dn_s,
    const uint16_t* __restrict__ dn_b, const uint8_t* __restrict__ sh_q, const uint16_t* __restrict__ sh_s,
    const uint16_t* __restrict__ sh_b, const int32_t* __restrict__ ids_ws, const float* __restrict__ w_ws,
    const uint16_t* __restrict__ h_ws, uint16_t* __restrict__ out) {
  extern __shared__ uint4 dsm[];
  __shared__ float red[kDownWaves][8];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x >> 1;                       // 16-row tile of the output
  const int row = 8 * (blockIdx.x & 1) + (lane & 7);   // the lane's row inside the tile
  const int q = lane >> 4, sub = (lane >> 3) & 1;      // K quarter, item of the pair

  const Staged<kDownPieces> hr = stage_load<kDownPieces>(h_ws, J * (I / 8));
  uint4* hl = dsm;  // [J][I] bf16: h of every expert of the step

  const size_t mat_codes = (size_t)H * I / 2;
  const size_t mat_groups = (size_t)H * (I / kGroup);
  const int G = I / kGroup, nfull = G / 2;
  const int NT = H / 16;
  const int nitems = J * nfull + ((G & 1) ? J : 0);
  const int npairs = (nitems + 1) / 2;

  float acc = 0.f;
  DownLoad f[kDownBatch];
  // loads are unconditional (item index clamped, surplus results unused), so
  // the expert ids arrive with one wait and the wait for h below is exact
  auto load_batch = [&](int p0) {
    int eb[kDownBatch];
#pragma unroll
    for (int i = 0; i < kDownBatch; ++i) {
      const DownItem d = down_item(min(2 * (p0 + kDownWaves * i) + sub, nitems - 1), nfull, J);
      const int jc = min(d.j, k - 1);
      eb[i] = ids_ws[jc];
      const float wl = w_ws[jc];
      f[i].w = d.j < k ? wl : 1.f;
    }
#pragma unroll
    for (int i = 0; i < kDownBatch; ++i) {
      const DownItem d = down_item(min(2 * (p0 + kDownWaves * i) + sub, nitems - 1), nfull, J);
      const uint8_t* mq = d.j < k ? dn_q + (size_t)eb[i] * mat_codes : sh_q;
      const uint16_t* ms = d.j < k ? dn_s + (size_t)eb[i] * mat_groups : sh_s;
      const uint16_t* mb = d.j < k ? dn_b + (size_t)eb[i] * mat_groups : sh_b;
      if (!d.tail) {
        f[i].codes = *(const uint4*)(mq + ((size_t)d.c * NT + t) * 1024 + 16 * (16 * q + row));
        const size_t g = 32 * ((size_t)d.c * NT + t) + 2 * row;
        f[i].s2 = *(const uint32_t*)(ms + g);
        f[i].b2 = *(const uint32_t*)(mb + g);
      } else {
        const uint2 cd = *(const uint2*)(mq + (size_t)d.c * NT * 1024 + (size_t)t * 512 + 8 * (16 * q + row));
        f[i].codes = make_uint4(cd.x, cd.y, 0u, 0u);
        const size_t g = 32 * (size_t)d.c * NT + 16 * (size_t)t + row;
        f[i].s2 = ms[g];
        f[i].b2 = mb[g];
      }
    }
  };
  auto compute_batch = [&](int p0) {
#pragma unroll
    for (int i = 0; i < kDownBatch; ++i) {
      const int it = 2 * (p0 + kDownWaves * i) + sub;
      if (it >= nitems) continue;
      const DownItem d = down_item(it, nfull, J);
      const uint4* x = hl + (size_t)d.j * I / 8;
      const int k0 = 128 * d.c + 16 * q;  // first K value of the lane's first 16
      const float s0 = bf16_bits_to_f32(f[i].s2 & 0xFFFFu), b0 = bf16_bits_to_f32(f[i].b2 & 0xFFFFu);
      float v = dot16(f[i].codes.x, f[i].codes.y, x[k0 / 8], x[k0 / 8 + 1], s0, b0);
      if (!d.tail) {
        const float s1 = bf16_bits_to_f32(f[i].s2 >> 16), b1 = bf16_bits_to_f32(f[i].b2 >> 16);
        v += dot16(f[i].codes.z, f[i].codes.w, x[(k0 + 64) / 8], x[(k0 + 64) / 8 + 1], s1, b1);
      }
      acc = __builtin_fmaf(f[i].w, v, acc);
    }
  };
  load_batch(wv);  // in flight while h is staged
  stage_store(hr, J * (I / 8), hl);
  __syncthreads();
  compute_batch(wv);
  for (int p0 = wv + kDownWaves * kDownBatch; p0 < npairs; p0 += kDownWaves * kDownBatch) {
    load_batch(p0);
    compute_batch(p0);
  }
  acc = sum_quarters(acc);         // the four K quarters of a row
  acc += __shfl_xor(acc, 8);       // the two items of a pair
  if (lane < 8) red[wv][lane] = acc;
  __syncthreads();
  if (threadIdx.x < 8) {
    float p = 0.f;
#pragma unroll
    for (int w = 0; w < kDownWaves; ++w) p += red[w][threadIdx.x];
    out[8 * blockIdx.x + threadIdx.x] = f32_to_bf16_bits(p);
  }
}

// ----------------------------------------------------------------------------
// Scratch of moe_decode_ffn_q4_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends, so that the call allocates nothing.  In host
// code `scratch` names a host-side stand-in, never the device memory: its
// address on a device comes from hipGetSymbolAddress, looked up once per device
// (with that device current) and kept.
static __device__ __align__(256) uint8_t scratch[MOEQ4_DECODE_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
static std::mutex g_scratch_mutex;

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) {
    note_hip_error(err, "hipGetDevice");
    return err;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) {
    note_hip_error(hipErrorInvalidDevice, "decode scratch: device index");
    return hipErrorInvalidDevice;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess || !p) {
        note_hip_error(err != hipSuccess ? err : hipErrorInvalidSymbol, "hipGetSymbolAddress(decode scratch)");
        return err != hipSuccess ? err : hipErrorInvalidSymbol;
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodePlan decode_plan(int E, int k, int H, int I, bool shared) {
  DecodePlan p{};
  p.J = k + (shared ? 1 : 0);
  p.ws_ids = 0;
  p.ws_w = align256(sizeof(int32_t) * (size_t)k);
  p.ws_h = p.ws_w + align256(sizeof(float) * (size_t)k);
  p.ws_bytes = p.ws_h + align256(sizeof(uint16_t) * (size_t)p.J * I);
  p.lds_gateup = (size_t)H * 2;
  p.lds_down = (size_t)p.J * I * 2;
  (void)E;
  return p;
}

hipError_t decode_launch(const DecodePlan& p, const float* logits, const uint16_t* x, int E, int k, int H, int I,
                         const uint8_t* gu_q, const uint16_t* gu_s, const uint16_t* gu_b, const uint8_t* dn_q,
                         const uint16_t* dn_s, const uint16_t* dn_b, const uint8_t* sh_gu_q,
                         const uint16_t* sh_gu_s, const uint16_t* sh_gu_b, const uint8_t* sh_dn_q,
                         const uint16_t* sh_dn_s, const uint16_t* sh_dn_b, int32_t* ids_out, float* w_out,
                         uint16_t* out, void* workspace, hipStream_t stream) {
  char* ws = (char*)workspace;
  int32_t* ids_ws = (int32_t*)(ws + p.ws_ids);
  float* w_ws = (float*)(ws + p.ws_w);
  uint16_t* h_ws = (uint16_t*)(ws + p.ws_h);
  const void* fn;
  if (E <= 64) fn = (const void*)&k_decode_gateup<1>;
  else if (E <= 128) fn = (const void*)&k_decode_gateup<2>;
  else if (E <= 256) fn = (const void*)&k_decode_gateup<4>;
  else if (E <= 512) fn = (const void*)&k_decode_gateup<8>;
  else fn = (const void*)&k_decode_gateup<16>;
  hipError_t err = launch("k_decode_gateup", fn, dim3(p.J * (I / 16)), dim3(kDecThreads), p.lds_gateup, stream,
                          logits, x, E, k, H, I, gu_q, gu_s, gu_b, sh_gu_q, sh_gu_s, sh_gu_b, ids_ws, w_ws, h_ws,
                          ids_out, w_out);
  if (err != hipSuccess) return err;
  return launch("k_decode_down", (const void*)&k_decode_down, dim3(H / 8), dim3(kDownThreads), p.lds_down,
                stream, k, H, I, p.J, dn_q, dn_s, dn_b, sh_dn_q, sh_dn_s, sh_dn_b, (const int32_t*)ids_ws,
                (const float*)w_ws, (const uint16_t*)h_ws, out);
}

}  // namespace moeq4
