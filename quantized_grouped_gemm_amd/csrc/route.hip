// route.hip -- GPU-resident MoE routing for gfx950.
//
// Perplexity Engineering, "Optimizing on-device inference for Apple Silicon",
// section "Keep expert routing on the GPU": after each token picks its
// experts, a histogram counts assignments per expert, a prefix scan turns the
// counts into start offsets, a scatter places rows into their expert groups,
// and a block map lists the fixed-size blocks the grouped GEMM processes.  The
// whole sequence stays on the GPU: the block count never goes to the host.
//
// Two kernels up to kSmallAssignMax assignments, three above, all on the
// caller's stream:
//   k_topk_rank      one wave per token (large inputs: workgroups of 16 waves
//                    per "chunk" of tokens; small: of 2): top-k by k rounds
//                    of a wave-wide argmax over order-preserving integer keys
//                    (DPP max + ballot), softmax over the k selected logits;
//                    then (large inputs only) the chunk's histogram and each
//                    assignment's stable rank among same-expert assignments
//                    of the chunk (ballot match masks over the expert-id bits
//                    + popcounts).
//   k_route_small    (small inputs) one workgroup does the rest from the
//                    expert ids alone: each wave ranks a contiguous range of
//                    assignments the same way, a scan over the waves gives
//                    each expert's count and per-wave bases; then offsets,
//                    block map and the scatter.
//   k_chunk_scan     (large inputs) one workgroup per 64 experts: per-expert
//                    exclusive scan over the chunks, and the counts.
//   k_scatter        (large inputs) one thread per assignment: perm and
//                    inv_perm from the offsets, which every workgroup scans
//                    from the counts; workgroup 0 also writes the offsets,
//                    the block counts' scan and the block map.
// moe_topk_softmax runs k_topk_rank alone; moe_route_grouped_gemm_q4 runs it
// and leaves the rest to the GEMM launch when that launch can rank the rows
// itself (gemm_q4.hip).
// Only integer adds decide positions, so every output is deterministic.
#include "common.h"

namespace moeq4 {

constexpr int kRouteWaves = 16;            // waves per chunk workgroup (with the histogram)
constexpr int kTopkSmallWaves = 2;         // waves (= tokens) per top-k workgroup for small inputs
constexpr int kRouteThreads = kRouteWaves * 64;
constexpr int kChunkAssignMax = 2048;      // assignments per chunk (LDS bound)
constexpr int kMaxSlicesPerWave = kChunkAssignMax / 64 / kRouteWaves;
constexpr int kSmallAssignMax = 8192;      // assignments one workgroup ranks and scatters
constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kSmallSlicesPerWave = kSmallAssignMax / 64 / kScanWaves;  // 64-assignment slices per wave

// ----------------------------------------------------------------------------
// top-k + softmax; for large inputs also the chunk histogram and in-chunk stable ranks.
// A workgroup of nw waves handles one chunk of tpc tokens; wave w takes tokens
// w, w+nw, ...  Lane l of a token's wave holds experts [l*VPT, (l+1)*VPT).
// Selection compares order-preserving integer keys of the logits (wave_topk).
// With the histogram the workgroup has kRouteWaves waves (the counters' rows);
// without it, small workgroups of one token per wave spread the selections
// over more CUs, and no LDS is used.
template <int VPT>
__global__ __launch_bounds__(kRouteThreads) void k_topk_rank(
    const float* __restrict__ logits, int T, int E, int k, int tpc, int nbits, int hist,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ local_rank) {
  extern __shared__ int smem[];
  constexpr int NW = kRouteWaves;
  int* sids = smem;                                  // [tpc * k] expert ids of the chunk
  uint16_t* cnt = (uint16_t*)(smem + tpc * k);       // [NW][E] per-wave counters, then bases

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int chunk = blockIdx.x;
  const int t0 = chunk * tpc;
  const int ntok = min(tpc, T - t0);

  const int nw = hist ? NW : (int)(blockDim.x >> 6);
  if (hist)
    for (int i = threadIdx.x; i < NW * E; i += blockDim.x) cnt[i] = 0;

  // the next token's logits are in flight while the current one is selected
  float vn[VPT];
  auto fetch = [&](int i) {
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
      const int e = lane * VPT + s;
      // clamped indices: the loads are unconditional, so they overlap
      vn[s] = logits[(size_t)(t0 + min(i, ntok - 1)) * E + min(e, E - 1)];
    }
  };
  fetch(wv);
  for (int i = wv; i < ntok; i += nw) {
    const int t = t0 + i;
    int key[VPT];
#pragma unroll
    for (int s = 0; s < VPT; ++s) key[s] = (lane * VPT + s < E) ? order_key(vn[s]) : kKeyTaken;
    fetch(i + nw);
    int my_id;
    float my_v, v0;
    wave_topk<VPT>(key, E, k, my_id, my_v, v0);
    const float ex = (lane < k) ? expf(my_v - v0) : 0.f;
    const float sum = wave_sum_f32(ex);
    if (lane < k) {
      ids_out[(size_t)t * k + lane] = my_id;
      w_out[(size_t)t * k + lane] = ex / sum;
      if (hist) sids[i * k + lane] = my_id;
    }
  }
  if (!hist) return;  // small inputs: k_route_small ranks from the ids
  __syncthreads();

  // ---- in-chunk histogram and stable ranks
  const int na = ntok * k;
  const int nslices = (na + 63) >> 6;
  const int spw = (nslices + NW - 1) / NW;  // contiguous slices per wave (<= kMaxSlicesPerWave)
  static_assert(kMaxSlicesPerWave * 64 * NW >= kChunkAssignMax, "slices per wave");
  const uint64_t lt = lanemask_lt();
  int rank[kMaxSlicesPerWave];
  int eid[kMaxSlicesPerWave];
#pragma unroll
  for (int s = 0; s < kMaxSlicesPerWave; ++s) {
    rank[s] = 0;
    eid[s] = -1;
    if (s >= spw) continue;
    const int slice = wv * spw + s;
    const int al = slice * 64 + lane;
    const bool valid = slice < nslices && al < na;
    const int e = valid ? sids[al] : 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      match &= bit ? bb : ~bb;
    }
    if (valid) {
      const int before = __popcll(match & lt);
      const int old = cnt[wv * E + e];
      rank[s] = old + before;
      eid[s] = e;
      // the highest lane of each match group publishes the new count
      if ((match >> lane) == 1ull) cnt[wv * E + e] = (uint16_t)(old + __popcll(match));
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    // all NW counters first (independent LDS reads), then the bases
    int c[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) c[w] = cnt[w * E + e];
    int run = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      cnt[w * E + e] = (uint16_t)run;
      run += c[w];
    }
    chunk_counts[(size_t)chunk * E + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kMaxSlicesPerWave; ++s) {
    if (eid[s] >= 0) {
      const int al = (wv * spw + s) * 64 + lane;
      local_rank[(size_t)t0 * k + al] = cnt[wv * E + eid[s]] + rank[s];
    }
  }
}

// ----------------------------------------------------------------------------
// Inclusive scan of an int over the 64 lanes of a wave: Hillis-Steele inside
// each row of 16 lanes (row_shr 1, 2, 4, 8), then row_bcast 15 / 31 carry the
// row totals upward.
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Block-wide exclusive scan over kScanThreads values (one per thread).
__device__ int block_exclusive_scan(int v, int* scratch /* >= kScanThreads/64 + 1 ints */,
                                    int* total) {
  constexpr int NW = kScanThreads / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int incl = wave_incl_scan_i32(v);
  if (lane == 63) scratch[wv] = incl;
  __syncthreads();
  if (wv == 0) {
    const int t = lane < NW ? scratch[lane] : 0;
    const int ti = wave_incl_scan_i32(t);
    if (lane < NW) scratch[lane] = ti - t;
    if (lane == NW - 1) scratch[NW] = ti;
  }
  __syncthreads();
  const int r = scratch[wv] + incl - v;
  *total = scratch[NW];
  __syncthreads();
  return r;
}

// From each expert's count (thread e < E holds cnt_e): counts (unless null),
// offsets, block offsets, the block count and the block map; offs_s / boffs_s
// (E + 1 ints in LDS) keep the offsets and block offsets for the caller.  Every
// thread of the kScanThreads workgroup calls it.
__device__ void counts_to_blockmap(int cnt_e, int E, int BM, int A, int32_t* __restrict__ counts,
                                   int32_t* __restrict__ offsets, int32_t* __restrict__ blocks,
                                   int32_t* __restrict__ num_blocks, int* offs_s, int* boffs_s, int* scratch) {
  const int tid = threadIdx.x;
  // Below 2^16 assignments both scans run as one over (count | blocks << 16):
  // the block total stays below E + A / BM < 2^15, so neither field carries
  // into the other.
  int total, nb_total, off, boff;
  const int nb = tid < E ? (cnt_e + BM - 1) / BM : 0;
  if (A < 65536) {
    const int pk = block_exclusive_scan(tid < E ? cnt_e | (nb << 16) : 0, scratch, &total);
    off = pk & 0xFFFF;
    boff = pk >> 16;
    nb_total = total >> 16;
    total &= 0xFFFF;
  } else {
    off = block_exclusive_scan(tid < E ? cnt_e : 0, scratch, &total);
    boff = block_exclusive_scan(nb, scratch, &nb_total);
  }
  if (tid < E) {
    if (counts) counts[tid] = cnt_e;
    offsets[tid] = off;
    offs_s[tid] = off;
    boffs_s[tid] = boff;
  }
  if (tid == 0) {
    offsets[E] = total;
    offs_s[E] = total;
    boffs_s[E] = nb_total;
    *num_blocks = nb_total;
  }
  __syncthreads();

  // block map: entry b belongs to the expert e with boffs[e] <= b < boffs[e+1]
  for (int b = tid; b < nb_total; b += kScanThreads) {
    int lo = 0, hi = E;  // invariant: boffs_s[lo] <= b < boffs_s[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (boffs_s[mid] <= b) lo = mid; else hi = mid;
    }
    const int i = b - boffs_s[lo];
    const int cnt = offs_s[lo + 1] - offs_s[lo];
    blocks[4 * (size_t)b + 0] = lo;
    blocks[4 * (size_t)b + 1] = offs_s[lo] + i * BM;
    blocks[4 * (size_t)b + 2] = min(BM, cnt - i * BM);
    blocks[4 * (size_t)b + 3] = i;
  }
}

// Large inputs: per expert, the exclusive scan over chunks, in place (chunk
// counts become chunk bases), and each expert's total into counts.  Workgroup
// g takes experts [64g, 64g + 64), one per lane, so every chunk row is read
// coalesced; its waves split the chunks into contiguous ranges, and a scan
// over the waves gives each range's base.  A range's first kChunkRegs counts
// stay in registers, loaded unconditionally (clamped rows) so they are in
// flight together.
constexpr int kChunkScanWaves = 16;
constexpr int kChunkRegs = 16;

__global__ __launch_bounds__(kChunkScanWaves * 64) void k_chunk_scan(int32_t* __restrict__ chunk_counts, int nchunks,
                                                                     int E, int32_t* __restrict__ counts) {
  __shared__ int part[kChunkScanWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = min(blockIdx.x * 64 + lane, E - 1);  // lanes past E repeat the last expert, unstored
  const bool act = blockIdx.x * 64 + lane < E;
  const int cpw = (nchunks + kChunkScanWaves - 1) / kChunkScanWaves;
  const int c_lo = min(nchunks, wv * cpw), c_hi = min(nchunks, c_lo + cpw);
  int vals[kChunkRegs];
#pragma unroll
  for (int i = 0; i < kChunkRegs; ++i) {
    const int c = c_lo + i;
    const int v = chunk_counts[(size_t)min(c, nchunks - 1) * E + e];
    vals[i] = c < c_hi ? v : 0;
  }
  int psum = 0;
#pragma unroll
  for (int i = 0; i < kChunkRegs; ++i) psum += vals[i];
  for (int c = c_lo + kChunkRegs; c < c_hi; ++c) psum += chunk_counts[(size_t)c * E + e];
  part[wv][lane] = psum;
  __syncthreads();
  if (wv == 0) {
    int run = 0;
    for (int w = 0; w < kChunkScanWaves; ++w) {
      const int x = part[w][lane];
      part[w][lane] = run;
      run += x;
    }
    if (act) counts[e] = run;
  }
  __syncthreads();
  if (!act) return;
  int run = part[wv][lane];
#pragma unroll
  for (int i = 0; i < kChunkRegs; ++i) {
    const int c = c_lo + i;
    if (c < c_hi) chunk_counts[(size_t)c * E + e] = run;
    run += vals[i];
  }
  for (int c = c_lo + kChunkRegs; c < c_hi; ++c) {
    const int x = chunk_counts[(size_t)c * E + e];
    chunk_counts[(size_t)c * E + e] = run;
    run += x;
  }
}

// ----------------------------------------------------------------------------
// Up to kSmallAssignMax assignments: histogram, stable ranks, offsets, block
// map and scatter in one workgroup, from the expert ids alone.  Wave w takes
// the contiguous assignments [w * spw * 64, (w + 1) * spw * 64) in slices of
// 64, in order: within a slice an assignment's rank among same-expert
// assignments comes from ballot match masks over the expert-id bits, across
// the wave's slices from its per-expert counter in LDS, across waves from
// the scan of those counters.  Position = offsets[e] + (same-expert
// assignments before it), the stable counting sort.
__global__ __launch_bounds__(kScanThreads) void k_route_small(
    const int32_t* __restrict__ ids, int A, int E, int BM, int nbits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ blocks, int32_t* __restrict__ num_blocks,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  __shared__ uint16_t cnt[kScanWaves][MOEQ4_MAX_EXPERTS];  // per-wave counts, then per-wave bases
  __shared__ int offs_s[MOEQ4_MAX_EXPERTS + 1];
  __shared__ int boffs_s[MOEQ4_MAX_EXPERTS + 1];
  __shared__ int scratch[kScanThreads / 64 + 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nslices = (A + 63) >> 6;
  const int spw = (nslices + kScanWaves - 1) / kScanWaves;  // <= kSmallSlicesPerWave

  // this wave's expert ids first (clamped indices: unconditional loads)
  int eid[kSmallSlicesPerWave];
#pragma unroll
  for (int s = 0; s < kSmallSlicesPerWave; ++s) {
    const int a = min((wv * spw + s) * 64 + lane, max(A - 1, 0));
    eid[s] = A > 0 ? ids[a] : 0;
  }
  for (int e = lane; e < E; e += 64) cnt[wv][e] = 0;  // this wave's own row

  const uint64_t lt = lanemask_lt();
  int rank[kSmallSlicesPerWave];
#pragma unroll
  for (int s = 0; s < kSmallSlicesPerWave; ++s) {
    rank[s] = -1;
    if (s >= spw) continue;
    const int a = (wv * spw + s) * 64 + lane;
    const bool valid = a < A;
    const int e = valid ? min(max(eid[s], 0), E - 1) : 0;
    eid[s] = e;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      match &= bit ? bb : ~bb;
    }
    if (valid) {
      const int old = cnt[wv][e];
      rank[s] = old + __popcll(match & lt);
      // the highest lane of each match group publishes the new count (a
      // wave's LDS operations complete in order, so the next slice sees it)
      if ((match >> lane) == 1ull) cnt[wv][e] = (uint16_t)(old + __popcll(match));
    }
  }
  __syncthreads();
  int cnt_e = 0;
  if (tid < E) {
    int c[kScanWaves];
#pragma unroll
    for (int w = 0; w < kScanWaves; ++w) c[w] = cnt[w][tid];
#pragma unroll
    for (int w = 0; w < kScanWaves; ++w) {
      cnt[w][tid] = (uint16_t)cnt_e;
      cnt_e += c[w];
    }
  }
  counts_to_blockmap(cnt_e, E, BM, A, counts, offsets, blocks, num_blocks, offs_s, boffs_s, scratch);
  // (counts_to_blockmap ends its scans with a barrier: the bases are visible)
  int pos[kSmallSlicesPerWave];
#pragma unroll
  for (int s = 0; s < kSmallSlicesPerWave; ++s) {
    pos[s] = -1;
    if (rank[s] < 0) continue;
    const int a = (wv * spw + s) * 64 + lane;
    const int p = offs_s[eid[s]] + cnt[wv][eid[s]] + rank[s];
    inv_perm[a] = p;
    if (p >= 0 && p < A) pos[s] = p;
  }
  // perm = the inverse, scattered in LDS (the counters' 32 KB, no longer
  // read, hold A <= kSmallAssignMax ints) and written out in order, so the
  // stores to memory are coalesced
  static_assert(sizeof(cnt) >= kSmallAssignMax * sizeof(int), "the counters hold the permutation");
  int* const perm_s = reinterpret_cast<int*>(&cnt[0][0]);
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kSmallSlicesPerWave; ++s)
    if (pos[s] >= 0) perm_s[pos[s]] = (wv * spw + s) * 64 + lane;
  __syncthreads();
  for (int i = tid; i < A; i += kScanThreads) perm[i] = perm_s[i];
}

// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void k_scatter(
    const int32_t* __restrict__ ids, int A, int E, int k, int tpc, int BM, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ local_rank, int32_t* __restrict__ offsets,
    int32_t* __restrict__ blocks, int32_t* __restrict__ num_blocks, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm) {
  __shared__ int offs_s[MOEQ4_MAX_EXPERTS + 1];
  __shared__ int boffs_s[MOEQ4_MAX_EXPERTS + 1];
  __shared__ int scratch[kScanThreads / 64 + 1];
  const int tid = threadIdx.x;
  const int a = blockIdx.x * kScanThreads + tid;
  const bool va = a < A;
  // the assignment's own loads go out together with the counts
  const int cnt_e = tid < E ? counts[tid] : 0;
  const int e = va ? ids[a] : 0;
  const int lr = va ? local_rank[a] : 0;
  if (blockIdx.x == 0) {
    counts_to_blockmap(cnt_e, E, BM, A, nullptr, offsets, blocks, num_blocks, offs_s, boffs_s, scratch);
  } else {
    int total;
    const int off = block_exclusive_scan(tid < E ? cnt_e : 0, scratch, &total);
    if (tid < E) offs_s[tid] = off;
    __syncthreads();
  }
  if (!va) return;
  const int c = a / (k * tpc);  // the chunk of token a / k
  const int p = offs_s[e] + chunk_base[(size_t)c * E + e] + lr;
  if (p >= 0 && p < A) perm[p] = a;
  inv_perm[a] = p;
}

// ----------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

RoutePlan route_plan(int T, int E, int k) {
  RoutePlan p{};
  const int nw = kRouteWaves;
  p.waves = nw;
  // about 256 chunks for long prompts; at least one token per wave
  int tpc = (T + 255) / 256;
  tpc = ((tpc + nw - 1) / nw) * nw;
  if (tpc < nw) tpc = nw;
  const int cap = kChunkAssignMax / k;
  if (tpc > cap) tpc = cap;
  if (tpc < 1) tpc = 1;
  p.tpc = tpc;
  p.nchunks = T > 0 ? (T + tpc - 1) / tpc : 0;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  p.nbits = nbits;
  p.ws_chunk_counts = 0;
  p.ws_local_rank = align256((size_t)p.nchunks * E * sizeof(int32_t));
  p.ws_bytes = p.ws_local_rank + align256((size_t)T * k * sizeof(int32_t));
  return p;
}

static const void* topk_kernel(int E) {
  if (E <= 64) return (const void*)&k_topk_rank<1>;
  if (E <= 128) return (const void*)&k_topk_rank<2>;
  if (E <= 256) return (const void*)&k_topk_rank<4>;
  if (E <= 512) return (const void*)&k_topk_rank<8>;
  return (const void*)&k_topk_rank<16>;
}

hipError_t topk_launch(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return launch("k_topk_rank", topk_kernel(E), dim3((T + kTopkSmallWaves - 1) / kTopkSmallWaves),
                dim3(64 * kTopkSmallWaves), 0, stream, logits, T, E, k, kTopkSmallWaves, nbits, 0, ids, w,
                (int32_t*)nullptr, (int32_t*)nullptr);
}

hipError_t route_launch(const RoutePlan& plan, const float* logits, int T, int E, int k, int BM,
                        int32_t* ids, float* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* inv_perm, int32_t* blocks, int32_t* num_blocks, void* workspace,
                        hipStream_t stream) {
  int32_t* chunk_counts = (int32_t*)((char*)workspace + plan.ws_chunk_counts);
  int32_t* local_rank = (int32_t*)((char*)workspace + plan.ws_local_rank);
  const int A = T * k;
  const int small = A <= kSmallAssignMax;
  hipError_t err = hipSuccess;
  if (plan.nchunks > 0) {
    if (small) {
      err = topk_launch(logits, T, E, k, ids, w, stream);
    } else {
      const size_t shmem = sizeof(int) * (size_t)plan.tpc * k + sizeof(uint16_t) * (size_t)kRouteWaves * E;
      err = launch("k_topk_rank", topk_kernel(E), dim3(plan.nchunks), dim3(kRouteThreads), shmem, stream, logits, T,
                   E, k, plan.tpc, plan.nbits, 1, ids, w, chunk_counts, local_rank);
    }
    if (err != hipSuccess) return err;
  }
  if (small)
    return launch("k_route_small", (const void*)&k_route_small, dim3(1), dim3(kScanThreads), 0, stream,
                  (const int32_t*)ids, A, E, BM, plan.nbits, counts, offsets, blocks, num_blocks, perm, inv_perm);
  err = launch("k_chunk_scan", (const void*)&k_chunk_scan, dim3((E + 63) / 64), dim3(kChunkScanWaves * 64), 0, stream,
               chunk_counts, plan.nchunks, E, counts);
  if (err != hipSuccess) return err;
  return launch("k_scatter", (const void*)&k_scatter, dim3((A + kScanThreads - 1) / kScanThreads), dim3(kScanThreads),
                0, stream, (const int32_t*)ids, A, E, k, plan.tpc, BM, (const int32_t*)counts,
                (const int32_t*)chunk_counts, (const int32_t*)local_rank, offsets, blocks, num_blocks, perm, inv_perm);
}

}  // namespace moeq4
