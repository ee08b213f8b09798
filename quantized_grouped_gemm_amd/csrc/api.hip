// api.hip -- the C ABI of include/moeq4.h: host-side argument checks, tile
// choice from the workload shape, and kernel launches on the caller's stream.
// Nothing here allocates, copies to the host or synchronises.
#include "common.h"

#include <stdio.h>

using namespace moeq4;

namespace {

thread_local char g_detail[256] = "";

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_block_rows(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 160 || bm == 256; }

int check_routing_shape(int T, int E, int k) {
  if (T < 0 || E < 1 || E > MOEQ4_MAX_EXPERTS || k < 1 || k > E) return MOEQ4_ERR_SHAPE;
  if (k > MOEQ4_MAX_TOPK) return MOEQ4_ERR_UNSUPPORTED;
  if ((long long)T * k > (long long)INT32_MAX / 2) return MOEQ4_ERR_SHAPE;
  return MOEQ4_OK;
}

// block_rows 0 -> default; returns <= 0 on error
int resolve_block_rows(int T, int E, int k, int block_rows) {
  if (block_rows == 0) return moe_default_block_rows(T, E, k);
  return valid_block_rows(block_rows) ? block_rows : MOEQ4_ERR_SHAPE;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the chunked prefill: the routing outputs and scratch of one
// chunk, then the FFN scratch of one chunk (each sized for the larger of a full
// chunk and the last, shorter one).
struct ChunkLayout {
  int tc, bm;  // chunk tokens in effect, block rows
  size_t ids, w, counts, offsets, perm, inv_perm, blocks, nblk, route_ws, ffn_ws, total;
};

int chunk_layout(int T, int chunk, int H, int I, int E, int k, int block_rows, int shared, ChunkLayout& L) {
  if (T < 0 || chunk < 4 || chunk % 4 != 0) return MOEQ4_ERR_SHAPE;
  L.tc = T > 0 && chunk > T ? T : chunk;
  int rc = check_routing_shape(L.tc, E, k);
  if (rc != MOEQ4_OK) return rc;
  if (H < 64 || H % 64 != 0 || I < 64 || I % 64 != 0) return MOEQ4_ERR_SHAPE;
  if ((long long)E * 2 * I * (H / 2) >= (1LL << 31) || (long long)E * H * (I / 2) >= (1LL << 31))
    return MOEQ4_ERR_SHAPE;
  const long long A = (long long)L.tc * k;
  if (A * I * 2 >= (1LL << 31) || (long long)L.tc * H * 2 >= (1LL << 31)) return MOEQ4_ERR_SHAPE;
  L.bm = resolve_block_rows(L.tc, E, k, block_rows);
  if (L.bm <= 0) return L.bm;
  const int last = T > 0 && T % L.tc != 0 ? T % L.tc : L.tc;
  const int mb = moe_max_blocks(L.tc, E, k, L.bm);
  if (mb < 0) return mb;
  size_t o = 0;
  L.ids = o;      o += align256(sizeof(int32_t) * (size_t)A);
  L.w = o;        o += align256(sizeof(float) * (size_t)A);
  L.counts = o;   o += align256(sizeof(int32_t) * (size_t)E);
  L.offsets = o;  o += align256(sizeof(int32_t) * (size_t)(E + 1));
  L.perm = o;     o += align256(sizeof(int32_t) * (size_t)A);
  L.inv_perm = o; o += align256(sizeof(int32_t) * (size_t)A);
  L.blocks = o;   o += align256(sizeof(int32_t) * 4 * (size_t)mb);
  L.nblk = o;     o += align256(sizeof(int32_t));
  const size_t rws0 = route_plan(L.tc, E, k).ws_bytes, rws1 = route_plan(last, E, k).ws_bytes;
  L.route_ws = o; o += align256(rws0 > rws1 ? rws0 : rws1);
  const size_t fws0 = ffn_plan(L.tc, H, I, k, shared != 0).ws_bytes, fws1 = ffn_plan(last, H, I, k, shared != 0).ws_bytes;
  L.ffn_ws = o;   o += align256(fws0 > fws1 ? fws0 : fws1);
  L.total = o;
  return MOEQ4_OK;
}

}  // namespace

namespace moeq4 {
void note_hip_error(hipError_t err, const char* what) {
  snprintf(g_detail, sizeof g_detail, "%s: %s (%d)", what, hipGetErrorString(err), (int)err);
}
}  // namespace moeq4

extern "C" {

const char* moe_last_error_detail(void) { return g_detail; }

const char* moe_strerror(int status) {
  switch (status) {
    case MOEQ4_OK: return "ok";
    case MOEQ4_ERR_NULL: return "a required pointer is NULL";
    case MOEQ4_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MOEQ4_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MOEQ4_ERR_WORKSPACE: return "workspace smaller than required";
    case MOEQ4_ERR_UNSUPPORTED: return "request not supported by this build";
    case MOEQ4_ERR_HIP: return "a HIP launch failed";
    default: return "unknown status";
  }
}

int moe_default_block_rows(int T, int E, int k) {
  const int rc = check_routing_shape(T, E, k);
  if (rc != MOEQ4_OK) return rc;
  // mean rows per expert, with headroom for the spread around it.  Below 64
  // rows the 64-row tall-block kernel (one filled 32-row tile per block)
  // measured fastest down to ~2 rows per expert; above 128, 160-row blocks
  // (five tiles) hold a typical expert of a heavy load in one block, so its
  // weights are streamed and rebuilt once (256-row blocks: on request,
  // measured slower)
  const long long A = (long long)T * k;
  const long long want = (A * 5 + 4LL * E - 1) / (4LL * E);  // ceil(1.25 * A / E)
  if (want > 128) return 160;
  return want > 64 ? 128 : 64;
}

int moe_max_blocks(int T, int E, int k, int block_rows) {
  const int rc = check_routing_shape(T, E, k);
  if (rc != MOEQ4_OK) return rc;
  const int bm = resolve_block_rows(T, E, k, block_rows);
  if (bm <= 0) return bm;
  const long long A = (long long)T * k;
  const long long m = A < E ? A : E;
  return (int)((A + m * (bm - 1)) / bm);
}

size_t moe_route_workspace_bytes(int T, int E, int k, int block_rows) {
  if (check_routing_shape(T, E, k) != MOEQ4_OK) return 0;
  if (resolve_block_rows(T, E, k, block_rows) <= 0) return 0;
  return route_plan(T, E, k).ws_bytes;
}

int moe_route(const float* logits, int T, int E, int k, int block_rows, int32_t* topk_ids,
              float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
              int32_t* blocks, int32_t* num_blocks, void* workspace, size_t ws_bytes,
              void* stream) {
  int rc = check_routing_shape(T, E, k);
  if (rc != MOEQ4_OK) return rc;
  const int bm = resolve_block_rows(T, E, k, block_rows);
  if (bm <= 0) return bm;
  if (!counts || !offsets || !num_blocks) return MOEQ4_ERR_NULL;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !perm || !inv_perm || !blocks))
    return MOEQ4_ERR_NULL;
  const RoutePlan plan = route_plan(T, E, k);
  if (ws_bytes < plan.ws_bytes) return MOEQ4_ERR_WORKSPACE;
  if (plan.ws_bytes > 0 && !workspace) return MOEQ4_ERR_NULL;
  const void* ptrs[] = {logits, topk_ids, topk_w, counts, offsets, perm, inv_perm, blocks,
                        num_blocks, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOEQ4_ERR_ALIGN;
  const hipError_t err = route_launch(plan, logits, T, E, k, bm, topk_ids, topk_w, counts, offsets,
                                      perm, inv_perm, blocks, num_blocks, workspace,
                                      (hipStream_t)stream);
  return err == hipSuccess ? MOEQ4_OK : MOEQ4_ERR_HIP;
}

int moe_topk_softmax(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w, void* stream) {
  const int rc = check_routing_shape(T, E, k);
  if (rc != MOEQ4_OK) return rc;
  if (T == 0) return MOEQ4_OK;
  if (!logits || !topk_ids || !topk_w) return MOEQ4_ERR_NULL;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return MOEQ4_ERR_ALIGN;
  return topk_launch(logits, T, E, k, topk_ids, topk_w, (hipStream_t)stream) == hipSuccess ? MOEQ4_OK : MOEQ4_ERR_HIP;
}

int moe_prepack_q4(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int E,
                   int N, int K, uint8_t* codes_t, uint16_t* scales_t, uint16_t* biases_t,
                   void* stream) {
  if (E < 1 || N < 16 || N % 16 != 0 || K < 64 || K % 64 != 0) return MOEQ4_ERR_SHAPE;
  if ((long long)E * N * (K / 2) >= (1LL << 31)) return MOEQ4_ERR_SHAPE;
  if (!codes || !scales || !biases || !codes_t || !scales_t || !biases_t) return MOEQ4_ERR_NULL;
  const void* ptrs[] = {codes, scales, biases, codes_t, scales_t, biases_t};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOEQ4_ERR_ALIGN;
  const hipError_t err = prepack_launch(codes, scales, biases, E, N, K, codes_t, scales_t,
                                        biases_t, (hipStream_t)stream);
  return err == hipSuccess ? MOEQ4_OK : MOEQ4_ERR_HIP;
}

int moe_dequant_q4(const uint8_t* codes_t, const uint16_t* scales_t, const uint16_t* biases_t, int E, int N,
                   int K, uint16_t* out, void* stream) {
  if (E < 1 || N < 16 || N % 16 != 0 || K < 64 || K % 64 != 0) return MOEQ4_ERR_SHAPE;
  if ((long long)E * N * (K / 2) >= (1LL << 31)) return MOEQ4_ERR_SHAPE;
  if (!codes_t || !scales_t || !biases_t || !out) return MOEQ4_ERR_NULL;
  const void* ptrs[] = {codes_t, scales_t, biases_t, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOEQ4_ERR_ALIGN;
  return moeq4::dequant_launch(codes_t, scales_t, biases_t, E, N, K, out, (hipStream_t)stream) == hipSuccess
             ? MOEQ4_OK
             : MOEQ4_ERR_HIP;
}

int moe_grouped_gemm_q4(const uint16_t* X, int T, int K, int N, int E, int k,
                        const uint8_t* codes_t, const uint16_t* scales_t,
                        const uint16_t* biases_t, const int32_t* perm, const int32_t* blocks,
                        const int32_t* num_blocks, int max_blocks, int block_rows, uint16_t* Y,
                        void* stream) {
  int rc = check_routing_shape(T, E, k);
  if (rc != MOEQ4_OK) return rc;
  if (K < 64 || K % 64 != 0 || N < 16 || N % 16 != 0) return MOEQ4_ERR_SHAPE;
  if ((long long)T * K * 2 >= (1LL << 31) || (long long)E * N * (K / 2) >= (1LL << 31))
    return MOEQ4_ERR_SHAPE;
  const int bm = resolve_block_rows(T, E, k, block_rows);
  if (bm <= 0) return bm;
  const int bound = moe_max_blocks(T, E, k, bm);
  if (bound < 0) return bound;
  if (max_blocks < bound) return MOEQ4_ERR_SHAPE;
  if (T == 0) return MOEQ4_OK;
  if (!X || !codes_t || !scales_t || !biases_t || !perm || !blocks || !num_blocks || !Y)
    return MOEQ4_ERR_NULL;
  const void* ptrs[] = {X, codes_t, scales_t, biases_t, perm, blocks, num_blocks, Y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOEQ4_ERR_ALIGN;
  const hipError_t err = gemm_q4_launch(X, T, K, N, E, k, codes_t, scales_t, biases_t, perm,
                                        blocks, num_blocks, max_blocks, bm, Y,
                                        (hipStream_t)stream);
  return err == hipSuccess ? MOEQ4_OK : MOEQ4_ERR_HIP;
}

int moe_route_grouped_gemm_q4(const float* logits, const uint16_t* X, int T, int K, int N, int E, int k,
                              const uint8_t* codes_t, const uint16_t* scales_t, const uint16_t* biases_t,
                              int block_rows, int32_t* topk_ids, float* topk_w, int32_t* counts,
                              int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* blocks,
                              int32_t* num_blocks, int max_blocks, uint16_t* Y, void* workspace,
                              size_t ws_bytes, void* stream) {
  int rc = check_routing_shape(T, E, k);
  if (rc != MOEQ4_OK) return rc;
  if (K < 64 || K % 64 != 0 || N < 16 || N % 16 != 0) return MOEQ4_ERR_SHAPE;
  if ((long long)T * K * 2 >= (1LL << 31) || (long long)E * N * (K / 2) >= (1LL << 31))
    return MOEQ4_ERR_SHAPE;
  const int bm = resolve_block_rows(T, E, k, block_rows);
  if (bm <= 0) return bm;
  const int bound = moe_max_blocks(T, E, k, bm);
  if (bound < 0) return bound;
  if (max_blocks < bound) return MOEQ4_ERR_SHAPE;
  if (!counts || !offsets || !num_blocks) return MOEQ4_ERR_NULL;
  if (T > 0 && (!logits || !X || !codes_t || !scales_t || !biases_t || !topk_ids || !topk_w || !perm ||
                !inv_perm || !blocks || !Y))
    return MOEQ4_ERR_NULL;
  const RoutePlan plan = route_plan(T, E, k);
  if (ws_bytes < plan.ws_bytes) return MOEQ4_ERR_WORKSPACE;
  if (plan.ws_bytes > 0 && !workspace) return MOEQ4_ERR_NULL;
  const void* ptrs[] = {logits, X, codes_t, scales_t, biases_t, topk_ids, topk_w, counts, offsets,
                        perm, inv_perm, blocks, num_blocks, Y, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOEQ4_ERR_ALIGN;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t err;
  static_assert(kRouteInLaunchMax == MOEQ4_ROUTE_IN_LAUNCH_MAX, "the launch's ranking limit");
  if (T > 0 && bm == 64 && (long long)T * k <= MOEQ4_ROUTE_IN_LAUNCH_MAX) {
    err = topk_launch(logits, T, E, k, topk_ids, topk_w, st);
    if (err == hipSuccess)
      err = route_gemm_q4_launch(topk_ids, X, T, K, N, E, k, codes_t, scales_t, biases_t, counts, offsets, perm,
                                 inv_perm, blocks, num_blocks, Y, st);
  } else {
    err = route_launch(plan, logits, T, E, k, bm, topk_ids, topk_w, counts, offsets, perm, inv_perm, blocks,
                       num_blocks, workspace, st);
    if (err == hipSuccess && T > 0)
      err = gemm_q4_launch(X, T, K, N, E, k, codes_t, scales_t, biases_t, perm, blocks, num_blocks, max_blocks, bm,
                           Y, st);
  }
  return err == hipSuccess ? MOEQ4_OK : MOEQ4_ERR_HIP;
}

static int check_decode_shape(int E, int k, int H, int I, int shared) {
  if (E < 1 || E > MOEQ4_MAX_EXPERTS || k < 1 || k > E) return MOEQ4_ERR_SHAPE;
  if (k > MOEQ4_MAX_TOPK) return MOEQ4_ERR_UNSUPPORTED;
  if (H < 128 || H % 64 != 0 || I < 128 || I % 64 != 0) return MOEQ4_ERR_SHAPE;
  if ((long long)E * 2 * I * (H / 2) >= (1LL << 31)) return MOEQ4_ERR_SHAPE;
  if (H > 8192) return MOEQ4_ERR_UNSUPPORTED;  // x staged as at most two 16-byte pieces per thread
  const DecodePlan p = decode_plan(E, k, H, I, shared != 0);
  if (p.lds_down > 65536 || p.lds_gateup > 65536) return MOEQ4_ERR_UNSUPPORTED;
  return MOEQ4_OK;
}

size_t moe_decode_workspace_bytes(int E, int k, int H, int I, int shared) {
  if (check_decode_shape(E, k, H, I, shared) != MOEQ4_OK) return 0;
  return decode_plan(E, k, H, I, shared != 0).ws_bytes;
}

// Checks and launch shared by moe_decode_ffn_q4 and moe_decode_ffn_q4_noalloc;
// workspace == nullptr with no_alloc: the library's per-device scratch array.
static int decode_call(const float* logits, const uint16_t* x, int E, int k, int H, int I,
                       const uint8_t* gu_codes_t, const uint16_t* gu_scales_t, const uint16_t* gu_biases_t,
                       const uint8_t* dn_codes_t, const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                       const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t,
                       const uint16_t* sh_gu_biases_t, const uint8_t* sh_dn_codes_t,
                       const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t, int32_t* topk_ids,
                       float* topk_w, uint16_t* out, void* workspace, size_t ws_bytes, bool no_alloc,
                       void* stream) {
  const void* sh[] = {sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                      sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t};
  int nsh = 0;
  for (const void* p : sh) nsh += p != nullptr;
  if (nsh != 0 && nsh != 6) return MOEQ4_ERR_NULL;
  const int shared = nsh == 6;
  const int rc = check_decode_shape(E, k, H, I, shared);
  if (rc != MOEQ4_OK) return rc;
  if (!logits || !x || !gu_codes_t || !gu_scales_t || !gu_biases_t || !dn_codes_t || !dn_scales_t ||
      !dn_biases_t || !out || (!no_alloc && !workspace))
    return MOEQ4_ERR_NULL;
  const void* ptrs[] = {logits, x, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t, dn_scales_t,
                        dn_biases_t, out, workspace, topk_ids, topk_w};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOEQ4_ERR_ALIGN;
  for (const void* p : sh)
    if (p && !aligned16(p)) return MOEQ4_ERR_ALIGN;
  const DecodePlan plan = decode_plan(E, k, H, I, shared);
  if (no_alloc) {
    if (plan.ws_bytes > (size_t)MOEQ4_DECODE_SCRATCH_BYTES) return MOEQ4_ERR_UNSUPPORTED;
    const hipError_t serr = decode_scratch(&workspace);
    if (serr != hipSuccess) return MOEQ4_ERR_HIP;
  } else if (ws_bytes < plan.ws_bytes) {
    return MOEQ4_ERR_WORKSPACE;
  }
  const hipError_t err = decode_launch(plan, logits, x, E, k, H, I, gu_codes_t, gu_scales_t, gu_biases_t,
                                       dn_codes_t, dn_scales_t, dn_biases_t, sh_gu_codes_t, sh_gu_scales_t,
                                       sh_gu_biases_t, sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t, topk_ids,
                                       topk_w, out, workspace, (hipStream_t)stream);
  return err == hipSuccess ? MOEQ4_OK : MOEQ4_ERR_HIP;
}

int moe_decode_ffn_q4(const float* logits, const uint16_t* x, int E, int k, int H, int I,
                      const uint8_t* gu_codes_t, const uint16_t* gu_scales_t,
                      const uint16_t* gu_biases_t, const uint8_t* dn_codes_t,
                      const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                      const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t,
                      const uint16_t* sh_gu_biases_t, const uint8_t* sh_dn_codes_t,
                      const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t,
                      int32_t* topk_ids, float* topk_w, uint16_t* out, void* workspace,
                      size_t ws_bytes, void* stream) {
  return decode_call(logits, x, E, k, H, I, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t, dn_scales_t,
                     dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t, sh_dn_codes_t, sh_dn_scales_t,
                     sh_dn_biases_t, topk_ids, topk_w, out, workspace, ws_bytes, false, stream);
}

int moe_decode_ffn_q4_noalloc(const float* logits, const uint16_t* x, int E, int k, int H, int I,
                              const uint8_t* gu_codes_t, const uint16_t* gu_scales_t,
                              const uint16_t* gu_biases_t, const uint8_t* dn_codes_t,
                              const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                              const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t,
                              const uint16_t* sh_gu_biases_t, const uint8_t* sh_dn_codes_t,
                              const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t,
                              int32_t* topk_ids, float* topk_w, uint16_t* out, void* stream) {
  return decode_call(logits, x, E, k, H, I, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t, dn_scales_t,
                     dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t, sh_dn_codes_t, sh_dn_scales_t,
                     sh_dn_biases_t, topk_ids, topk_w, out, nullptr, 0, true, stream);
}

static int check_small_shape(int T, int E, int k, int H, int I) {
  if (T < 1 || E < 1 || E > MOEQ4_MAX_EXPERTS || k < 1 || k > E) return MOEQ4_ERR_SHAPE;
  if (k > MOEQ4_MAX_TOPK || T > MOEQ4_SMALL_MAX_T) return MOEQ4_ERR_UNSUPPORTED;
  if (H < 128 || H % 64 != 0 || I < 128 || I % 64 != 0) return MOEQ4_ERR_SHAPE;
  if ((long long)E * 2 * I * (H / 2) >= (1LL << 31)) return MOEQ4_ERR_SHAPE;
  if (!small_fits(T, E, k, H, I)) return MOEQ4_ERR_UNSUPPORTED;
  return MOEQ4_OK;
}

size_t moe_small_batch_workspace_bytes(int T, int E, int k, int H, int I, int shared) {
  (void)shared;
  if (check_small_shape(T, E, k, H, I) != MOEQ4_OK) return 0;
  return small_plan(T, E, k, H, I).ws_bytes;
}

int moe_small_batch_ffn_q4(const float* logits, const uint16_t* x, int T, int E, int k, int H, int I,
                           const uint8_t* gu_codes_t, const uint16_t* gu_scales_t,
                           const uint16_t* gu_biases_t, const uint8_t* dn_codes_t,
                           const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                           const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t,
                           const uint16_t* sh_gu_biases_t, const uint8_t* sh_dn_codes_t,
                           const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t,
                           int32_t* topk_ids, float* topk_w, uint16_t* out, void* workspace,
                           size_t ws_bytes, void* stream) {
  const void* sh[] = {sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                      sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t};
  int nsh = 0;
  for (const void* p : sh) nsh += p != nullptr;
  if (nsh != 0 && nsh != 6) return MOEQ4_ERR_NULL;
  const int rc = check_small_shape(T, E, k, H, I);
  if (rc != MOEQ4_OK) return rc;
  if (!logits || !x || !gu_codes_t || !gu_scales_t || !gu_biases_t || !dn_codes_t || !dn_scales_t ||
      !dn_biases_t || !out || !workspace)
    return MOEQ4_ERR_NULL;
  const void* ptrs[] = {logits, x, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t, dn_scales_t,
                        dn_biases_t, out, workspace, topk_ids, topk_w};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOEQ4_ERR_ALIGN;
  for (const void* p : sh)
    if (p && !aligned16(p)) return MOEQ4_ERR_ALIGN;
  const SmallPlan plan = small_plan(T, E, k, H, I);
  if (ws_bytes < plan.ws_bytes) return MOEQ4_ERR_WORKSPACE;
  const hipError_t err = small_launch(plan, logits, x, T, E, k, H, I, gu_codes_t, gu_scales_t, gu_biases_t,
                                      dn_codes_t, dn_scales_t, dn_biases_t, sh_gu_codes_t, sh_gu_scales_t,
                                      sh_gu_biases_t, sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t, topk_ids,
                                      topk_w, out, workspace, (hipStream_t)stream);
  return err == hipSuccess ? MOEQ4_OK : MOEQ4_ERR_HIP;
}

static int check_ffn_shape(int T, int H, int I, int E, int k) {
  const int rc = check_routing_shape(T, E, k);
  if (rc != MOEQ4_OK) return rc;
  if (H < 64 || H % 64 != 0 || I < 64 || I % 64 != 0) return MOEQ4_ERR_SHAPE;
  const long long A = (long long)T * k;
  if ((long long)T * H * 2 >= (1LL << 31) || A * I * 2 >= (1LL << 31) ||
      (long long)E * 2 * I * (H / 2) >= (1LL << 31) || (long long)E * H * (I / 2) >= (1LL << 31))
    return MOEQ4_ERR_SHAPE;
  return MOEQ4_OK;
}

size_t moe_expert_ffn_workspace_bytes(int T, int H, int I, int E, int k, int shared) {
  if (check_ffn_shape(T, H, I, E, k) != MOEQ4_OK) return 0;
  return ffn_plan(T, H, I, k, shared != 0).ws_bytes;
}

size_t moe_prefill_ffn_chunked_workspace_bytes(int T, int chunk_tokens, int H, int I, int E, int k,
                                               int block_rows, int shared) {
  ChunkLayout L;
  if (chunk_layout(T, chunk_tokens, H, I, E, k, block_rows, shared, L) != MOEQ4_OK) return 0;
  return L.total;
}

int moe_prefill_ffn_chunked_q4(const float* logits, const uint16_t* X, int T, int H, int I, int E, int k,
                               const uint8_t* gu_codes_t, const uint16_t* gu_scales_t,
                               const uint16_t* gu_biases_t, const uint8_t* dn_codes_t,
                               const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                               const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t,
                               const uint16_t* sh_gu_biases_t, const uint8_t* sh_dn_codes_t,
                               const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t,
                               int chunk_tokens, int block_rows, int32_t* topk_ids, float* topk_w,
                               uint16_t* out, void* workspace, size_t ws_bytes, void* stream) {
  const void* sh[] = {sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                      sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t};
  int nsh = 0;
  for (const void* p : sh) nsh += p != nullptr;
  if (nsh != 0 && nsh != 6) return MOEQ4_ERR_NULL;
  const int shared = nsh == 6;
  ChunkLayout L;
  const int rc = chunk_layout(T, chunk_tokens, H, I, E, k, block_rows, shared, L);
  if (rc != MOEQ4_OK) return rc;
  if (T == 0) return MOEQ4_OK;
  if (!logits || !X || !gu_codes_t || !gu_scales_t || !gu_biases_t || !dn_codes_t || !dn_scales_t ||
      !dn_biases_t || !out || !workspace)
    return MOEQ4_ERR_NULL;
  const void* ptrs[] = {logits, X, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t, dn_scales_t,
                        dn_biases_t, out, workspace, topk_ids, topk_w};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOEQ4_ERR_ALIGN;
  for (const void* p : sh)
    if (p && !aligned16(p)) return MOEQ4_ERR_ALIGN;
  if (ws_bytes < L.total) return MOEQ4_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* perm = (int32_t*)(ws + L.perm);
  int32_t* inv_perm = (int32_t*)(ws + L.inv_perm);
  int32_t* blocks = (int32_t*)(ws + L.blocks);
  int32_t* nblk = (int32_t*)(ws + L.nblk);
  const hipStream_t st = (hipStream_t)stream;
  // Every chunk: route its tokens, then run the FFN on them, reusing the same
  // scratch (stream order keeps a chunk's reads before the next chunk's
  // writes).  Chunk starts are multiples of chunk_tokens (a multiple of 4), so
  // every per-chunk pointer stays 16-byte aligned.
  for (int t0 = 0; t0 < T; t0 += L.tc) {
    const int tn = T - t0 < L.tc ? T - t0 : L.tc;
    int32_t* ids = topk_ids ? topk_ids + (size_t)t0 * k : (int32_t*)(ws + L.ids);
    float* w = topk_w ? topk_w + (size_t)t0 * k : (float*)(ws + L.w);
    hipError_t err = route_launch(route_plan(tn, E, k), logits + (size_t)t0 * E, tn, E, k, L.bm, ids, w, counts,
                                  offsets, perm, inv_perm, blocks, nblk, ws + L.route_ws, st);
    if (err != hipSuccess) return MOEQ4_ERR_HIP;
    err = ffn_launch(ffn_plan(tn, H, I, k, shared), X + (size_t)t0 * H, tn, H, I, E, k, gu_codes_t, gu_scales_t,
                     gu_biases_t, dn_codes_t, dn_scales_t, dn_biases_t, sh_gu_codes_t, sh_gu_scales_t,
                     sh_gu_biases_t, sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t, w, perm, blocks, nblk,
                     moe_max_blocks(tn, E, k, L.bm), L.bm, out + (size_t)t0 * H, ws + L.ffn_ws, st);
    if (err != hipSuccess) return MOEQ4_ERR_HIP;
  }
  return MOEQ4_OK;
}

int moe_expert_ffn_q4(const uint16_t* X, int T, int H, int I, int E, int k, const uint8_t* gu_codes_t,
                      const uint16_t* gu_scales_t, const uint16_t* gu_biases_t, const uint8_t* dn_codes_t,
                      const uint16_t* dn_scales_t, const uint16_t* dn_biases_t, const uint8_t* sh_gu_codes_t,
                      const uint16_t* sh_gu_scales_t, const uint16_t* sh_gu_biases_t,
                      const uint8_t* sh_dn_codes_t, const uint16_t* sh_dn_scales_t,
                      const uint16_t* sh_dn_biases_t, const float* topk_w, const int32_t* perm,
                      const int32_t* blocks, const int32_t* num_blocks, int max_blocks, int block_rows,
                      uint16_t* out, void* workspace, size_t ws_bytes, void* stream) {
  const void* sh[] = {sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                      sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t};
  int nsh = 0;
  for (const void* p : sh) nsh += p != nullptr;
  if (nsh != 0 && nsh != 6) return MOEQ4_ERR_NULL;
  const int shared = nsh == 6;
  int rc = check_ffn_shape(T, H, I, E, k);
  if (rc != MOEQ4_OK) return rc;
  const int bm = resolve_block_rows(T, E, k, block_rows);
  if (bm <= 0) return bm;
  const int bound = moe_max_blocks(T, E, k, bm);
  if (bound < 0) return bound;
  if (max_blocks < bound) return MOEQ4_ERR_SHAPE;
  if (T == 0) return MOEQ4_OK;
  if (!X || !gu_codes_t || !gu_scales_t || !gu_biases_t || !dn_codes_t || !dn_scales_t || !dn_biases_t ||
      !topk_w || !perm || !blocks || !num_blocks || !out || !workspace)
    return MOEQ4_ERR_NULL;
  const void* ptrs[] = {X, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t, dn_scales_t, dn_biases_t,
                        topk_w, perm, blocks, num_blocks, out, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOEQ4_ERR_ALIGN;
  for (const void* p : sh)
    if (p && !aligned16(p)) return MOEQ4_ERR_ALIGN;
  const FfnPlan plan = ffn_plan(T, H, I, k, shared);
  if (ws_bytes < plan.ws_bytes) return MOEQ4_ERR_WORKSPACE;
  const hipError_t err = ffn_launch(plan, X, T, H, I, E, k, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t,
                                    dn_scales_t, dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                                    sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t, topk_w, perm, blocks,
                                    num_blocks, max_blocks, bm, out, workspace, (hipStream_t)stream);
  return err == hipSuccess ? MOEQ4_OK : MOEQ4_ERR_HIP;
}

// ---- the layer call: the path is chosen from the number of rows
static int layer_chunk(int T) { return T < 4 ? 4 : (T + 3) / 4 * 4; }  // the whole batch as one chunk

int moe_layer_ffn_path(int T, int E, int k, int H, int I, int shared) {
  if (T < 0) return MOEQ4_ERR_SHAPE;
  if (T == 1 && check_decode_shape(E, k, H, I, shared != 0) == MOEQ4_OK) return MOEQ4_PATH_DECODE;
  if (T >= 1 && T <= MOEQ4_SMALL_MAX_T && check_small_shape(T, E, k, H, I) == MOEQ4_OK) return MOEQ4_PATH_FEW_ROWS;
  ChunkLayout L;
  const int rc = chunk_layout(T, layer_chunk(T), H, I, E, k, 0, shared != 0, L);
  return rc == MOEQ4_OK ? MOEQ4_PATH_PREFILL : rc;
}

size_t moe_layer_ffn_workspace_bytes(int T, int H, int I, int E, int k, int block_rows, int shared) {
  const int path = moe_layer_ffn_path(T, E, k, H, I, shared);
  if (path == MOEQ4_PATH_DECODE) return moe_decode_workspace_bytes(E, k, H, I, shared);
  if (path == MOEQ4_PATH_FEW_ROWS) return moe_small_batch_workspace_bytes(T, E, k, H, I, shared);
  if (path == MOEQ4_PATH_PREFILL)
    return moe_prefill_ffn_chunked_workspace_bytes(T, layer_chunk(T), H, I, E, k, block_rows, shared);
  return 0;
}

int moe_layer_ffn_q4(const float* logits, const uint16_t* X, int T, int H, int I, int E, int k,
                     const uint8_t* gu_codes_t, const uint16_t* gu_scales_t, const uint16_t* gu_biases_t,
                     const uint8_t* dn_codes_t, const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                     const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t, const uint16_t* sh_gu_biases_t,
                     const uint8_t* sh_dn_codes_t, const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t,
                     int block_rows, int32_t* topk_ids, float* topk_w, uint16_t* out, void* workspace,
                     size_t ws_bytes, void* stream) {
  const void* sh[] = {sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                      sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t};
  int nsh = 0;
  for (const void* p : sh) nsh += p != nullptr;
  if (nsh != 0 && nsh != 6) return MOEQ4_ERR_NULL;
  const int shared = nsh == 6;
  if (block_rows != 0 && !valid_block_rows(block_rows)) return MOEQ4_ERR_SHAPE;
  const int path = moe_layer_ffn_path(T, E, k, H, I, shared);
  if (path < 0) return path;
  if (path == MOEQ4_PATH_DECODE)
    return moe_decode_ffn_q4(logits, X, E, k, H, I, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t, dn_scales_t,
                             dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t, sh_dn_codes_t,
                             sh_dn_scales_t, sh_dn_biases_t, topk_ids, topk_w, out, workspace, ws_bytes, stream);
  if (path == MOEQ4_PATH_FEW_ROWS)
    return moe_small_batch_ffn_q4(logits, X, T, E, k, H, I, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t,
                                  dn_scales_t, dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                                  sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t, topk_ids, topk_w, out, workspace,
                                  ws_bytes, stream);
  return moe_prefill_ffn_chunked_q4(logits, X, T, H, I, E, k, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t,
                                    dn_scales_t, dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                                    sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t, layer_chunk(T), block_rows,
                                    topk_ids, topk_w, out, workspace, ws_bytes, stream);
}

int moe_calibrate_mfma(int workgroups, int iters, float* out, void* stream) {
  if (!out) return MOEQ4_ERR_NULL;
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 0) return MOEQ4_ERR_SHAPE;
  if (!aligned16(out)) return MOEQ4_ERR_ALIGN;
  return moeq4::calib_mfma_launch(workgroups, iters, out, (hipStream_t)stream) == hipSuccess ? MOEQ4_OK
                                                                                            : MOEQ4_ERR_HIP;
}

}  // extern "C"
