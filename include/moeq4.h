/*
 * moeq4.h -- C ABI of the MoE routing + group-wise affine 4-bit grouped GEMM
 * library for AMD Instinct MI355X (gfx950).
 *
 * The calls follow the problem statement of Perplexity Engineering,
 * "Optimizing on-device inference for Apple Silicon" (2026):
 *   - section "Keep expert routing on the GPU": after the per-token expert
 *     selection, a histogram counts assignments per expert, a prefix scan
 *     turns the counts into start offsets, a scatter places rows into their
 *     expert groups and a block map lists the fixed-size blocks the grouped
 *     GEMM processes; nothing waits on the host inside the layer.
 *   - section "Dequantize weights during matrix multiplication": each weight is
 *     a 4-bit code, 64 weights along K share one bf16 scale and one bf16 bias;
 *     the weights are rebuilt in bf16 a small tile at a time on chip and never
 *     written back to memory as a bf16 array; fp32 accumulation, bf16 output.
 *   - section "Qwen creates three workload shapes": a router scores the
 *     experts and picks 8 of 256 per token.
 *
 * Conventions for every call below.
 *   - Array arguments are DEVICE pointers owned by the caller (allocate them
 *     with hipMalloc or any device allocator); scalar sizes are host ints.
 *     All arrays are dense and row-major.  bf16 values travel as uint16_t bit
 *     patterns.  The library never allocates, frees, copies to the host or
 *     synchronises; it enqueues kernels on `stream` (a hipStream_t passed as
 *     void*; NULL is the null stream) and returns.
 *   - Return value: MOEQ4_OK (0) or a negative MOEQ4_ERR_* code.  All argument
 *     checks run on the host before anything is enqueued; on an error nothing
 *     is written.  MOEQ4_ERR_HIP reports a failed launch; faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - Alignment: every array pointer must be 16-byte aligned.
 *   - Calls on different streams may run concurrently as long as their output
 *     and workspace buffers do not overlap.
 *
 * Group-wise affine 4-bit matrix [N, K] (K % 64 == 0):
 *   codes  uint8  [N, K/2]   byte i of a row holds the code of K index 2i in
 *                             its low nibble and of 2i+1 in its high nibble
 *   scales uint16 [N, K/64]  bf16
 *   biases uint16 [N, K/64]  bf16
 *   weight(n, kk) = bf16( scale[n, kk/64] * code(n, kk) + bias[n, kk/64] )
 *   (scale * code + bias formed in fp32 with one rounding, as fma does).
 *   Scales must be finite with magnitude below 2^100 (the kernels scale them by
 *   2^24 on the way); biases must be finite.
 * A stack of E such matrices is [E, N, K/2] / [E, N, K/64].
 */
#ifndef MOEQ4_H
#define MOEQ4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEQ4_OK 0
#define MOEQ4_ERR_NULL (-1)        /* a required pointer is NULL */
#define MOEQ4_ERR_SHAPE (-2)       /* a size is out of range or inconsistent */
#define MOEQ4_ERR_ALIGN (-3)       /* a pointer is not 16-byte aligned */
#define MOEQ4_ERR_WORKSPACE (-4)   /* workspace smaller than required */
#define MOEQ4_ERR_UNSUPPORTED (-5) /* valid request this build does not implement */
#define MOEQ4_ERR_HIP (-6)         /* a HIP launch failed (no device, bad stream, ...) */

#define MOEQ4_MAX_EXPERTS 1024
#define MOEQ4_MAX_TOPK 64
#define MOEQ4_SMALL_MAX_T 8   /* tokens moe_small_batch_ffn_q4 takes at most */

/* Human-readable text for a status code.  Never NULL; static storage. */
const char* moe_strerror(int status);

/* Diagnostics: the HIP error text and the kernel of the calling thread's most
 * recent MOEQ4_ERR_HIP ("" if none).  Never NULL; valid until the thread's next
 * library call. */
const char* moe_last_error_detail(void);

/* Block-map tile height used when a call passes block_rows = 0: chosen from
 * the mean rows per expert, T*k/E (section "Match tile size to expert load":
 * tile height is matched to the expert load): 64 up to a mean of about 51
 * rows per expert, 128 up to about 102, 160 above (an expert of up to 160 rows
 * is then one block, its weights streamed and rebuilt once).  Negative error
 * code for invalid T, E, k. */
int moe_default_block_rows(int T, int E, int k);

/* Host-side upper bound on the number of block-map entries for any routing of
 * T tokens to k of E experts with tile height block_rows (0 = default):
 *   floor((A + m*(block_rows-1)) / block_rows),  A = T*k,  m = min(E, A).
 * Size `blocks` for this many entries and pass it to the GEMM as max_blocks.
 * Negative error code on invalid arguments. */
int moe_max_blocks(int T, int E, int k, int block_rows);

/* Bytes of device scratch moe_route needs (0 is possible).  Returns 0 on
 * invalid arguments as well; moe_route then reports the error. */
size_t moe_route_workspace_bytes(int T, int E, int k, int block_rows);

/* Routing on the GPU (section "Keep expert routing on the GPU").
 *
 * In:  logits     float [T, E]   router scores; must be finite.
 * Out: topk_ids   int32 [T, k]   per token the k largest logits, in
 *                                descending order; equal logits are ordered
 *                                by ascending expert id; -0 equals +0.
 *      topk_w     float [T, k]   softmax over the k selected logits (fp32).
 *      counts     int32 [E]      assignments per expert (histogram).
 *      offsets    int32 [E+1]    exclusive prefix sum of counts; offsets[E] = T*k.
 *      perm       int32 [T*k]    sorted position p -> assignment a = t*k + j;
 *                                experts in ascending order, and inside an
 *                                expert group ascending a (a stable sort).
 *      inv_perm   int32 [T*k]    assignment a -> sorted position p.
 *      blocks     int32 [max_blocks, 4]  entries {expert, first sorted row,
 *                                rows (1..block_rows), block index inside the
 *                                expert}, expert by expert; only the first
 *                                *num_blocks entries are written.
 *      num_blocks int32 [1]      number of block-map entries (stays on the device).
 * workspace: device scratch of at least moe_route_workspace_bytes(...) bytes
 *            (may be NULL when that is 0).
 * Sizes: T >= 0, 1 <= k <= min(E, MOEQ4_MAX_TOPK), E <= MOEQ4_MAX_EXPERTS,
 *        block_rows in {0 (default), 16, 32, 64, 128, 160, 256}.
 * T = 0 writes zero counts and offsets and num_blocks = 0.
 * Output buffers must not overlap each other or the workspace. */
int moe_route(const float* logits, int T, int E, int k, int block_rows, int32_t* topk_ids,
              float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
              int32_t* blocks, int32_t* num_blocks, void* workspace, size_t ws_bytes, void* stream);

/* The first step of moe_route alone (section "Keep expert routing on the
 * GPU"): each token's k largest logits and the softmax over them.
 * In:  logits float32 [T, E].
 * Out: topk_ids int32 [T, k], topk_w float [T, k], exactly as moe_route writes
 *      them (same selection, same order, same weights).
 * Sizes: as moe_route.  T = 0 writes nothing.  Errors: MOEQ4_ERR_SHAPE,
 * MOEQ4_ERR_UNSUPPORTED (k > MOEQ4_MAX_TOPK), MOEQ4_ERR_NULL, MOEQ4_ERR_ALIGN,
 * MOEQ4_ERR_HIP. */
int moe_topk_softmax(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                     void* stream);

/* Tiled copy of a stack of group-wise affine 4-bit matrices, the layout the
 * grouped GEMM streams.  It holds the same bytes as the row-major format
 * (codes E*N*K/2 bytes, scales and biases E*N*K/64 values each), re-ordered so
 * that one wave's load of one MFMA weight fragment is 1 KB of contiguous memory
 * (section "Dequantize weights during matrix multiplication": the weights stay
 * packed until they are rebuilt inside the GEMM; this only re-orders them once,
 * at load time).  With NT = N/16 row tiles, G = K/64 groups and C = ceil(G/2)
 * chunks of 128 K values; chunk c is full when group 2c+1 exists:
 *   codes_t:  the bytes of (expert e, chunk c, row tile t) start at
 *             e*N*K/2 + c*NT*1024 + t*1024 (full chunk) or t*512 (the last
 *             chunk of an odd G), so all tiles of one expert and chunk are
 *             adjacent.  In a full chunk, bytes [16*l, 16*l+16) belong to lane
 *             l = 16*q + r (q in 0..3, r in 0..15): row n = 16*t + r, first the
 *             8 bytes of K indices 128c + 16q + [0,16), then the 8 bytes of
 *             128c + 64 + 16q + [0,16).  Each little-endian 32-bit word holds 8
 *             consecutive codes c0..c7 as the nibbles (bits 4p..4p+3, p = 0..7)
 *             c0, c2, c4, c6, c1, c3, c5, c7.  The last chunk of an odd G holds
 *             only the first 8 bytes per lane, at [8*l, 8*l+8).
 *   scales_t, biases_t: the value of row 16*t + r, group g (chunk c = g/2) is at
 *             element e*N*G + 32*c*NT + 32*t + 2*r + (g - 2c) in a full chunk and
 *             e*N*G + 32*c*NT + 16*t + r in the last chunk of an odd G.
 * In:  codes [E, N, K/2], scales [E, N, K/64], biases [E, N, K/64] (row-major).
 * Out: codes_t, scales_t, biases_t of the same sizes; must not overlap the inputs.
 * Sizes: E >= 1, N % 16 == 0, N >= 16, K % 64 == 0, K >= 64, E*N*K/2 < 2^31. */
int moe_prepack_q4(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int E,
                   int N, int K, uint8_t* codes_t, uint16_t* scales_t, uint16_t* biases_t,
                   void* stream);

/* Dequantization into memory: every weight of E tiled matrices rebuilt as
 * bf16(scale*code + bias) (same rounding as the grouped GEMM's rebuild) into a
 * row-major bf16 array.  This is the unfused path that section "Dequantize
 * weights during matrix multiplication" compares the in-GEMM rebuild against
 * (a separate pass that writes the expanded weights to memory); it exists for
 * that comparison and for inspection, not on the fused path.
 * In:  codes_t, scales_t, biases_t  [E, N, K] in the tiled layout of moe_prepack_q4.
 * Out: out  uint16 (bf16) [E, N, K], 16-byte aligned; E*N*K*2 bytes.
 * Sizes: as moe_prepack_q4.  Errors: MOEQ4_ERR_SHAPE, MOEQ4_ERR_NULL,
 * MOEQ4_ERR_ALIGN, MOEQ4_ERR_HIP. */
int moe_dequant_q4(const uint8_t* codes_t, const uint16_t* scales_t, const uint16_t* biases_t, int E,
                   int N, int K, uint16_t* out, void* stream);

/* Grouped GEMM over group-wise affine 4-bit expert weights (section
 * "Dequantize weights during matrix multiplication").
 *
 * For every block-map entry b < *num_blocks with expert e and sorted rows
 * [r0, r0 + rows):
 *   Y[p, n] = bf16( sum_kk X[perm[p] / k, kk] * weight_e(n, kk) ),  p in [r0, r0+rows)
 * with fp32 accumulation.  Weights are rebuilt on chip, tile by tile, as
 * bf16(scale*code + bias) and never written back to memory; the result agrees
 * with the definition within the fp32 rounding of the sums.
 *
 * In:  X        uint16 (bf16) [T, K]  token activations (rows gathered via perm).
 *      codes_t, scales_t, biases_t   the experts' weights [E, N, K] in the tiled
 *                            layout written by moe_prepack_q4.
 *      perm, blocks, num_blocks  as produced by moe_route for the same T, E, k,
 *                            block_rows.
 *      max_blocks            host bound from moe_max_blocks (sizes the grid;
 *                            entries past *num_blocks exit at once).
 * Out: Y        uint16 (bf16) [T*k, N]  in sorted order (row p belongs to
 *                            assignment perm[p]); rows not covered by a block
 *                            are not written.
 * Sizes: T >= 0, K % 64 == 0, K >= 64, N % 16 == 0, N >= 16, 1 <= k <= E,
 *        E <= MOEQ4_MAX_EXPERTS, block_rows in {0, 16, 32, 64, 128, 160, 256} and equal
 *        to the value given to moe_route, max_blocks >= moe_max_blocks(T, E,
 *        k, block_rows), T*K*2 and E*N*K/2 below 2^31.  Y must not overlap the
 *        inputs. */
int moe_grouped_gemm_q4(const uint16_t* X, int T, int K, int N, int E, int k,
                        const uint8_t* codes_t, const uint16_t* scales_t,
                        const uint16_t* biases_t, const int32_t* perm, const int32_t* blocks,
                        const int32_t* num_blocks, int max_blocks, int block_rows, uint16_t* Y,
                        void* stream);

/* Most assignments (T*k) whose rows moe_route_grouped_gemm_q4 ranks inside
 * its GEMM launch. */
#define MOEQ4_ROUTE_IN_LAUNCH_MAX 4096

/* Routing and the grouped GEMM of one prefill chunk in one call (section
 * "Keep expert routing on the GPU": selection, histogram, scan, scatter and
 * block map stay on the GPU next to the grouped GEMM; section "Dequantize
 * weights during matrix multiplication" for the GEMM).  Outputs are exactly
 * those of moe_route followed by moe_grouped_gemm_q4 with the same block_rows:
 * topk_ids, topk_w, counts, offsets, perm, inv_perm, blocks, num_blocks and Y,
 * bit for bit.
 *
 * With 64-row blocks (block_rows 64, or 0 when moe_default_block_rows picks
 * 64) and T*k <= MOEQ4_ROUTE_IN_LAUNCH_MAX it runs two kernels: the top-k, then one GEMM launch in
 * which each workgroup takes one expert and one 256-column tile, starts
 * streaming that expert's weights at once, ranks the expert's assignments
 * from the ids with wave ballots (the stable counting sort), writes the
 * expert's part of perm and inv_perm (from its first column tile) and
 * multiplies its rows 64 at a time; one more workgroup writes counts,
 * offsets and the block map.  Otherwise it runs moe_route's kernels and then
 * the grouped GEMM.
 *
 * In:  logits, X, codes_t, scales_t, biases_t as for moe_route and
 *      moe_grouped_gemm_q4; block_rows, max_blocks as there.
 * Out: the outputs of both calls.
 * workspace: at least moe_route_workspace_bytes(T, E, k, block_rows) bytes.
 * Sizes: those of both calls.  T = 0 writes what moe_route writes for T = 0.
 * Errors: as for the two calls.  Output buffers must not overlap each other,
 * the inputs or the workspace. */
int moe_route_grouped_gemm_q4(const float* logits, const uint16_t* X, int T, int K, int N, int E, int k,
                              const uint8_t* codes_t, const uint16_t* scales_t, const uint16_t* biases_t,
                              int block_rows, int32_t* topk_ids, float* topk_w, int32_t* counts,
                              int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* blocks,
                              int32_t* num_blocks, int max_blocks, uint16_t* Y, void* workspace,
                              size_t ws_bytes, void* stream);

/* Bytes of device scratch moe_expert_ffn_q4 needs (0 on invalid sizes):
 * 2*T*k*(I + H) bytes, plus 2*T*(I + H) with a shared expert, rounded up.
 * shared: 1 when a shared expert is given, else 0. */
size_t moe_expert_ffn_workspace_bytes(int T, int H, int I, int E, int k, int shared);

/* The MoE layer's expert FFNs over a batch of T tokens, after moe_route
 * (section "Reduce intermediate and state traffic": the two input projections
 * run with their gated activation, the output projection with the routing
 * score and the shared expert's result; section "Qwen creates three workload
 * shapes": one shared expert sees every token):
 *   for each assignment a = t*k + j routed to expert e (rows grouped by expert
 *   through perm / blocks, as for moe_grouped_gemm_q4):
 *     h_a = bf16( silu(G_e x_t) * (U_e x_t) ),  G_e / U_e = rows [0, I) / [I, 2I)
 *                                               of e's gate+up matrix [2I, H]
 *   and with a shared expert (no routing, weight 1) h_t likewise;
 *     out[t] = bf16( D_sh h_t + sum_j w_a * D_e h_a )
 * silu(z) = z / (1 + exp(-z)) in fp32 from the fp32 projections; every weight
 * is rebuilt exactly as bf16(scale * code + bias); fp32 accumulation.  Each
 * weighted routed term and the shared term are held once in the workspace as
 * fp16 of term * 2^-8 (11-bit significand, |term| up to ~1.6e7) before the
 * combine, which adds in a fixed order (shared term, then j ascending): the
 * result is the same run after run.
 *
 * In:  X        uint16 (bf16) [T, H]   token activations.
 *      gu_*     [E, 2I, H] gate+up weights, dn_* [E, H, I] down weights, both
 *               in the tiled layout of moe_prepack_q4.
 *      sh_*     the shared expert's [1, 2I, H] and [1, H, I] matrices (tiled):
 *               all six given or all six NULL.
 *      topk_w, perm, blocks, num_blocks   from moe_route(T, E, k, block_rows).
 *      max_blocks   >= moe_max_blocks(T, E, k, block_rows).
 *      workspace    moe_expert_ffn_workspace_bytes(...) bytes, 16-byte
 *               aligned; no initial contents needed.
 * Out: out      uint16 (bf16) [T, H]; must not overlap the inputs.
 * Sizes: as moe_grouped_gemm_q4 for both matrices; H and I multiples of 64;
 *        T*k*I*2, T*H*2 and the weight arrays below 2^31 bytes. */
int moe_expert_ffn_q4(const uint16_t* X, int T, int H, int I, int E, int k, const uint8_t* gu_codes_t,
                      const uint16_t* gu_scales_t, const uint16_t* gu_biases_t, const uint8_t* dn_codes_t,
                      const uint16_t* dn_scales_t, const uint16_t* dn_biases_t, const uint8_t* sh_gu_codes_t,
                      const uint16_t* sh_gu_scales_t, const uint16_t* sh_gu_biases_t,
                      const uint8_t* sh_dn_codes_t, const uint16_t* sh_dn_scales_t,
                      const uint16_t* sh_dn_biases_t, const float* topk_w, const int32_t* perm,
                      const int32_t* blocks, const int32_t* num_blocks, int max_blocks, int block_rows,
                      uint16_t* out, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of device scratch moe_prefill_ffn_chunked_q4 needs for T tokens in
 * chunks of chunk_tokens (0 on invalid sizes).  It is that of one chunk, not
 * of the whole prompt.  shared: 1 when a shared expert is given, else 0. */
size_t moe_prefill_ffn_chunked_workspace_bytes(int T, int chunk_tokens, int H, int I, int E, int k,
                                               int block_rows, int shared);

/* The routed expert FFN (+ shared expert) of a long prompt, run as a sequence
 * of bounded chunks (section "Bound temporary memory with prompt chunking": the
 * temporary matrices of one chunk at a time, reused for the next, so the
 * scratch no longer grows with the prompt while the weights stay resident;
 * the output is unchanged).  For each chunk of chunk_tokens tokens (the last
 * one shorter), in order on the stream: moe_route over its logits, then
 * moe_expert_ffn_q4 over its rows, into the chunk's rows of out.  Every token's
 * result is the one moe_route + moe_expert_ffn_q4 give for it (the per-token
 * arithmetic does not depend on the other tokens of the call; the kernels
 * chosen for a chunk size may sum in another fp32 order than those for T).
 *
 * In:  logits float [T, E]; X uint16 (bf16) [T, H]; weights as moe_expert_ffn_q4.
 *      chunk_tokens  tokens per chunk: a multiple of 4, at least 4 (a chunk
 *                    longer than T means one chunk).
 *      block_rows    0 (the default for a full chunk) or 16/32/64/128/160/256; the
 *                    same for every chunk.
 *      workspace     device scratch of moe_prefill_ffn_chunked_workspace_bytes(
 *                    T, chunk_tokens, H, I, E, k, block_rows, shared) bytes,
 *                    16-byte aligned; no initial contents needed.
 * Out: out uint16 (bf16) [T, H].
 *      topk_ids int32 [T, k], topk_w float [T, k]: the routing (each may be
 *                    NULL; then it lives in the workspace, one chunk at a time).
 * Sizes: as moe_expert_ffn_q4 for one chunk.
 * Errors: MOEQ4_ERR_NULL, MOEQ4_ERR_SHAPE (also chunk_tokens not a positive
 *         multiple of 4), MOEQ4_ERR_UNSUPPORTED, MOEQ4_ERR_ALIGN,
 *         MOEQ4_ERR_WORKSPACE, MOEQ4_ERR_HIP; every check runs before the first
 *         chunk is enqueued.  MOEQ4_ERR_HIP (a kernel launch the runtime
 *         refused) stops the sequence at that chunk: the chunks before it are
 *         already enqueued and write their rows of out. */
int moe_prefill_ffn_chunked_q4(const float* logits, const uint16_t* X, int T, int H, int I, int E, int k,
                               const uint8_t* gu_codes_t, const uint16_t* gu_scales_t,
                               const uint16_t* gu_biases_t, const uint8_t* dn_codes_t,
                               const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                               const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t,
                               const uint16_t* sh_gu_biases_t, const uint8_t* sh_dn_codes_t,
                               const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t,
                               int chunk_tokens, int block_rows, int32_t* topk_ids, float* topk_w,
                               uint16_t* out, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of device scratch moe_decode_ffn_q4 needs (0 on invalid sizes).
 * shared: 1 when a shared expert is given, else 0. */
size_t moe_decode_workspace_bytes(int E, int k, int H, int I, int shared);

/* One batch-1 decode step of the MoE layer: routing, the selected experts'
 * FFNs and the shared expert, fused into two kernels (sections "Decode:
 * minimize bytes moved per token", "Optimize the single-row weight path" and
 * "Reduce intermediate and state traffic": the step is bound by the bytes it
 * moves, a row-parallel GEMV reads the weights; the two input projections run with their
 * gated activation, the output projection with the routing scores and the
 * shared expert's result).
 *
 *   ids, w   = top-k of logits and softmax over the k selected (as moe_route)
 *   h_j      = bf16( silu(G_j x) * (U_j x) ),  G_j / U_j = rows [0, I) / [I, 2I)
 *              of expert ids[j]'s gate+up matrix [2I, H]
 *   out      = bf16( sum_j w_j * D_j h_j  +  D_sh h_sh )
 * where D_j is expert ids[j]'s down matrix [H, I] and the shared expert's terms
 * (weight 1, no routing) are present when its matrices are given.  silu(z) =
 * z / (1 + exp(-z)) in fp32 from the fp32 projections.  Every weight is
 * rebuilt exactly as bf16(scale * code + bias) before it is multiplied (fp32
 * accumulation).  The result is the same for the same inputs, run after run.
 *
 * In:  logits  float  [E]           the token's router logits (finite).
 *      x       uint16 (bf16) [H]    the token's activations.
 *      gu_codes_t, gu_scales_t, gu_biases_t   [E, 2I, H] gate+up weights in the
 *                                   tiled layout of moe_prepack_q4 (N = 2I, K = H).
 *      dn_codes_t, dn_scales_t, dn_biases_t   [E, H, I] down weights, tiled
 *                                   (N = H, K = I).
 *      sh_*    the shared expert's two matrices ([1, 2I, H] and [1, H, I],
 *              tiled), all six given or all six NULL.
 *      workspace  device scratch of moe_decode_workspace_bytes(E, k, H, I,
 *              shared) bytes, 16-byte aligned; no initial contents needed.
 * Out: out     uint16 (bf16) [H].
 *      topk_ids int32 [k], topk_w float [k]   the routing (each may be NULL).
 * Sizes: 1 <= k <= min(E, MOEQ4_MAX_TOPK), E <= MOEQ4_MAX_EXPERTS, H and I
 *        multiples of 64 and at least 128, H <= 8192, (k + shared) * I * 2 bytes
 *        <= 64 KiB, E*2I*H/2 below 2^31.  Returns MOEQ4_ERR_UNSUPPORTED when
 *        the sizes exceed the kernels' LDS budget. */
int moe_decode_ffn_q4(const float* logits, const uint16_t* x, int E, int k, int H, int I,
                      const uint8_t* gu_codes_t, const uint16_t* gu_scales_t,
                      const uint16_t* gu_biases_t, const uint8_t* dn_codes_t,
                      const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                      const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t,
                      const uint16_t* sh_gu_biases_t, const uint8_t* sh_dn_codes_t,
                      const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t,
                      int32_t* topk_ids, float* topk_w, uint16_t* out, void* workspace,
                      size_t ws_bytes, void* stream);

/* Size of the per-GPU static scratch array of moe_decode_ffn_q4_noalloc. */
#define MOEQ4_DECODE_SCRATCH_BYTES (256 * 1024)

/* moe_decode_ffn_q4 with no workspace argument and no allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments (less
 * workspace and ws_bytes), checks, kernels and results as moe_decode_ffn_q4.
 * Its scratch is a static device array of MOEQ4_DECODE_SCRATCH_BYTES bytes, one
 * per GPU, held by the library until the process ends; the first call on a
 * device looks its address up (hipGetSymbolAddress, with the calling thread's
 * current device, which must be the device `stream` belongs to).  The call
 * itself never calls hipMalloc or hipFree.  Every call on one GPU shares that
 * array: calls that may overlap in time on one GPU (other streams, other
 * threads) race and give undefined results; calls ordered on one stream are
 * safe.  The array needs no initial contents (each call writes every byte it
 * reads).  Sizes whose scratch (moe_decode_workspace_bytes) exceeds
 * MOEQ4_DECODE_SCRATCH_BYTES return MOEQ4_ERR_UNSUPPORTED (no shape the decode
 * kernels accept needs that much); a failed address lookup returns
 * MOEQ4_ERR_HIP. */
int moe_decode_ffn_q4_noalloc(const float* logits, const uint16_t* x, int E, int k, int H, int I,
                              const uint8_t* gu_codes_t, const uint16_t* gu_scales_t,
                              const uint16_t* gu_biases_t, const uint8_t* dn_codes_t,
                              const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                              const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t,
                              const uint16_t* sh_gu_biases_t, const uint8_t* sh_dn_codes_t,
                              const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t,
                              int32_t* topk_ids, float* topk_w, uint16_t* out, void* stream);

/* Bytes of device scratch moe_small_batch_ffn_q4 needs (0 on invalid or
 * unsupported sizes).  shared: 1 when a shared expert is given, else 0. */
size_t moe_small_batch_workspace_bytes(int T, int E, int k, int H, int I, int shared);

/* The MoE layer for a small group of tokens (1 <= T <= MOEQ4_SMALL_MAX_T), such
 * as the two to five rows of a speculative-decoding verification step
 * (section "Limits of further optimization": that shape suits neither the
 * matrix path nor the one-row path, and its rows often select different
 * experts).  Same result, token by token, as moe_decode_ffn_q4 and as
 * moe_route + moe_expert_ffn_q4 (up to fp32 summation order):
 *
 *   ids[t], w[t] = top-k of logits[t] and softmax over the k selected
 *   out[t]       = bf16( sum_j w[t][j] * D_{ids[t][j]} h[t][j]  +  D_sh h_sh[t] )
 *   h[t][j]      = bf16( silu(G x[t]) * (U x[t]) ) with expert ids[t][j]'s gate
 *                  and up rows (the shared expert's for h_sh)
 *
 * in two kernels, with every distinct selected expert's weights read once for
 * all the tokens that selected it (and the shared expert's once for all T).
 * The routing stays on the GPU: nothing is copied to the host.  The result is
 * the same for the same inputs, run after run.
 *
 * In:  logits  float  [T, E]        router logits (finite).
 *      x       uint16 (bf16) [T, H] activations.
 *      gu_*, dn_*, sh_*              as moe_decode_ffn_q4 (tiled layout of
 *                                   moe_prepack_q4; the six sh_* all given or
 *                                   all NULL).
 *      workspace  device scratch of moe_small_batch_workspace_bytes(T, E, k,
 *              H, I, shared) bytes, 16-byte aligned; no initial contents needed.
 * Out: out     uint16 (bf16) [T, H].
 *      topk_ids int32 [T, k], topk_w float [T, k]   the routing (each may be NULL).
 * Sizes: 1 <= T <= MOEQ4_SMALL_MAX_T, 1 <= k <= min(E, MOEQ4_MAX_TOPK),
 *        E <= MOEQ4_MAX_EXPERTS, H and I multiples of 64 and at least 128,
 *        T*H <= 16384, T*(k+1)*I <= 49152 (the activations and the gated
 *        outputs are staged in LDS), E*2I*H/2 below 2^31.  Larger sizes give
 *        MOEQ4_ERR_UNSUPPORTED (use moe_route + moe_expert_ffn_q4).
 * Errors: MOEQ4_ERR_NULL, MOEQ4_ERR_SHAPE, MOEQ4_ERR_UNSUPPORTED,
 *         MOEQ4_ERR_ALIGN, MOEQ4_ERR_WORKSPACE, MOEQ4_ERR_HIP; on error nothing
 *         is enqueued. */
int moe_small_batch_ffn_q4(const float* logits, const uint16_t* x, int T, int E, int k, int H, int I,
                           const uint8_t* gu_codes_t, const uint16_t* gu_scales_t,
                           const uint16_t* gu_biases_t, const uint8_t* dn_codes_t,
                           const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                           const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t,
                           const uint16_t* sh_gu_biases_t, const uint8_t* sh_dn_codes_t,
                           const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t,
                           int32_t* topk_ids, float* topk_w, uint16_t* out, void* workspace,
                           size_t ws_bytes, void* stream);

/* Paths of moe_layer_ffn_q4, chosen from the number of rows T. */
#define MOEQ4_PATH_DECODE 1     /* T = 1: moe_decode_ffn_q4 */
#define MOEQ4_PATH_FEW_ROWS 2   /* 2 <= T <= MOEQ4_SMALL_MAX_T: moe_small_batch_ffn_q4 */
#define MOEQ4_PATH_PREFILL 3    /* otherwise: moe_route + moe_expert_ffn_q4 */

/* Which path moe_layer_ffn_q4 takes for these sizes: MOEQ4_PATH_DECODE for
 * T = 1, MOEQ4_PATH_FEW_ROWS for 2 <= T <= MOEQ4_SMALL_MAX_T, else
 * MOEQ4_PATH_PREFILL; a shape beyond a smaller path's limits (see those calls)
 * takes the next one.  Negative error code when no path takes the sizes.
 * shared: 1 when a shared expert is given, else 0. */
int moe_layer_ffn_path(int T, int E, int k, int H, int I, int shared);

/* Bytes of device scratch moe_layer_ffn_q4 needs for these sizes (that of
 * the path it takes; 0 on invalid sizes). */
size_t moe_layer_ffn_workspace_bytes(int T, int H, int I, int E, int k, int block_rows, int shared);

/* The MoE layer from router logits to output for T tokens, with the kernels
 * chosen from the shape (section "Optimization strategy": the runtime selects
 * kernels by row count and shape; section "Apple silicon provides different
 * paths for different workloads": one row is a bandwidth-bound matrix-vector
 * product, many rows a matrix product that reuses each weight):
 *   T = 1          the batch-1 decode step (moe_decode_ffn_q4);
 *   2 <= T <= 8    the few-row step (moe_small_batch_ffn_q4);
 *   otherwise      moe_route + moe_expert_ffn_q4 over all T rows, the routing
 *                  tables held in the workspace.
 * Every path computes, per token t:
 *   ids[t], w[t] = top-k of logits[t] (descending, ties by ascending expert id)
 *                  and softmax over the k selected
 *   out[t] = bf16( sum_j w[t][j] * D_{ids[t][j]} h[t][j]  +  D_sh h_sh[t] )
 *   h[t][j] = bf16( silu(G x_t) * (U x_t) ) with expert ids[t][j]'s gate/up rows
 * (as moe_expert_ffn_q4; the paths differ only in fp32 summation order).
 * In:  logits float [T, E]; X uint16 (bf16) [T, H]; weights as moe_expert_ffn_q4
 *      (tiled layout of moe_prepack_q4; the six sh_* all given or all NULL).
 *      block_rows  0 (default) or 16/32/64/128/160/256: the block height of the
 *                  routed path (unused by the other two).
 *      workspace   moe_layer_ffn_workspace_bytes(...) bytes, 16-byte aligned;
 *                  no initial contents needed.
 * Out: out uint16 (bf16) [T, H]; topk_ids int32 [T, k] and topk_w float [T, k]
 *      (each may be NULL).
 * Errors: those of the call the path makes (every check runs before anything
 * is enqueued); T = 0 enqueues nothing. */
int moe_layer_ffn_q4(const float* logits, const uint16_t* X, int T, int H, int I, int E, int k,
                     const uint8_t* gu_codes_t, const uint16_t* gu_scales_t, const uint16_t* gu_biases_t,
                     const uint8_t* dn_codes_t, const uint16_t* dn_scales_t, const uint16_t* dn_biases_t,
                     const uint8_t* sh_gu_codes_t, const uint16_t* sh_gu_scales_t, const uint16_t* sh_gu_biases_t,
                     const uint8_t* sh_dn_codes_t, const uint16_t* sh_dn_scales_t, const uint16_t* sh_dn_biases_t,
                     int block_rows, int32_t* topk_ids, float* topk_w, uint16_t* out, void* workspace,
                     size_t ws_bytes, void* stream);

/* Measured MFMA ceiling (measurement only, not a step of the method): each of
 * `workgroups` workgroups of 4 waves issues iters x 8 independent
 * v_mfma_f32_32x32x16_bf16 per wave (32768 flops each), the instruction of the
 * tall-block grouped GEMM, so flops / kernel time is the matrix-core
 * throughput that kernel can reach on this GPU at its clock.
 *   out  float [workgroups * 256], device, 16-byte aligned (results, unused).
 * Errors: MOEQ4_ERR_NULL, MOEQ4_ERR_SHAPE (workgroups < 1 or > 2^20,
 * iters < 0), MOEQ4_ERR_ALIGN, MOEQ4_ERR_HIP. */
int moe_calibrate_mfma(int workgroups, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ4_H */
