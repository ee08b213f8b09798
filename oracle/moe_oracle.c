/*
 * moe_oracle.c -- plain, slow, obviously correct CPU oracle for the MoE
 * routing + group-wise affine 4-bit grouped GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; the product path never calls it.
 *
 * What it follows (Perplexity Engineering, "Optimizing on-device inference
 * for Apple Silicon", 2026):
 *   - section "Qwen creates three workload shapes": a router scores the
 *     experts and selects 8 of 256 per token; one shared expert processes
 *     every token.
 *   - section "Keep expert routing on the GPU": a histogram counts the
 *     assignments per expert, a prefix scan turns the counts into start
 *     offsets, a scatter places the rows into their expert groups, and a block
 *     map lists the fixed-size matrix blocks the grouped GEMM processes.
 *   - section "Dequantize weights during matrix multiplication": each weight
 *     is a 4-bit integer code; each group of 64 weights shares a bf16 scale and
 *     a bf16 bias; the weights are rebuilt in bf16 before the multiply;
 *     accumulation is 32-bit float; the output is bf16.
 *   - section "Reduce intermediate and state traffic": the two expert input
 *     projections with their gated activation, then the output projection with
 *     its routing score and the shared-expert result.
 *
 * Arithmetic: every floating-point sum here is taken in fp64 over bf16
 * operands, whose products are exact in fp64, so the results are the exact
 * values up to fp64 rounding.  The GEMM outputs are returned unrounded
 * (double); the caller compares them with the rounding-aware rule.
 *
 * Readings of points the pages leave open (each one is listed in the design doc):
 *   R1 top-k order: descending logit; equal logits -> lower expert id first;
 *      -0 and +0 compare equal.  Inputs must be finite.
 *   R2 routing weights: softmax over the k selected logits.
 *   R3 order inside an expert group: ascending assignment id a = t*k + j
 *      (a stable counting sort).
 *   R4 block map entry {expert, first sorted row, rows (<= BM), block index
 *      inside the expert}; blocks listed expert by expert.
 *   R5 nibble order: byte i of a row holds K index 2i in its low nibble and
 *      2i+1 in its high nibble; scales/biases are [.., N, K/64] arrays.
 *   R6 rebuilt weight = bf16(scale*code + bias), rounded to nearest even once
 *      from the exact value.
 *   R7 FFN: gate rows 0..I-1 and up rows I..2I-1 of one [2I, H] matrix;
 *      h = bf16(silu(g) * u) from the unrounded projections; the shared expert
 *      is added with weight 1; the combine sums j ascending.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 64
#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

/* ---------------------------------------------------------------- bf16 -- */

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a real (held exactly in a double) to the nearest bf16, ties to even.
 * bf16 keeps 8 significant bits; quantum = 2^(e-8) for x in [2^(e-1), 2^e),
 * never below the subnormal quantum 2^-133. */
uint16_t oracle_bf16_round(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double ax = fabs(x);
  if (ax == 0.0) return sign;
  int e;
  frexp(ax, &e);
  int qe = e - 8;
  if (qe < -133) qe = -133;
  double r = nearbyint(ldexp(ax, -qe)); /* default rounding mode: ties to even */
  double y = ldexp(r, qe);
  if (y >= ldexp(1.0, 128)) return sign | 0x7F80; /* overflow -> inf */
  float f = (float)y;                             /* exact: y has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* ------------------------------------------------------------ dequant -- */

/* One rebuilt weight (reading R6). */
double oracle_dequant_one(uint16_t scale, uint16_t bias, int code) {
  double v = bf16_value(scale) * (double)code + bf16_value(bias); /* exact in fp64 */
  return bf16_value(oracle_bf16_round(v));
}

/* Code of K index kk in a packed row (reading R5). */
static int code_at(const uint8_t* row, int kk) {
  uint8_t byte = row[kk >> 1];
  return (kk & 1) ? (byte >> 4) : (byte & 0x0F);
}

/* Rebuild a whole [N, K] matrix as doubles holding bf16 values. */
int oracle_dequant_q4(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases,
                      int N, int K, double* W) {
  if (!codes || !scales || !biases || !W || N < 0 || K <= 0 || K % GROUP) return ORC_EINVAL;
  for (int n = 0; n < N; ++n) {
    const uint8_t* row = codes + (size_t)n * (K / 2);
    for (int kk = 0; kk < K; ++kk) {
      size_t g = (size_t)n * (K / GROUP) + kk / GROUP;
      W[(size_t)n * K + kk] = oracle_dequant_one(scales[g], biases[g], code_at(row, kk));
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------- top-k ---- */

/* Reading R1 and R2.  ids [T, k], w [T, k] (fp64). */
int oracle_topk_softmax(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return ORC_EINVAL;
  if (T > 0 && (!logits || !ids || !w)) return ORC_EINVAL;
  int fail = 0;
#pragma omp parallel
  {
    char* taken = (char*)malloc((size_t)E);
    if (!taken) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
      if (!taken) continue;
      const float* l = logits + (size_t)t * E;
      memset(taken, 0, (size_t)E);
      for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
          if (taken[e]) continue;
          /* scanning e upward, a strictly greater logit is needed to replace:
           * equal logits keep the lower id; -0 == +0 under this compare */
          if (best < 0 || l[e] > l[best]) best = e;
        }
        taken[best] = 1;
        ids[(size_t)t * k + j] = best;
      }
      double m = (double)l[ids[(size_t)t * k]];
      double sum = 0.0;
      for (int j = 0; j < k; ++j) sum += exp((double)l[ids[(size_t)t * k + j]] - m);
      for (int j = 0; j < k; ++j)
        w[(size_t)t * k + j] = exp((double)l[ids[(size_t)t * k + j]] - m) / sum;
    }
    free(taken);
  }
  return fail ? ORC_ENOMEM : ORC_OK;
}

/* ----------------------------------------------------------- routing ---- */

/* Histogram, exclusive scan, stable counting sort and block map
 * (section "Keep expert routing on the GPU"; readings R3, R4).
 * counts [E], offsets [E+1], perm [A], inv_perm [A], blocks [*,4] with room
 * for every block, num_blocks scalar. */
int oracle_route(const int32_t* ids, int T, int E, int k, int block_rows, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* blocks,
                 int32_t* num_blocks) {
  if (T < 0 || E <= 0 || k <= 0 || k > E || block_rows <= 0) return ORC_EINVAL;
  if (!counts || !offsets || !num_blocks) return ORC_EINVAL;
  long A = (long)T * k;
  if (A > 0 && (!ids || !perm || !inv_perm || !blocks)) return ORC_EINVAL;
  for (long a = 0; a < A; ++a)
    if (ids[a] < 0 || ids[a] >= E) return ORC_EINVAL;

  /* histogram */
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (long a = 0; a < A; ++a) counts[ids[a]] += 1;
  /* exclusive prefix scan */
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  /* scatter: visiting a in ascending order makes the sort stable */
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!cursor) return ORC_ENOMEM;
  for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (long a = 0; a < A; ++a) {
    int32_t p = cursor[ids[a]]++;
    perm[p] = (int32_t)a;
    inv_perm[a] = p;
  }
  free(cursor);
  /* block map */
  int32_t nb = 0;
  for (int e = 0; e < E; ++e) {
    for (int i = 0; (long)i * block_rows < counts[e]; ++i) {
      int32_t rows = counts[e] - i * block_rows;
      if (rows > block_rows) rows = block_rows;
      blocks[4 * (size_t)nb + 0] = e;
      blocks[4 * (size_t)nb + 1] = offsets[e] + i * block_rows;
      blocks[4 * (size_t)nb + 2] = rows;
      blocks[4 * (size_t)nb + 3] = i;
      ++nb;
    }
  }
  *num_blocks = nb;
  return ORC_OK;
}

/* ------------------------------------------------------ grouped GEMM ---- */

/* Y[p, n] = sum_kk X[perm[p] / k, kk] * Wdq[e, n, kk] for p in expert e's
 * group [offsets[e], offsets[e+1]); Y is [A, N] fp64 in sorted order.
 * Each touched expert's matrix is rebuilt once, then multiplied
 * ("dequantize, then matmul"). */
int oracle_grouped_gemm_q4(const uint16_t* X, int T, int K, int N, int E, int k,
                           const uint8_t* Wq, const uint16_t* S, const uint16_t* B,
                           const int32_t* perm, const int32_t* offsets, double* Y) {
  if (T < 0 || K <= 0 || K % GROUP || N <= 0 || E <= 0 || k <= 0) return ORC_EINVAL;
  if (!X || !Wq || !S || !B || !perm || !offsets || !Y) return ORC_EINVAL;
  int fail = 0;
#pragma omp parallel
  {
    double* W = (double*)malloc(sizeof(double) * (size_t)N * K);
    double* x = (double*)malloc(sizeof(double) * (size_t)K);
    if (!W || !x) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int e = 0; e < E; ++e) {
      if (!W || !x) continue;
      if (offsets[e + 1] == offsets[e]) continue;
      const size_t mat = (size_t)e * N;
      oracle_dequant_q4(Wq + mat * (K / 2), S + mat * (K / GROUP), B + mat * (K / GROUP), N, K, W);
      for (int32_t p = offsets[e]; p < offsets[e + 1]; ++p) {
        int t = perm[p] / k;
        for (int kk = 0; kk < K; ++kk) x[kk] = bf16_value(X[(size_t)t * K + kk]);
        for (int n = 0; n < N; ++n) {
          const double* wr = W + (size_t)n * K;
          double acc = 0.0;
          for (int kk = 0; kk < K; ++kk) acc += x[kk] * wr[kk];
          Y[(size_t)p * N + n] = acc;
        }
      }
    }
    free(W);
    free(x);
  }
  return fail ? ORC_ENOMEM : ORC_OK;
}

/* Sampled rows: Y[r, n] = sum_kk X[tokens[r], kk] * Wdq[experts[r], n, kk],
 * rebuilding each weight on the fly (for spot checks at full sizes). */
int oracle_expert_rows_q4(const uint16_t* X, int K, int N, const uint8_t* Wq, const uint16_t* S,
                          const uint16_t* B, const int32_t* tokens, const int32_t* experts,
                          int nrows, double* Y) {
  if (K <= 0 || K % GROUP || N <= 0 || nrows < 0) return ORC_EINVAL;
  if (nrows > 0 && (!X || !Wq || !S || !B || !tokens || !experts || !Y)) return ORC_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nrows; ++r) {
    const uint16_t* xr = X + (size_t)tokens[r] * K;
    for (int n = 0; n < N; ++n) {
      size_t row = (size_t)experts[r] * N + n;
      const uint8_t* cr = Wq + row * (K / 2);
      double acc = 0.0;
      for (int kk = 0; kk < K; ++kk) {
        size_t g = row * (K / GROUP) + kk / GROUP;
        acc += bf16_value(xr[kk]) * oracle_dequant_one(S[g], B[g], code_at(cr, kk));
      }
      Y[(size_t)r * N + n] = acc;
    }
  }
  return ORC_OK;
}

/* ---------------------------------------------------------- expert FFN -- */

/* out[i, :] for token tokens[i]:
 *   sum_j w[t, j] * FFN_{ids[t, j]}(x_t)  +  FFN_shared(x_t)   (reading R7)
 * FFN_e(x) = Wdn_e . bf16(silu(g) * u),  [g; u] = Wgu_e . x.
 * gu_*: [E, 2I, H];  dn_*: [E, H, I];  sh_*: [1, 2I, H] / [1, H, I] or NULL.
 * Weights are rebuilt on the fly for each (token, expert). */
static void ffn_one(const double* x, int H, int I, const uint8_t* guq, const uint16_t* gus,
                    const uint16_t* gub, const uint8_t* dnq, const uint16_t* dns,
                    const uint16_t* dnb, double scale, double* gu, double* h, double* out) {
  for (int n = 0; n < 2 * I; ++n) {
    const uint8_t* cr = guq + (size_t)n * (H / 2);
    double acc = 0.0;
    for (int kk = 0; kk < H; ++kk) {
      size_t g = (size_t)n * (H / GROUP) + kk / GROUP;
      acc += x[kk] * oracle_dequant_one(gus[g], gub[g], code_at(cr, kk));
    }
    gu[n] = acc;
  }
  for (int i = 0; i < I; ++i) {
    double gt = gu[i], up = gu[I + i];
    double silu = gt / (1.0 + exp(-gt));
    h[i] = bf16_value(oracle_bf16_round(silu * up));
  }
  for (int n = 0; n < H; ++n) {
    const uint8_t* cr = dnq + (size_t)n * (I / 2);
    double acc = 0.0;
    for (int kk = 0; kk < I; ++kk) {
      size_t g = (size_t)n * (I / GROUP) + kk / GROUP;
      acc += h[kk] * oracle_dequant_one(dns[g], dnb[g], code_at(cr, kk));
    }
    out[n] += scale * acc;
  }
}

int oracle_expert_ffn_q4(const uint16_t* X, int T, int H, int I, int E, int k,
                         const uint8_t* gu_q, const uint16_t* gu_s, const uint16_t* gu_b,
                         const uint8_t* dn_q, const uint16_t* dn_s, const uint16_t* dn_b,
                         const uint8_t* sh_gu_q, const uint16_t* sh_gu_s, const uint16_t* sh_gu_b,
                         const uint8_t* sh_dn_q, const uint16_t* sh_dn_s, const uint16_t* sh_dn_b,
                         const int32_t* ids, const double* w, const int32_t* tokens, int ntok,
                         double* out) {
  if (T < 0 || H <= 0 || H % GROUP || I <= 0 || I % GROUP || E <= 0 || k <= 0 || ntok < 0)
    return ORC_EINVAL;
  if (ntok > 0 && (!X || !gu_q || !gu_s || !gu_b || !dn_q || !dn_s || !dn_b || !ids || !w ||
                   !tokens || !out))
    return ORC_EINVAL;
  int has_shared = sh_gu_q && sh_gu_s && sh_gu_b && sh_dn_q && sh_dn_s && sh_dn_b;
  int fail = 0;
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)H);
    double* gu = (double*)malloc(sizeof(double) * 2 * (size_t)I);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    if (!x || !gu || !h) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int r = 0; r < ntok; ++r) {
      if (!x || !gu || !h) continue;
      int t = tokens[r];
      double* o = out + (size_t)r * H;
      for (int n = 0; n < H; ++n) o[n] = 0.0;
      for (int kk = 0; kk < H; ++kk) x[kk] = bf16_value(X[(size_t)t * H + kk]);
      for (int j = 0; j < k; ++j) {
        size_t e = (size_t)ids[(size_t)t * k + j];
        size_t gm = e * 2 * I, dm = e * H;
        ffn_one(x, H, I, gu_q + gm * (H / 2), gu_s + gm * (H / GROUP), gu_b + gm * (H / GROUP),
                dn_q + dm * (I / 2), dn_s + dm * (I / GROUP), dn_b + dm * (I / GROUP),
                w[(size_t)t * k + j], gu, h, o);
      }
      if (has_shared)
        ffn_one(x, H, I, sh_gu_q, sh_gu_s, sh_gu_b, sh_dn_q, sh_dn_s, sh_dn_b, 1.0, gu, h, o);
    }
    free(x);
    free(gu);
    free(h);
  }
  return fail ? ORC_ENOMEM : ORC_OK;
}

/* The same layer output, computed expert by expert ("dequantize, then
 * matmul"): each expert's two matrices are rebuilt once (reading R6), then
 * applied to every assignment routed to it, and the combine runs per token
 * afterwards.  Every dot product and the combine take their terms in the same
 * order as oracle_expert_ffn_q4 (kk ascending; routed terms j ascending, then
 * the shared term), so the two functions agree bit for bit; this one rebuilds
 * each weight once instead of once per (token, expert) and so finishes the
 * full-size workloads in seconds.  out [T, H] fp64. */
static void rebuild_matrix(const uint8_t* q, const uint16_t* s, const uint16_t* b, int N, int K, double* W) {
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    const uint8_t* cr = q + (size_t)n * (K / 2);
    for (int kk = 0; kk < K; ++kk) {
      size_t g = (size_t)n * (K / GROUP) + kk / GROUP;
      W[(size_t)n * K + kk] = oracle_dequant_one(s[g], b[g], code_at(cr, kk));
    }
  }
}

/* FFN of one row x through rebuilt matrices Wgu [2I, H] and Wdn [H, I]:
 * d = Wdn . bf16(silu(g) * u), [g; u] = Wgu . x (reading R7). */
static void ffn_rebuilt(const double* x, int H, int I, const double* Wgu, const double* Wdn, double* gu,
                        double* h, double* d) {
  for (int n = 0; n < 2 * I; ++n) {
    const double* wr = Wgu + (size_t)n * H;
    double acc = 0.0;
    for (int kk = 0; kk < H; ++kk) acc += x[kk] * wr[kk];
    gu[n] = acc;
  }
  for (int i = 0; i < I; ++i) {
    double gt = gu[i], up = gu[I + i];
    double silu = gt / (1.0 + exp(-gt));
    h[i] = bf16_value(oracle_bf16_round(silu * up));
  }
  for (int n = 0; n < H; ++n) {
    const double* wr = Wdn + (size_t)n * I;
    double acc = 0.0;
    for (int kk = 0; kk < I; ++kk) acc += h[kk] * wr[kk];
    d[n] = acc;
  }
}

/* rows[r] of X through one expert's rebuilt matrices into D[dst[r]] */
static int ffn_rows(const uint16_t* X, int H, int I, const double* Wgu, const double* Wdn, const int32_t* rows,
                    const int32_t* dst, int nrows, double* D) {
  int fail = 0;
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)H);
    double* gu = (double*)malloc(sizeof(double) * 2 * (size_t)I);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    if (!x || !gu || !h) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int r = 0; r < nrows; ++r) {
      if (!x || !gu || !h) continue;
      for (int kk = 0; kk < H; ++kk) x[kk] = bf16_value(X[(size_t)rows[r] * H + kk]);
      ffn_rebuilt(x, H, I, Wgu, Wdn, gu, h, D + (size_t)dst[r] * H);
    }
    free(x);
    free(gu);
    free(h);
  }
  return fail;
}

int oracle_expert_ffn_grouped_q4(const uint16_t* X, int T, int H, int I, int E, int k,
                                 const uint8_t* gu_q, const uint16_t* gu_s, const uint16_t* gu_b,
                                 const uint8_t* dn_q, const uint16_t* dn_s, const uint16_t* dn_b,
                                 const uint8_t* sh_gu_q, const uint16_t* sh_gu_s, const uint16_t* sh_gu_b,
                                 const uint8_t* sh_dn_q, const uint16_t* sh_dn_s, const uint16_t* sh_dn_b,
                                 const int32_t* ids, const double* w, double* out) {
  if (T < 0 || H <= 0 || H % GROUP || I <= 0 || I % GROUP || E <= 0 || k <= 0) return ORC_EINVAL;
  if (T > 0 && (!X || !gu_q || !gu_s || !gu_b || !dn_q || !dn_s || !dn_b || !ids || !w || !out))
    return ORC_EINVAL;
  const long A = (long)T * k;
  for (long a = 0; a < A; ++a)
    if (ids[a] < 0 || ids[a] >= E) return ORC_EINVAL;
  int has_shared = sh_gu_q && sh_gu_s && sh_gu_b && sh_dn_q && sh_dn_s && sh_dn_b;
  double* Wgu = (double*)malloc(sizeof(double) * 2 * (size_t)I * H);
  double* Wdn = (double*)malloc(sizeof(double) * (size_t)H * I);
  double* D = (double*)malloc(sizeof(double) * (size_t)(A > 0 ? A : 1) * H);          /* routed terms */
  double* Dsh = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * H);        /* shared term */
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A > T ? A : (T > 0 ? T : 1)));
  int32_t* dst = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A > T ? A : (T > 0 ? T : 1)));
  int fail = !Wgu || !Wdn || !D || !Dsh || !rows || !dst;
  for (int e = 0; e < E && !fail && A > 0; ++e) {
    int n = 0;
    for (long a = 0; a < A; ++a)
      if (ids[a] == e) {
        rows[n] = (int32_t)(a / k);
        dst[n] = (int32_t)a;
        ++n;
      }
    if (n == 0) continue;
    const size_t gm = (size_t)e * 2 * I, dm = (size_t)e * H;
    rebuild_matrix(gu_q + gm * (H / 2), gu_s + gm * (H / GROUP), gu_b + gm * (H / GROUP), 2 * I, H, Wgu);
    rebuild_matrix(dn_q + dm * (I / 2), dn_s + dm * (I / GROUP), dn_b + dm * (I / GROUP), H, I, Wdn);
    fail |= ffn_rows(X, H, I, Wgu, Wdn, rows, dst, n, D);
  }
  if (!fail && has_shared && T > 0) {
    for (int t = 0; t < T; ++t) rows[t] = dst[t] = t;
    rebuild_matrix(sh_gu_q, sh_gu_s, sh_gu_b, 2 * I, H, Wgu);
    rebuild_matrix(sh_dn_q, sh_dn_s, sh_dn_b, H, I, Wdn);
    fail |= ffn_rows(X, H, I, Wgu, Wdn, rows, dst, T, Dsh);
  }
  if (!fail) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
      double* o = out + (size_t)t * H;
      for (int n = 0; n < H; ++n) o[n] = 0.0;
      for (int j = 0; j < k; ++j) {
        const double wj = w[(size_t)t * k + j];
        const double* d = D + ((size_t)t * k + j) * H;
        for (int n = 0; n < H; ++n) o[n] += wj * d[n];
      }
      if (has_shared) {
        const double* d = Dsh + (size_t)t * H;
        for (int n = 0; n < H; ++n) o[n] += 1.0 * d[n];
      }
    }
  }
  free(Wgu);
  free(Wdn);
  free(D);
  free(Dsh);
  free(rows);
  free(dst);
  return fail ? ORC_ENOMEM : ORC_OK;
}

int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}
