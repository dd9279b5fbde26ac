/*
 * moe_oracle.c -- the ORACLE: a plain, slow CPU implementation of one GPU's
 * share of a grouped-GEMM Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library: it includes only the C standard library (and OpenMP for the
 * token-parallel outer loop).
 *
 * Arithmetic: every floating-point input arrives as the exact bit pattern the
 * GPU receives (bf16 / fp16 as uint16, logits as fp32).  Widening to double is
 * exact, every product and sum is done in double, in ascending index order,
 * and nothing is rounded to a narrow type except where stated (the routing
 * weights are returned as fp32; other outputs are returned as double).
 *
 * What is computed, and where it is defined:
 *   - the serial MoE layer dataflow  gate/up expert GEMM -> SiLU -> down GEMM
 *     is the one drawn in "Comm-compute fusion (1): why write communication
 *     into the GEMM kernel", section 1 (the problem);
 *   - "grouped" = rows bucketed by expert, each bucket multiplied by its own
 *     weights, with 128-row blocks as the expert alignment unit:
 *     "Comm-compute fusion (3): ThunderKittens multi-GPU programming and a
 *     fusable GEMM template", section 4 (gemm_config and the template);
 *   - the route-dependent reorder before the GEMM and the top-k weighted
 *     reduction after it: part (1), section 4 (the four-dataflow table, MoE
 *     layer0 / layer1 rows).
 * The pages leave routing, tie-breaks, row order and padding open; the
 * readings taken here (top-k on logits, ties to the lower expert id, softmax
 * over the k chosen logits, stable expert-major row order, zero-length
 * padding for empty experts) are listed with reasons in the design notes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ROW_BLOCK 128 /* expert alignment unit (part 3, section 4) */

/* ------------------------------------------------------------------ */
/* exact decoding of the 16-bit storage formats                          */
/* ------------------------------------------------------------------ */

/* bfloat16: the upper half of an IEEE binary32. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double fp16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1f;
  int fr = h & 0x3ff;
  double v;
  if (ex == 0)
    v = ldexp((double)fr, -24); /* subnormal: fr * 2^-14 / 2^10 */
  else if (ex == 31)
    v = fr ? NAN : INFINITY;
  else
    v = ldexp((double)(fr | 0x400), ex - 25); /* (1024+fr) * 2^(ex-15-10) */
  return sign ? -v : v;
}

static double decode16(uint16_t v, int is_fp16) {
  return is_fp16 ? fp16_to_double(v) : bf16_to_double(v);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* O0 router logits, the input of O1: the pages take the logits as given */
/* (part (1), section 4: the route that the reorder follows); the reading */
/* taken is the plain linear router, logits[t][e] = x[t] . W[e] with W   */
/* stored [E][H] (one row of hidden weights per expert, no bias).        */
/* ------------------------------------------------------------------ */
void oracle_router_logits(const uint16_t *x, const uint16_t *w, int T, int H, int E,
                          double *logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int h = 0; h < H; ++h)
        s += bf16_to_double(x[(size_t)t * H + h]) * bf16_to_double(w[(size_t)e * H + h]);
      logits[(size_t)t * E + e] = s;
    }
  }
}

/* ------------------------------------------------------------------ */
/* O1 route: top-k of each token's router logits, softmax over the k    */
/* selected logits.  Slot 0 holds the largest logit; equal logits go to  */
/* the lower expert id.                                                  */
/* ------------------------------------------------------------------ */
void oracle_route(const float *logits, int T, int E, int k, int32_t *idx,
                  float *w) {
  unsigned char *taken = (unsigned char *)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    const float *l = logits + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        /* strict '>' keeps the lower id on equal logits */
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      idx[(size_t)t * k + j] = best;
    }
    double m = (double)l[idx[(size_t)t * k]];
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += exp((double)l[idx[(size_t)t * k + j]] - m);
    for (int j = 0; j < k; ++j)
      w[(size_t)t * k + j] =
          (float)(exp((double)l[idx[(size_t)t * k + j]] - m) / z);
  }
  free(taken);
}

/* ------------------------------------------------------------------ */
/* O2 permute: bucket the T*k (token, slot) pairs by expert into         */
/* expert-contiguous runs, each run padded to a multiple of 128 rows.    */
/* Pair p = t*k + j.  Within an expert, rows follow ascending p.         */
/* Returns M_pad (= offsets[E]), or -1 if cap is smaller than M_pad.     */
/* ------------------------------------------------------------------ */
int oracle_permute(const int32_t *idx, int T, int k, int E, int cap,
                   int32_t *counts, int32_t *offsets, int32_t *pair_to_row,
                   int32_t *row_to_pair, int32_t *block_expert) {
  long R = (long)T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (long p = 0; p < R; ++p) counts[idx[p]] += 1;

  offsets[0] = 0;
  for (int e = 0; e < E; ++e) {
    int padded = ((counts[e] + ROW_BLOCK - 1) / ROW_BLOCK) * ROW_BLOCK;
    offsets[e + 1] = offsets[e] + padded;
  }
  int m_pad = offsets[E];
  if (m_pad > cap) return -1;

  for (int r = 0; r < cap; ++r) row_to_pair[r] = -1;
  int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  for (long p = 0; p < R; ++p) {
    int e = idx[p];
    int row = offsets[e] + fill[e];
    fill[e] += 1;
    pair_to_row[p] = row;
    row_to_pair[row] = (int32_t)p;
  }
  free(fill);

  int nblk = cap / ROW_BLOCK;
  for (int b = 0; b < nblk; ++b) block_expert[b] = -1;
  for (int e = 0; e < E; ++e)
    for (int r = offsets[e]; r < offsets[e + 1]; r += ROW_BLOCK)
      block_expert[r / ROW_BLOCK] = e;
  return m_pad;
}

/* x_perm[row] = x[token of the row's pair], zero for padding rows. */
void oracle_gather(const uint16_t *x, int H, const int32_t *row_to_pair,
                   int k, int cap, uint16_t *x_perm) {
  for (int r = 0; r < cap; ++r) {
    int p = row_to_pair[r];
    if (p < 0)
      memset(x_perm + (size_t)r * H, 0, (size_t)H * sizeof(uint16_t));
    else
      memcpy(x_perm + (size_t)r * H, x + (size_t)(p / k) * H,
             (size_t)H * sizeof(uint16_t));
  }
}

/* ------------------------------------------------------------------ */
/* O3-O5 grouped GEMM: output row r uses group g = block_group[r/128]     */
/* and A row  a(r) = a_src_row ? a_src_row[r] / a_src_div : r            */
/* (a negative a_src_row entry marks a row with no source: its output is */
/* NaN here and unspecified on the GPU).                                 */
/*   b_layout 0: B[g] is [K][N] (N contiguous)                            */
/*   b_layout 1: B[g] is [N][K] (K contiguous)                            */
/*   epi 0: D = A.B          epi 1: D = SiLU(A.B) * (A.B2)                */
/* Only the rows listed in `rows` (or all M rows when rows == NULL) are  */
/* computed; D has one row of N doubles per listed row.                  */
/* ------------------------------------------------------------------ */
static double b_at(const uint16_t *B, int layout, int is_fp16, int g, int K,
                   int N, int kk, int n) {
  size_t base = (size_t)g * K * N;
  size_t off = layout == 0 ? (size_t)kk * N + n : (size_t)n * K + kk;
  return decode16(B[base + off], is_fp16);
}

void oracle_grouped_gemm(int is_fp16, int M, int N, int K, const uint16_t *A,
                         const int32_t *a_src_row, int a_src_div,
                         const uint16_t *B, const uint16_t *B2, int b_layout,
                         const int32_t *block_group, int epi,
                         const int32_t *rows, int nrows, double *D) {
  int n_out = rows ? nrows : M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n_out; ++i) {
    int r = rows ? rows[i] : i;
    double *d = D + (size_t)i * N;
    int src = r;
    if (a_src_row) src = a_src_row[r] < 0 ? -1 : a_src_row[r] / a_src_div;
    int g = block_group[r / ROW_BLOCK];
    if (src < 0 || g < 0) {
      for (int n = 0; n < N; ++n) d[n] = NAN;
      continue;
    }
    const uint16_t *a = A + (size_t)src * K;
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int kk = 0; kk < K; ++kk)
        acc += decode16(a[kk], is_fp16) *
               b_at(B, b_layout, is_fp16, g, K, N, kk, n);
      if (epi == 1) {
        double up = 0.0;
        for (int kk = 0; kk < K; ++kk)
          up += decode16(a[kk], is_fp16) *
                b_at(B2, b_layout, is_fp16, g, K, N, kk, n);
        acc = silu(acc) * up;
      }
      d[n] = acc;
    }
  }
}

/* ------------------------------------------------------------------ */
/* O6 combine: out[t] = sum_j w[t][j] * y[pair_to_row[t*k+j]], slots in  */
/* ascending order, y given as bf16 rows.                               */
/* ------------------------------------------------------------------ */
void oracle_combine(const uint16_t *y, int H, const int32_t *pair_to_row,
                    const float *w, int T, int k, double *out) {
  for (int t = 0; t < T; ++t) {
    double *o = out + (size_t)t * H;
    for (int n = 0; n < H; ++n) o[n] = 0.0;
    for (int j = 0; j < k; ++j) {
      long p = (long)t * k + j;
      const uint16_t *yr = y + (size_t)pair_to_row[p] * H;
      double wj = (double)w[p];
      for (int n = 0; n < H; ++n) o[n] += wj * bf16_to_double(yr[n]);
    }
  }
}

/* ------------------------------------------------------------------ */
/* O6' weighted scatter (the combine folded into the down GEMM's         */
/* epilogue, part (1), section 4, MoE layer1 row): every real row r of   */
/* the row-ordered products Y [M][N] (double) adds w[p] * Y[r] into the  */
/* token row p / k of out [T][N], p = row_to_pair[r]; padding rows       */
/* (p < 0) add nothing.  Rows are visited in ascending order.            */
/* ------------------------------------------------------------------ */
void oracle_weighted_scatter(const double *Y, int M, int N,
                             const int32_t *row_to_pair, const float *w,
                             int k, int T, double *out) {
  for (size_t i = 0; i < (size_t)T * N; ++i) out[i] = 0.0;
  for (int r = 0; r < M; ++r) {
    int p = row_to_pair[r];
    if (p < 0) continue;
    double wp = (double)w[p];
    double *o = out + (size_t)(p / k) * N;
    const double *yr = Y + (size_t)r * N;
    for (int n = 0; n < N; ++n) o[n] += wp * yr[n];
  }
}

/* ------------------------------------------------------------------ */
/* The whole layer for a list of tokens, by its definition:              */
/*   out[t] = sum_j w[t][j] * FFN_{idx[t][j]}(x[t])                       */
/*   FFN_e(z) = (SiLU(z.Wg[e]) * (z.Wu[e])) . Wd[e]                      */
/* with Wg, Wu [E][H][I] and Wd [E][I][H] (bf16), x [T][H] (bf16).        */
/* No permutation, no padding, no blocking: one token at a time.         */
/* out has one row of H doubles per listed token.                        */
/* ------------------------------------------------------------------ */
void oracle_moe_tokens(const uint16_t *x, const int32_t *idx, const float *w,
                       const uint16_t *Wg, const uint16_t *Wu,
                       const uint16_t *Wd, int H, int E, int k, int I,
                       const int32_t *tokens, int ntok, double *out) {
  (void)E;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < ntok; ++i) {
    int t = tokens[i];
    double *o = out + (size_t)i * H;
    double *g = (double *)malloc((size_t)I * sizeof(double));
    double *u = (double *)malloc((size_t)I * sizeof(double));
    double *y = (double *)malloc((size_t)H * sizeof(double));
    for (int n = 0; n < H; ++n) o[n] = 0.0;
    const uint16_t *xt = x + (size_t)t * H;
    for (int j = 0; j < k; ++j) {
      int e = idx[(size_t)t * k + j];
      double wj = (double)w[(size_t)t * k + j];
      const uint16_t *wg = Wg + (size_t)e * H * I;
      const uint16_t *wu = Wu + (size_t)e * H * I;
      const uint16_t *wd = Wd + (size_t)e * I * H;
      for (int c = 0; c < I; ++c) g[c] = u[c] = 0.0;
      for (int h = 0; h < H; ++h) {
        double xv = bf16_to_double(xt[h]);
        for (int c = 0; c < I; ++c) {
          g[c] += xv * bf16_to_double(wg[(size_t)h * I + c]);
          u[c] += xv * bf16_to_double(wu[(size_t)h * I + c]);
        }
      }
      for (int n = 0; n < H; ++n) y[n] = 0.0;
      for (int c = 0; c < I; ++c) {
        double a = silu(g[c]) * u[c];
        for (int n = 0; n < H; ++n) y[n] += a * bf16_to_double(wd[(size_t)c * H + n]);
      }
      for (int n = 0; n < H; ++n) o[n] += wj * y[n];
    }
    free(g);
    free(u);
    free(y);
  }
}
