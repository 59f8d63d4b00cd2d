/*
 * fp64 reference GEMM and convolution -- the oracle.
 *
 * TEST INFRASTRUCTURE ONLY: the product library never links, loads or calls
 * this file.  It is compiled on its own with gcc (no fast-math, no FP
 * contraction) and loaded by oracle/gemm_conv.py through ctypes.
 *
 * What it computes (plain definitions, no blocking, no reordering):
 *
 *  GEMM  C[b][i][j] = sum_{k=0}^{K-1} A[b][i][k] * B[b][k][j]
 *        ("Tiling（分块）" page: every C[i,j] takes K multiplies and K adds
 *        over a row of A and a column of B).  Loop order i, k, j with k
 *        ascending; S[b][i][j] = sum_k |A[b][i][k] * B[b][k][j]| is returned
 *        beside it for the error bound.
 *
 *  conv  y[n][co][oh][ow] = sum_{ci, r, s} x[n][ci][oh*sh - ph + r*dh]
 *                                           [ow*sw - pw + s*dw] * w[co][ci][r][s]
 *        with x outside the image equal to zero; NCHW input, OIHW weights.
 *
 *  H-tiled conv: the same output built one output-row tile at a time, each
 *        tile a sub-convolution over its input slice with the sub-operator
 *        pads pt' (top) and pb' (bottom) of the Tiling page's H/W tiling
 *        formulas.  The slice table comes from the caller.  The (ci, r, s)
 *        summation order equals the direct conv's, so the two agree bit for
 *        bit.
 *
 *  Tiled conv: tiles over images, output rows and output columns; rows and
 *        columns each take their slice and pads from the same formulas.
 *
 * Inputs are the exact fp16 / bf16 values the device receives, widened to
 * double by the caller.  All arrays are dense row-major.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

void oracle_gemm(int64_t batch, int64_t M, int64_t N, int64_t K,
                 const double *A, const double *B, double *C, double *S) {
  int64_t rows = batch * M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bi = 0; bi < rows; ++bi) {
    int64_t b = bi / M, i = bi % M;
    const double *a = A + (b * M + i) * K;
    const double *bm = B + b * K * N;
    double *c = C + (b * M + i) * N;
    double *s = S ? S + (b * M + i) * N : NULL;
    for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
    if (s)
      for (int64_t j = 0; j < N; ++j) s[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double aik = a[k];
      const double *brow = bm + k * N;
      for (int64_t j = 0; j < N; ++j) c[j] += aik * brow[j];
      if (s)
        for (int64_t j = 0; j < N; ++j) s[j] += fabs(aik * brow[j]);
    }
  }
}

/* Individual entries (b, i, j): the same dot product, k ascending. */
void oracle_gemm_entries(int64_t M, int64_t N, int64_t K, const double *A, const double *B,
                         int64_t n, const int64_t *bb, const int64_t *ii, const int64_t *jj,
                         double *C, double *S) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    const double *a = A + (bb[t] * M + ii[t]) * K;
    const double *bm = B + bb[t] * K * N + jj[t];
    double c = 0.0, s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double p = a[k] * bm[k * N];
      c += p;
      s += fabs(p);
    }
    C[t] = c;
    if (S) S[t] = s;
  }
}

static int64_t out_extent(int64_t size, int64_t k, int64_t stride, int64_t pad_lo, int64_t pad_hi,
                          int64_t d) {
  return (size + pad_lo + pad_hi - ((k - 1) * d + 1)) / stride + 1;
}

void oracle_conv2d(int64_t N, int64_t Ci, int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw,
                   int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                   const double *x, const double *w, double *y, double *S) {
  int64_t OH = out_extent(H, kh, sh, ph, ph, dh), OW = out_extent(W, kw, sw, pw, pw, dw);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t co = 0; co < Co; ++co)
      for (int64_t oh = 0; oh < OH; ++oh)
        for (int64_t ow = 0; ow < OW; ++ow) {
          double acc = 0.0, sa = 0.0;
          for (int64_t ci = 0; ci < Ci; ++ci)
            for (int64_t r = 0; r < kh; ++r)
              for (int64_t s = 0; s < kw; ++s) {
                int64_t ih = oh * sh - ph + r * dh, iw = ow * sw - pw + s * dw;
                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                double p = x[((n * Ci + ci) * H + ih) * W + iw] * w[((co * Ci + ci) * kh + r) * kw + s];
                acc += p;
                sa += fabs(p);
              }
          int64_t o = ((n * Co + co) * OH + oh) * OW + ow;
          y[o] = acc;
          if (S) S[o] = sa;
        }
}

/*
 * tiles: ntiles rows of (o0, o1, in_start, in_end, pt', pb').
 * Each tile materialises its zero-padded slice -- pt' zero rows, input rows
 * [in_start, min(in_end, H)), pb' zero rows; pw zero columns each side -- and
 * runs an unpadded strided conv over it, writing output rows [o0, o1).
 */
int oracle_conv2d_htiled(int64_t N, int64_t Ci, int64_t H, int64_t W, int64_t Co, int64_t kh,
                         int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                         int64_t dw, int64_t ntiles, const int64_t *tiles, const double *x,
                         const double *w, double *y) {
  int64_t OH = out_extent(H, kh, sh, ph, ph, dh), OW = out_extent(W, kw, sw, pw, pw, dw);
  int64_t WP = W + 2 * pw;
  (void)ph;
  for (int64_t t = 0; t < ntiles; ++t) {
    const int64_t *tt = tiles + 6 * t;
    int64_t o0 = tt[0], o1 = tt[1], in_start = tt[2], in_end = tt[3], ptp = tt[4], pbp = tt[5];
    int64_t rows_in = (in_end < H ? in_end : H) - in_start;
    int64_t HP = ptp + rows_in + pbp;
    int64_t sub_oh = out_extent(HP, kh, sh, 0, 0, dh);
    if (sub_oh != o1 - o0) return -1; /* the slice does not produce the tile's rows */
    double *xs = (double *)calloc((size_t)(N * Ci * HP * WP), sizeof(double));
    if (!xs) return -2;
    /* rows_in < 0: the tile's windows lie wholly in the padding (empty slice) */
    for (int64_t n = 0; n < N; ++n)
      for (int64_t ci = 0; ci < Ci; ++ci)
        for (int64_t r = 0; r < rows_in; ++r)
          memcpy(xs + ((n * Ci + ci) * HP + ptp + r) * WP + pw,
                 x + ((n * Ci + ci) * H + in_start + r) * W, (size_t)W * sizeof(double));
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t co = 0; co < Co; ++co)
        for (int64_t oh = 0; oh < sub_oh; ++oh)
          for (int64_t ow = 0; ow < OW; ++ow) {
            double acc = 0.0;
            for (int64_t ci = 0; ci < Ci; ++ci)
              for (int64_t r = 0; r < kh; ++r)
                for (int64_t s = 0; s < kw; ++s)
                  acc += xs[((n * Ci + ci) * HP + oh * sh + r * dh) * WP + ow * sw + s * dw] *
                         w[((co * Ci + ci) * kh + r) * kw + s];
            y[((n * Co + co) * OH + o0 + oh) * OW + ow] = acc;
          }
    free(xs);
  }
  return 0;
}

/*
 * Tiles over images, output rows and output columns.  tiles: ntiles rows of
 * (n0, n1, o0, o1, h_start, h_end, pt', pb', q0, q1, w_start, w_end, pl', pr'):
 * images [n0, n1), output rows [o0, o1) and columns [q0, q1).  The H/W tiling
 * formulas of the Tiling page hold for either dimension, so the columns get
 * their own slice [w_start, min(w_end, W)) and pads pl' (left), pr' (right),
 * as the rows do; images split without any halo.  Each tile materialises its
 * zero-padded slice and runs an unpadded strided conv over it, in the direct
 * conv's (ci, r, s) order, writing y[n0:n1, :, o0:o1, q0:q1].
 */
int oracle_conv2d_tiled(int64_t N, int64_t Ci, int64_t H, int64_t W, int64_t Co, int64_t kh,
                        int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                        int64_t dw, int64_t ntiles, const int64_t *tiles, const double *x,
                        const double *w, double *y) {
  int64_t OH = out_extent(H, kh, sh, ph, ph, dh), OW = out_extent(W, kw, sw, pw, pw, dw);
  for (int64_t t = 0; t < ntiles; ++t) {
    const int64_t *tt = tiles + 14 * t;
    int64_t n0 = tt[0], n1 = tt[1];
    int64_t o0 = tt[2], o1 = tt[3], h_start = tt[4], h_end = tt[5], ptp = tt[6], pbp = tt[7];
    int64_t q0 = tt[8], q1 = tt[9], w_start = tt[10], w_end = tt[11], plp = tt[12], prp = tt[13];
    if (n0 < 0 || n1 > N || n0 >= n1) return -3;
    int64_t rows_in = (h_end < H ? h_end : H) - h_start;
    int64_t cols_in = (w_end < W ? w_end : W) - w_start;
    int64_t HP = ptp + rows_in + pbp, WP = plp + cols_in + prp;
    int64_t sub_oh = out_extent(HP, kh, sh, 0, 0, dh), sub_ow = out_extent(WP, kw, sw, 0, 0, dw);
    if (sub_oh != o1 - o0 || sub_ow != q1 - q0) return -1; /* the slice does not produce the tile */
    int64_t nb = n1 - n0;
    double *xs = (double *)calloc((size_t)(nb * Ci * HP * WP), sizeof(double));
    if (!xs) return -2;
    /* A tile whose windows lie wholly in the padding has an empty slice: the
     * formulas give min(end, size) <= start there (a negative count, which the
     * pads' sum above still turns into the window span), and nothing is copied. */
    for (int64_t n = 0; n < nb && cols_in > 0; ++n)
      for (int64_t ci = 0; ci < Ci; ++ci)
        for (int64_t r = 0; r < rows_in; ++r)
          memcpy(xs + ((n * Ci + ci) * HP + ptp + r) * WP + plp,
                 x + (((n0 + n) * Ci + ci) * H + h_start + r) * W + w_start, (size_t)cols_in * sizeof(double));
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t n = 0; n < nb; ++n)
      for (int64_t co = 0; co < Co; ++co)
        for (int64_t oh = 0; oh < sub_oh; ++oh)
          for (int64_t ow = 0; ow < sub_ow; ++ow) {
            double acc = 0.0;
            for (int64_t ci = 0; ci < Ci; ++ci)
              for (int64_t r = 0; r < kh; ++r)
                for (int64_t s = 0; s < kw; ++s)
                  acc += xs[((n * Ci + ci) * HP + oh * sh + r * dh) * WP + ow * sw + s * dw] *
                         w[((co * Ci + ci) * kh + r) * kw + s];
            y[(((n0 + n) * Co + co) * OH + o0 + oh) * OW + q0 + ow] = acc;
          }
    free(xs);
  }
  return 0;
}

/* Threads the OpenMP loops above run on. */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
