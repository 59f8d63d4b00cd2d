/*
 * The fp64 oracle (oracle/gemm_conv.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer (host code only; built with gcc, without OpenMP,
 * by tests/test_host_sanitizers.py).  Small ragged GEMMs with a batch, sampled
 * entries, direct convolutions with stride, padding and dilation, and the
 * H-tiled convolution over one whole-height tile and over two tiles, whose
 * results must equal the direct convolution's bit for bit (the same sum
 * order).  Exit status 0, 3 on a mismatch; a sanitizer finding aborts with
 * its report.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_gemm(int64_t batch, int64_t M, int64_t N, int64_t K, const double *A, const double *B, double *C,
                 double *S);
void oracle_gemm_entries(int64_t M, int64_t N, int64_t K, const double *A, const double *B, int64_t n,
                         const int64_t *bb, const int64_t *ii, const int64_t *jj, double *C, double *S);
void oracle_conv2d(int64_t N, int64_t Ci, int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw, int64_t sh,
                   int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, const double *x, const double *w,
                   double *y, double *S);
int oracle_conv2d_htiled(int64_t N, int64_t Ci, int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw,
                         int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, int64_t ntiles,
                         const int64_t *tiles, const double *x, const double *w, double *y);

static double *fill(int64_t n, unsigned seed) {
  double *p = malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  unsigned s = seed;
  for (int64_t i = 0; i < n; ++i) {
    s = s * 1103515245u + 12345u;
    p[i] = (double)((int)((s >> 16) % 5) - 2);
  }
  return p;
}

static int64_t extent(int64_t size, int64_t k, int64_t stride, int64_t pad, int64_t d) {
  return (size + 2 * pad - ((k - 1) * d + 1)) / stride + 1;
}

/* One H-tile row (o0, o1, in_start, in_end, pt', pb') from the Tiling page's
   formulas: input rows [o0*sh - ph, (o1-1)*sh - ph + (kh-1)*d + 1) clipped
   at 0 on top (the clipped rows become pt'), pb' the rows past H. */
static void htile(int64_t H, int64_t kh, int64_t sh, int64_t ph, int64_t d, int64_t o0, int64_t o1, int64_t *t) {
  const int64_t start = o0 * sh - ph, end = (o1 - 1) * sh - ph + (kh - 1) * d + 1;
  t[0] = o0;
  t[1] = o1;
  t[2] = start > 0 ? start : 0;
  t[3] = end;
  t[4] = start < 0 ? -start : 0;
  t[5] = end > H ? end - H : 0;
}

int main(void) {
  int bad = 0;
  /* batched ragged GEMMs */
  const int64_t shapes[][4] = {{1, 1, 1, 1}, {2, 7, 9, 13}, {3, 17, 5, 33}, {1, 64, 64, 0}, {1, 0, 8, 8}};
  for (int t = 0; t < 5; ++t) {
    const int64_t b = shapes[t][0], M = shapes[t][1], N = shapes[t][2], K = shapes[t][3];
    double *A = fill(b * M * K, 1 + t), *B = fill(b * K * N, 7 + t);
    double *C = malloc((size_t)(b * M * N + 1) * sizeof(double)), *S = malloc((size_t)(b * M * N + 1) * sizeof(double));
    oracle_gemm(b, M, N, K, A, B, C, S);
    if (b * M * N > 0) {
      int64_t bb[3] = {0, b - 1, b / 2}, ii[3] = {0, M - 1, M / 2}, jj[3] = {0, N - 1, N / 3};
      double c[3], s[3];
      oracle_gemm_entries(M, N, K, A, B, 3, bb, ii, jj, c, s);
      for (int e = 0; e < 3; ++e) {
        const int64_t o = (bb[e] * M + ii[e]) * N + jj[e];
        if (c[e] != C[o] || s[e] != S[o]) bad = 1;
      }
    }
    free(A);
    free(B);
    free(C);
    free(S);
  }
  /* convolutions: direct, one whole tile and two tiles */
  const int64_t geo[][10] = {{2, 3, 9, 7, 4, 3, 3, 2, 1, 1}, {1, 2, 12, 12, 3, 5, 5, 2, 2, 1},
                             {2, 4, 10, 13, 5, 3, 1, 1, 3, 2}, {1, 1, 5, 5, 2, 5, 5, 1, 4, 1}};
  for (int t = 0; t < 4; ++t) {
    const int64_t N = geo[t][0], Ci = geo[t][1], H = geo[t][2], W = geo[t][3], Co = geo[t][4], kh = geo[t][5],
                  kw = geo[t][6], st = geo[t][7], pad = geo[t][8], dil = geo[t][9];
    const int64_t OH = extent(H, kh, st, pad, dil), OW = extent(W, kw, st, pad, dil);
    double *x = fill(N * Ci * H * W, 11 + t), *w = fill(Co * Ci * kh * kw, 13 + t);
    const int64_t ny = N * Co * OH * OW;
    double *y = malloc((size_t)ny * sizeof(double)), *y1 = malloc((size_t)ny * sizeof(double));
    double *y2 = malloc((size_t)ny * sizeof(double)), *S = malloc((size_t)ny * sizeof(double));
    oracle_conv2d(N, Ci, H, W, Co, kh, kw, st, st, pad, pad, dil, dil, x, w, y, S);
    int64_t one[6], two[12];
    htile(H, kh, st, pad, dil, 0, OH, one);
    htile(H, kh, st, pad, dil, 0, OH / 2 > 0 ? OH / 2 : 1, two);
    htile(H, kh, st, pad, dil, OH / 2 > 0 ? OH / 2 : 1, OH, two + 6);
    memset(y1, 0, (size_t)ny * sizeof(double));
    memset(y2, 0, (size_t)ny * sizeof(double));
    if (oracle_conv2d_htiled(N, Ci, H, W, Co, kh, kw, st, st, pad, pad, dil, dil, 1, one, x, w, y1) != 0) bad = 1;
    if (OH > 1 &&
        oracle_conv2d_htiled(N, Ci, H, W, Co, kh, kw, st, st, pad, pad, dil, dil, 2, two, x, w, y2) != 0)
      bad = 1;
    if (memcmp(y, y1, (size_t)ny * sizeof(double)) != 0) bad = 1;
    if (OH > 1 && memcmp(y, y2, (size_t)ny * sizeof(double)) != 0) bad = 1;
    free(x);
    free(w);
    free(y);
    free(y1);
    free(y2);
    free(S);
  }
  printf("oracle driver: %s\n", bad ? "MISMATCH" : "ok");
  return bad ? 3 : 0;
}
