/*
 * CPU oracle for fused scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file; it exists so that tests, the smoke check and the CPU leg of
 * the benchmark can compare the GPU library against a plain, slow and
 * obviously correct definition.  It shares no code with the GPU library.
 *
 * What it computes: softmax attention written out from its definition.  The
 * page "Não escreva kernels, derive-os" (section "Aprofundamento", first
 * paragraph) gets the fused attention kernel by treating the streaming softmax
 * state as a monoid; regrouping a monoid fold does not change its value, so
 * the fused kernel must equal this plain definition up to rounding:
 *
 *   s[i][j] = scale * sum_c Q[b,h,i,c] * K[b,kv(h),j,c]      (j visible to i)
 *   O[b,h,i,:] = sum_j softmax_j(s[i][:]) * V[b,kv(h),j,:]
 *   LSE[b,h,i] = log sum_j exp(s[i][j])                      (natural log)
 *
 * Readings taken where the pages are silent:
 *   - causal visibility is bottom-right aligned: j <= i + (Nk - Nq);
 *   - grouped-query heads: kv(h) = h / (Hq / Hkv);
 *   - a row with no visible key has O = 0 and LSE = -inf (gradients 0);
 *   - tensors are [B, H, N, d] contiguous with d fastest.
 *
 * Arithmetic is fp64 throughout on the exact input values (fp32 arrays; bf16
 * inputs are passed as their exact fp32 values).  The forward is the naive
 * three-pass form: max, then sum of exponentials, then the weighted sum of V.
 * The backward is the analytic gradient of O with respect to Q, K and V (the
 * same page, FAQ entry "O que o Tang propõe de diferente?", says its backward
 * kernel is obtained by rewriting; here the gradient is written out by hand):
 *
 *   P = exp(s - LSE);  dP = dO V^T;  D_i = sum_j P_ij dP_ij;
 *   dS = P (dP - D);   dQ = scale dS K;  dK = scale dS^T Q;  dV = P^T dO,
 *   with dK and dV summed over the query heads that share a kv head.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int visible(int64_t i, int64_t j, int64_t Nq, int64_t Nk, int causal) {
  if (j < 0 || j >= Nk) return 0;
  if (!causal) return 1;
  return j <= i + (Nk - Nq);
}

static double dot(const float* a, const float* b, int64_t d) {
  double s = 0.0;
  for (int64_t c = 0; c < d; c++) s += (double)a[c] * (double)b[c];
  return s;
}

/* One query row.  q_row: d values; kh, vh: the kv head's [Nk, d] blocks.
 * s_buf: Nk doubles of scratch.  Writes d values to o_row and one LSE. */
static void fwd_row(const float* q_row, const float* kh, const float* vh, int64_t i, int64_t Nq, int64_t Nk,
                    int64_t d, double scale, int causal, double* s_buf, double* o_row, double* lse) {
  int64_t j, c;
  int any = 0;
  double m = -INFINITY, l = 0.0;
  for (j = 0; j < Nk; j++)
    if (visible(i, j, Nq, Nk, causal)) s_buf[j] = scale * dot(q_row, kh + j * d, d);
  /* pass 1: row maximum */
  for (j = 0; j < Nk; j++)
    if (visible(i, j, Nq, Nk, causal)) {
      if (!any || s_buf[j] > m) m = s_buf[j];
      any = 1;
    }
  for (c = 0; c < d; c++) o_row[c] = 0.0;
  if (!any) {
    *lse = -INFINITY;
    return;
  }
  /* pass 2: sum of exponentials */
  for (j = 0; j < Nk; j++)
    if (visible(i, j, Nq, Nk, causal)) l += exp(s_buf[j] - m);
  /* pass 3: normalised weights times V */
  for (j = 0; j < Nk; j++)
    if (visible(i, j, Nq, Nk, causal)) {
      double p = exp(s_buf[j] - m) / l;
      for (c = 0; c < d; c++) o_row[c] += p * (double)vh[j * d + c];
    }
  *lse = m + log(l);
}

/* Full forward.  q: [B,Hq,Nq,d]; k, v: [B,Hkv,Nk,d]; o: [B,Hq,Nq,d]; lse: [B,Hq,Nq]. */
int oracle_fwd(const float* q, const float* k, const float* v, double* o, double* lse, int64_t B, int64_t Hq,
               int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, double scale, int causal) {
  int64_t rows = B * Hq * Nq, r;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || d <= 0 || Hq % Hkv) return 1;
  int64_t g = Hq / Hkv;
#pragma omp parallel
  {
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
#pragma omp for schedule(dynamic, 16)
    for (r = 0; r < rows; r++) {
      int64_t i = r % Nq, h = (r / Nq) % Hq, b = r / (Nq * Hq);
      int64_t kvh = h / g;
      const float* kh = k + (b * Hkv + kvh) * Nk * d;
      const float* vh = v + (b * Hkv + kvh) * Nk * d;
      fwd_row(q + r * d, kh, vh, i, Nq, Nk, d, scale, causal, s_buf, o + r * d, lse + r);
    }
    free(s_buf);
  }
  return 0;
}

/* Forward on a list of rows.  rows_bhi: n triples (b, h, i).  o_rows: [n, d]; lse_rows: [n]. */
int oracle_fwd_rows(const float* q, const float* k, const float* v, const int64_t* rows_bhi, int64_t n,
                    double* o_rows, double* lse_rows, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                    int64_t d, double scale, int causal) {
  int64_t t;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0) return 1;
  for (t = 0; t < n; t++) {
    int64_t b = rows_bhi[3 * t], h = rows_bhi[3 * t + 1], i = rows_bhi[3 * t + 2];
    if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Nq) return 2;
  }
  int64_t g = Hq / Hkv;
#pragma omp parallel
  {
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
#pragma omp for schedule(dynamic, 1)
    for (t = 0; t < n; t++) {
      int64_t b = rows_bhi[3 * t], h = rows_bhi[3 * t + 1], i = rows_bhi[3 * t + 2];
      int64_t kvh = h / g;
      const float* kh = k + (b * Hkv + kvh) * Nk * d;
      const float* vh = v + (b * Hkv + kvh) * Nk * d;
      fwd_row(q + ((b * Hq + h) * Nq + i) * d, kh, vh, i, Nq, Nk, d, scale, causal, s_buf, o_rows + t * d,
              lse_rows + t);
    }
    free(s_buf);
  }
  return 0;
}

/* Backward.  Inputs q, k, v, dout as in the forward; outputs dq [B,Hq,Nq,d],
 * dk, dv [B,Hkv,Nk,d] (fp64, fully overwritten).  The oracle recomputes its
 * own scores, LSE and P; it never takes O or LSE from anywhere else.  One
 * OpenMP task per (b, kv head) owns that head's dK, dV and its group's dQ. */
int oracle_bwd(const float* q, const float* k, const float* v, const float* dout, double* dq, double* dk,
               double* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, double scale,
               int causal) {
  int64_t units = B * Hkv, u;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || d <= 0 || Hq % Hkv) return 1;
  int64_t g = Hq / Hkv;
  memset(dq, 0, sizeof(double) * (size_t)(B * Hq * Nq * d));
  memset(dk, 0, sizeof(double) * (size_t)(B * Hkv * Nk * d));
  memset(dv, 0, sizeof(double) * (size_t)(B * Hkv * Nk * d));
#pragma omp parallel
  {
    size_t nk1 = (size_t)(Nk > 0 ? Nk : 1);
    double* s = (double*)malloc(sizeof(double) * nk1);
    double* p = (double*)malloc(sizeof(double) * nk1);
    double* dp = (double*)malloc(sizeof(double) * nk1);
#pragma omp for schedule(dynamic, 1)
    for (u = 0; u < units; u++) {
      int64_t b = u / Hkv, kvh = u % Hkv, hh, i, j, c;
      const float* kh = k + (b * Hkv + kvh) * Nk * d;
      const float* vh = v + (b * Hkv + kvh) * Nk * d;
      double* dkh = dk + (b * Hkv + kvh) * Nk * d;
      double* dvh = dv + (b * Hkv + kvh) * Nk * d;
      for (hh = 0; hh < g; hh++) {
        int64_t h = kvh * g + hh;
        for (i = 0; i < Nq; i++) {
          const float* qi = q + ((b * Hq + h) * Nq + i) * d;
          const float* doi = dout + ((b * Hq + h) * Nq + i) * d;
          double* dqi = dq + ((b * Hq + h) * Nq + i) * d;
          double m = -INFINITY, l = 0.0, lse, Di = 0.0;
          int any = 0;
          for (j = 0; j < Nk; j++)
            if (visible(i, j, Nq, Nk, causal)) {
              s[j] = scale * dot(qi, kh + j * d, d);
              if (!any || s[j] > m) m = s[j];
              any = 1;
            }
          if (!any) continue; /* no visible key: every gradient of this row is 0 */
          for (j = 0; j < Nk; j++)
            if (visible(i, j, Nq, Nk, causal)) l += exp(s[j] - m);
          lse = m + log(l);
          for (j = 0; j < Nk; j++)
            if (visible(i, j, Nq, Nk, causal)) {
              p[j] = exp(s[j] - lse);
              dp[j] = dot(doi, vh + j * d, d);
              Di += p[j] * dp[j];
            }
          for (j = 0; j < Nk; j++)
            if (visible(i, j, Nq, Nk, causal)) {
              double ds = p[j] * (dp[j] - Di);
              for (c = 0; c < d; c++) {
                dqi[c] += scale * ds * (double)kh[j * d + c];
                dkh[j * d + c] += scale * ds * (double)qi[c];
                dvh[j * d + c] += p[j] * (double)doi[c];
              }
            }
        }
      }
    }
    free(s);
    free(p);
    free(dp);
  }
  return 0;
}

/* Row statistics D_i = sum_j P_ij dP_ij computed from the definition (for
 * checking the identity D_i = dO_i . O_i).  out: [B,Hq,Nq]. */
int oracle_bwd_rowdot(const float* q, const float* k, const float* v, const float* dout, double* out, int64_t B,
                      int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, double scale, int causal) {
  int64_t rows = B * Hq * Nq, r;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || d <= 0 || Hq % Hkv) return 1;
  int64_t g = Hq / Hkv;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
#pragma omp for schedule(dynamic, 16)
    for (r = 0; r < rows; r++) {
      int64_t i = r % Nq, h = (r / Nq) % Hq, b = r / (Nq * Hq), j;
      const float* kh = k + (b * Hkv + h / g) * Nk * d;
      const float* vh = v + (b * Hkv + h / g) * Nk * d;
      double m = -INFINITY, l = 0.0, acc = 0.0;
      int any = 0;
      for (j = 0; j < Nk; j++)
        if (visible(i, j, Nq, Nk, causal)) {
          s[j] = scale * dot(q + r * d, kh + j * d, d);
          if (!any || s[j] > m) m = s[j];
          any = 1;
        }
      if (any) {
        for (j = 0; j < Nk; j++)
          if (visible(i, j, Nq, Nk, causal)) l += exp(s[j] - m);
        for (j = 0; j < Nk; j++)
          if (visible(i, j, Nq, Nk, causal)) acc += exp(s[j] - m) / l * dot(dout + r * d, vh + j * d, d);
      }
      out[r] = acc;
    }
    free(s);
  }
  return 0;
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
