/*
 * CPU oracle for the VC-Attention hot path: the C half (k-means grouping and an
 * element-wise fused multiply-add).  TEST INFRASTRUCTURE ONLY: the product path
 * never links or calls this file; only the tests, the smoke check and the
 * bench's CPU-baseline leg do.  It shares no code with the HIP kernels.
 *
 * Built with -ffp-contract=off so that no multiply-add is fused unless the
 * code says fmaf() explicitly.
 *
 * Source of the method: "VC-Attention: Value Smoothing and Softmax Casting for
 * Low-bit Attention" (paper digest page, V-Smooth paragraph) and the news page
 * "Nunchux open-sources VC-Attention" (section "V-Smooth", item "Group"): per
 * batch and per head, Value tokens are clustered with k-means at inference time,
 * then Key and Value are reordered by cluster label.
 *
 * The pages do not fix the arithmetic of the k-means; the reading used here is
 * one that a GPU can reproduce bit for bit:
 *   - init: centroid c = V[floor(c * N / k)]  (no random draw)
 *   - assign: dot = fmaf chain over channels 0..d-1 starting from 0,
 *             cc  = the same chain for c.c,  score = fmaf(-2, dot, cc),
 *             label = argmin score, lowest centroid index on ties
 *   - update: per-cluster sums of llrint(v * 2^24) in int64 (order-free),
 *             centroid = (float)(((double)sum * 2^-24) / (double)count),
 *             an empty cluster keeps its previous centroid
 *   - iterations: assign then update, repeated `iters` times; the labels are
 *     those of the last assign, the centroids those after the last update.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* out[i] = fmaf(a[i], b[i], c[i]): one rounding of the exact a*b+c (C99 fmaf). */
void vco_fmaf(const float* a, const float* b, const float* c, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = fmaf(a[i], b[i], c[i]);
}

/* cc[c] = sum over channels of C[c][i]^2 as a fmaf chain in channel order. */
static void centroid_norms(const float* C, int k, int d, float* cc) {
  for (int c = 0; c < k; ++c) {
    float acc = 0.0f;
    for (int i = 0; i < d; ++i) acc = fmaf(C[(int64_t)c * d + i], C[(int64_t)c * d + i], acc);
    cc[c] = acc;
  }
}

/* Assign every token to its nearest centroid.  The loop over centroids is the
   inner one so that the k independent chains advance together; each chain still
   runs over channels 0..d-1 in order, so every score is the fixed-order value. */
static void assign(const float* V, int64_t N, int d, int k, const float* C, const float* cc,
                   int32_t* labels) {
  float* Ct = (float*)malloc(sizeof(float) * (size_t)k * d); /* Ct[i][c] = C[c][i] */
  for (int c = 0; c < k; ++c)
    for (int i = 0; i < d; ++i) Ct[(int64_t)i * k + c] = C[(int64_t)c * d + i];
#pragma omp parallel
  {
    float* dot = (float*)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(static)
    for (int64_t j = 0; j < N; ++j) {
      const float* x = V + j * d;
      for (int c = 0; c < k; ++c) dot[c] = 0.0f;
      for (int i = 0; i < d; ++i) {
        const float xi = x[i];
        const float* row = Ct + (int64_t)i * k;
        for (int c = 0; c < k; ++c) dot[c] = fmaf(xi, row[c], dot[c]);
      }
      int best = 0;
      float best_s = fmaf(-2.0f, dot[0], cc[0]);
      for (int c = 1; c < k; ++c) {
        const float s = fmaf(-2.0f, dot[c], cc[c]);
        if (s < best_s) { best_s = s; best = c; } /* strict: lowest index wins ties */
      }
      labels[j] = best;
    }
    free(dot);
  }
  free(Ct);
}

/* Centroid update from integer fixed-point sums (24 fractional bits). */
static void update(const float* V, int64_t N, int d, int k, const int32_t* labels, float* C,
                   int64_t* counts_out) {
  int64_t* sums = (int64_t*)calloc((size_t)k * d, sizeof(int64_t));
  int64_t* counts = (int64_t*)calloc((size_t)k, sizeof(int64_t));
  for (int64_t j = 0; j < N; ++j) {
    const int c = labels[j];
    counts[c] += 1;
    for (int i = 0; i < d; ++i) sums[(int64_t)c * d + i] += llrint((double)V[j * d + i] * 16777216.0);
  }
  for (int c = 0; c < k; ++c) {
    if (counts[c] == 0) continue; /* empty cluster: keep the old centroid */
    for (int i = 0; i < d; ++i)
      C[(int64_t)c * d + i] =
          (float)(((double)sums[(int64_t)c * d + i] * 0x1p-24) / (double)counts[c]);
  }
  if (counts_out) memcpy(counts_out, counts, sizeof(int64_t) * (size_t)k);
  free(sums);
  free(counts);
}

/* k-means on one (batch, head): V is fp32 [N][d] holding exact bf16 values.
   Writes labels[N] (last assign) and centroids[k][d] (after the last update). */
int vco_kmeans(const float* V, int64_t N, int d, int k, int iters, int32_t* labels,
               float* centroids, int64_t* counts) {
  if (N < 1 || d < 1 || k < 1 || iters < 1) return -1;
  for (int c = 0; c < k; ++c) {
    const int64_t src = ((int64_t)c * N) / k;
    memcpy(centroids + (int64_t)c * d, V + src * d, sizeof(float) * (size_t)d);
  }
  float* cc = (float*)malloc(sizeof(float) * (size_t)k);
  for (int it = 0; it < iters; ++it) {
    centroid_norms(centroids, k, d, cc);
    assign(V, N, d, k, centroids, cc, labels);
    update(V, N, d, k, labels, centroids, counts);
  }
  free(cc);
  return 0;
}

/* One assign step alone (for pinning the arithmetic on tiny inputs). */
void vco_assign(const float* V, int64_t N, int d, int k, const float* C, int32_t* labels) {
  float* cc = (float*)malloc(sizeof(float) * (size_t)k);
  centroid_norms(C, k, d, cc);
  assign(V, N, d, k, C, cc, labels);
  free(cc);
}
