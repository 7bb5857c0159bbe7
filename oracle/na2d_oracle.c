/*
 * na2d_oracle.c -- fp64 CPU oracle for 2D Neighborhood Attention (forward).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU path is checked against.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links or calls it, and it shares no header, helper
 * or table with the GPU code.
 *
 * What it computes follows "Neighborhood Attention Transformer" (the CVPR 2023
 * paper as translated on the CSDN page "[CVPR2023] Neighborhood Attention
 * Transformer"), section 3.1, equations 2-4, restated in the qiita article
 * "NAT: スライディングウィンドウアテンションの革新", section "Neighborhood
 * Attention(NA)":
 *
 *   A_i   = [ Q_i . K_rho_j(i) + B(i, rho_j(i)) ]_j          (Eq. 2)
 *   V_i   = [ V_rho_j(i) ]_j                                  (Eq. 3)
 *   NA(i) = softmax( A_i / sqrt(d) ) V_i                      (Eq. 4)
 *
 * repeated for every pixel (same section, text after Eq. 4).
 *
 * Readings taken where the pages leave a step open (each also listed in the
 * design notes of the repository):
 *  - In 2D the neighbourhood of kernel size k is a k x k window (CSDN page,
 *    section 3.4 and Fig. 4: "kernel size 7^2"), so a query has k*k keys.
 *  - The neighbourhood is the per-axis k-nearest set: along an axis of length
 *    L the window starts at clamp(i - k/2, 0, L - k), so a border pixel keeps
 *    the full span and its window is pushed inward (CSDN page, section 1
 *    "Introduction" and section 3.1; qiita ASCII figure of NA windows at the
 *    border; paperlayer summary, appendix C "repeated windows at edge pixels").
 *  - The bias is indexed by the relative offset of key to query,
 *    B[head][ky - y + k - 1][kx - x + k - 1], a (2k-1) x (2k-1) table per head,
 *    and it is divided by sqrt(d) together with Q.K, as Eq. 4 writes it.
 *  - rpb == NULL means "no positional bias" (the paperlayer summary,
 *    appendix B.1, ablates NA with and without it).
 *  - Layout: q, k, v, out are [B, heads, H, W, d] with d fastest.
 *
 * Every value is double; callers widen their (possibly 16-bit) inputs to
 * double exactly, so input quantisation is not part of any error measured
 * against this oracle.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

/* Start of the clamped window along one axis: the k indices of [0, L)
 * nearest to i.  Needs 1 <= k <= L. */
int na2d_oracle_window_start(int i, int k, int L)
{
    int s = i - k / 2;
    if (s < 0) s = 0;
    if (s > L - k) s = L - k;
    return s;
}

/* One output vector: query (b, h, y, x).  `logit` is scratch of k*k doubles.
 * When lse is not NULL it receives ln of the softmax denominator of Eq. 4,
 * ln sum_j exp((Q.K_j + B_j) / sqrt(d)), the per-query statistic a backward
 * pass can reuse. */
static void one_query(const double *q, const double *kk, const double *v,
                      const double *rpb, int heads, int H, int W, int d, int k,
                      int64_t b, int h, int y, int x, double *logit, double *o, double *lse)
{
    const int64_t map = ((int64_t)b * heads + h) * H * W;   /* first pixel of this (b, h) map */
    const double *qi = q + (map + (int64_t)y * W + x) * d;
    const int sy = na2d_oracle_window_start(y, k, H);
    const int sx = na2d_oracle_window_start(x, k, W);
    const int nb = 2 * k - 1;
    const double scale = 1.0 / sqrt((double)d);

    /* Eq. 2 and the division of Eq. 4: (Q.K + B) / sqrt(d) for every neighbour. */
    for (int a = 0; a < k; ++a) {
        for (int c = 0; c < k; ++c) {
            const int ky = sy + a, kx = sx + c;
            const double *kj = kk + (map + (int64_t)ky * W + kx) * d;
            double dot = 0.0;
            for (int t = 0; t < d; ++t) dot += qi[t] * kj[t];
            double bias = 0.0;
            if (rpb) bias = rpb[((int64_t)h * nb + (ky - y + k - 1)) * nb + (kx - x + k - 1)];
            logit[a * k + c] = (dot + bias) * scale;
        }
    }
    /* softmax over the k*k neighbours (max subtracted; same value exactly). */
    double m = -INFINITY;
    for (int j = 0; j < k * k; ++j) if (logit[j] > m) m = logit[j];
    double z = 0.0;
    for (int j = 0; j < k * k; ++j) { logit[j] = exp(logit[j] - m); z += logit[j]; }
    if (lse) *lse = m + log(z);
    /* Eq. 4: weights times the neighbour values (Eq. 3). */
    for (int t = 0; t < d; ++t) o[t] = 0.0;
    for (int a = 0; a < k; ++a) {
        for (int c = 0; c < k; ++c) {
            const double *vj = v + (map + (int64_t)(sy + a) * W + (sx + c)) * d;
            const double w = logit[a * k + c] / z;
            for (int t = 0; t < d; ++t) o[t] += w * vj[t];
        }
    }
}

static int bad_args(int B, int heads, int H, int W, int d, int k)
{
    if (B <= 0 || heads <= 0 || H <= 0 || W <= 0 || d <= 0) return 1;
    if (k < 1 || (k % 2) == 0 || k > H || k > W) return 1;
    return 0;
}

/* Whole forward pass; lse ([B, heads, H, W], may be NULL) receives each
 * query's log softmax denominator.  Returns 0, or -1 on invalid sizes.
 * nthreads <= 0 uses the OpenMP default. */
int na2d_oracle_f64_lse(const double *q, const double *k, const double *v,
                        const double *rpb, double *out, double *lse,
                        int B, int heads, int H, int W, int d, int ksize, int nthreads)
{
    if (bad_args(B, heads, H, W, d, ksize)) return -1;
    const int64_t rows = (int64_t)B * heads * H;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)ksize * ksize);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < rows; ++r) {
            const int y = (int)(r % H);
            const int h = (int)((r / H) % heads);
            const int64_t b = r / ((int64_t)H * heads);
            for (int x = 0; x < W; ++x)
                one_query(q, k, v, rpb, heads, H, W, d, ksize, b, h, y, x, logit,
                          out + (r * W + x) * d, lse ? lse + r * W + x : NULL);
        }
        free(logit);
    }
    return 0;
}

/* Whole forward pass.  Returns 0, or -1 on invalid sizes.  nthreads <= 0 uses
 * the OpenMP default. */
int na2d_oracle_f64(const double *q, const double *k, const double *v,
                    const double *rpb, double *out,
                    int B, int heads, int H, int W, int d, int ksize, int nthreads)
{
    return na2d_oracle_f64_lse(q, k, v, rpb, out, NULL, B, heads, H, W, d, ksize, nthreads);
}

/* The same definition for a list of queries given by their linear index
 * ((b * heads + h) * H + y) * W + x; out is [n, d].  Used to check large
 * launches on sampled outputs. */
int na2d_oracle_f64_sampled(const double *q, const double *k, const double *v,
                            const double *rpb, const int64_t *idx, int64_t n,
                            double *out, int B, int heads, int H, int W, int d,
                            int ksize, int nthreads)
{
    if (bad_args(B, heads, H, W, d, ksize)) return -1;
    const int64_t total = (int64_t)B * heads * H * W;
    for (int64_t i = 0; i < n; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)ksize * ksize);
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < n; ++i) {
            const int64_t p = idx[i];
            const int x = (int)(p % W);
            const int y = (int)((p / W) % H);
            const int h = (int)((p / ((int64_t)W * H)) % heads);
            const int64_t b = p / ((int64_t)W * H * heads);
            one_query(q, k, v, rpb, heads, H, W, d, ksize, b, h, y, x, logit, out + i * d, NULL);
        }
        free(logit);
    }
    return 0;
}
