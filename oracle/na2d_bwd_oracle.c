/*
 * na2d_bwd_oracle.c -- fp64 CPU oracle for the gradients of 2D Neighborhood
 * Attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Like the forward oracle this is the slow,
 * obviously correct definition the GPU path is checked against; only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark load it,
 * and it shares no code with the GPU library.
 *
 * Forward (CSDN translation of "Neighborhood Attention Transformer", section
 * 3.1, Eq. 2-4), for query i of a (b, h) map and the keys j of its clamped
 * k x k window N(i):
 *   s_ij = (q_i . k_j + B[h][j - i + k - 1]) / sqrt(d)
 *   p_ij = exp(s_ij) / sum_j' exp(s_ij')
 *   o_i  = sum_j p_ij v_j
 * The pages name the backward pass (NATTEN computes the gradients of QK+B and
 * AV, qiita article, section "NATTEN") without writing it out; it is the
 * chain rule applied to the three lines above.  For an upstream gradient
 * g_i = dL/do_i:
 *   dL/dv_j  = sum over queries i with j in N(i) of p_ij g_i
 *   dL/dp_ij = g_i . v_j
 *   dL/ds_ij = p_ij (dL/dp_ij - sum_j' p_ij' dL/dp_ij')       (softmax)
 *            = p_ij (g_i . v_j - g_i . o_i)
 *   dL/dq_i  = sum_j dL/ds_ij k_j / sqrt(d)
 *   dL/dk_j  = sum over queries i with j in N(i) of dL/ds_ij q_i / sqrt(d)
 *   dL/dB[h][off] = sum over all (b, i, j) with j - i = off of dL/ds_ij / sqrt(d)
 * Each query's terms are formed once and scattered to the keys of its window,
 * so the "queries whose window holds j" sets never need to be enumerated.
 * Layout as in the forward: [B][heads][H][W][d]; rpb and drpb
 * [heads][2k-1][2k-1]; rpb == NULL means no bias (drpb may then be NULL).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

static int wstart(int i, int k, int L)
{
    int s = i - k / 2;
    if (s < 0) s = 0;
    if (s > L - k) s = L - k;
    return s;
}

/* Gradients of one (b, h) map.  Every pointer is offset to the map; drpb_map
 * is this map's own (2k-1)^2 partial table.  `scr` holds 2 k*k doubles. */
static void one_map(const double *q, const double *kk, const double *v, const double *rpb_h,
                    const double *g, double *dq, double *dk, double *dv, double *drpb_map,
                    int H, int W, int d, int k, double *scr)
{
    const int nb = 2 * k - 1, n = k * k;
    const double scale = 1.0 / sqrt((double)d);
    double *p = scr, *ds = scr + n;
    for (int y = 0; y < H; ++y) {
        for (int x = 0; x < W; ++x) {
            const int64_t iq = (int64_t)y * W + x;
            const double *qi = q + iq * d, *gi = g + iq * d;
            const int sy = wstart(y, k, H), sx = wstart(x, k, W);
            /* forward: logits, softmax */
            double m = -INFINITY;
            for (int a = 0; a < k; ++a)
                for (int c = 0; c < k; ++c) {
                    const int64_t j = (int64_t)(sy + a) * W + (sx + c);
                    double dot = 0.0;
                    for (int t = 0; t < d; ++t) dot += qi[t] * kk[j * d + t];
                    const double b = rpb_h ? rpb_h[(sy + a - y + k - 1) * nb + (sx + c - x + k - 1)] : 0.0;
                    p[a * k + c] = (dot + b) * scale;
                    if (p[a * k + c] > m) m = p[a * k + c];
                }
            double z = 0.0;
            for (int e = 0; e < n; ++e) { p[e] = exp(p[e] - m); z += p[e]; }
            for (int e = 0; e < n; ++e) p[e] /= z;
            /* g_i . o_i with o_i = sum_j p_ij v_j */
            double go = 0.0;
            for (int a = 0; a < k; ++a)
                for (int c = 0; c < k; ++c) {
                    const int64_t j = (int64_t)(sy + a) * W + (sx + c);
                    double gv = 0.0;
                    for (int t = 0; t < d; ++t) gv += gi[t] * v[j * d + t];
                    ds[a * k + c] = gv;  /* dL/dp_ij for now */
                    go += p[a * k + c] * gv;
                }
            /* dL/ds, then the scatters */
            for (int a = 0; a < k; ++a)
                for (int c = 0; c < k; ++c) {
                    const int e = a * k + c;
                    const int64_t j = (int64_t)(sy + a) * W + (sx + c);
                    ds[e] = p[e] * (ds[e] - go);
                    for (int t = 0; t < d; ++t) {
                        dq[iq * d + t] += ds[e] * kk[j * d + t] * scale;
                        dk[j * d + t] += ds[e] * qi[t] * scale;
                        dv[j * d + t] += p[e] * gi[t];
                    }
                    if (drpb_map)
                        drpb_map[(sy + a - y + k - 1) * nb + (sx + c - x + k - 1)] += ds[e] * scale;
                }
        }
    }
}

/* dq, dk, dv [B][heads][H][W][d] and drpb [heads][2k-1][2k-1] (may be NULL)
 * are overwritten.  Returns 0, or -1 on invalid sizes. */
int na2d_oracle_backward_f64(const double *q, const double *k, const double *v,
                             const double *rpb, const double *g, double *dq, double *dk,
                             double *dv, double *drpb, int B, int heads, int H, int W, int d,
                             int ksize, int nthreads)
{
    if (B <= 0 || heads <= 0 || H <= 0 || W <= 0 || d <= 0) return -1;
    if (ksize < 1 || ksize % 2 == 0 || ksize > H || ksize > W) return -1;
    const int nb = 2 * ksize - 1;
    const int64_t maps = (int64_t)B * heads, per_map = (int64_t)H * W * d;
    memset(dq, 0, sizeof(double) * (size_t)(maps * per_map));
    memset(dk, 0, sizeof(double) * (size_t)(maps * per_map));
    memset(dv, 0, sizeof(double) * (size_t)(maps * per_map));
    double *part = NULL;
    if (drpb) part = (double *)calloc((size_t)(maps * nb * nb), sizeof(double));
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
        double *scr = (double *)malloc(sizeof(double) * 2 * (size_t)ksize * ksize);
#pragma omp for schedule(dynamic, 1)
        for (int64_t mp = 0; mp < maps; ++mp) {
            const int h = (int)(mp % heads);
            const int64_t o = mp * per_map;
            one_map(q + o, k + o, v + o, rpb ? rpb + (int64_t)h * nb * nb : NULL, g + o, dq + o,
                    dk + o, dv + o, part ? part + mp * nb * nb : NULL, H, W, d, ksize, scr);
        }
        free(scr);
    }
    if (drpb) {  /* sum the per-map tables over the batch, in batch order */
        memset(drpb, 0, sizeof(double) * (size_t)heads * nb * nb);
        for (int64_t mp = 0; mp < maps; ++mp) {
            const int h = (int)(mp % heads);
            for (int e = 0; e < nb * nb; ++e) drpb[(int64_t)h * nb * nb + e] += part[mp * nb * nb + e];
        }
        free(part);
    }
    return 0;
}
