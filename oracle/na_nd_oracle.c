/*
 * na_nd_oracle.c -- fp64 CPU oracle for Neighborhood Attention over one, two
 * or three axes, and for SASA windows (zero padding).
 *
 * TEST INFRASTRUCTURE ONLY.  Like na2d_oracle.c this is the slow, obviously
 * correct definition the GPU path is checked against; only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark load it, and it
 * shares no code with the GPU library.
 *
 * Definition.  Eq. 2-4 of "Neighborhood Attention Transformer" (CSDN
 * translation, section 3.1; the same equations in the qiita article
 * "NAT: スライディングウィンドウアテンションの革新", section "Neighborhood
 * Attention(NA)") for a query at position i = (i0, i1, i2) of a grid with
 * axes of length (L0, L1, L2):
 *
 *   A_i   = [ Q_i . K_p + B(i, p) ]  over the neighbours p of i
 *   NA(i) = softmax( A_i / sqrt(d) ) [ V_p ]
 *
 * The neighbourhood is a product of per-axis windows of k_a positions:
 *  - mode 0, Neighborhood Attention: the k_a indices of the axis nearest to
 *    i_a, window start clamp(i_a - k_a/2, 0, L_a - k_a) (CSDN page, section 1
 *    and section 3.1; qiita figure of NA windows at the border).  One and two
 *    axes are the 1D and 2D NA of NATTEN (CSDN page, section 3.2); three axes
 *    are the 3D case the qiita article's NATTEN section names.
 *  - mode 1, SASA: the window centred on the query, start i_a - k_a/2, on the
 *    input zero-padded by k_a/2 at both ends of every axis.  The CSDN page
 *    (section 3.1, the paragraph after Eq. 4, and section 3.2) describes SASA
 *    as exactly this: NA on a zero-padded input.  Read plainly, a padded
 *    position is a key and a value equal to zero: its logit is B / sqrt(d)
 *    and it takes part in the softmax, but adds nothing to the output.
 * The bias table is [heads][2k0-1][2k1-1][2k2-1], indexed on every axis by
 * key position minus query position plus k_a - 1.  rpb == NULL means no bias.
 * Layout: q, k, v, out are [B][heads][L0][L1][L2][d], d fastest.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

/* Window start along one axis (see the modes above). */
int na_nd_window_start(int i, int k, int L, int mode)
{
    int s = i - k / 2;
    if (mode == 0) {
        if (s < 0) s = 0;
        if (s > L - k) s = L - k;
    }
    return s;
}

typedef struct {
    int B, heads, L[3], d, k[3], mode;
} nd_shape;

/* One output vector.  `logit` is scratch of k0*k1*k2 doubles. */
static void one_query(const double *q, const double *kk, const double *v, const double *rpb,
                      const nd_shape *s, int64_t b, int h, const int pos[3], double *logit,
                      double *o)
{
    const int d = s->d;
    const int64_t map = ((int64_t)b * s->heads + h) * s->L[0] * s->L[1] * s->L[2];
    const double *qi = q + (map + ((int64_t)pos[0] * s->L[1] + pos[1]) * s->L[2] + pos[2]) * d;
    int st[3], nb[3];
    for (int a = 0; a < 3; ++a) {
        st[a] = na_nd_window_start(pos[a], s->k[a], s->L[a], s->mode);
        nb[a] = 2 * s->k[a] - 1;
    }
    const double scale = 1.0 / sqrt((double)d);
    const int n = s->k[0] * s->k[1] * s->k[2];

    /* logits (Eq. 2 and the division of Eq. 4) */
    for (int j = 0; j < n; ++j) {
        const int c2 = j % s->k[2], c1 = (j / s->k[2]) % s->k[1], c0 = j / (s->k[2] * s->k[1]);
        const int p0 = st[0] + c0, p1 = st[1] + c1, p2 = st[2] + c2;
        const int inside = p0 >= 0 && p0 < s->L[0] && p1 >= 0 && p1 < s->L[1] && p2 >= 0 &&
                           p2 < s->L[2];
        double dot = 0.0;
        if (inside) {
            const double *kj = kk + (map + ((int64_t)p0 * s->L[1] + p1) * s->L[2] + p2) * d;
            for (int t = 0; t < d; ++t) dot += qi[t] * kj[t];
        }
        double bias = 0.0;
        if (rpb) {
            const int64_t r0 = p0 - pos[0] + s->k[0] - 1, r1 = p1 - pos[1] + s->k[1] - 1,
                          r2 = p2 - pos[2] + s->k[2] - 1;
            bias = rpb[(((int64_t)h * nb[0] + r0) * nb[1] + r1) * nb[2] + r2];
        }
        logit[j] = (dot + bias) * scale;
    }
    /* softmax over the neighbourhood (max subtracted; same value exactly) */
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) if (logit[j] > m) m = logit[j];
    double z = 0.0;
    for (int j = 0; j < n; ++j) { logit[j] = exp(logit[j] - m); z += logit[j]; }
    /* weighted sum of the neighbour values (Eq. 3-4); padded values are zero */
    for (int t = 0; t < d; ++t) o[t] = 0.0;
    for (int j = 0; j < n; ++j) {
        const int c2 = j % s->k[2], c1 = (j / s->k[2]) % s->k[1], c0 = j / (s->k[2] * s->k[1]);
        const int p0 = st[0] + c0, p1 = st[1] + c1, p2 = st[2] + c2;
        if (p0 < 0 || p0 >= s->L[0] || p1 < 0 || p1 >= s->L[1] || p2 < 0 || p2 >= s->L[2])
            continue;
        const double *vj = v + (map + ((int64_t)p0 * s->L[1] + p1) * s->L[2] + p2) * d;
        const double w = logit[j] / z;
        for (int t = 0; t < d; ++t) o[t] += w * vj[t];
    }
}

static int bad_shape(const nd_shape *s)
{
    if (s->B <= 0 || s->heads <= 0 || s->d <= 0 || (s->mode != 0 && s->mode != 1)) return 1;
    for (int a = 0; a < 3; ++a) {
        if (s->L[a] <= 0 || s->k[a] < 1 || (s->k[a] % 2) == 0) return 1;
        if (s->mode == 0 && s->k[a] > s->L[a]) return 1;
    }
    return 0;
}

static void split_index(const nd_shape *s, int64_t p, int64_t *b, int *h, int pos[3])
{
    pos[2] = (int)(p % s->L[2]);
    p /= s->L[2];
    pos[1] = (int)(p % s->L[1]);
    p /= s->L[1];
    pos[0] = (int)(p % s->L[0]);
    p /= s->L[0];
    *h = (int)(p % s->heads);
    *b = p / s->heads;
}

/* The outputs for the queries with linear index
 * (((b * heads + h) * L0 + i0) * L1 + i1) * L2 + i2 listed in idx (all of
 * them, in order, when idx is NULL); out is [n][d].  Returns 0, or -1 on
 * invalid sizes or indices.  nthreads <= 0 uses the OpenMP default. */
int na_nd_oracle_f64(const double *q, const double *k, const double *v, const double *rpb,
                     const int64_t *idx, int64_t n, double *out, int B, int heads, int L0,
                     int L1, int L2, int d, int k0, int k1, int k2, int mode, int nthreads)
{
    const nd_shape s = {B, heads, {L0, L1, L2}, d, {k0, k1, k2}, mode};
    if (bad_shape(&s)) return -1;
    const int64_t total = (int64_t)B * heads * L0 * L1 * L2;
    if (!idx) n = total;
    for (int64_t i = 0; idx && i < n; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)k0 * k1 * k2);
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < n; ++i) {
            int64_t b;
            int h, pos[3];
            split_index(&s, idx ? idx[i] : i, &b, &h, pos);
            one_query(q, k, v, rpb, &s, b, h, pos, logit, out + i * d);
        }
        free(logit);
    }
    return 0;
}
