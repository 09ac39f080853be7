/*
 * attn_oracle.c -- fp64 CPU oracle for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or helper with the GPU library; the two are compared, never combined.
 *
 * What it computes (the plain definition; no tiling, no online softmax):
 *
 *   FlashAttention-4 pages, "The Asymmetric Hardware Scaling Wall" (three
 *   phases per tile: the scaled scores QK^T/sqrt(d), the softmax
 *   P = exp(S - m)/l, and O = PV) and the guide's "Functional Validation
 *   Harness", which checks the tiled result against plain
 *   softmax(QK^T * scale) V.  Tiling and the running max/sum rescale are
 *   exact up to rounding, so the oracle is the untiled definition written out
 *   in double precision:
 *
 *     s_ij = scale * sum_c q_ic k_jc              (j in the valid set V_i)
 *     m_i  = max_j s_ij,  p_ij = exp(s_ij - m_i),  l_i = sum_j p_ij
 *     O_i  = (sum_j p_ij v_j) / l_i,   LSE_i = m_i + ln(l_i)
 *
 *   Causal masking keeps key j for query i iff j <= i (the guide's simulator,
 *   "End-to-End Implementation", masks keys after the query inside each
 *   tile).  A causal sliding window of W >= 1 keys (the banded mask a
 *   score/mask hook of the FlexAttention kind expresses; the guide's
 *   deployment section names such custom masks) further drops keys
 *   j <= i - W: query i sees keys max(0, i - W + 1) .. i.  W <= 0 means no
 *   window.
 *   Linear position bias: with per-query-head slopes a_h, every score gets
 *   a_h * (j - i) added after the scale,
 *     s_ij = scale * sum_c q_ic k_jc + a_h * (j - i),
 *   the additive score modification of the FlexAttention kind the guide's
 *   deployment section points to (ALiBi form); softmax, O, LSE and the
 *   gradients below are unchanged in form (the bias does not depend on Q, K
 *   or V, so it only enters through s).  slopes == NULL means no bias.
 *   Grouped-query attention: query head h reads key/value head
 *   h / (Hq / Hkv) (contiguous groups).
 *
 *   Backward (the pages give no formulas; these are the analytic gradients of
 *   the definition above, with P_ij = p_ij / l_i):
 *     dP_ij = dO_i . v_j
 *     D_i   = sum_c dO_ic O_ic
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = scale * sum_j dS_ij k_j
 *     dK_j  = scale * sum_{h in group} sum_i dS_ij q_i
 *     dV_j  =         sum_{h in group} sum_i P_ij dO_i
 *
 * Inputs are bf16 bit patterns (uint16), widened exactly to double once per
 * call.  The scale used is the float argument widened exactly to double.
 * Every sum runs sequentially in index order: each dot product over c, each
 * row sum over j, each gradient sum over j or over (head, i).  Dot products
 * are computed four at a time (four independent sums side by side, each in
 * c order), which gives the same values as one at a time.  Outputs are
 * double.
 *
 * Layout: row-major [B, H, N, d] for Q/K/V/dO/O/dQ/dK/dV, [B, H, N] for LSE.
 *
 * Build: gcc -O3 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math; without
 * contraction or reassociation, -O3 vectorises only element-wise loops).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1
#define ORACLE_NO_MEMORY 2

/* bf16 bit pattern -> double (exact: bf16 is the top half of an fp32). */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* n bf16 values -> double, exactly.  NULL when out of memory. */
static double *widen(const uint16_t *src, size_t n)
{
    double *dst = (double *)malloc(sizeof(double) * (n ? n : 1));
    if (!dst) return NULL;
    for (size_t t = 0; t < n; t++) dst[t] = bf16_to_double(src[t]);
    return dst;
}

static int check_shape(int B, int Hq, int Hkv, int N, int d)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1) return 0;
    if (Hq % Hkv != 0) return 0;
    return 1;
}

/* Keys query i may attend to: key_lo .. key_hi (inclusive). */
static int key_hi(int i, int N, int causal) { return causal ? i : N - 1; }
static int key_lo(int i, int causal, int window)
{
    return (causal && window > 0 && i - window + 1 > 0) ? i - window + 1 : 0;
}

/* Offset of row n of head h of batch b in a [B, H, N, d] tensor. */
static size_t row_off(int b, int h, int H, int n, int N, int d)
{
    return (((size_t)b * H + h) * N + n) * (size_t)d;
}

/*
 * out[j] = sum_c x_c * rows_j,c for the n rows of length d starting at
 * `rows`, each sum over c in index order.  Four rows are summed side by side
 * (independent sums), one row at a time for the remainder.
 */
static void row_dots(const double *x, const double *rows, int n, int d, double *out)
{
    int j = 0;
    for (; j + 4 <= n; j += 4) {
        const double *r0 = rows + (size_t)j * d, *r1 = r0 + d, *r2 = r1 + d, *r3 = r2 + d;
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
        for (int c = 0; c < d; c++) {
            a0 += x[c] * r0[c];
            a1 += x[c] * r1[c];
            a2 += x[c] * r2[c];
            a3 += x[c] * r3[c];
        }
        out[j] = a0;
        out[j + 1] = a1;
        out[j + 2] = a2;
        out[j + 3] = a3;
    }
    for (; j < n; j++) {
        const double *r = rows + (size_t)j * d;
        double a = 0.0;
        for (int c = 0; c < d; c++) a += x[c] * r[c];
        out[j] = a;
    }
}

/*
 * Scores of query row i (head h) against its keys lo .. lo + n - 1 (rows of
 * kh from key lo on): s[j] = scale * (q_i . k_{lo+j}) [+ slope * (lo + j - i)].
 * Returns max_j s[j].
 */
static double scores_row(const double *qi, const double *kh_lo, int n, int d, double sc,
                         const double *slope, int lo, int i, double *s)
{
    row_dots(qi, kh_lo, n, d, s);
    double m = -INFINITY;
    for (int j = 0; j < n; j++) {
        s[j] = slope ? sc * s[j] + *slope * (double)(lo + j - i) : sc * s[j];
        if (s[j] > m) m = s[j];
    }
    return m;
}

/*
 * Forward of one query row: m, l, O_i (into o_row, length d) and returns
 * the row's scores turned into p_ij = exp(s_ij - m) in s[0 .. n-1].
 */
static void forward_row(const double *qi, const double *kh_lo, const double *vh_lo, int n,
                        int d, double sc, const double *slope, int lo, int i, double *s,
                        double *o_row, double *m_out, double *l_out)
{
    const double m = scores_row(qi, kh_lo, n, d, sc, slope, lo, i, s);
    double l = 0.0;
    for (int j = 0; j < n; j++) {
        s[j] = exp(s[j] - m); /* p_ij */
        l += s[j];
    }
    for (int c = 0; c < d; c++) o_row[c] = 0.0;
    for (int j = 0; j < n; j++) {
        const double *vj = vh_lo + (size_t)j * d;
        for (int c = 0; c < d; c++) o_row[c] += s[j] * vj[c];
    }
    for (int c = 0; c < d; c++) o_row[c] /= l;
    *m_out = m;
    *l_out = l;
}

/*
 * Forward for an arbitrary list of query rows.  rows[r] is the flat index
 * (b * Hq + h) * N + i.  o_rows is [nrows, d], lse_rows is [nrows] (either
 * may be NULL).  Used for whole tensors (all rows) and for selected rows.
 */
int oracle_fwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int Hq,
                    int Hkv, int N, int d, float scale, int causal, int window,
                    const double *slopes, const int64_t *rows, int64_t nrows, double *o_rows,
                    double *lse_rows, int nthreads)
{
    if (!q || !k || !v || !rows || nrows < 0) return ORACLE_BAD_ARGS;
    if (!check_shape(B, Hq, Hkv, N, d)) return ORACLE_BAD_ARGS;
    if (window > 0 && !causal) return ORACLE_BAD_ARGS;
    const int64_t total = (int64_t)B * Hq * N;
    for (int64_t r = 0; r < nrows; r++)
        if (rows[r] < 0 || rows[r] >= total) return ORACLE_BAD_ARGS;
    const double sc = (double)scale;
    const int group = Hq / Hkv;
    if (nthreads < 1) nthreads = 1;
    const size_t kv_elems = (size_t)B * Hkv * N * d;
    double *kd = widen(k, kv_elems), *vd = widen(v, kv_elems);
    if (!kd || !vd) {
        free(kd);
        free(vd);
        return ORACLE_NO_MEMORY;
    }
    int failed = 0;

#pragma omp parallel num_threads(nthreads)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *qi = (double *)malloc(sizeof(double) * (size_t)d);
        double *oi = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qi || !oi) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; r++) {
            if (!s || !qi || !oi) continue;
            const int64_t flat = rows[r];
            const int i = (int)(flat % N);
            const int h = (int)((flat / N) % Hq);
            const int b = (int)(flat / ((int64_t)N * Hq));
            const int g = h / group;
            for (int c = 0; c < d; c++) qi[c] = bf16_to_double(q[row_off(b, h, Hq, i, N, d) + c]);
            const int lo = key_lo(i, causal, window);
            const int n = key_hi(i, N, causal) - lo + 1;
            double m, l;
            forward_row(qi, kd + row_off(b, g, Hkv, lo, N, d), vd + row_off(b, g, Hkv, lo, N, d),
                        n, d, sc, slopes ? slopes + h : NULL, lo, i, s, oi, &m, &l);
            if (o_rows) memcpy(o_rows + (size_t)r * d, oi, sizeof(double) * d);
            if (lse_rows) lse_rows[r] = m + log(l);
        }
        free(s);
        free(qi);
        free(oi);
    }
    free(kd);
    free(vd);
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Backward for a list of key/value groups, restricted to a block:
 *   dQ (and O, LSE) for query rows r0 .. r1 - 1 of each of the group's heads,
 *   dK and dV for keys k0 .. k1 - 1 of the group.
 * groups[t] is the flat index b * Hkv + g.  Outputs, group-major:
 *   dq [ngroups, Hq/Hkv, r1 - r0, d], o likewise, lse [ngroups, Hq/Hkv, r1 - r0]
 *   dk, dv [ngroups, k1 - k0, d]
 * (o, lse may be NULL).  r0 = k0 = 0, r1 = k1 = N is the whole backward.
 * stat_lse and stat_D (each may be NULL) receive LSE_i and D_i of every row
 * whose statistics the block computes, rows s0 .. s1 - 1 (defined below),
 * [ngroups, Hq/Hkv, s1 - s0]; stat_range (may be NULL) receives s0 and s1.
 *
 * The forward statistics (m, l, O, D) are computed here for every row the
 * block needs: rows r0 .. r1 - 1, and every row that sees a key of
 * k0 .. k1 - 1 (causal: rows j .. j + W - 1 for key j, all of them later
 * rows; otherwise every row).  Each such row's statistics still run over
 * all of that row's keys, so every block result equals the same slice of the
 * whole backward, bit for bit.
 *
 * Pass A walks query rows (dQ_i only touches row i); pass B walks key rows
 * (dK_j, dV_j only touch row j), recomputing s_ij, P_ij and dP_ij, so no two
 * threads write the same element and every sum runs in index order.
 */
int oracle_bwd_block(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const uint16_t *dout, int B, int Hq, int Hkv, int N, int d, float scale,
                     int causal, int window, const double *slopes, int r0, int r1, int k0, int k1,
                     const int64_t *groups, int64_t ngroups, double *dq, double *dk, double *dv,
                     double *o, double *lse, double *stat_lse, double *stat_D, int *stat_range,
                     int nthreads)
{
    if (!q || !k || !v || !dout || !groups || !dq || !dk || !dv || ngroups < 0)
        return ORACLE_BAD_ARGS;
    if (!check_shape(B, Hq, Hkv, N, d)) return ORACLE_BAD_ARGS;
    if (window > 0 && !causal) return ORACLE_BAD_ARGS;
    if (r0 < 0 || r1 <= r0 || r1 > N || k0 < 0 || k1 <= k0 || k1 > N) return ORACLE_BAD_ARGS;
    for (int64_t t = 0; t < ngroups; t++)
        if (groups[t] < 0 || groups[t] >= (int64_t)B * Hkv) return ORACLE_BAD_ARGS;
    const double sc = (double)scale;
    const int group = Hq / Hkv;
    if (nthreads < 1) nthreads = 1;

    /* Rows whose statistics are needed: [s0, s1). */
    int kr0 = 0, kr1 = N; /* rows that see some key of k0 .. k1 - 1 */
    if (causal) {
        kr0 = k0;
        kr1 = (window > 0 && (int64_t)k1 - 1 + window < N) ? k1 - 1 + window : N;
    }
    const int s0 = r0 < kr0 ? r0 : kr0;
    const int s1 = r1 > kr1 ? r1 : kr1;
    const int NS = s1 - s0, NR = r1 - r0, NK = k1 - k0;
    const size_t stat_rows = (size_t)group * NS;
    if (stat_range) {
        stat_range[0] = s0;
        stat_range[1] = s1;
    }

    double *m_buf = (double *)malloc(sizeof(double) * stat_rows);
    double *l_buf = (double *)malloc(sizeof(double) * stat_rows);
    double *D_buf = (double *)malloc(sizeof(double) * stat_rows);
    double *kh = (double *)malloc(sizeof(double) * (size_t)N * d);
    double *vh = (double *)malloc(sizeof(double) * (size_t)N * d);
    double *qg = (double *)malloc(sizeof(double) * (size_t)group * N * d);
    double *dog = (double *)malloc(sizeof(double) * (size_t)group * N * d);
    int failed = !m_buf || !l_buf || !D_buf || !kh || !vh || !qg || !dog;

    for (int64_t t = 0; t < ngroups && !failed; t++) {
        const int b = (int)(groups[t] / Hkv);
        const int g = (int)(groups[t] % Hkv);
        for (size_t e = 0; e < (size_t)N * d; e++) {
            kh[e] = bf16_to_double(k[row_off(b, g, Hkv, 0, N, d) + e]);
            vh[e] = bf16_to_double(v[row_off(b, g, Hkv, 0, N, d) + e]);
        }
        for (int hl = 0; hl < group; hl++)
            for (size_t e = 0; e < (size_t)N * d; e++) {
                const size_t src = row_off(b, g * group + hl, Hq, 0, N, d) + e;
                qg[(size_t)hl * N * d + e] = bf16_to_double(q[src]);
                dog[(size_t)hl * N * d + e] = bf16_to_double(dout[src]);
            }
        double *dq_t = dq + (size_t)t * group * NR * d;
        double *dk_t = dk + (size_t)t * NK * d;
        double *dv_t = dv + (size_t)t * NK * d;
        double *o_t = o ? o + (size_t)t * group * NR * d : NULL;
        double *lse_t = lse ? lse + (size_t)t * group * NR : NULL;

        /* Pass A: per query row of each head of the group -> m, l, O, D; dQ, O
         * and LSE for the block's rows. */
#pragma omp parallel num_threads(nthreads)
        {
            double *s = (double *)malloc(sizeof(double) * (size_t)N);
            double *dp = (double *)malloc(sizeof(double) * (size_t)N);
            double *oi = (double *)malloc(sizeof(double) * (size_t)d);
            double *acc = (double *)malloc(sizeof(double) * (size_t)d);
            if (!s || !dp || !oi || !acc) {
#pragma omp atomic write
                failed = 1;
            }
#pragma omp for schedule(dynamic, 4)
            for (int64_t rr = 0; rr < (int64_t)stat_rows; rr++) {
                if (!s || !dp || !oi || !acc) continue;
                const int hl = (int)(rr / NS); /* head within the group */
                const int i = s0 + (int)(rr % NS);
                const int h = g * group + hl;
                const double *qi = qg + ((size_t)hl * N + i) * d;
                const double *doi = dog + ((size_t)hl * N + i) * d;
                const int lo = key_lo(i, causal, window);
                const int n = key_hi(i, N, causal) - lo + 1;
                const double *khi = kh + (size_t)lo * d; /* keys lo .. lo + n - 1 */
                const double *vhi = vh + (size_t)lo * d;
                double m, l;
                forward_row(qi, khi, vhi, n, d, sc, slopes ? slopes + h : NULL, lo, i, s, oi, &m,
                            &l);
                double Di = 0.0;
                for (int c = 0; c < d; c++) Di += doi[c] * oi[c];
                m_buf[rr] = m;
                l_buf[rr] = l;
                D_buf[rr] = Di;
                if (stat_lse) stat_lse[(size_t)t * stat_rows + rr] = m + log(l);
                if (stat_D) stat_D[(size_t)t * stat_rows + rr] = Di;
                if (i < r0 || i >= r1) continue;
                const size_t out = (size_t)hl * NR + (i - r0);
                if (o_t) memcpy(o_t + out * d, oi, sizeof(double) * d);
                if (lse_t) lse_t[out] = m + log(l);

                /* dQ_i = scale * sum_j dS_ij k_j, dS_ij = P_ij (dP_ij - D_i) */
                row_dots(doi, vhi, n, d, dp); /* dP_ij */
                for (int c = 0; c < d; c++) acc[c] = 0.0;
                for (int j = 0; j < n; j++) {
                    const double dS = (s[j] / l) * (dp[j] - Di);
                    const double *kj = khi + (size_t)j * d;
                    for (int c = 0; c < d; c++) acc[c] += dS * kj[c];
                }
                double *dqi = dq_t + out * d;
                for (int c = 0; c < d; c++) dqi[c] = sc * acc[c];
            }
            free(s);
            free(dp);
            free(oi);
            free(acc);
        }
        if (failed) break;

        /* Pass B: per key row j of the block -> dK_j, dV_j over the group's
         * heads and the rows that see key j, in (head, row) order. */
#pragma omp parallel num_threads(nthreads)
        {
            double *sv = (double *)malloc(sizeof(double) * (size_t)N);
            double *dp = (double *)malloc(sizeof(double) * (size_t)N);
            double *acck = (double *)malloc(sizeof(double) * (size_t)d);
            double *accv = (double *)malloc(sizeof(double) * (size_t)d);
            if (!sv || !dp || !acck || !accv) {
#pragma omp atomic write
                failed = 1;
            }
#pragma omp for schedule(dynamic, 2)
            for (int j = k0; j < k1; j++) {
                if (!sv || !dp || !acck || !accv) continue;
                const double *kj = kh + (size_t)j * d;
                const double *vj = vh + (size_t)j * d;
                for (int c = 0; c < d; c++) acck[c] = accv[c] = 0.0;
                /* rows that see key j: j .. j + W - 1 (causal), all (otherwise) */
                const int i0 = causal ? j : 0;
                const int i1 = (causal && window > 0 && (int64_t)j + window < N) ? j + window : N;
                for (int hl = 0; hl < group; hl++) {
                    const int h = g * group + hl;
                    const double *qrows = qg + ((size_t)hl * N + i0) * d;
                    const double *dorows = dog + ((size_t)hl * N + i0) * d;
                    row_dots(kj, qrows, i1 - i0, d, sv); /* q_i . k_j */
                    row_dots(vj, dorows, i1 - i0, d, dp); /* dO_i . v_j */
                    for (int i = i0; i < i1; i++) {
                        const size_t rr = (size_t)hl * NS + (i - s0);
                        const double sij = slopes ? sc * sv[i - i0] + slopes[h] * (double)(j - i)
                                                  : sc * sv[i - i0];
                        const double P = exp(sij - m_buf[rr]) / l_buf[rr];
                        const double dS = P * (dp[i - i0] - D_buf[rr]);
                        const double *qi = qrows + (size_t)(i - i0) * d;
                        const double *doi = dorows + (size_t)(i - i0) * d;
                        for (int c = 0; c < d; c++) {
                            accv[c] += P * doi[c];
                            acck[c] += dS * qi[c];
                        }
                    }
                }
                for (int c = 0; c < d; c++) {
                    dv_t[(size_t)(j - k0) * d + c] = accv[c];
                    dk_t[(size_t)(j - k0) * d + c] = sc * acck[c];
                }
            }
            free(sv);
            free(dp);
            free(acck);
            free(accv);
        }
    }
    free(m_buf);
    free(l_buf);
    free(D_buf);
    free(kh);
    free(vh);
    free(qg);
    free(dog);
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}
