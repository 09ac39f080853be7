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
 *   phases per tile: S = QK^T/sqrt(d); P = exp(S - m)/l; O = PV) and the
 *   simulator's validation harness ("Functional Validation Harness"), which
 *   states that the tiled result equals softmax(QK^T * scale) V.  Tiling and
 *   the running max/sum rescale are exact up to rounding, so the oracle is the
 *   untiled definition written out in double precision:
 *
 *     s_ij = scale * sum_c q_ic k_jc              (j in the valid set V_i)
 *     m_i  = max_j s_ij,  p_ij = exp(s_ij - m_i),  l_i = sum_j p_ij
 *     O_i  = (sum_j p_ij v_j) / l_i,   LSE_i = m_i + ln(l_i)
 *
 *   Causal masking keeps key j for query i iff j <= i (the simulator's
 *   "Apply causal mask inside tile" step keeps q_idx >= kv_idx).  A causal
 *   sliding window of W >= 1 keys (the banded mask a score/mask hook of the
 *   FlexAttention kind expresses; the guide's deployment section names such
 *   custom masks) further drops keys j <= i - W: query i sees keys
 *   max(0, i - W + 1) .. i.  W <= 0 means no window.
 *   Linear position bias (the `_b` entry points): with per-query-head slopes
 *   a_h, every score gets a_h * (j - i) added after the scale,
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
 * Inputs are bf16 bit patterns (uint16), widened exactly to double.  The
 * scale used is the float argument widened exactly to double.  Every sum runs
 * sequentially in index order.  Outputs are double.
 *
 * Layout: row-major [B, H, N, d] for Q/K/V/dO/O/dQ/dK/dV, [B, H, N] for LSE.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
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

static int check_shape(int B, int Hq, int Hkv, int N, int d)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1) return 0;
    if (Hq % Hkv != 0) return 0;
    return 1;
}

/* Keys query i may attend to: lo .. hi (inclusive). */
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
 * Scores of query row i against keys 0..n-1 into s[], returns the max.
 * s_ij = scale * (q_i . k_j), dot product summed over c in order.
 */
static double scores_row(const uint16_t *qi, const uint16_t *kh, int n, int d,
                         double sc, double *s)
{
    double m = -INFINITY;
    for (int j = 0; j < n; j++) {
        const uint16_t *kj = kh + (size_t)j * d;
        double dot = 0.0;
        for (int c = 0; c < d; c++) dot += bf16_to_double(qi[c]) * bf16_to_double(kj[c]);
        s[j] = sc * dot;
        if (s[j] > m) m = s[j];
    }
    return m;
}

/* The same with the linear position bias: the keys are lo .. lo + n - 1,
 * s_ij = scale * (q_i . k_j) + slope * (j - i). */
static double scores_row_bias(const uint16_t *qi, const uint16_t *kh, int n, int d, double sc,
                              double slope, int lo, int i, double *s)
{
    double m = -INFINITY;
    for (int j = 0; j < n; j++) {
        const uint16_t *kj = kh + (size_t)j * d;
        double dot = 0.0;
        for (int c = 0; c < d; c++) dot += bf16_to_double(qi[c]) * bf16_to_double(kj[c]);
        s[j] = sc * dot + slope * (double)(lo + j - i);
        if (s[j] > m) m = s[j];
    }
    return m;
}

/*
 * Forward for an arbitrary list of query rows.  rows[r] is the flat index
 * (b * Hq + h) * N + i.  o_rows is [nrows, d], lse_rows is [nrows] (either
 * may be NULL).  Used for whole tensors (all rows) and for sampled rows of
 * tensors too large to check in full.
 */
int oracle_fwd_rows_b(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      int B, int Hq, int Hkv, int N, int d, float scale, int causal, int window,
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
    int failed = 0;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel num_threads(nthreads)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; r++) {
            if (!s || !acc) continue;
            const int64_t flat = rows[r];
            const int i = (int)(flat % N);
            const int h = (int)((flat / N) % Hq);
            const int b = (int)(flat / ((int64_t)N * Hq));
            const int g = h / group;
            const uint16_t *qi = q + row_off(b, h, Hq, i, N, d);
            const int lo = key_lo(i, causal, window);
            const int n = key_hi(i, N, causal) - lo + 1;
            /* keys lo .. lo + n - 1, indexed 0 .. n - 1 below */
            const uint16_t *kh = k + row_off(b, g, Hkv, lo, N, d);
            const uint16_t *vh = v + row_off(b, g, Hkv, lo, N, d);

            const double m = slopes ? scores_row_bias(qi, kh, n, d, sc, slopes[h], lo, i, s)
                                    : scores_row(qi, kh, n, d, sc, s);
            double l = 0.0;
            for (int j = 0; j < n; j++) {
                s[j] = exp(s[j] - m); /* p_ij */
                l += s[j];
            }
            for (int c = 0; c < d; c++) acc[c] = 0.0;
            for (int j = 0; j < n; j++) {
                const uint16_t *vj = vh + (size_t)j * d;
                for (int c = 0; c < d; c++) acc[c] += s[j] * bf16_to_double(vj[c]);
            }
            if (o_rows)
                for (int c = 0; c < d; c++) o_rows[r * d + c] = acc[c] / l;
            if (lse_rows) lse_rows[r] = m + log(l);
        }
        free(s);
        free(acc);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

int oracle_fwd_rows_w(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      int B, int Hq, int Hkv, int N, int d, float scale, int causal, int window,
                      const int64_t *rows, int64_t nrows, double *o_rows, double *lse_rows,
                      int nthreads)
{
    return oracle_fwd_rows_b(q, k, v, B, Hq, Hkv, N, d, scale, causal, window, NULL, rows, nrows,
                             o_rows, lse_rows, nthreads);
}

int oracle_fwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                    const int64_t *rows, int64_t nrows, double *o_rows, double *lse_rows,
                    int nthreads)
{
    return oracle_fwd_rows_w(q, k, v, B, Hq, Hkv, N, d, scale, causal, 0, rows, nrows, o_rows,
                             lse_rows, nthreads);
}

/* Whole forward: O [B,Hq,N,d], LSE [B,Hq,N] (LSE may be NULL). */
int oracle_fwd_w(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *o, double *lse,
                 int B, int Hq, int Hkv, int N, int d, float scale, int causal, int window,
                 int nthreads)
{
    if (!o) return ORACLE_BAD_ARGS;
    if (!check_shape(B, Hq, Hkv, N, d)) return ORACLE_BAD_ARGS;
    const int64_t total = (int64_t)B * Hq * N;
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)total);
    if (!rows) return ORACLE_NO_MEMORY;
    for (int64_t r = 0; r < total; r++) rows[r] = r;
    int st = oracle_fwd_rows_w(q, k, v, B, Hq, Hkv, N, d, scale, causal, window, rows, total, o,
                               lse, nthreads);
    free(rows);
    return st;
}

/* Whole forward with the linear position bias (slopes [Hq]). */
int oracle_fwd_b(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *o, double *lse,
                 int B, int Hq, int Hkv, int N, int d, float scale, int causal, int window,
                 const double *slopes, int nthreads)
{
    if (!o || !slopes) return ORACLE_BAD_ARGS;
    if (!check_shape(B, Hq, Hkv, N, d)) return ORACLE_BAD_ARGS;
    const int64_t total = (int64_t)B * Hq * N;
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)total);
    if (!rows) return ORACLE_NO_MEMORY;
    for (int64_t r = 0; r < total; r++) rows[r] = r;
    int st = oracle_fwd_rows_b(q, k, v, B, Hq, Hkv, N, d, scale, causal, window, slopes, rows,
                               total, o, lse, nthreads);
    free(rows);
    return st;
}

int oracle_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *o, double *lse,
               int B, int Hq, int Hkv, int N, int d, float scale, int causal, int nthreads)
{
    return oracle_fwd_w(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, 0, nthreads);
}

/*
 * Backward for a list of key/value groups.  groups[t] is the flat index
 * b * Hkv + g.  For each listed group it writes, group-major:
 *   dq  [ngroups, Hq/Hkv, N, d]   (the group's query heads, in head order)
 *   dk  [ngroups, N, d], dv [ngroups, N, d]
 *   o   [ngroups, Hq/Hkv, N, d] and lse [ngroups, Hq/Hkv, N]  (may be NULL)
 * The forward quantities it needs (m, l, O, D) are its own, computed here.
 *
 * Pass A walks query rows (dQ_i only touches row i); pass B walks key rows
 * (dK_j, dV_j only touch row j), recomputing s_ij, P_ij and dP_ij, so no two
 * threads write the same element and every sum runs in index order.
 */
/*
 * The same backward restricted to the tail block of a causal problem: rows
 * and keys row0 .. N - 1.  Under the causal mask key j only receives gradient
 * from rows i >= j, so dK_j and dV_j for j >= row0 need only the tail rows
 * (whose forward statistics still run over all their keys), and dQ_i for
 * i >= row0 is the ordinary row result.  Outputs hold the tail only:
 * dq [ngroups, Hq/Hkv, N - row0, d], dk and dv [ngroups, N - row0, d], o and
 * lse likewise.  row0 = 0 is the full backward (and the only value allowed
 * without the causal mask).  With a window, key j receives gradient from rows
 * j .. j + W - 1 only, still all >= j.
 */
int oracle_bwd_groups_tail_b(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const uint16_t *dout, int B, int Hq, int Hkv, int N, int d,
                             float scale, int causal, int window, const double *slopes,
                             int row0, const int64_t *groups, int64_t ngroups, double *dq,
                             double *dk, double *dv, double *o, double *lse, int nthreads)
{
    if (!q || !k || !v || !dout || !groups || !dq || !dk || !dv || ngroups < 0)
        return ORACLE_BAD_ARGS;
    if (!check_shape(B, Hq, Hkv, N, d)) return ORACLE_BAD_ARGS;
    if (window > 0 && !causal) return ORACLE_BAD_ARGS;
    if (row0 < 0 || row0 >= N || (!causal && row0 != 0)) return ORACLE_BAD_ARGS;
    for (int64_t t = 0; t < ngroups; t++)
        if (groups[t] < 0 || groups[t] >= (int64_t)B * Hkv) return ORACLE_BAD_ARGS;
    const double sc = (double)scale;
    const int group = Hq / Hkv;
    const int NT = N - row0; /* tail rows per head */
    const size_t rows_per_group = (size_t)group * NT;
    if (nthreads < 1) nthreads = 1;

    /* Per-row forward statistics of the group being processed. */
    double *m_buf = (double *)malloc(sizeof(double) * rows_per_group);
    double *l_buf = (double *)malloc(sizeof(double) * rows_per_group);
    double *D_buf = (double *)malloc(sizeof(double) * rows_per_group);
    double *o_buf = (double *)malloc(sizeof(double) * rows_per_group * (size_t)d);
    if (!m_buf || !l_buf || !D_buf || !o_buf) {
        free(m_buf); free(l_buf); free(D_buf); free(o_buf);
        return ORACLE_NO_MEMORY;
    }
    int failed = 0;

    for (int64_t t = 0; t < ngroups && !failed; t++) {
        const int b = (int)(groups[t] / Hkv);
        const int g = (int)(groups[t] % Hkv);
        const uint16_t *kh = k + row_off(b, g, Hkv, 0, N, d);
        const uint16_t *vh = v + row_off(b, g, Hkv, 0, N, d);
        double *dq_t = dq + (size_t)t * rows_per_group * d;
        double *dk_t = dk + (size_t)t * NT * d;
        double *dv_t = dv + (size_t)t * NT * d;

        /* Pass A: per query row of each head of the group -> m, l, O, D, dQ. */
#pragma omp parallel num_threads(nthreads)
        {
            double *s = (double *)malloc(sizeof(double) * (size_t)N);
            double *acc = (double *)malloc(sizeof(double) * (size_t)d);
            if (!s || !acc) {
#pragma omp atomic write
                failed = 1;
            }
#pragma omp for schedule(dynamic, 4)
            for (int64_t rr = 0; rr < (int64_t)rows_per_group; rr++) {
                if (!s || !acc) continue;
                const int hl = (int)(rr / NT); /* head within the group */
                const int i = row0 + (int)(rr % NT);
                const int h = g * group + hl;
                const uint16_t *qi = q + row_off(b, h, Hq, i, N, d);
                const uint16_t *doi = dout + row_off(b, h, Hq, i, N, d);
                const int lo = key_lo(i, causal, window);
                const int n = key_hi(i, N, causal) - lo + 1;
                const uint16_t *khi = kh + (size_t)lo * d; /* keys lo .. lo + n - 1 */
                const uint16_t *vhi = vh + (size_t)lo * d;

                const double m = slopes ? scores_row_bias(qi, khi, n, d, sc, slopes[h], lo, i, s)
                                        : scores_row(qi, khi, n, d, sc, s);
                double l = 0.0;
                for (int j = 0; j < n; j++) {
                    s[j] = exp(s[j] - m);
                    l += s[j];
                }
                for (int c = 0; c < d; c++) acc[c] = 0.0;
                for (int j = 0; j < n; j++) {
                    const uint16_t *vj = vhi + (size_t)j * d;
                    for (int c = 0; c < d; c++) acc[c] += s[j] * bf16_to_double(vj[c]);
                }
                double *oi = o_buf + (size_t)rr * d;
                for (int c = 0; c < d; c++) oi[c] = acc[c] / l;
                double Di = 0.0;
                for (int c = 0; c < d; c++) Di += bf16_to_double(doi[c]) * oi[c];
                m_buf[rr] = m;
                l_buf[rr] = l;
                D_buf[rr] = Di;

                /* dQ_i = scale * sum_j dS_ij k_j */
                for (int c = 0; c < d; c++) acc[c] = 0.0;
                for (int j = 0; j < n; j++) {
                    const uint16_t *vj = vhi + (size_t)j * d;
                    const uint16_t *kj = khi + (size_t)j * d;
                    double dp = 0.0;
                    for (int c = 0; c < d; c++) dp += bf16_to_double(doi[c]) * bf16_to_double(vj[c]);
                    const double P = s[j] / l;
                    const double dS = P * (dp - Di);
                    for (int c = 0; c < d; c++) acc[c] += dS * bf16_to_double(kj[c]);
                }
                double *dqi = dq_t + (size_t)rr * d;
                for (int c = 0; c < d; c++) dqi[c] = sc * acc[c];
            }
            free(s);
            free(acc);
        }
        if (failed) break;

        /* Pass B: per key row j -> dK_j, dV_j over the group's heads and rows. */
#pragma omp parallel num_threads(nthreads)
        {
            double *acck = (double *)malloc(sizeof(double) * (size_t)d);
            double *accv = (double *)malloc(sizeof(double) * (size_t)d);
            if (!acck || !accv) {
#pragma omp atomic write
                failed = 1;
            }
#pragma omp for schedule(dynamic, 4)
            for (int j = row0; j < N; j++) {
                if (!acck || !accv) continue;
                const uint16_t *kj = kh + (size_t)j * d;
                const uint16_t *vj = vh + (size_t)j * d;
                for (int c = 0; c < d; c++) acck[c] = accv[c] = 0.0;
                for (int hl = 0; hl < group; hl++) {
                    const int h = g * group + hl;
                    /* queries that see key j (>= row0): j .. j + W - 1 with a window */
                    const int i0 = causal ? j : 0;
                    const int i1 = (causal && window > 0 && j + window < N) ? j + window : N;
                    for (int i = i0; i < i1; i++) {
                        const size_t rr = (size_t)hl * NT + (i - row0);
                        const uint16_t *qi = q + row_off(b, h, Hq, i, N, d);
                        const uint16_t *doi = dout + row_off(b, h, Hq, i, N, d);
                        double dot = 0.0, dp = 0.0;
                        for (int c = 0; c < d; c++) dot += bf16_to_double(qi[c]) * bf16_to_double(kj[c]);
                        for (int c = 0; c < d; c++) dp += bf16_to_double(doi[c]) * bf16_to_double(vj[c]);
                        const double sij = slopes ? sc * dot + slopes[h] * (double)(j - i) : sc * dot;
                        const double P = exp(sij - m_buf[rr]) / l_buf[rr];
                        const double dS = P * (dp - D_buf[rr]);
                        for (int c = 0; c < d; c++) {
                            accv[c] += P * bf16_to_double(doi[c]);
                            acck[c] += dS * bf16_to_double(qi[c]);
                        }
                    }
                }
                for (int c = 0; c < d; c++) {
                    dv_t[(size_t)(j - row0) * d + c] = accv[c];
                    dk_t[(size_t)(j - row0) * d + c] = sc * acck[c];
                }
            }
            free(acck);
            free(accv);
        }

        if (o) memcpy(o + (size_t)t * rows_per_group * d, o_buf, sizeof(double) * rows_per_group * d);
        if (lse)
            for (size_t rr = 0; rr < rows_per_group; rr++)
                lse[(size_t)t * rows_per_group + rr] = m_buf[rr] + log(l_buf[rr]);
    }
    free(m_buf);
    free(l_buf);
    free(D_buf);
    free(o_buf);
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

int oracle_bwd_groups_tail_w(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const uint16_t *dout, int B, int Hq, int Hkv, int N, int d,
                             float scale, int causal, int window, int row0,
                             const int64_t *groups, int64_t ngroups, double *dq, double *dk,
                             double *dv, double *o, double *lse, int nthreads)
{
    return oracle_bwd_groups_tail_b(q, k, v, dout, B, Hq, Hkv, N, d, scale, causal, window, NULL,
                                    row0, groups, ngroups, dq, dk, dv, o, lse, nthreads);
}

int oracle_bwd_groups_tail(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const uint16_t *dout, int B, int Hq, int Hkv, int N, int d,
                           float scale, int causal, int row0, const int64_t *groups,
                           int64_t ngroups, double *dq, double *dk, double *dv, double *o,
                           double *lse, int nthreads)
{
    return oracle_bwd_groups_tail_w(q, k, v, dout, B, Hq, Hkv, N, d, scale, causal, 0, row0,
                                    groups, ngroups, dq, dk, dv, o, lse, nthreads);
}

int oracle_bwd_groups(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const uint16_t *dout, int B, int Hq, int Hkv, int N, int d, float scale,
                      int causal, const int64_t *groups, int64_t ngroups, double *dq, double *dk,
                      double *dv, double *o, double *lse, int nthreads)
{
    return oracle_bwd_groups_tail_w(q, k, v, dout, B, Hq, Hkv, N, d, scale, causal, 0, 0, groups,
                                    ngroups, dq, dk, dv, o, lse, nthreads);
}
