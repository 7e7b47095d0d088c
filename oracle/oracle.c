/*
 * fp64 CPU oracle for fused graph attention over a CSR neighbourhood, and for
 * min/max reduction aggregation over the same neighbourhood (last section).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code, header or constant with the HIP library.
 *
 * What it computes is the plain definition of the two attention-GNN layers the
 * pages name (Graph Transformer dot-product attention and GATv2 additive
 * attention: DF-GNN abstract; IO-aware layers abstract, "attention-based layers
 * (GATv2/Graph Transformer)"). The fused kernels the pages describe (Yandex
 * Research blog, paragraph on attention-based layers) evaluate exactly this
 * result with an online softmax; an online softmax is an algebraic
 * rearrangement, so the oracle deliberately does the textbook two-pass form:
 * scores, row max, exponentials, normalisation, weighted sum.
 *
 * Conventions (readings of the pages, which give no formulas):
 *   - CSR by destination: row i holds edges e in [rowptr[i], rowptr[i+1]),
 *     each an edge colidx[e] -> i. Softmax runs over the edges of a row.
 *   - Repeated edges are separate softmax terms (multiset semantics).
 *   - Empty row: out = 0, lse = -inf, all gradients from it zero.
 *   - lse is the natural-log log-sum-exp of the row's scores.
 *   - Graph Transformer score: <Q_i, K_j> / sqrt(D), per head.
 *   - GATv2 score: sum_d a[h,d] * LeakyReLU(Xs[i,h,d] + Xt[j,h,d]); the value
 *     aggregated is Xt[j]; LeakyReLU'(z) is 1 for z > 0 and `slope` otherwise.
 *   - The backward uses the softmax Jacobian written out,
 *     dS_e = alpha_e * (dP_e - sum_e' alpha_e' dP_e'), for the loss
 *     L = sum(out * dout). No stored statistics are reused.
 *
 * Inputs are read in their stored type (fp32, bf16 bits, or fp64) and widened
 * exactly to fp64. Every sum is taken in fp64. Row-parallel loops use OpenMP;
 * every reduction that crosses rows is done over fixed row blocks, summed in
 * block order, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

static double ld(const void* p, int dtype, int64_t k)
{
    if (dtype == ORC_F64) return ((const double*)p)[k];
    if (dtype == ORC_F32) return (double)((const float*)p)[k];
    uint32_t u = (uint32_t)((const uint16_t*)p)[k] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int check_csr(int64_t n, const int64_t* rowptr, const int32_t* colidx)
{
    if (n < 0) return 1;
    if (rowptr[0] != 0) return 2;
    for (int64_t i = 0; i < n; ++i)
        if (rowptr[i + 1] < rowptr[i]) return 2;
    for (int64_t e = 0; e < rowptr[n]; ++e)
        if (colidx[e] < 0 || colidx[e] >= n) return 2;
    return 0;
}

static int64_t max_degree(int64_t n, const int64_t* rowptr)
{
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i)
        if (rowptr[i + 1] - rowptr[i] > m) m = rowptr[i + 1] - rowptr[i];
    return m;
}

/* ------------------------------------------------------------------------ */
/* scores                                                                     */
/* ------------------------------------------------------------------------ */

/* Graph Transformer score of edge j -> i, head h. */
static double gt_score(const void* Q, const void* K, int dt, int64_t i, int64_t j,
                       int H, int D, int h)
{
    double s = 0.0;
    for (int d = 0; d < D; ++d)
        s += ld(Q, dt, (i * H + h) * D + d) * ld(K, dt, (j * H + h) * D + d);
    return s / sqrt((double)D);
}

static double lrelu(double z, double slope) { return z > 0.0 ? z : slope * z; }
static double lrelu_grad(double z, double slope) { return z > 0.0 ? 1.0 : slope; }

/* GATv2 score of edge j -> i, head h. */
static double gat_score(const void* Xs, const void* Xt, const double* a, int dt,
                        int64_t i, int64_t j, int H, int D, int h, double slope)
{
    double s = 0.0;
    for (int d = 0; d < D; ++d) {
        double z = ld(Xs, dt, (i * H + h) * D + d) + ld(Xt, dt, (j * H + h) * D + d);
        s += a[h * D + d] * lrelu(z, slope);
    }
    return s;
}

/* Softmax of scores s[0..deg) in place: returns lse, leaves alpha in s. */
static double softmax_inplace(double* s, int64_t deg)
{
    double m = -INFINITY;
    for (int64_t t = 0; t < deg; ++t) if (s[t] > m) m = s[t];
    double l = 0.0;
    for (int64_t t = 0; t < deg; ++t) l += exp(s[t] - m);
    for (int64_t t = 0; t < deg; ++t) s[t] = exp(s[t] - m) / l;
    return m + log(l);
}

/* ------------------------------------------------------------------------ */
/* forward                                                                    */
/* ------------------------------------------------------------------------ */

/* op 0: Graph Transformer (A=Q, B=K, C=V). op 1: GATv2 (A=Xs, B=Xt, C=Xt). */
static int attn_fwd(int op, int64_t n, const int64_t* rowptr, const int32_t* colidx,
                    int H, int D, int dt, const void* A, const void* B, const void* C,
                    const double* a, double slope,
                    int64_t nsel, const int64_t* sel, double* out, double* lse)
{
    int rc = check_csr(n, rowptr, colidx);
    if (rc) return rc;
    int64_t cnt = sel ? nsel : n;
    int64_t maxd = max_degree(n, rowptr);
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(maxd > 0 ? maxd : 1));
        if (!s) {
#pragma omp atomic write
            bad = 3;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < cnt; ++r) {
            if (!s) continue;
            int64_t i = sel ? sel[r] : r;
            int64_t b = rowptr[i], deg = rowptr[i + 1] - rowptr[i];
            for (int h = 0; h < H; ++h) {
                double* o = out + (r * H + h) * D;
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                if (deg == 0) { lse[r * H + h] = -INFINITY; continue; }
                for (int64_t t = 0; t < deg; ++t) {
                    int64_t j = colidx[b + t];
                    s[t] = op == 0 ? gt_score(A, B, dt, i, j, H, D, h)
                                   : gat_score(A, B, a, dt, i, j, H, D, h, slope);
                }
                lse[r * H + h] = softmax_inplace(s, deg);
                for (int64_t t = 0; t < deg; ++t) {
                    int64_t j = colidx[b + t];
                    for (int d = 0; d < D; ++d)
                        o[d] += s[t] * ld(C, dt, (j * H + h) * D + d);
                }
            }
        }
        free(s);
    }
    return bad;
}

int oracle_gt_fwd(int64_t n, const int64_t* rowptr, const int32_t* colidx, int H, int D,
                  int dtype, const void* Q, const void* K, const void* V,
                  int64_t nsel, const int64_t* sel, double* out, double* lse)
{
    return attn_fwd(0, n, rowptr, colidx, H, D, dtype, Q, K, V, NULL, 0.0, nsel, sel, out, lse);
}

int oracle_gat_fwd(int64_t n, const int64_t* rowptr, const int32_t* colidx, int H, int D,
                   int dtype, const void* Xs, const void* Xt, const double* a, double slope,
                   int64_t nsel, const int64_t* sel, double* out, double* lse)
{
    return attn_fwd(1, n, rowptr, colidx, H, D, dtype, Xs, Xt, Xt, a, slope, nsel, sel, out, lse);
}

/* ------------------------------------------------------------------------ */
/* backward                                                                   */
/* ------------------------------------------------------------------------ */

/*
 * Pass 1, over destination rows: for every edge e of row i and head h,
 *   alpha[e,h] and dS[e,h] = alpha (dP - sum_row alpha dP), with
 *   dP = dout[i,h] . V[j,h] (GT) or dout[i,h] . Xt[j,h] (GATv2).
 * Edge arrays are [E, H], fp64.
 */
static int edge_pass(int op, int64_t n, const int64_t* rowptr, const int32_t* colidx,
                     int H, int D, int dt, const void* A, const void* B, const void* C,
                     const double* a, double slope, const void* dout,
                     double* alpha, double* dS)
{
    int64_t maxd = max_degree(n, rowptr);
    int bad = 0;
#pragma omp parallel
    {
        double* dp = (double*)malloc(sizeof(double) * (size_t)(maxd > 0 ? maxd : 1));
        if (!dp) {
#pragma omp atomic write
            bad = 3;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < n; ++i) {
            if (!dp) continue;
            int64_t b = rowptr[i], deg = rowptr[i + 1] - rowptr[i];
            if (deg == 0) continue;
            for (int h = 0; h < H; ++h) {
                double s_max = -INFINITY;
                for (int64_t t = 0; t < deg; ++t) {
                    int64_t j = colidx[b + t];
                    double s = op == 0 ? gt_score(A, B, dt, i, j, H, D, h)
                                       : gat_score(A, B, a, dt, i, j, H, D, h, slope);
                    alpha[(b + t) * H + h] = s;
                    if (s > s_max) s_max = s;
                }
                double l = 0.0;
                for (int64_t t = 0; t < deg; ++t) l += exp(alpha[(b + t) * H + h] - s_max);
                double c = 0.0;
                for (int64_t t = 0; t < deg; ++t) {
                    int64_t j = colidx[b + t];
                    double al = exp(alpha[(b + t) * H + h] - s_max) / l;
                    alpha[(b + t) * H + h] = al;
                    double p = 0.0;
                    for (int d = 0; d < D; ++d)
                        p += ld(dout, dt, (i * H + h) * D + d) * ld(C, dt, (j * H + h) * D + d);
                    dp[t] = p;
                    c += al * p;
                }
                for (int64_t t = 0; t < deg; ++t)
                    dS[(b + t) * H + h] = alpha[(b + t) * H + h] * (dp[t] - c);
            }
        }
        free(dp);
    }
    return bad;
}

/* Edge ids grouped by source (stable counting sort), and the row of each edge. */
static int build_csc(int64_t n, const int64_t* rowptr, const int32_t* colidx,
                     int64_t** colptr_out, int64_t** eid_out, int64_t** erow_out)
{
    int64_t E = rowptr[n];
    int64_t* colptr = (int64_t*)calloc((size_t)n + 1, sizeof(int64_t));
    int64_t* eid = (int64_t*)malloc(sizeof(int64_t) * (size_t)(E > 0 ? E : 1));
    int64_t* erow = (int64_t*)malloc(sizeof(int64_t) * (size_t)(E > 0 ? E : 1));
    int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    if (!colptr || !eid || !erow || !fill) {
        free(colptr); free(eid); free(erow); free(fill);
        return 3;
    }
    for (int64_t e = 0; e < E; ++e) colptr[colidx[e] + 1]++;
    for (int64_t j = 0; j < n; ++j) colptr[j + 1] += colptr[j];
    for (int64_t j = 0; j < n; ++j) fill[j] = colptr[j];
    for (int64_t i = 0; i < n; ++i)
        for (int64_t e = rowptr[i]; e < rowptr[i + 1]; ++e) {
            erow[e] = i;
            eid[fill[colidx[e]]++] = e;
        }
    free(fill);
    *colptr_out = colptr; *eid_out = eid; *erow_out = erow;
    return 0;
}

int oracle_gt_bwd(int64_t n, const int64_t* rowptr, const int32_t* colidx, int H, int D,
                  int dtype, const void* Q, const void* K, const void* V, const void* dout,
                  int64_t nsel_dst, const int64_t* sel_dst, double* dQ,
                  int64_t nsel_src, const int64_t* sel_src, double* dK, double* dV)
{
    int rc = check_csr(n, rowptr, colidx);
    if (rc) return rc;
    int64_t E = rowptr[n];
    size_t eh = (size_t)(E > 0 ? E : 1) * (size_t)H;
    double* alpha = (double*)malloc(sizeof(double) * eh);
    double* dS = (double*)malloc(sizeof(double) * eh);
    if (!alpha || !dS) { free(alpha); free(dS); return 3; }
    rc = edge_pass(0, n, rowptr, colidx, H, D, dtype, Q, K, V, NULL, 0.0, dout, alpha, dS);
    if (rc) { free(alpha); free(dS); return rc; }
    const double inv = 1.0 / sqrt((double)D);

    /* dQ[i,h] = sum over the edges e = (j -> i) of row i of dS[e,h] K[j,h] / sqrt(D) */
    int64_t cd = sel_dst ? nsel_dst : n;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < cd; ++r) {
        int64_t i = sel_dst ? sel_dst[r] : r;
        for (int h = 0; h < H; ++h) {
            double* g = dQ + (r * H + h) * D;
            for (int d = 0; d < D; ++d) g[d] = 0.0;
            for (int64_t e = rowptr[i]; e < rowptr[i + 1]; ++e) {
                int64_t j = colidx[e];
                for (int d = 0; d < D; ++d)
                    g[d] += dS[e * H + h] * ld(K, dtype, (j * H + h) * D + d) * inv;
            }
        }
    }

    /* dK[j,h] = sum over edges e = (j -> i) of dS[e,h] Q[i,h] / sqrt(D);
       dV[j,h] = sum over the same edges of alpha[e,h] dout[i,h]. */
    int64_t *colptr, *eid, *erow;
    rc = build_csc(n, rowptr, colidx, &colptr, &eid, &erow);
    if (rc) { free(alpha); free(dS); return rc; }
    int64_t cs = sel_src ? nsel_src : n;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < cs; ++r) {
        int64_t j = sel_src ? sel_src[r] : r;
        for (int h = 0; h < H; ++h) {
            double* gk = dK + (r * H + h) * D;
            double* gv = dV + (r * H + h) * D;
            for (int d = 0; d < D; ++d) { gk[d] = 0.0; gv[d] = 0.0; }
            for (int64_t t = colptr[j]; t < colptr[j + 1]; ++t) {
                int64_t e = eid[t], i = erow[e];
                for (int d = 0; d < D; ++d) {
                    gk[d] += dS[e * H + h] * ld(Q, dtype, (i * H + h) * D + d) * inv;
                    gv[d] += alpha[e * H + h] * ld(dout, dtype, (i * H + h) * D + d);
                }
            }
        }
    }
    free(colptr); free(eid); free(erow); free(alpha); free(dS);
    return 0;
}

int oracle_gat_bwd(int64_t n, const int64_t* rowptr, const int32_t* colidx, int H, int D,
                   int dtype, const void* Xs, const void* Xt, const double* a, double slope,
                   const void* dout,
                   int64_t nsel_dst, const int64_t* sel_dst, double* dXs,
                   int64_t nsel_src, const int64_t* sel_src, double* dXt, double* da)
{
    int rc = check_csr(n, rowptr, colidx);
    if (rc) return rc;
    int64_t E = rowptr[n];
    size_t eh = (size_t)(E > 0 ? E : 1) * (size_t)H;
    double* alpha = (double*)malloc(sizeof(double) * eh);
    double* dE = (double*)malloc(sizeof(double) * eh);
    if (!alpha || !dE) { free(alpha); free(dE); return 3; }
    rc = edge_pass(1, n, rowptr, colidx, H, D, dtype, Xs, Xt, Xt, a, slope, dout, alpha, dE);
    if (rc) { free(alpha); free(dE); return rc; }

    /* dXs[i,h,d] = sum over row i of dE[e,h] a[h,d] LReLU'(z_e,d),
       z_e = Xs[i] + Xt[j]. */
    int64_t cd = sel_dst ? nsel_dst : n;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < cd; ++r) {
        int64_t i = sel_dst ? sel_dst[r] : r;
        for (int h = 0; h < H; ++h) {
            double* g = dXs + (r * H + h) * D;
            for (int d = 0; d < D; ++d) g[d] = 0.0;
            for (int64_t e = rowptr[i]; e < rowptr[i + 1]; ++e) {
                int64_t j = colidx[e];
                for (int d = 0; d < D; ++d) {
                    double z = ld(Xs, dtype, (i * H + h) * D + d) + ld(Xt, dtype, (j * H + h) * D + d);
                    g[d] += dE[e * H + h] * a[h * D + d] * lrelu_grad(z, slope);
                }
            }
        }
    }

    /* da[h,d] = sum over all edges of dE[e,h] LReLU(z_e,d); fixed row blocks. */
    const int64_t BLK = 1024;
    int64_t nblk = (n + BLK - 1) / BLK;
    int HD = H * D;
    double* part = (double*)calloc((size_t)(nblk > 0 ? nblk : 1) * (size_t)HD, sizeof(double));
    if (!part) { free(alpha); free(dE); return 3; }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bk = 0; bk < nblk; ++bk) {
        double* p = part + bk * HD;
        int64_t i1 = (bk + 1) * BLK < n ? (bk + 1) * BLK : n;
        for (int64_t i = bk * BLK; i < i1; ++i)
            for (int64_t e = rowptr[i]; e < rowptr[i + 1]; ++e) {
                int64_t j = colidx[e];
                for (int h = 0; h < H; ++h)
                    for (int d = 0; d < D; ++d) {
                        double z = ld(Xs, dtype, (i * H + h) * D + d) + ld(Xt, dtype, (j * H + h) * D + d);
                        p[h * D + d] += dE[e * H + h] * lrelu(z, slope);
                    }
            }
    }
    for (int k = 0; k < HD; ++k) da[k] = 0.0;
    for (int64_t bk = 0; bk < nblk; ++bk)
        for (int k = 0; k < HD; ++k) da[k] += part[bk * HD + k];
    free(part);

    /* dXt[j,h,d] = sum over edges e = (j -> i) of
       dE[e,h] a[h,d] LReLU'(z_e,d) + alpha[e,h] dout[i,h,d]. */
    int64_t *colptr, *eid, *erow;
    rc = build_csc(n, rowptr, colidx, &colptr, &eid, &erow);
    if (rc) { free(alpha); free(dE); return rc; }
    int64_t cs = sel_src ? nsel_src : n;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < cs; ++r) {
        int64_t j = sel_src ? sel_src[r] : r;
        for (int h = 0; h < H; ++h) {
            double* g = dXt + (r * H + h) * D;
            for (int d = 0; d < D; ++d) g[d] = 0.0;
            for (int64_t t = colptr[j]; t < colptr[j + 1]; ++t) {
                int64_t e = eid[t], i = erow[e];
                for (int d = 0; d < D; ++d) {
                    double z = ld(Xs, dtype, (i * H + h) * D + d) + ld(Xt, dtype, (j * H + h) * D + d);
                    g[d] += dE[e * H + h] * a[h * D + d] * lrelu_grad(z, slope)
                          + alpha[e * H + h] * ld(dout, dtype, (i * H + h) * D + d);
                }
            }
        }
    }
    free(colptr); free(eid); free(erow); free(alpha); free(dE);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* reduction aggregation: min / max pooling over the in-neighbours            */
/* ------------------------------------------------------------------------ */

/*
 * The reduction-based aggregation family (IO-aware layers abstract; Yandex
 * Research blog, paragraph on aggregation layers: min/max pooling). Readings:
 * the message of edge j -> i is the source row X[j] (F features); for every
 * destination i and feature f the result is the extreme value over the row's
 * edges; the winning edge is the first one in CSR order whose value is
 * strictly below (min) or above (max) every earlier value of the row, so ties
 * go to the lowest position; an empty row gives 0 and no winner (arg -1).
 * op 0 = min, op 1 = max.
 */
int oracle_reduce_fwd(int64_t n, const int64_t* rowptr, const int32_t* colidx, int F, int dtype,
                      int op, const void* X, int64_t nsel, const int64_t* sel, double* out,
                      int64_t* arg)
{
    int rc = check_csr(n, rowptr, colidx);
    if (rc) return rc;
    if (F < 1 || (op != 0 && op != 1)) return 1;
    int64_t cnt = sel ? nsel : n;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < cnt; ++r) {
        int64_t i = sel ? sel[r] : r;
        double* v = out + r * F;
        int64_t* w = arg + r * F;
        for (int f = 0; f < F; ++f) { v[f] = 0.0; w[f] = -1; }
        for (int64_t e = rowptr[i]; e < rowptr[i + 1]; ++e) {
            int64_t j = colidx[e];
            for (int f = 0; f < F; ++f) {
                double x = ld(X, dtype, j * F + f);
                int better = op == 0 ? x < v[f] : x > v[f];
                if (w[f] < 0 || better) { v[f] = x; w[f] = e; }
            }
        }
    }
    return 0;
}

/*
 * Backward of L = sum(out * dout). out[i,f] = X[colidx[arg[i,f]], f], so each
 * (i, f) with a winner passes dout[i,f] to feature f of the winning edge's
 * source: dX[j,f] = sum of dout[i,f] over those (i, f). `arg` is the
 * forward's winner array over all n rows; an entry that is neither -1 nor an
 * edge of its own row is rejected (return 1).
 */
int oracle_reduce_bwd(int64_t n, const int64_t* rowptr, const int32_t* colidx, int F, int dtype,
                      const int64_t* arg, const void* dout, double* dX)
{
    int rc = check_csr(n, rowptr, colidx);
    if (rc) return rc;
    if (F < 1) return 1;
    for (int64_t k = 0; k < n * F; ++k) dX[k] = 0.0;
    /* Threads own disjoint feature blocks; each sums its entries in row order. */
    const int FB = 16;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int f0 = 0; f0 < F; f0 += FB) {
        int f1 = f0 + FB < F ? f0 + FB : F;
        for (int64_t i = 0; i < n; ++i)
            for (int f = f0; f < f1; ++f) {
                int64_t e = arg[i * F + f];
                if (e < 0) continue;
                if (e < rowptr[i] || e >= rowptr[i + 1]) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                dX[(int64_t)colidx[e] * F + f] += ld(dout, dtype, i * F + f);
            }
    }
    return bad;
}
