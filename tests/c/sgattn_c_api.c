/*
 * A plain C99 consumer of the library's C ABI (include/sgattn.h): no C++, no
 * torch. Test code.
 *
 *   sgattn_c_api        host-only calls: plan creation, statistics, array
 *                       export, workspace sizes, argument errors
 *   sgattn_c_api gpu    also runs, on device memory from hipMalloc, the Graph
 *                       Transformer forward and backward and the min/max
 *                       aggregation, and compares them with the fp64 oracle
 *                       (oracle/oracle.c, linked into this test program)
 *
 * Exit status 0 when every check passes; each failure prints one line.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sgattn.h"

/* the oracle's entry points (oracle/oracle.c) */
int oracle_gt_fwd(int64_t n, const int64_t* rowptr, const int32_t* colidx, int H, int D,
                  int dtype, const void* Q, const void* K, const void* V, int64_t nsel,
                  const int64_t* sel, double* out, double* lse);
int oracle_gt_bwd(int64_t n, const int64_t* rowptr, const int32_t* colidx, int H, int D,
                  int dtype, const void* Q, const void* K, const void* V, const void* dout,
                  int64_t nsel_dst, const int64_t* sel_dst, double* dQ, int64_t nsel_src,
                  const int64_t* sel_src, double* dK, double* dV);
int oracle_reduce_fwd(int64_t n, const int64_t* rowptr, const int32_t* colidx, int F, int dtype,
                      int op, const void* X, int64_t nsel, const int64_t* sel, double* out,
                      int64_t* arg);
int oracle_reduce_bwd(int64_t n, const int64_t* rowptr, const int32_t* colidx, int F, int dtype,
                      const int64_t* arg, const void* dout, double* dX);

static int failures = 0;

#define CHECK(cond, ...)                                                \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);        \
            fprintf(stderr, __VA_ARGS__);                               \
            fprintf(stderr, "\n");                                      \
            ++failures;                                                 \
        }                                                               \
    } while (0)

/* 64-bit LCG (Knuth's MMIX constants), the upper bits as the draw */
static uint64_t lcg_state = 12345;
static uint32_t lcg(void)
{
    lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(lcg_state >> 32);
}
static float unif(void) { return (float)lcg() / 4294967296.0f * 2.0f - 1.0f; }

/* A CSR by destination: degrees 0..20, rows 3 and 11 with 700 in-edges */
static void make_graph(int64_t n, int64_t** rowptr, int32_t** colidx)
{
    int64_t* rp = malloc(sizeof(int64_t) * (size_t)(n + 1));
    rp[0] = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t deg = (i == 3 || i == 11) ? 700 : (int64_t)(lcg() % 21);
        rp[i + 1] = rp[i] + deg;
    }
    int32_t* ci = malloc(sizeof(int32_t) * (size_t)(rp[n] > 0 ? rp[n] : 1));
    for (int64_t e = 0; e < rp[n]; ++e) ci[e] = (int32_t)(lcg() % (uint32_t)n);
    *rowptr = rp;
    *colidx = ci;
}

static double max_rel(const float* got, const double* ref, size_t count)
{
    double scale = 0.0, err = 0.0;
    for (size_t k = 0; k < count; ++k) {
        if (fabs(ref[k]) > scale) scale = fabs(ref[k]);
        if (fabs((double)got[k] - ref[k]) > err) err = fabs((double)got[k] - ref[k]);
    }
    return scale > 0.0 ? err / scale : err;
}

static void host_checks(void)
{
    const int64_t n = 300;
    int64_t* rp;
    int32_t* ci;
    make_graph(n, &rp, &ci);
    const int64_t nnz = rp[n];

    sgat_plan_opts opts;
    memset(&opts, 0, sizeof opts);
    opts.chunk = 64;
    sgat_plan* plan = NULL;
    CHECK(sgat_plan_create(n, nnz, rp, ci, &opts, &plan) == SGAT_OK && plan, "plan_create");

    sgat_plan_stats st;
    CHECK(sgat_plan_stats_get(plan, &st) == SGAT_OK, "stats");
    CHECK(st.n == n && st.nnz == nnz && st.chunk == 64, "stats fields");
    CHECK(st.max_in_degree == 700, "max in-degree %lld", (long long)st.max_in_degree);
    CHECK(st.row_splits == 2 && st.row_slots == 2 * 11, "two rows of 700 split into 11 chunks");

    /* the exported work list covers every edge exactly once */
    size_t bytes = 0;
    CHECK(sgat_plan_array_bytes(plan, SGAT_ARR_ROW_ITEMS, &bytes) == SGAT_OK, "array bytes");
    CHECK(bytes == (size_t)st.row_items * sizeof(sgat_work_item), "work list size");
    sgat_work_item* items = malloc(bytes);
    CHECK(sgat_plan_export(plan, SGAT_ARR_ROW_ITEMS, items, bytes) == SGAT_OK, "export");
    int64_t covered = 0;
    for (int64_t k = 0; k < st.row_items; ++k) covered += items[k].len;
    CHECK(covered == nnz, "work list covers %lld of %lld edges", (long long)covered,
          (long long)nnz);
    free(items);

    size_t ws = 0;
    for (int op = SGAT_OP_GT_FWD; op <= SGAT_OP_GAT_BWD; ++op)
        CHECK(sgat_workspace_bytes(plan, op, 4, 32, SGAT_F32, &ws) == SGAT_OK && ws % 256 == 0,
              "workspace op %d", op);
    CHECK(sgat_workspace_bytes(plan, SGAT_OP_REDUCE_FWD, 1, 512, SGAT_BF16, &ws) == SGAT_OK,
          "reduce workspace");
    CHECK(sgat_workspace_bytes(plan, SGAT_OP_GT_FWD, 4, 48, SGAT_F32, &ws) ==
              SGAT_INVALID_ARGUMENT, "D = 48 rejected");

    /* argument errors are reported before any HIP call */
    CHECK(gt_fwd(plan, n, nnz, rp, ci, 4, 32, SGAT_F32, rp, rp, rp, rp, (float*)rp, rp, 1 << 20,
                 0, NULL) == SGAT_NOT_UPLOADED, "not uploaded");
    CHECK(gt_fwd(plan, n + 1, nnz, rp, ci, 4, 32, SGAT_F32, rp, rp, rp, rp, (float*)rp, rp,
                 1 << 20, 0, NULL) == SGAT_PLAN_MISMATCH, "n mismatch");
    CHECK(reduce_fwd(NULL, n, nnz, rp, ci, 64, SGAT_F32, SGAT_REDUCE_MIN, rp, rp, NULL, rp, 0,
                     NULL) == SGAT_INVALID_ARGUMENT, "null plan");

    /* invalid CSR: a source outside [0, n) */
    int32_t saved = ci[5];
    ci[5] = (int32_t)n;
    sgat_plan* bad = NULL;
    CHECK(sgat_plan_create(n, nnz, rp, ci, NULL, &bad) == SGAT_INVALID_CSR && !bad,
          "invalid CSR rejected");
    ci[5] = saved;
    CHECK(strcmp(sgat_status_string(SGAT_INVALID_CSR), "invalid CSR") == 0, "status string");

    sgat_plan_destroy(plan);
    sgat_plan_destroy(NULL);
    free(rp);
    free(ci);
}

#define HIP_OK(call) CHECK((call) == hipSuccess, #call)

/* device buffer of `bytes`, filled from `host` unless it is NULL */
static void* dev_copy(const void* host, size_t bytes)
{
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes > 0 ? bytes : 16));
    if (host && bytes > 0) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static void gpu_checks(void)
{
    const int64_t n = 300;
    const int H = 4, D = 32, F = 64;
    int64_t* rp;
    int32_t* ci;
    make_graph(n, &rp, &ci);
    const int64_t nnz = rp[n];
    const size_t ne = (size_t)n * H * D, fb = sizeof(float);

    sgat_plan_opts opts;
    memset(&opts, 0, sizeof opts);
    opts.chunk = 64;
    sgat_plan* plan = NULL;
    CHECK(sgat_plan_create(n, nnz, rp, ci, &opts, &plan) == SGAT_OK, "plan_create");
    size_t pb = 0;
    CHECK(sgat_plan_device_bytes(plan, &pb) == SGAT_OK, "device bytes");
    void* dplan = NULL;
    HIP_OK(hipMalloc(&dplan, pb));
    CHECK(sgat_plan_upload(plan, dplan, pb, NULL) == SGAT_OK, "upload");

    float *q = malloc(ne * fb), *k = malloc(ne * fb), *v = malloc(ne * fb), *g = malloc(ne * fb);
    for (size_t t = 0; t < ne; ++t) {
        q[t] = unif();
        k[t] = unif();
        v[t] = unif();
        g[t] = unif();
    }
    void *drp = dev_copy(rp, sizeof(int64_t) * (size_t)(n + 1)),
         *dci = dev_copy(ci, sizeof(int32_t) * (size_t)nnz);
    void *dq = dev_copy(q, ne * fb), *dk = dev_copy(k, ne * fb), *dv = dev_copy(v, ne * fb),
         *dg = dev_copy(g, ne * fb);
    void *dout = dev_copy(NULL, ne * fb), *dlse = dev_copy(NULL, (size_t)n * H * fb);
    void *ddq = dev_copy(NULL, ne * fb), *ddk = dev_copy(NULL, ne * fb),
         *ddv = dev_copy(NULL, ne * fb);
    size_t wf = 0, wb = 0;
    CHECK(sgat_workspace_bytes(plan, SGAT_OP_GT_FWD, H, D, SGAT_F32, &wf) == SGAT_OK, "ws fwd");
    CHECK(sgat_workspace_bytes(plan, SGAT_OP_GT_BWD, H, D, SGAT_F32, &wb) == SGAT_OK, "ws bwd");
    void *wsf = dev_copy(NULL, wf), *wsb = dev_copy(NULL, wb);

    CHECK(gt_fwd(plan, n, nnz, drp, dci, H, D, SGAT_F32, dq, dk, dv, dout, dlse, wsf, wf - 256, 0,
                 NULL) == (wf >= 256 ? SGAT_WORKSPACE_TOO_SMALL : SGAT_OK), "workspace too small");
    CHECK(gt_fwd(plan, n, nnz, drp, dci, H, D, SGAT_F32, dq, dk, dv, dout, dlse, wsf, wf, 0,
                 NULL) == SGAT_OK, "gt_fwd");
    CHECK(gt_bwd(plan, n, nnz, drp, dci, H, D, SGAT_F32, dq, dk, dv, dout, dlse, dg, ddq, ddk, ddv,
                 wsb, wb, 0, NULL) == SGAT_OK, "gt_bwd");
    HIP_OK(hipDeviceSynchronize());

    float *out = malloc(ne * fb), *lse = malloc((size_t)n * H * fb);
    float *gq = malloc(ne * fb), *gk = malloc(ne * fb), *gv = malloc(ne * fb);
    HIP_OK(hipMemcpy(out, dout, ne * fb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse, dlse, (size_t)n * H * fb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gq, ddq, ne * fb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gk, ddk, ne * fb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gv, ddv, ne * fb, hipMemcpyDeviceToHost));

    double *ro = malloc(ne * sizeof(double)), *rl = malloc((size_t)n * H * sizeof(double));
    double *rq = malloc(ne * sizeof(double)), *rk = malloc(ne * sizeof(double)),
           *rv = malloc(ne * sizeof(double));
    CHECK(oracle_gt_fwd(n, rp, ci, H, D, 0, q, k, v, 0, NULL, ro, rl) == 0, "oracle fwd");
    CHECK(oracle_gt_bwd(n, rp, ci, H, D, 0, q, k, v, g, 0, NULL, rq, 0, NULL, rk, rv) == 0,
          "oracle bwd");
    CHECK(max_rel(out, ro, ne) <= 1e-4, "out rel err %.3g", max_rel(out, ro, ne));
    int lse_ok = 1;
    for (int64_t t = 0; t < n * H; ++t) {
        if (isinf(rl[t])) lse_ok &= isinf(lse[t]) && lse[t] < 0;
        else lse_ok &= fabs(lse[t] - rl[t]) <= 1e-4 * (1.0 + fabs(rl[t]));
    }
    CHECK(lse_ok, "lse");
    CHECK(max_rel(gq, rq, ne) <= 1e-4, "dQ rel err %.3g", max_rel(gq, rq, ne));
    CHECK(max_rel(gk, rk, ne) <= 1e-4, "dK rel err %.3g", max_rel(gk, rk, ne));
    CHECK(max_rel(gv, rv, ne) <= 1e-4, "dV rel err %.3g", max_rel(gv, rv, ne));

    /* min aggregation, F = 64 fp32: values and winners exact */
    const size_t nf = (size_t)n * F;
    float* x = malloc(nf * fb);
    for (size_t t = 0; t < nf; ++t) x[t] = (float)(lcg() % 9) * 0.25f - 1.0f;   /* many ties */
    void *dx = dev_copy(x, nf * fb), *dro = dev_copy(NULL, nf * fb),
         *darg = dev_copy(NULL, nf * sizeof(int32_t)), *ddx = dev_copy(NULL, nf * fb),
         *dgo = dev_copy(g, nf * fb);
    size_t rf = 0, rb = 0;
    CHECK(sgat_workspace_bytes(plan, SGAT_OP_REDUCE_FWD, 1, F, SGAT_F32, &rf) == SGAT_OK, "ws");
    CHECK(sgat_workspace_bytes(plan, SGAT_OP_REDUCE_BWD, 1, F, SGAT_F32, &rb) == SGAT_OK, "ws");
    void *wrf = dev_copy(NULL, rf), *wrb = dev_copy(NULL, rb);
    CHECK(reduce_fwd(plan, n, nnz, drp, dci, F, SGAT_F32, SGAT_REDUCE_MIN, dx, dro, darg, wrf, rf,
                     NULL) == SGAT_OK, "reduce_fwd");
    CHECK(reduce_bwd(plan, n, nnz, drp, dci, F, SGAT_F32, darg, dgo, ddx, wrb, rb, NULL) ==
              SGAT_OK, "reduce_bwd");
    HIP_OK(hipDeviceSynchronize());
    float *mo = malloc(nf * fb), *mdx = malloc(nf * fb);
    int32_t* ma = malloc(nf * sizeof(int32_t));
    HIP_OK(hipMemcpy(mo, dro, nf * fb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ma, darg, nf * sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(mdx, ddx, nf * fb, hipMemcpyDeviceToHost));
    double *xo = malloc(nf * sizeof(double)), *xdx = malloc(nf * sizeof(double));
    int64_t* xa = malloc(nf * sizeof(int64_t));
    CHECK(oracle_reduce_fwd(n, rp, ci, F, 0, 0, x, 0, NULL, xo, xa) == 0, "oracle reduce");
    CHECK(oracle_reduce_bwd(n, rp, ci, F, 0, xa, g, xdx) == 0, "oracle reduce bwd");
    int exact = 1;
    for (size_t t = 0; t < nf; ++t) exact &= (double)mo[t] == xo[t] && (int64_t)ma[t] == xa[t];
    CHECK(exact, "min aggregation values and winners");
    CHECK(max_rel(mdx, xdx, nf) <= 1e-6, "dX rel err %.3g", max_rel(mdx, xdx, nf));

    void* bufs[] = {dplan, drp, dci, dq, dk, dv, dg, dout, dlse, ddq, ddk, ddv, wsf, wsb,
                    dx, dro, darg, ddx, dgo, wrf, wrb};
    for (size_t t = 0; t < sizeof bufs / sizeof bufs[0]; ++t) HIP_OK(hipFree(bufs[t]));
    free(q); free(k); free(v); free(g); free(out); free(lse); free(gq); free(gk); free(gv);
    free(ro); free(rl); free(rq); free(rk); free(rv); free(x); free(mo); free(mdx); free(ma);
    free(xo); free(xdx); free(xa);
    sgat_plan_destroy(plan);
    free(rp);
    free(ci);
}

int main(int argc, char** argv)
{
    host_checks();
    if (argc > 1 && strcmp(argv[1], "gpu") == 0) {
        int count = 0;
        CHECK(hipGetDeviceCount(&count) == hipSuccess && count > 0, "no GPU");
        if (count > 0) {
            HIP_OK(hipSetDevice(0));
            gpu_checks();
        }
    }
    printf("%s: %d failure(s)\n", argc > 1 ? argv[1] : "host", failures);
    return failures == 0 ? 0 : 1;
}
