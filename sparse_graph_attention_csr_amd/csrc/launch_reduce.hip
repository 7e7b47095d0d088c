// Min/max reduction aggregation launchers: forward rows (+ merge of split
// rows); backward: route the contributions by winning edge on the CSR side,
// gather them over the transposed CSR (+ fixed-order sum of split sources).
#include "launch.hpp"
#include "reduce.hpp"

namespace sgat {

#ifndef SGAT_UNROLL_REDUCE_FWD
#define SGAT_UNROLL_REDUCE_FWD 8
#endif
#ifndef SGAT_UNROLL_REDUCE_BWD
#define SGAT_UNROLL_REDUCE_BWD 4
#endif

namespace {
// Rows in flight per wave: fewer when a lane holds several fragments of a row
// or when many edges already sit side by side in the wave.
constexpr int unroll_rf(int lpe, int nf)
{
    const int u = lpe <= 16 ? 2 : SGAT_UNROLL_REDUCE_FWD;
    return u / nf > 0 ? u / nf : 1;
}
}  // namespace

// Every (dtype, lanes per edge, fragments per lane) compiled.
#define SGAT_REDUCE_CONFIGS(X)                                                             \
    X(SGAT_BF16, 1, 1) X(SGAT_BF16, 2, 1) X(SGAT_BF16, 4, 1) X(SGAT_BF16, 8, 1)            \
    X(SGAT_BF16, 16, 1) X(SGAT_BF16, 32, 1) X(SGAT_BF16, 64, 1) X(SGAT_BF16, 64, 2)        \
    X(SGAT_BF16, 64, 3) X(SGAT_BF16, 64, 4)                                                \
    X(SGAT_F32, 1, 1) X(SGAT_F32, 2, 1) X(SGAT_F32, 4, 1) X(SGAT_F32, 8, 1)                \
    X(SGAT_F32, 16, 1) X(SGAT_F32, 32, 1) X(SGAT_F32, 64, 1) X(SGAT_F32, 64, 2)            \
    X(SGAT_F32, 64, 3) X(SGAT_F32, 64, 4) X(SGAT_F32, 64, 5) X(SGAT_F32, 64, 6)            \
    X(SGAT_F32, 64, 7) X(SGAT_F32, 64, 8)

ReduceGeom reduce_geometry(int dt, int F)
{
    const int vec = dt == SGAT_F32 ? 4 : 8;
    const int frags = F / vec;
    int lpe = 1;
    while (lpe < frags && lpe < kWave) lpe <<= 1;
    return {lpe, (frags + kWave - 1) / kWave};
}

bool reduce_supported(int dt, int F)
{
    if (dt != SGAT_F32 && dt != SGAT_BF16) return false;
    const int vec = dt == SGAT_F32 ? 4 : 8;
    return F >= vec && F <= kReduceMaxF && F % vec == 0;
}

int launch_reduce_fwd(const Plan& p, int F, int dt, int op, const int32_t* colidx, const void* X,
                      void* out, int32_t* arg, float* part_val, int32_t* part_pos, hipStream_t s)
{
    const ReduceGeom g = reduce_geometry(dt, F);
    ReduceFwdArgs a;
    a.items = p.dptr<sgat_work_item>(SGAT_ARR_ROW_ITEMS);
    a.n_items = static_cast<int64_t>(p.row_items.size());
    a.F = F;
    a.colidx = colidx;
    a.X = X;
    a.out = out;
    a.arg = arg;
    a.part_val = part_val;
    a.part_pos = part_pos;
    const void* fn = nullptr;
#define X(DT_, L_, N_)                                                                          \
    if (dt == DT_ && g.lpe == L_ && g.nf == N_)                                                 \
        fn = op == SGAT_REDUCE_MAX                                                              \
                 ? reinterpret_cast<const void*>(&reduce_fwd_rows<DT_, L_, N_, true, unroll_rf(L_, N_)>) \
                 : reinterpret_cast<const void*>(&reduce_fwd_rows<DT_, L_, N_, false, unroll_rf(L_, N_)>);
    SGAT_REDUCE_CONFIGS(X)
#undef X
    if (!fn) return SGAT_INVALID_ARGUMENT;
    int rc;
    if (a.n_items > 0 &&
        (rc = launch("reduce_fwd_rows", fn, dim3(static_cast<unsigned>(wave_grid(a.n_items))),
                     dim3(kBlock), &a, s)))
        return rc;
    if (p.row_splits.empty()) return SGAT_OK;
    ReduceMergeArgs m{p.dptr<sgat_split>(SGAT_ARR_ROW_SPLITS), F, part_val, part_pos, out, arg};
    const bool mx = op == SGAT_REDUCE_MAX;
    const void* mf = dt == SGAT_F32
        ? (mx ? reinterpret_cast<const void*>(&reduce_merge<SGAT_F32, true>)
              : reinterpret_cast<const void*>(&reduce_merge<SGAT_F32, false>))
        : (mx ? reinterpret_cast<const void*>(&reduce_merge<SGAT_BF16, true>)
              : reinterpret_cast<const void*>(&reduce_merge<SGAT_BF16, false>));
    return launch("reduce_fwd_merge", mf,
                  dim3(static_cast<unsigned>(p.row_splits.size()),
                       static_cast<unsigned>((F + kBlock - 1) / kBlock)),
                  dim3(kBlock), &m, s);
}

int launch_reduce_bwd(const Plan& p, int F, int dt, const int64_t* rowptr, const int32_t* arg,
                      const void* dO, void* dX, float* part, uint32_t* sc, void* entries,
                      hipStream_t s)
{
    const int nr = reduce_geometry(dt, F).nf;
    ReduceRouteArgs r;
    r.items = p.dptr<sgat_work_item>(SGAT_ARR_ROW_ITEMS);
    r.n_items = static_cast<int64_t>(p.row_items.size());
    r.F = F;
    r.rowptr = rowptr;
    r.arg = arg;
    r.dO = dO;
    r.sc = sc;
    r.entries = entries;
    ReduceGatherArgs g;
    g.items = p.dptr<sgat_work_item>(SGAT_ARR_COL_ITEMS);
    g.n_items = static_cast<int64_t>(p.col_items.size());
    g.F = F;
    g.rowidx = p.dptr<int32_t>(SGAT_ARR_ROWIDX);
    g.col_edge = p.dptr<int32_t>(SGAT_ARR_COL_EDGE);
    g.sc = sc;
    g.entries = entries;
    g.dX = dX;
    g.part = part;
    const void *fr = nullptr, *fg = nullptr;
#define X(DT_, N_)                                                                        \
    if (dt == DT_ && nr == N_) {                                                          \
        fr = reinterpret_cast<const void*>(&reduce_bwd_route<DT_, N_>);                   \
        fg = reinterpret_cast<const void*>(&reduce_bwd_gather<DT_, N_, SGAT_UNROLL_REDUCE_BWD>); \
    }
    X(SGAT_BF16, 1) X(SGAT_BF16, 2) X(SGAT_BF16, 3) X(SGAT_BF16, 4)
    X(SGAT_F32, 1) X(SGAT_F32, 2) X(SGAT_F32, 3) X(SGAT_F32, 4)
    X(SGAT_F32, 5) X(SGAT_F32, 6) X(SGAT_F32, 7) X(SGAT_F32, 8)
#undef X
    if (!fr || !fg) return SGAT_INVALID_ARGUMENT;
    int rc;
    if (r.n_items > 0 &&
        (rc = launch("reduce_bwd_route", fr, dim3(static_cast<unsigned>(wave_grid(r.n_items))),
                     dim3(kBlock), &r, s)))
        return rc;
    if (g.n_items > 0 &&
        (rc = launch("reduce_bwd_gather", fg, dim3(static_cast<unsigned>(wave_grid(g.n_items))),
                     dim3(kBlock), &g, s)))
        return rc;
    return merge_sum("reduce_bwd_merge", p.col_splits, p.dptr<sgat_split>(SGAT_ARR_COL_SPLITS), F,
                     part, 1.f, dX, nullptr, 0.f, nullptr, dt, s);
}

}  // namespace sgat
