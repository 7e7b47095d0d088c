// Graph Transformer launchers: forward rows (+ log-sum-exp merge of split
// rows), backward CSR pass (+ merge), backward transposed-CSR pass (+ merge).
#include "gather.hpp"
#include "launch.hpp"

namespace sgat {

// Neighbour rows each wave gathers before their first use (compile-time
// tunables; -DSGAT_UNROLL_FWD=... etc. override them).
#ifndef SGAT_UNROLL_FWD
#define SGAT_UNROLL_FWD 8
#endif
#ifndef SGAT_UNROLL_BWD
#define SGAT_UNROLL_BWD 4
#endif
#ifndef SGAT_UNROLL_ROWS
#define SGAT_UNROLL_ROWS 8
#endif

namespace {
// With several edges per wave side by side, each unrolled step already holds
// EPW neighbour rows, so fewer steps keep the same bytes in flight with fewer
// registers.
constexpr int unroll_fwd(int epw) { return epw >= 4 ? (SGAT_UNROLL_FWD + 3) / 4 : SGAT_UNROLL_FWD; }
constexpr int unroll_bwd(int epw) { return epw >= 4 ? (SGAT_UNROLL_BWD + 1) / 2 : SGAT_UNROLL_BWD; }
constexpr int unroll_rows(int epw) { return epw >= 4 ? (SGAT_UNROLL_ROWS + 1) / 2 : SGAT_UNROLL_ROWS; }
}

int launch_gt_fwd(const Plan& p, int H, int D, int dt, const int32_t* colidx, const void* Q,
                  const void* K, const void* V, void* out, float* lse, const FwdWs& ws,
                  hipStream_t s)
{
    const Decomp dc = decompose(dt, D, H);
    GtFwdArgs a;
    a.items = p.dptr<sgat_work_item>(SGAT_ARR_ROW_ITEMS);
    a.n_units = static_cast<int64_t>(p.row_items.size()) * dc.n_hg;
    a.n_hg = dc.n_hg;
    a.H = H;
    a.colidx = colidx;
    a.Q = Q; a.K = K; a.V = V;
    a.out = out;
    a.lse = lse;
    a.part_acc = ws.part_acc;
    a.part_ml = ws.part_ml;
    a.scale2 = kLog2e / sqrtf(static_cast<float>(D));
    const void* fn = nullptr;
#define X(DT_, D_, E_) \
    if (dt == DT_ && D == D_ && dc.epw == E_) fn = reinterpret_cast<const void*>(&gt_fwd_rows<DT_, D_, E_, unroll_fwd(E_)>);
    SGAT_GATHER_CONFIGS(X)
#undef X
    if (!fn) return SGAT_INVALID_ARGUMENT;
    if (a.n_units > 0) {
        int rc = launch("gt_fwd_rows", fn, dim3(static_cast<unsigned>(wave_grid(a.n_units))),
                        dim3(kBlock), &a, s);
        if (rc) return rc;
    }
    if (!p.row_splits.empty()) {
        LseMergeArgs m{p.dptr<sgat_split>(SGAT_ARR_ROW_SPLITS), H, D, ws.part_acc, ws.part_ml,
                       out, lse};
        const void* mf = dt == SGAT_F32 ? reinterpret_cast<const void*>(&lse_merge<SGAT_F32>)
                                        : reinterpret_cast<const void*>(&lse_merge<SGAT_BF16>);
        int rc = launch("gt_fwd_merge", mf,
                        dim3(static_cast<unsigned>(p.row_splits.size()),
                             static_cast<unsigned>((H * D + kBlock - 1) / kBlock)),
                        dim3(kBlock), &m, s);
        if (rc) return rc;
    }
    return SGAT_OK;
}

int merge_sum(const char* name, const std::vector<sgat_split>& sp, const sgat_split* dsp, int HD,
              const float* part0, float scale0, void* out0, const float* part1, float scale1,
              void* out1, int dt, hipStream_t s)
{
    if (sp.empty()) return SGAT_OK;
    SumMergeArgs m;
    m.splits = dsp;
    m.HD = HD;
    m.part[0] = part0; m.scale[0] = scale0; m.out[0] = out0;
    m.part[1] = part1; m.scale[1] = scale1; m.out[1] = out1;
    m.n_out = part1 ? 2 : 1;
    const void* mf = dt == SGAT_F32 ? reinterpret_cast<const void*>(&sum_merge<SGAT_F32>)
                                    : reinterpret_cast<const void*>(&sum_merge<SGAT_BF16>);
    return launch(name, mf,
                  dim3(static_cast<unsigned>(sp.size()), static_cast<unsigned>((HD + kBlock - 1) / kBlock)),
                  dim3(kBlock), &m, s);
}

int launch_gt_bwd(const Plan& p, int H, int D, int dt, const int32_t* colidx, const void* Q,
                  const void* K, const void* V, const void* O, const float* lse, const void* dO,
                  void* dQ, void* dK, void* dV, const BwdWs& ws, hipStream_t s)
{
    const Decomp dc = decompose(dt, D, H);
    const float scale2 = kLog2e / sqrtf(static_cast<float>(D));
    const float oscale = 1.f / sqrtf(static_cast<float>(D));
    const int HD = H * D;

    DeltaArgs d;
    d.n = p.n;
    d.n_units = (p.n + dc.epw - 1) / dc.epw * dc.n_hg;
    d.n_hg = dc.n_hg;
    d.H = H;
    d.O = O; d.dO = dO;
    d.lse = lse;
    d.stats = static_cast<RowStat*>(ws.stats);

    GtBwdColArgs c;
    c.items = p.dptr<sgat_work_item>(SGAT_ARR_COL_ITEMS);
    c.n_units = static_cast<int64_t>(p.col_items.size()) * dc.n_hg;
    c.n_hg = dc.n_hg;
    c.H = H;
    c.rowidx = p.dptr<int32_t>(SGAT_ARR_ROWIDX);
    c.col_edge = p.dptr<int32_t>(SGAT_ARR_COL_EDGE);
    c.Q = Q; c.K = K; c.V = V; c.dO = dO;
    c.stats = static_cast<const RowStat*>(ws.stats);
    c.dK = dK; c.dV = dV;
    c.part_k = ws.part_col0;
    c.part_v = ws.part_col1;
    c.ds = ws.ds;
    c.scale2 = scale2;
    c.oscale = oscale;

    GtBwdRowArgs r;
    r.items = p.dptr<sgat_work_item>(SGAT_ARR_ROW_ITEMS);
    r.n_units = static_cast<int64_t>(p.row_items.size()) * dc.n_hg;
    r.n_hg = dc.n_hg;
    r.H = H;
    r.colidx = colidx;
    const bool tpos = p.ds_transposed(H);
    r.tpos = tpos ? p.dptr<int32_t>(SGAT_ARR_ROW_TPOS) : nullptr;
    r.K = K;
    r.ds = ws.ds;
    r.dQ = dQ;
    r.part = ws.part_row;
    r.oscale = oscale;

    const void *fd = nullptr, *fr = nullptr, *fc = nullptr;
#define X(DT_, D_, E_)                                                                      \
    if (dt == DT_ && D == D_ && dc.epw == E_) {                                             \
        fd = reinterpret_cast<const void*>(&bwd_delta<DT_, D_, E_>);                        \
        fr = tpos ? reinterpret_cast<const void*>(&gt_bwd_rows<DT_, D_, E_, unroll_rows(E_), true>)  \
                  : reinterpret_cast<const void*>(&gt_bwd_rows<DT_, D_, E_, unroll_rows(E_), false>); \
        fc = tpos ? reinterpret_cast<const void*>(&gt_bwd_cols<DT_, D_, E_, unroll_bwd(E_), true>)   \
                  : reinterpret_cast<const void*>(&gt_bwd_cols<DT_, D_, E_, unroll_bwd(E_), false>);  \
    }
    SGAT_GATHER_CONFIGS(X)
#undef X
    if (!fd || !fr || !fc) return SGAT_INVALID_ARGUMENT;
    int rc;
    if ((rc = launch("gt_bwd_delta", fd, dim3(static_cast<unsigned>(wave_grid(d.n_units))),
                     dim3(kBlock), &d, s)))
        return rc;
    if (c.n_units > 0 &&
        (rc = launch("gt_bwd_cols", fc, dim3(static_cast<unsigned>(wave_grid(c.n_units))),
                     dim3(kBlock), &c, s)))
        return rc;
    if ((rc = merge_sum("gt_bwd_cols_merge", p.col_splits, p.dptr<sgat_split>(SGAT_ARR_COL_SPLITS),
                        HD, ws.part_col0, oscale, dK, ws.part_col1, 1.f, dV, dt, s)))
        return rc;
    if (r.n_units > 0 &&
        (rc = launch("gt_bwd_rows", fr, dim3(static_cast<unsigned>(wave_grid(r.n_units))),
                     dim3(kBlock), &r, s)))
        return rc;
    return merge_sum("gt_bwd_rows_merge", p.row_splits, p.dptr<sgat_split>(SGAT_ARR_ROW_SPLITS),
                     HD, ws.part_row, oscale, dQ, nullptr, 0.f, nullptr, dt, s);
}

}  // namespace sgat
