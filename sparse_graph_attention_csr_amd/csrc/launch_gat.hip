// GATv2 launchers: forward rows (+ log-sum-exp merge), backward CSR pass with
// da partials (+ merge, + fixed-order da reduction), transposed-CSR pass (+ merge).
#include <algorithm>

#include "gather.hpp"
#include "launch.hpp"

namespace sgat {

// Neighbour rows each wave gathers before their first use (compile-time
// tunables; -DSGAT_UNROLL_FWD=... etc. override them). The CSR backward pass
// gathers SGAT_UNROLL_BWD rows per edge group into each of two register
// buffers, one in flight while the other is used.
#ifndef SGAT_UNROLL_FWD
#define SGAT_UNROLL_FWD 8
#endif
#ifndef SGAT_UNROLL_BWD
#define SGAT_UNROLL_BWD 2
#endif
#ifndef SGAT_UNROLL_ROWS
#define SGAT_UNROLL_ROWS 8
#endif
// Items shorter than 2^SGAT_SHORT_LOG2 edges at the end of the work list go
// several to a wavefront (one per edge group) when a wave has more than one
// edge group; SGAT_UNROLL_MULTI neighbour rows per group and step.
#ifndef SGAT_SHORT_LOG2
#define SGAT_SHORT_LOG2 7
#endif
#ifndef SGAT_UNROLL_MULTI
#define SGAT_UNROLL_MULTI 4
#endif
// one source row per step and edge group in the transposed pass: with its
// per-node da terms a second one costs occupancy
#ifndef SGAT_UNROLL_COLS
#define SGAT_UNROLL_COLS 1
#endif
#ifndef SGAT_UNROLL_MULTI_COLS
#define SGAT_UNROLL_MULTI_COLS 1
#endif

namespace {
// With several edges per wave side by side, each unrolled step already holds
// EPW neighbour rows, so fewer steps keep the same bytes in flight with fewer
// registers.
constexpr int unroll_fwd(int epw) { return epw >= 4 ? (SGAT_UNROLL_FWD + 1) / 2 : SGAT_UNROLL_FWD; }
constexpr int unroll_bwd(int epw) { return epw >= 4 ? (SGAT_UNROLL_BWD + 1) / 2 : SGAT_UNROLL_BWD; }
// The backward passes take one work unit per wave up to this grid and
// stride beyond it; every workgroup writes one row of da partials, so the
// cap also bounds that workspace (3 * 2^16 rows of H*D floats at most).
constexpr int kGatBwdMaxBlocks = 1 << 16;
// da partials summed per run of this many by the first reduction level
constexpr int kDaRun = 64;
// above this many partials the reduction takes two levels
constexpr int kDaOneLevel = 1024;
}

int64_t gat_da_part_rows(const GatRowGrid& g)
{
    const int64_t n = static_cast<int64_t>(g.single) + g.shorts + g.cols;
    return n > kDaOneLevel ? n + (n + kDaRun - 1) / kDaRun : n;
}

// First level of the da reduction when there are many partials: workgroup b
// sums partials [b*kDaRun, (b+1)*kDaRun) in order, one thread per element.
__global__ __launch_bounds__(kBlock) void da_reduce_runs(DaReduceArgs a)
{
    const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kDaRun;
    const int nb = static_cast<int>(std::min<int64_t>(kDaRun, a.G - b0));
    for (int e = threadIdx.x; e < a.HD; e += kBlock) {
        const float* src = a.da_part + b0 * a.HD + e;
        float s = 0.f;
#pragma unroll 8
        for (int r = 0; r < nb; ++r) s += src[static_cast<int64_t>(r) * a.HD];
        a.da[static_cast<int64_t>(blockIdx.x) * a.HD + e] = s;
    }
}

// Fixed-order sum of the per-workgroup da partials: one workgroup per element
// of da; thread t sums partials t, t+256, ... in order, then a fixed LDS tree
// combines the 256 thread sums. The result does not depend on timing.
__global__ __launch_bounds__(kBlock) void da_reduce(DaReduceArgs a)
{
    __shared__ float red[kBlock];
    const int e = blockIdx.x;
    float s = 0.f;
    for (int b = threadIdx.x; b < a.G; b += kBlock) s += a.da_part[static_cast<int64_t>(b) * a.HD + e];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kBlock / 2; w > 0; w >>= 1) {
        if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.da[e] = red[0];
}

GatRowGrid gat_bwd_row_grid(const Plan& p, int dt, int D, int H)
{
    const Decomp dc = decompose(dt, D, H);
    const int64_t n_items = static_cast<int64_t>(p.row_items.size());
    const int64_t n_single = dc.epw > 1 ? p.row_short_from[SGAT_SHORT_LOG2] : n_items;
    const int64_t short_units = (n_items - n_single + dc.epw - 1) / dc.epw;
    const int64_t c_items = static_cast<int64_t>(p.col_items.size());
    const int64_t c_single = dc.epw > 1 ? p.col_short_from[SGAT_SHORT_LOG2] : c_items;
    const int64_t c_units = c_single + (c_items - c_single + dc.epw - 1) / dc.epw;
    auto blocks = [](int64_t waves) {
        const int64_t need = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
        return static_cast<int>(std::min<int64_t>(need, kGatBwdMaxBlocks));
    };
    GatRowGrid g{blocks(n_single), blocks(short_units),
                 static_cast<int>(std::min<int64_t>(wave_grid(c_units), kGatBwdMaxBlocks))};
    if (g.cols == 0) g.cols = kGridQuantum;   // da is still written (as zeros)
    return g;
}

int launch_da_zero(float* da, int HD, hipStream_t s)
{
    DaReduceArgs d{nullptr, 0, HD, da};
    return launch("gat_bwd_da_reduce", reinterpret_cast<const void*>(&da_reduce),
                  dim3(static_cast<unsigned>(HD)), dim3(kBlock), &d, s);
}

int launch_gat_fwd(const Plan& p, int H, int D, int dt, const int32_t* colidx, const void* Xs,
                   const void* Xt, const float* att, float slope, void* out, float* lse,
                   const FwdWs& ws, hipStream_t s)
{
    const Decomp dc = decompose(dt, D, H);
    GatFwdArgs a;
    a.items = p.dptr<sgat_work_item>(SGAT_ARR_ROW_ITEMS);
    a.n_items = static_cast<int64_t>(p.row_items.size());
    a.n_single = dc.epw > 1 ? p.row_short_from[SGAT_SHORT_LOG2] : a.n_items;
    a.n_units = (a.n_single + (a.n_items - a.n_single + dc.epw - 1) / dc.epw) * dc.n_hg;
    a.n_hg = dc.n_hg;
    a.H = H;
    a.colidx = colidx;
    a.Xs = Xs; a.Xt = Xt;
    a.att = att;
    a.slope = slope;
    a.out = out;
    a.lse = lse;
    a.part_acc = ws.part_acc;
    a.part_ml = ws.part_ml;
    const void* fn = nullptr;
#define X(DT_, D_, E_) \
    if (dt == DT_ && D == D_ && dc.epw == E_) fn = reinterpret_cast<const void*>(&gat_fwd_rows<DT_, D_, E_, unroll_fwd(E_), SGAT_UNROLL_MULTI>);
    SGAT_GATHER_CONFIGS(X)
#undef X
    if (!fn) return SGAT_INVALID_ARGUMENT;
    if (a.n_units > 0) {
        int rc = launch("gat_fwd_rows", fn, dim3(static_cast<unsigned>(wave_grid(a.n_units))),
                        dim3(kBlock), &a, s);
        if (rc) return rc;
    }
    if (!p.row_splits.empty()) {
        LseMergeArgs m{p.dptr<sgat_split>(SGAT_ARR_ROW_SPLITS), H, D, ws.part_acc, ws.part_ml,
                       out, lse};
        const void* mf = dt == SGAT_F32 ? reinterpret_cast<const void*>(&lse_merge<SGAT_F32>)
                                        : reinterpret_cast<const void*>(&lse_merge<SGAT_BF16>);
        int rc = launch("gat_fwd_merge", mf,
                        dim3(static_cast<unsigned>(p.row_splits.size()),
                             static_cast<unsigned>((H * D + kBlock - 1) / kBlock)),
                        dim3(kBlock), &m, s);
        if (rc) return rc;
    }
    return SGAT_OK;
}

int64_t gat_edge_record_dwords(int dt, int D, int H)
{
    const Decomp dc = decompose(dt, D, H);
    return static_cast<int64_t>(dc.n_hg) * gat_rec_dwords(dc.hg, dc.hg * dc.sph);
}

int launch_gat_bwd(const Plan& p, int H, int D, int dt, const int32_t* colidx, const void* Xs,
                   const void* Xt, const float* att, float slope, const void* O, const float* lse,
                   const void* dO, void* dXs, void* dXt, float* da, const BwdWs& ws,
                   hipStream_t s)
{
    const Decomp dc = decompose(dt, D, H);
    const int HD = H * D;
    const GatRowGrid gx = gat_bwd_row_grid(p, dt, D, H);

    GatBwdRowArgs r;
    r.items = p.dptr<sgat_work_item>(SGAT_ARR_ROW_ITEMS);
    r.n_items = static_cast<int64_t>(p.row_items.size());
    r.n_single = dc.epw > 1 ? p.row_short_from[SGAT_SHORT_LOG2] : r.n_items;
    r.H = H;
    r.colidx = colidx;
    r.Xs = Xs; r.Xt = Xt; r.O = O; r.dO = dO;
    r.att = att;
    r.slope = slope;
    r.lse = lse;
    r.edge_rec = static_cast<uint32_t*>(ws.edge_rec);
    r.nnz = p.nnz;
    r.dXs = dXs;
    r.part = ws.part_row;
    r.da_part = ws.da_part;

    GatBwdColArgs c;
    c.items = p.dptr<sgat_work_item>(SGAT_ARR_COL_ITEMS);
    c.n_items = static_cast<int64_t>(p.col_items.size());
    c.n_single = dc.epw > 1 ? p.col_short_from[SGAT_SHORT_LOG2] : c.n_items;
    c.H = H;
    c.rowidx = p.dptr<int32_t>(SGAT_ARR_ROWIDX);
    c.col_edge = p.dptr<int32_t>(SGAT_ARR_COL_EDGE);
    c.Xt = Xt;
    c.dO = dO;
    c.att = att;
    c.slope = slope;
    c.edge_rec = static_cast<const uint32_t*>(ws.edge_rec);
    c.nnz = p.nnz;
    c.dXt = dXt;
    c.part = ws.part_col0;
    c.da_part = ws.da_part + static_cast<int64_t>(gx.single + gx.shorts) * HD;

    const void *fr = nullptr, *frs = nullptr, *fc = nullptr;
#define X(DT_, D_, E_)                                                                        \
    if (dt == DT_ && D == D_ && dc.epw == E_) {                                               \
        fr = reinterpret_cast<const void*>(                                                   \
            &gat_bwd_rows<DT_, D_, E_, unroll_bwd(E_), false>);                               \
        if constexpr (E_ > 1)                                                                 \
            frs = reinterpret_cast<const void*>(                                              \
                &gat_bwd_rows<DT_, D_, E_, unroll_bwd(E_), true>);                            \
        fc = reinterpret_cast<const void*>(                                                   \
            &gat_bwd_cols<DT_, D_, E_, SGAT_UNROLL_COLS, SGAT_UNROLL_MULTI_COLS>);            \
    }
    SGAT_GATHER_CONFIGS(X)
#undef X
    if (!fr || !fc || (gx.shorts > 0 && !frs)) return SGAT_INVALID_ARGUMENT;
    int rc;
    // every workgroup of the row passes writes its da partial (zeros if it had no item)
    if (gx.single > 0 &&
        (rc = launch("gat_bwd_rows", fr,
                     dim3(static_cast<unsigned>(gx.single), static_cast<unsigned>(dc.n_hg)),
                     dim3(kBlock), &r, s)))
        return rc;
    if (gx.shorts > 0) {
        GatBwdRowArgs rs = r;
        rs.da_part = ws.da_part + static_cast<int64_t>(gx.single) * HD;
        if ((rc = launch("gat_bwd_rows_short", frs,
                         dim3(static_cast<unsigned>(gx.shorts), static_cast<unsigned>(dc.n_hg)),
                         dim3(kBlock), &rs, s)))
            return rc;
    }
    if ((rc = merge_sum("gat_bwd_rows_merge", p.row_splits, p.dptr<sgat_split>(SGAT_ARR_ROW_SPLITS),
                        HD, ws.part_row, 1.f, dXs, nullptr, 0.f, nullptr, dt, s)))
        return rc;
    // every workgroup of the transposed pass writes its da partial too
    if ((rc = launch("gat_bwd_cols", fc,
                     dim3(static_cast<unsigned>(gx.cols), static_cast<unsigned>(dc.n_hg)),
                     dim3(kBlock), &c, s)))
        return rc;
    if ((rc = merge_sum("gat_bwd_cols_merge", p.col_splits, p.dptr<sgat_split>(SGAT_ARR_COL_SPLITS),
                        HD, ws.part_col0, 1.f, dXt, nullptr, 0.f, nullptr, dt, s)))
        return rc;
    DaReduceArgs d{ws.da_part, gx.single + gx.shorts + gx.cols, HD, da};
    if (d.G > kDaOneLevel) {
        // runs of kDaRun partials first, into the rows after the partials
        const int runs = (d.G + kDaRun - 1) / kDaRun;
        float* lvl = ws.da_part + static_cast<int64_t>(d.G) * HD;
        DaReduceArgs r{ws.da_part, d.G, HD, lvl};
        if ((rc = launch("gat_bwd_da_reduce_runs", reinterpret_cast<const void*>(&da_reduce_runs),
                         dim3(static_cast<unsigned>(runs)), dim3(kBlock), &r, s)))
            return rc;
        d = DaReduceArgs{lvl, runs, HD, da};
    }
    return launch("gat_bwd_da_reduce", reinterpret_cast<const void*>(&da_reduce),
                  dim3(static_cast<unsigned>(HD)), dim3(kBlock), &d, s);
}

}  // namespace sgat
