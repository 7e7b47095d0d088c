// Launchers of the block-sparse (16x16 tile, bf16 MFMA) Graph Transformer path.
#include "blocksparse.hpp"
#include "launch.hpp"

namespace sgat {

int launch_gt_bs_fwd(const Plan& p, int H, int D, const void* Q, const void* K, const void* V,
                     void* out, float* lse, hipStream_t s)
{
    BsFwdArgs a;
    a.n = p.n;
    a.n_tile_rows = (p.n + kTileDim - 1) / kTileDim;
    a.H = H;
    a.tile_rowptr = p.dptr<int64_t>(SGAT_ARR_TILE_ROWPTR);
    a.tile_col = p.dptr<int32_t>(SGAT_ARR_TILE_COL);
    a.tile_mask = p.dptr<uint16_t>(SGAT_ARR_TILE_MASK);
    a.res_rowptr = p.dptr<int64_t>(SGAT_ARR_RES_ROWPTR);
    a.res_colidx = p.dptr<int32_t>(SGAT_ARR_RES_COLIDX);
    a.res_row = p.dptr<int32_t>(SGAT_ARR_RES_ROW);
    a.Q = Q; a.K = K; a.V = V;
    a.out = out;
    a.lse = lse;
    a.scale2 = kLog2e / sqrtf(static_cast<float>(D));
    const void* fn = D == 32 ? reinterpret_cast<const void*>(&gt_bs_fwd<32>)
                   : D == 64 ? reinterpret_cast<const void*>(&gt_bs_fwd<64>)
                             : reinterpret_cast<const void*>(&gt_bs_fwd<128>);
    // one wave per (tile row, head): ceil(H / 4) workgroups per tile row
    return launch("gt_bs_fwd", fn,
                  dim3(static_cast<unsigned>(wave_grid(a.n_tile_rows * head_groups(H) * kWavesPerBlock))),
                  dim3(kBlock), &a, s);
}

int launch_gt_bs_bwd(const Plan& p, int H, int D, const void* Q, const void* K, const void* V,
                     const void* O, const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                     void* tile_pd, void* res_pd, hipStream_t s)
{
    BsBwdArgs a;
    a.n = p.n;
    a.n_blocks = (p.n + kTileDim - 1) / kTileDim;
    a.H = H;
    a.tile_rowptr = p.dptr<int64_t>(SGAT_ARR_TILE_ROWPTR);
    a.tile_col = p.dptr<int32_t>(SGAT_ARR_TILE_COL);
    a.tile_mask = p.dptr<uint16_t>(SGAT_ARR_TILE_MASK);
    a.tile_colptr = p.dptr<int64_t>(SGAT_ARR_TILE_COLPTR);
    a.tile_bycol = p.dptr<int32_t>(SGAT_ARR_TILE_BYCOL);
    a.res_rowptr = p.dptr<int64_t>(SGAT_ARR_RES_ROWPTR);
    a.res_colidx = p.dptr<int32_t>(SGAT_ARR_RES_COLIDX);
    a.res_colptr = p.dptr<int64_t>(SGAT_ARR_RES_COLPTR);
    a.res_rowidx = p.dptr<int32_t>(SGAT_ARR_RES_ROWIDX);
    a.res_col_edge = p.dptr<int32_t>(SGAT_ARR_RES_COL_EDGE);
    a.res_row = p.dptr<int32_t>(SGAT_ARR_RES_ROW);
    a.res_colsrc = p.dptr<int32_t>(SGAT_ARR_RES_COLSRC);
    a.tile_row_bycol = p.dptr<int32_t>(SGAT_ARR_TILE_ROW_BYCOL);
    a.Q = Q; a.K = K; a.V = V; a.O = O; a.dO = dO;
    a.lse = lse;
    a.tile_pd = static_cast<uint2*>(tile_pd);
    a.res_pd = static_cast<uint32_t*>(res_pd);
    a.dQ = dQ; a.dK = dK; a.dV = dV;
    a.scale2 = kLog2e / sqrtf(static_cast<float>(D));
    a.oscale = 1.f / sqrtf(static_cast<float>(D));
    const void *fr, *fc;
    if (D == 32) {
        fr = reinterpret_cast<const void*>(&gt_bs_bwd_rows<32>);
        fc = reinterpret_cast<const void*>(&gt_bs_bwd_cols<32>);
    } else if (D == 64) {
        fr = reinterpret_cast<const void*>(&gt_bs_bwd_rows<64>);
        fc = reinterpret_cast<const void*>(&gt_bs_bwd_cols<64>);
    } else {
        fr = reinterpret_cast<const void*>(&gt_bs_bwd_rows<128>);
        fc = reinterpret_cast<const void*>(&gt_bs_bwd_cols<128>);
    }
    // one wave per (block, head): ceil(H / 4) workgroups per tile row or column
    const dim3 grid(static_cast<unsigned>(wave_grid(a.n_blocks * head_groups(H) * kWavesPerBlock)));
    int rc = launch("gt_bs_bwd_rows", fr, grid, dim3(kBlock), &a, s);
    if (rc) return rc;
    return launch("gt_bs_bwd_cols", fc, grid, dim3(kBlock), &a, s);
}

}  // namespace sgat
