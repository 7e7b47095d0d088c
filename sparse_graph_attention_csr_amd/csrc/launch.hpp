// Internal host interface between the C ABI and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "device.hpp"
#include "plan.hpp"

namespace sgat {

// Work decomposition for element type dt, head dim D and H heads: lanes per
// head SPH = D / VEC; a head group is the largest power of two of heads (at
// most H rounded up) whose 16-byte fragments fit 64 lanes; EPW = edges a wave
// processes side by side; n_hg = head groups per row.
struct Decomp {
    int vec, sph, hg, epw, n_hg;
};
Decomp decompose(int dt, int D, int H);

// Grids of the GATv2 backward: the CSR pass's long items one per wave, its
// short ones several per wave, and the transposed pass (a multiple of the XCD
// remap quantum); da partials are one per workgroup of all three.
struct GatRowGrid {
    int single, shorts, cols;
};
GatRowGrid gat_bwd_row_grid(const Plan& p, int dt, int D, int H);
// rows of H*D floats the da partials (and their reduction) take in the workspace
int64_t gat_da_part_rows(const GatRowGrid& g);

struct FwdWs {
    float* part_acc;   // [row_slots][H*D]
    float* part_ml;    // [row_slots][H][2]
};
struct BwdWs {
    void* stats;       // [n][H] (lse * log2 e, Delta) (Graph Transformer only)
    float* part_row;   // [row_slots][H*D]
    float* part_col0;  // [col_slots][H*D]
    float* part_col1;  // [col_slots][H*D] (GT only)
    float* da_part;    // [single + shorts + cols workgroups][H*D] (GATv2 only)
    float* ds;         // [nnz][H] dS per edge (Graph Transformer only)
    void* edge_rec;    // [nnz][gat_edge_record_dwords] (GATv2 only)
};

// Dwords per edge (over all head groups) of the records the GATv2 CSR
// backward pass leaves for the transposed pass: (p, dE) per head and one sign
// bit of z per channel.
int64_t gat_edge_record_dwords(int dt, int D, int H);

int launch_gt_fwd(const Plan& p, int H, int D, int dt, const int32_t* colidx, const void* Q,
                  const void* K, const void* V, void* out, float* lse, const FwdWs& ws,
                  hipStream_t s);
int launch_gt_bwd(const Plan& p, int H, int D, int dt, const int32_t* colidx, const void* Q,
                  const void* K, const void* V, const void* O, const float* lse, const void* dO,
                  void* dQ, void* dK, void* dV, const BwdWs& ws, hipStream_t s);
int launch_gat_fwd(const Plan& p, int H, int D, int dt, const int32_t* colidx, const void* Xs,
                   const void* Xt, const float* att, float slope, void* out, float* lse,
                   const FwdWs& ws, hipStream_t s);
int launch_gat_bwd(const Plan& p, int H, int D, int dt, const int32_t* colidx, const void* Xs,
                   const void* Xt, const float* att, float slope, const void* O, const float* lse,
                   const void* dO, void* dXs, void* dXt, float* da, const BwdWs& ws,
                   hipStream_t s);

// Block-sparse forward (bf16 only): dense tiles and residual pseudo-tiles.
int launch_gt_bs_fwd(const Plan& p, int H, int D, const void* Q, const void* K, const void* V,
                     void* out, float* lse, hipStream_t s);

// Block-sparse backward (bf16 only): dQ and (lse, Delta) per tile row, then
// dK and dV per tile column. `stats` is the [n][H] (lse*log2 e, Delta) region.
int launch_gt_bs_bwd(const Plan& p, int H, int D, const void* Q, const void* K, const void* V,
                     const void* O, const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                     void* tile_pd, void* res_pd, hipStream_t s);

// Min/max aggregation: lanes per edge and fragments per lane for F features.
constexpr int kReduceMaxF = 2048;
struct ReduceGeom {
    int lpe, nf;
};
ReduceGeom reduce_geometry(int dt, int F);
bool reduce_supported(int dt, int F);
int launch_reduce_fwd(const Plan& p, int F, int dt, int op, const int32_t* colidx, const void* X,
                      void* out, int32_t* arg, float* part_val, int32_t* part_pos, hipStream_t s);
int launch_reduce_bwd(const Plan& p, int F, int dt, const int64_t* rowptr, const int32_t* arg,
                      const void* dO, void* dX, float* part, uint32_t* sc, void* entries,
                      hipStream_t s);

// da = 0 (the empty sum, for a graph without nodes), by a kernel.
int launch_da_zero(float* da, int HD, hipStream_t s);

// Fixed-order sum of split-row partial gradients into one or two outputs
// (part1 == nullptr: one), scaled, in the output dtype.
int merge_sum(const char* name, const std::vector<sgat_split>& sp, const sgat_split* dsp, int HD,
              const float* part0, float scale0, void* out0, const float* part1, float scale1,
              void* out1, int dt, hipStream_t s);

// Launch one kernel through hipLaunchKernel, bracketed by trace events when
// tracing is on. Returns SGAT_OK or SGAT_HIP_ERROR.
int launch(const char* name, const void* fn, dim3 grid, dim3 block, void* arg, hipStream_t s);

// Blocks for `units` one-wave units, rounded up to the XCD remap quantum.
int64_t wave_grid(int64_t units);

}  // namespace sgat

// Every (dtype, D, EPW) the gather kernels are compiled for.
#define SGAT_GATHER_CONFIGS(X)                                                        \
    X(SGAT_BF16, 32, 1) X(SGAT_BF16, 32, 2) X(SGAT_BF16, 32, 4) X(SGAT_BF16, 32, 8)   \
    X(SGAT_BF16, 32, 16) X(SGAT_BF16, 64, 1) X(SGAT_BF16, 64, 2) X(SGAT_BF16, 64, 4)  \
    X(SGAT_BF16, 64, 8) X(SGAT_BF16, 128, 1) X(SGAT_BF16, 128, 2) X(SGAT_BF16, 128, 4) \
    X(SGAT_F32, 32, 1) X(SGAT_F32, 32, 2) X(SGAT_F32, 32, 4) X(SGAT_F32, 32, 8)       \
    X(SGAT_F32, 64, 1) X(SGAT_F32, 64, 2) X(SGAT_F32, 64, 4) X(SGAT_F32, 128, 1)      \
    X(SGAT_F32, 128, 2)
