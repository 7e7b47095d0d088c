// Host-side plan: the integer preprocessing of one CSR graph.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "sgattn.h"

namespace sgat {

constexpr int64_t kDefaultChunk = 1024;
constexpr int32_t kDefaultTileMinNnz = 32;
constexpr int kTile = 16;
constexpr size_t kAlign = 256;
// edge_order 0: dS goes in transposed order above this many bytes, and the
// inverse map is built when some H <= 16 could get there
constexpr int64_t kDsTransposedBytes = int64_t(128) << 20;
constexpr int64_t kTposMinEdges = int64_t(1) << 21;

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

struct Plan {
    int64_t n = 0, nnz = 0;
    int64_t chunk = kDefaultChunk;
    int32_t tile_min_nnz = kDefaultTileMinNnz;
    bool block_sparse = false;
    bool locality = false;
    int32_t edge_order = 0;             // sgat_plan_opts.edge_order
    int64_t max_in_degree = 0, max_out_degree = 0;

    std::vector<sgat_work_item> row_items;
    std::vector<sgat_split> row_splits;
    int64_t row_slots = 0;
    // short_from[b]: first work item from which every item has fewer than 2^b edges
    int64_t row_short_from[33] = {};
    int64_t col_short_from[33] = {};

    std::vector<int64_t> colptr;
    std::vector<int32_t> rowidx;
    std::vector<int32_t> col_edge;      // CSR edge id of each transposed entry
    std::vector<int32_t> row_tpos;      // transposed position of each CSR edge (may be empty)
    std::vector<sgat_work_item> col_items;
    std::vector<sgat_split> col_splits;
    int64_t col_slots = 0;

    std::vector<int64_t> tile_rowptr;
    std::vector<int32_t> tile_col;
    std::vector<uint16_t> tile_mask;   // [tiles][16]
    std::vector<int64_t> res_rowptr;
    std::vector<int32_t> res_colidx;
    std::vector<int32_t> tile_row;      // block row of each tile
    std::vector<int64_t> tile_colptr;   // tiles grouped by block column
    std::vector<int32_t> tile_bycol;
    std::vector<int64_t> res_colptr;    // transposed residual CSR
    std::vector<int32_t> res_rowidx;
    std::vector<int32_t> res_col_edge;  // residual-CSR edge id of each transposed residual entry
    std::vector<int32_t> res_row;       // destination of each residual edge
    std::vector<int32_t> res_colsrc;    // source of each transposed residual entry
    std::vector<int32_t> tile_row_bycol;// block row of each tile, in tile_bycol order
    int64_t tile_edges = 0;

    // device image: every array at a 256-byte aligned offset of one buffer
    size_t offset[SGAT_ARR_COUNT] = {};
    size_t bytes[SGAT_ARR_COUNT] = {};
    size_t device_bytes = 0;
    const unsigned char* dev = nullptr;
    bool uploaded = false;

    const void* host_array(int id) const;
    // Graph Transformer backward: dS in transposed order for H heads?
    bool ds_transposed(int H) const;
    void layout();
    template <class T>
    const T* dptr(int id) const { return reinterpret_cast<const T*>(dev + offset[id]); }
};

// A1: returns SGAT_OK or SGAT_INVALID_CSR / SGAT_INVALID_ARGUMENT.
int validate_csr(int64_t n, int64_t nnz, const int64_t* rowptr, const int32_t* colidx);

// A2: degree-binned work list over any CSR-like pointer array. Whole rows of
// one bin come in ascending `rank` (ascending id when rank is null).
void build_work_list(int64_t n, const int64_t* ptr, int64_t chunk,
                     std::vector<sgat_work_item>& items, std::vector<sgat_split>& splits,
                     int64_t& nslots, const int32_t* rank = nullptr);

// out[b] = first index from which every item has fewer than 2^b edges (b = 0..32).
void short_suffixes(const std::vector<sgat_work_item>& items, int64_t out[33]);

// Cuthill-McKee rank of every node of the undirected simple graph underlying
// the CSR (in- and out-neighbours, self-loops and repeats dropped).
std::vector<int32_t> cuthill_mckee_rank(int64_t n, const int64_t* rowptr, const int32_t* colidx,
                                        const int64_t* colptr, const int32_t* rowidx);

// A3: transposed CSR by stable counting sort of edges by source; with
// `edge_ids` also the CSR edge id of every transposed entry.
void build_transpose(int64_t n, const int64_t* rowptr, const int32_t* colidx,
                     std::vector<int64_t>& colptr, std::vector<int32_t>& rowidx,
                     std::vector<int32_t>* edge_ids = nullptr);

// A4: 16x16 dense tiles with at least `min_nnz` distinct edges, plus residual CSR.
void build_tiles(int64_t n, const int64_t* rowptr, const int32_t* colidx, int32_t min_nnz,
                 std::vector<int64_t>& tile_rowptr, std::vector<int32_t>& tile_col,
                 std::vector<uint16_t>& tile_mask, std::vector<int64_t>& res_rowptr,
                 std::vector<int32_t>& res_colidx, int64_t& tile_edges);

// The row of every entry of a CSR-like pointer array (out[e] = i for e in
// [ptr[i], ptr[i+1])).
void expand_pointer(int64_t n, const std::vector<int64_t>& ptr, std::vector<int32_t>& out);

// A4 (column side): tiles grouped by block column (stable in block row) and
// the block row of each tile.
void build_tile_columns(int64_t n, const std::vector<int64_t>& tile_rowptr,
                        const std::vector<int32_t>& tile_col, std::vector<int32_t>& tile_row,
                        std::vector<int64_t>& tile_colptr, std::vector<int32_t>& tile_bycol);

}  // namespace sgat

struct sgat_plan {
    sgat::Plan p;
};
