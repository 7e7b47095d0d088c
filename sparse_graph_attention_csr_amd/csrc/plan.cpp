// Host preprocessing of a CSR graph into the arrays the kernels read.
//
// Everything here is integer work and deterministic: the same CSR and options
// always give byte-identical arrays.
//
// Heavy-tailed degree distributions let a few high-degree nodes dominate the
// run time and starve the GPU of parallelism (Yandex Research blog "On
// efficient scaling of GNNs via IO-aware layer implementations", paragraph on
// aggregation layers; the super nodes of the DF-GNN paper, Abstract). The
// work list answers that by cutting every row longer than `chunk` edges into
// chunks of `chunk` edges, each its own wavefront, and by ordering the rest by
// a coarse degree bin so the longest work is dispatched first while rows of
// similar id stay together.
#include "plan.hpp"

#include <algorithm>
#include <cstring>
#include <new>

namespace sgat {

int validate_csr(int64_t n, int64_t nnz, const int64_t* rowptr, const int32_t* colidx)
{
    if (n < 0 || nnz < 0 || n > INT32_MAX || nnz > INT32_MAX) return SGAT_INVALID_ARGUMENT;
    if (!rowptr || (nnz > 0 && !colidx)) return SGAT_INVALID_ARGUMENT;
    if (rowptr[0] != 0) return SGAT_INVALID_CSR;
    for (int64_t i = 0; i < n; ++i)
        if (rowptr[i + 1] < rowptr[i]) return SGAT_INVALID_CSR;
    if (rowptr[n] != nnz) return SGAT_INVALID_CSR;
    for (int64_t e = 0; e < nnz; ++e)
        if (colidx[e] < 0 || colidx[e] >= n) return SGAT_INVALID_CSR;
    return SGAT_OK;
}

static int degree_bin(int64_t deg)
{
    if (deg <= 0) return -1;
    return 63 - __builtin_clzll(static_cast<unsigned long long>(deg));
}

void build_work_list(int64_t n, const int64_t* ptr, int64_t chunk,
                     std::vector<sgat_work_item>& items, std::vector<sgat_split>& splits,
                     int64_t& nslots, const int32_t* rank)
{
    items.clear();
    splits.clear();
    nslots = 0;
    // 1. chunks of split rows, rows ascending, chunks in edge order
    for (int64_t i = 0; i < n; ++i) {
        int64_t deg = ptr[i + 1] - ptr[i];
        if (deg <= chunk) continue;
        int64_t nk = (deg + chunk - 1) / chunk;
        splits.push_back({static_cast<int32_t>(i), static_cast<int32_t>(nslots),
                          static_cast<int32_t>(nk), 0});
        for (int64_t k = 0; k < nk; ++k) {
            int64_t b = ptr[i] + k * chunk;
            int64_t len = std::min(chunk, ptr[i + 1] - b);
            items.push_back({b, static_cast<int32_t>(len), static_cast<int32_t>(i),
                             static_cast<int32_t>(nslots + k), k == 0 ? 1 : 0});
        }
        nslots += nk;
    }
    // 2. whole rows, by degree bin floor(log2(deg)) descending, empty rows
    //    last; inside a bin ascending rank, or ascending id (a counting sort)
    std::vector<int32_t> by_rank;
    if (rank) {
        by_rank.assign(static_cast<size_t>(n), 0);
        for (int64_t i = 0; i < n; ++i) by_rank[static_cast<size_t>(rank[i])] = static_cast<int32_t>(i);
    }
    std::vector<int64_t> count(65, 0);
    for (int64_t i = 0; i < n; ++i) {
        int64_t deg = ptr[i + 1] - ptr[i];
        if (deg > chunk) continue;
        count[64 - (degree_bin(deg) + 1)]++;   // bin 63 -> slot 0, ..., empty -> slot 64
    }
    std::vector<int64_t> start(65, 0);
    for (int s = 1; s < 65; ++s) start[s] = start[s - 1] + count[s - 1];
    size_t base = items.size();
    items.resize(base + static_cast<size_t>(start[64] + count[64]));
    for (int64_t q = 0; q < n; ++q) {
        const int64_t i = rank ? by_rank[static_cast<size_t>(q)] : q;
        int64_t deg = ptr[i + 1] - ptr[i];
        if (deg > chunk) continue;
        int s = 64 - (degree_bin(deg) + 1);
        items[base + static_cast<size_t>(start[s]++)] =
            {ptr[i], static_cast<int32_t>(deg), static_cast<int32_t>(i), -1, 1};
    }
}

void short_suffixes(const std::vector<sgat_work_item>& items, int64_t out[33])
{
    // the suffix maximum of the lengths never increases along the list, so
    // the items from out[b] on are exactly the suffix whose maximum is < 2^b
    const int64_t m = static_cast<int64_t>(items.size());
    int64_t longest = 0;
    for (int b = 0; b <= 32; ++b) out[b] = m;
    for (int64_t i = m - 1; i >= 0; --i) {
        longest = std::max<int64_t>(longest, items[static_cast<size_t>(i)].len);
        for (int b = 0; b <= 32; ++b)
            if ((int64_t{1} << b) > longest) out[b] = i;
    }
}

std::vector<int32_t> cuthill_mckee_rank(int64_t n, const int64_t* rowptr, const int32_t* colidx,
                                        const int64_t* colptr, const int32_t* rowidx)
{
    // undirected simple adjacency: in- and out-neighbours, sorted, unique, no self
    std::vector<int64_t> aptr(static_cast<size_t>(n) + 1, 0);
    std::vector<int32_t> adj;
    adj.reserve(static_cast<size_t>(rowptr[n]) * 2);
    std::vector<int32_t> tmp;
    for (int64_t v = 0; v < n; ++v) {
        tmp.clear();
        for (int64_t e = rowptr[v]; e < rowptr[v + 1]; ++e)
            if (colidx[e] != v) tmp.push_back(colidx[e]);
        for (int64_t e = colptr[v]; e < colptr[v + 1]; ++e)
            if (rowidx[e] != v) tmp.push_back(rowidx[e]);
        std::sort(tmp.begin(), tmp.end());
        tmp.erase(std::unique(tmp.begin(), tmp.end()), tmp.end());
        adj.insert(adj.end(), tmp.begin(), tmp.end());
        aptr[static_cast<size_t>(v) + 1] = static_cast<int64_t>(adj.size());
    }
    std::vector<int64_t> deg(static_cast<size_t>(n));
    for (int64_t v = 0; v < n; ++v) deg[static_cast<size_t>(v)] = aptr[v + 1] - aptr[v];
    auto less = [&](int32_t a, int32_t b) {
        return deg[static_cast<size_t>(a)] != deg[static_cast<size_t>(b)]
                   ? deg[static_cast<size_t>(a)] < deg[static_cast<size_t>(b)]
                   : a < b;
    };
    for (int64_t v = 0; v < n; ++v)
        std::sort(adj.begin() + aptr[v], adj.begin() + aptr[v + 1], less);
    std::vector<int32_t> seeds(static_cast<size_t>(n));
    for (int64_t v = 0; v < n; ++v) seeds[static_cast<size_t>(v)] = static_cast<int32_t>(v);
    std::stable_sort(seeds.begin(), seeds.end(), less);
    std::vector<unsigned char> seen(static_cast<size_t>(n), 0);
    std::vector<int32_t> order;
    order.reserve(static_cast<size_t>(n));
    for (int32_t s0 : seeds) {
        if (seen[static_cast<size_t>(s0)]) continue;
        seen[static_cast<size_t>(s0)] = 1;
        size_t head = order.size();
        order.push_back(s0);
        while (head < order.size()) {
            const int32_t v = order[head++];
            for (int64_t e = aptr[v]; e < aptr[v + 1]; ++e) {
                const int32_t u = adj[static_cast<size_t>(e)];
                if (!seen[static_cast<size_t>(u)]) {
                    seen[static_cast<size_t>(u)] = 1;
                    order.push_back(u);
                }
            }
        }
    }
    std::vector<int32_t> rank(static_cast<size_t>(n));
    for (size_t k = 0; k < order.size(); ++k) rank[static_cast<size_t>(order[k])] = static_cast<int32_t>(k);
    return rank;
}

void build_transpose(int64_t n, const int64_t* rowptr, const int32_t* colidx,
                     std::vector<int64_t>& colptr, std::vector<int32_t>& rowidx,
                     std::vector<int32_t>* edge_ids)
{
    int64_t nnz = rowptr[n];
    colptr.assign(static_cast<size_t>(n) + 1, 0);
    for (int64_t e = 0; e < nnz; ++e) colptr[static_cast<size_t>(colidx[e]) + 1]++;
    for (int64_t j = 0; j < n; ++j) colptr[j + 1] += colptr[j];
    std::vector<int64_t> fill(colptr.begin(), colptr.end() - 1);
    rowidx.assign(static_cast<size_t>(nnz), 0);
    if (edge_ids) edge_ids->assign(static_cast<size_t>(nnz), 0);
    for (int64_t i = 0; i < n; ++i)
        for (int64_t e = rowptr[i]; e < rowptr[i + 1]; ++e) {
            const size_t t = static_cast<size_t>(fill[colidx[e]]++);
            rowidx[t] = static_cast<int32_t>(i);
            if (edge_ids) (*edge_ids)[t] = static_cast<int32_t>(e);
        }
}

void build_tiles(int64_t n, const int64_t* rowptr, const int32_t* colidx, int32_t min_nnz,
                 std::vector<int64_t>& tile_rowptr, std::vector<int32_t>& tile_col,
                 std::vector<uint16_t>& tile_mask, std::vector<int64_t>& res_rowptr,
                 std::vector<int32_t>& res_colidx, int64_t& tile_edges)
{
    const int64_t nbr = (n + kTile - 1) / kTile;
    const int64_t nnz = rowptr[n];
    tile_rowptr.assign(static_cast<size_t>(nbr) + 1, 0);
    tile_col.clear();
    tile_mask.clear();
    tile_edges = 0;
    std::vector<unsigned char> in_tile(static_cast<size_t>(nnz), 0);

    // key = (block column, row in tile, column in tile), edge id breaks ties so a
    // stable order puts the first occurrence of every (i, j) first
    struct Ent { int64_t key; int64_t e; };
    std::vector<Ent> ents;
    for (int64_t br = 0; br < nbr; ++br) {
        int64_t r0 = br * kTile, r1 = std::min(n, r0 + kTile);
        ents.clear();
        for (int64_t i = r0; i < r1; ++i)
            for (int64_t e = rowptr[i]; e < rowptr[i + 1]; ++e) {
                int64_t j = colidx[e];
                int64_t key = ((j / kTile) << 8) | ((i - r0) << 4) | (j % kTile);
                ents.push_back({key, e});
            }
        std::sort(ents.begin(), ents.end(), [](const Ent& a, const Ent& b) {
            return a.key != b.key ? a.key < b.key : a.e < b.e;
        });
        size_t t = 0;
        while (t < ents.size()) {
            int64_t bc = ents[t].key >> 8;
            size_t u = t;
            int64_t distinct = 0;
            while (u < ents.size() && (ents[u].key >> 8) == bc) {
                if (u == t || ents[u].key != ents[u - 1].key) ++distinct;
                ++u;
            }
            if (distinct >= min_nnz) {
                uint16_t mask[kTile] = {};
                for (size_t w = t; w < u; ++w) {
                    if (w != t && ents[w].key == ents[w - 1].key) continue;  // repeat -> residual
                    int r = static_cast<int>((ents[w].key >> 4) & 15);
                    int c = static_cast<int>(ents[w].key & 15);
                    mask[r] = static_cast<uint16_t>(mask[r] | (1u << c));
                    in_tile[static_cast<size_t>(ents[w].e)] = 1;
                    ++tile_edges;
                }
                tile_col.push_back(static_cast<int32_t>(bc));
                tile_mask.insert(tile_mask.end(), mask, mask + kTile);
            }
            t = u;
        }
        tile_rowptr[static_cast<size_t>(br) + 1] = static_cast<int64_t>(tile_col.size());
    }
    res_rowptr.assign(static_cast<size_t>(n) + 1, 0);
    res_colidx.clear();
    res_colidx.reserve(static_cast<size_t>(nnz - tile_edges));
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t e = rowptr[i]; e < rowptr[i + 1]; ++e)
            if (!in_tile[static_cast<size_t>(e)]) res_colidx.push_back(colidx[e]);
        res_rowptr[static_cast<size_t>(i) + 1] = static_cast<int64_t>(res_colidx.size());
    }
}

void build_tile_columns(int64_t n, const std::vector<int64_t>& tile_rowptr,
                        const std::vector<int32_t>& tile_col, std::vector<int32_t>& tile_row,
                        std::vector<int64_t>& tile_colptr, std::vector<int32_t>& tile_bycol)
{
    const int64_t nb = (n + kTile - 1) / kTile;
    const size_t T = tile_col.size();
    tile_row.assign(T, 0);
    for (int64_t br = 0; br < nb; ++br)
        for (int64_t t = tile_rowptr[br]; t < tile_rowptr[br + 1]; ++t)
            tile_row[static_cast<size_t>(t)] = static_cast<int32_t>(br);
    tile_colptr.assign(static_cast<size_t>(nb) + 1, 0);
    for (size_t t = 0; t < T; ++t) tile_colptr[static_cast<size_t>(tile_col[t]) + 1]++;
    for (int64_t b = 0; b < nb; ++b) tile_colptr[b + 1] += tile_colptr[b];
    std::vector<int64_t> fill(tile_colptr.begin(), tile_colptr.end() - 1);
    tile_bycol.assign(T, 0);
    for (size_t t = 0; t < T; ++t)
        tile_bycol[static_cast<size_t>(fill[tile_col[t]]++)] = static_cast<int32_t>(t);
}

void expand_pointer(int64_t n, const std::vector<int64_t>& ptr, std::vector<int32_t>& out)
{
    out.assign(static_cast<size_t>(ptr[static_cast<size_t>(n)]), 0);
    for (int64_t i = 0; i < n; ++i)
        for (int64_t e = ptr[static_cast<size_t>(i)]; e < ptr[static_cast<size_t>(i) + 1]; ++e)
            out[static_cast<size_t>(e)] = static_cast<int32_t>(i);
}

const void* Plan::host_array(int id) const
{
    switch (id) {
    case SGAT_ARR_ROW_ITEMS: return row_items.data();
    case SGAT_ARR_ROW_SPLITS: return row_splits.data();
    case SGAT_ARR_COLPTR: return colptr.data();
    case SGAT_ARR_ROWIDX: return rowidx.data();
    case SGAT_ARR_COL_ITEMS: return col_items.data();
    case SGAT_ARR_COL_SPLITS: return col_splits.data();
    case SGAT_ARR_TILE_ROWPTR: return tile_rowptr.data();
    case SGAT_ARR_TILE_COL: return tile_col.data();
    case SGAT_ARR_TILE_MASK: return tile_mask.data();
    case SGAT_ARR_RES_ROWPTR: return res_rowptr.data();
    case SGAT_ARR_RES_COLIDX: return res_colidx.data();
    case SGAT_ARR_TILE_ROW: return tile_row.data();
    case SGAT_ARR_TILE_COLPTR: return tile_colptr.data();
    case SGAT_ARR_TILE_BYCOL: return tile_bycol.data();
    case SGAT_ARR_RES_COLPTR: return res_colptr.data();
    case SGAT_ARR_RES_ROWIDX: return res_rowidx.data();
    case SGAT_ARR_RES_COL_EDGE: return res_col_edge.data();
    case SGAT_ARR_COL_EDGE: return col_edge.data();
    case SGAT_ARR_ROW_TPOS: return row_tpos.data();
    case SGAT_ARR_RES_ROW: return res_row.data();
    case SGAT_ARR_RES_COLSRC: return res_colsrc.data();
    case SGAT_ARR_TILE_ROW_BYCOL: return tile_row_bycol.data();
    default: return nullptr;
    }
}

bool Plan::ds_transposed(int H) const
{
    if (edge_order == 1 || row_tpos.empty()) return false;
    return edge_order == 2 || nnz * static_cast<int64_t>(H) * 4 > kDsTransposedBytes;
}

void Plan::layout()
{
    bytes[SGAT_ARR_ROW_ITEMS] = row_items.size() * sizeof(sgat_work_item);
    bytes[SGAT_ARR_ROW_SPLITS] = row_splits.size() * sizeof(sgat_split);
    bytes[SGAT_ARR_COLPTR] = colptr.size() * sizeof(int64_t);
    bytes[SGAT_ARR_ROWIDX] = rowidx.size() * sizeof(int32_t);
    bytes[SGAT_ARR_COL_ITEMS] = col_items.size() * sizeof(sgat_work_item);
    bytes[SGAT_ARR_COL_SPLITS] = col_splits.size() * sizeof(sgat_split);
    bytes[SGAT_ARR_TILE_ROWPTR] = tile_rowptr.size() * sizeof(int64_t);
    bytes[SGAT_ARR_TILE_COL] = tile_col.size() * sizeof(int32_t);
    bytes[SGAT_ARR_TILE_MASK] = tile_mask.size() * sizeof(uint16_t);
    bytes[SGAT_ARR_RES_ROWPTR] = res_rowptr.size() * sizeof(int64_t);
    bytes[SGAT_ARR_RES_COLIDX] = res_colidx.size() * sizeof(int32_t);
    bytes[SGAT_ARR_TILE_ROW] = tile_row.size() * sizeof(int32_t);
    bytes[SGAT_ARR_TILE_COLPTR] = tile_colptr.size() * sizeof(int64_t);
    bytes[SGAT_ARR_TILE_BYCOL] = tile_bycol.size() * sizeof(int32_t);
    bytes[SGAT_ARR_RES_COLPTR] = res_colptr.size() * sizeof(int64_t);
    bytes[SGAT_ARR_RES_ROWIDX] = res_rowidx.size() * sizeof(int32_t);
    bytes[SGAT_ARR_RES_COL_EDGE] = res_col_edge.size() * sizeof(int32_t);
    bytes[SGAT_ARR_COL_EDGE] = col_edge.size() * sizeof(int32_t);
    bytes[SGAT_ARR_ROW_TPOS] = row_tpos.size() * sizeof(int32_t);
    bytes[SGAT_ARR_RES_ROW] = res_row.size() * sizeof(int32_t);
    bytes[SGAT_ARR_RES_COLSRC] = res_colsrc.size() * sizeof(int32_t);
    bytes[SGAT_ARR_TILE_ROW_BYCOL] = tile_row_bycol.size() * sizeof(int32_t);
    size_t off = 0;
    for (int a = 0; a < SGAT_ARR_COUNT; ++a) {
        offset[a] = off;
        off = align_up(off + bytes[a]);
    }
    device_bytes = std::max<size_t>(off, kAlign);
}

}  // namespace sgat

using sgat::Plan;

extern "C" {

int sgat_plan_create(int64_t n, int64_t nnz, const int64_t* rowptr, const int32_t* colidx,
                     const sgat_plan_opts* opts, sgat_plan** out)
{
    if (!out) return SGAT_INVALID_ARGUMENT;
    *out = nullptr;
    int rc = sgat::validate_csr(n, nnz, rowptr, colidx);
    if (rc != SGAT_OK) return rc;
    int64_t chunk = sgat::kDefaultChunk;
    int32_t tmin = sgat::kDefaultTileMinNnz;
    bool bs = false, loc = false;
    int32_t order = 0;
    if (opts) {
        if (opts->chunk < 0 || opts->chunk > INT32_MAX) return SGAT_INVALID_ARGUMENT;
        if (opts->tile_min_nnz < 0 || opts->tile_min_nnz > 256) return SGAT_INVALID_ARGUMENT;
        if (opts->block_sparse != 0 && opts->block_sparse != 1) return SGAT_INVALID_ARGUMENT;
        if (opts->locality != 0 && opts->locality != 1) return SGAT_INVALID_ARGUMENT;
        if (opts->edge_order < 0 || opts->edge_order > 2) return SGAT_INVALID_ARGUMENT;
        if (opts->chunk > 0) chunk = opts->chunk;
        if (opts->tile_min_nnz > 0) tmin = opts->tile_min_nnz;
        bs = opts->block_sparse == 1;
        loc = opts->locality == 1;
        order = opts->edge_order;
    }
    sgat_plan* h = new (std::nothrow) sgat_plan;
    if (!h) return SGAT_OUT_OF_HOST_MEMORY;
    try {
        Plan& p = h->p;
        p.n = n;
        p.nnz = nnz;
        p.chunk = chunk;
        p.tile_min_nnz = tmin;
        p.block_sparse = bs;
        p.locality = loc;
        p.edge_order = order;
        for (int64_t i = 0; i < n; ++i)
            p.max_in_degree = std::max(p.max_in_degree, rowptr[i + 1] - rowptr[i]);
        sgat::build_transpose(n, rowptr, colidx, p.colptr, p.rowidx, &p.col_edge);
        if (order == 2 || (order == 0 && nnz > sgat::kTposMinEdges)) {
            p.row_tpos.assign(static_cast<size_t>(nnz), 0);
            for (int64_t q = 0; q < nnz; ++q)
                p.row_tpos[static_cast<size_t>(p.col_edge[static_cast<size_t>(q)])] =
                    static_cast<int32_t>(q);
        }
        for (int64_t j = 0; j < n; ++j)
            p.max_out_degree = std::max(p.max_out_degree, p.colptr[j + 1] - p.colptr[j]);
        std::vector<int32_t> rank;
        if (loc) rank = sgat::cuthill_mckee_rank(n, rowptr, colidx, p.colptr.data(), p.rowidx.data());
        const int32_t* rk = loc ? rank.data() : nullptr;
        sgat::build_work_list(n, rowptr, chunk, p.row_items, p.row_splits, p.row_slots, rk);
        sgat::build_work_list(n, p.colptr.data(), chunk, p.col_items, p.col_splits, p.col_slots, rk);
        sgat::short_suffixes(p.row_items, p.row_short_from);
        sgat::short_suffixes(p.col_items, p.col_short_from);
        if (bs) {
            sgat::build_tiles(n, rowptr, colidx, tmin, p.tile_rowptr, p.tile_col, p.tile_mask,
                              p.res_rowptr, p.res_colidx, p.tile_edges);
            sgat::build_tile_columns(n, p.tile_rowptr, p.tile_col, p.tile_row, p.tile_colptr,
                                     p.tile_bycol);
            sgat::build_transpose(n, p.res_rowptr.data(), p.res_colidx.data(), p.res_colptr,
                                  p.res_rowidx, &p.res_col_edge);
            sgat::expand_pointer(n, p.res_rowptr, p.res_row);
            sgat::expand_pointer(n, p.res_colptr, p.res_colsrc);
            p.tile_row_bycol.resize(p.tile_bycol.size());
            for (size_t x = 0; x < p.tile_bycol.size(); ++x)
                p.tile_row_bycol[x] = p.tile_row[static_cast<size_t>(p.tile_bycol[x])];
        }
        p.layout();
    } catch (const std::bad_alloc&) {
        delete h;
        return SGAT_OUT_OF_HOST_MEMORY;
    } catch (...) {
        delete h;
        return SGAT_OUT_OF_HOST_MEMORY;
    }
    *out = h;
    return SGAT_OK;
}

int sgat_plan_device_bytes(const sgat_plan* plan, size_t* bytes)
{
    if (!plan || !bytes) return SGAT_INVALID_ARGUMENT;
    *bytes = plan->p.device_bytes;
    return SGAT_OK;
}

int sgat_plan_stats_get(const sgat_plan* plan, sgat_plan_stats* s)
{
    if (!plan || !s) return SGAT_INVALID_ARGUMENT;
    const Plan& p = plan->p;
    s->n = p.n;
    s->nnz = p.nnz;
    s->chunk = p.chunk;
    s->max_in_degree = p.max_in_degree;
    s->max_out_degree = p.max_out_degree;
    s->row_items = static_cast<int64_t>(p.row_items.size());
    s->row_splits = static_cast<int64_t>(p.row_splits.size());
    s->row_slots = p.row_slots;
    s->col_items = static_cast<int64_t>(p.col_items.size());
    s->col_splits = static_cast<int64_t>(p.col_splits.size());
    s->col_slots = p.col_slots;
    s->tiles = static_cast<int64_t>(p.tile_col.size());
    s->tile_edges = p.tile_edges;
    s->residual_edges = p.block_sparse ? static_cast<int64_t>(p.res_colidx.size()) : 0;
    s->device_bytes = static_cast<int64_t>(p.device_bytes);
    return SGAT_OK;
}

int sgat_plan_array_bytes(const sgat_plan* plan, int id, size_t* bytes)
{
    if (!plan || !bytes || id < 0 || id >= SGAT_ARR_COUNT) return SGAT_INVALID_ARGUMENT;
    *bytes = plan->p.bytes[id];
    return SGAT_OK;
}

int sgat_plan_export(const sgat_plan* plan, int id, void* dst, size_t bytes)
{
    if (!plan || id < 0 || id >= SGAT_ARR_COUNT) return SGAT_INVALID_ARGUMENT;
    size_t need = plan->p.bytes[id];
    if (bytes < need) return SGAT_WORKSPACE_TOO_SMALL;
    if (need == 0) return SGAT_OK;
    if (!dst) return SGAT_INVALID_ARGUMENT;
    std::memcpy(dst, plan->p.host_array(id), need);
    return SGAT_OK;
}

void sgat_plan_destroy(sgat_plan* plan) { delete plan; }

}  // extern "C"
