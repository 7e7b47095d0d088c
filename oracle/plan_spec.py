"""Independent numpy statement of the integer preprocessing arrays.

TEST INFRASTRUCTURE ONLY (see the package docstring). Written from the
specification of the arrays, not from the C++ builder, so that tests can
require byte equality between the two.

Work list over a pointer array ``ptr`` (the CSR rowptr, or the transposed
CSR's colptr) with chunk size C -- the degree-aware split of high-degree
nodes (Yandex Research blog "On efficient scaling of GNNs via IO-aware layer
implementations", paragraph on aggregation layers):
  1. every row with deg > C, rows ascending: chunks k = 0..ceil(deg/C)-1 of
     edges [ptr[i] + kC, min(ptr[i] + (k+1)C, ptr[i+1])), each with the next
     free partial slot; flags = 1 for k = 0; one split record
     (row, first slot, number of chunks) per such row;
  2. then every other row as one item (slot -1, flags 1), ordered by
     floor(log2(deg)) descending, rows with deg 0 last, row id ascending
     within a bin.

Transposed CSR: edges grouped by source with a stable sort, so the
destinations of a source appear in edge order.

16x16 tiles: tile (br, bc) holds the edges j -> i with i // 16 = br and
j // 16 = bc. Only the first occurrence of a pair (i, j) in row i counts. A tile
with at least ``min_nnz`` distinct pairs is dense; dense tiles are listed by
block row, then block column. Bit c of mask word r marks edge
(16 bc + c) -> (16 br + r). Every edge not marked in a dense tile (including
repeats) goes to the residual CSR, in its original order.

Column side of the tiles: the block row of every tile, and the tile ids grouped
by block column with block rows ascending inside a column; the residual CSR
transposed like the main one.
"""
from __future__ import annotations

import numpy as np

WORK_ITEM = np.dtype([("begin", "<i8"), ("len", "<i4"), ("row", "<i4"),
                      ("slot", "<i4"), ("flags", "<i4")])
SPLIT = np.dtype([("row", "<i4"), ("first_slot", "<i4"), ("nslots", "<i4"),
                  ("reserved", "<i4")])


def floor_log2(deg: np.ndarray) -> np.ndarray:
    deg = np.asarray(deg, dtype=np.int64)
    b = np.full(deg.shape, -1, dtype=np.int64)
    for k in range(63):
        b += deg >= (np.int64(1) << k)
    return b            # -1 for deg == 0


def cuthill_mckee_rank(rowptr: np.ndarray, colidx: np.ndarray) -> np.ndarray:
    """Cuthill-McKee rank of each node of the undirected simple graph under the
    CSR (in- and out-neighbours, no self-loops, no repeats). Components start
    from the unvisited node of least degree (then least id); a visited node's
    unvisited neighbours are appended by (degree, id)."""
    rowptr = np.asarray(rowptr, dtype=np.int64)
    n = rowptr.size - 1
    dst = np.repeat(np.arange(n, dtype=np.int64), np.diff(rowptr))
    src = np.asarray(colidx, dtype=np.int64)
    keep = dst != src
    a = np.concatenate([dst[keep], src[keep]])
    b = np.concatenate([src[keep], dst[keep]])
    code = np.unique(a * max(n, 1) + b)
    u = code // max(n, 1)
    v = code - u * max(n, 1)
    deg = np.bincount(u, minlength=n).astype(np.int64)
    adj = [[] for _ in range(n)]
    for x, y in zip(u.tolist(), v.tolist()):
        adj[x].append(y)
    for x in range(n):
        adj[x].sort(key=lambda y: (deg[y], y))
    seeds = sorted(range(n), key=lambda y: (deg[y], y))
    seen = np.zeros(n, dtype=bool)
    order = []
    for s0 in seeds:
        if seen[s0]:
            continue
        seen[s0] = True
        head = len(order)
        order.append(s0)
        while head < len(order):
            x = order[head]
            head += 1
            for y in adj[x]:
                if not seen[y]:
                    seen[y] = True
                    order.append(y)
    rank = np.empty(n, dtype=np.int32)
    rank[np.asarray(order, dtype=np.int64)] = np.arange(n, dtype=np.int32)
    return rank


def work_list(ptr: np.ndarray, chunk: int, rank: np.ndarray | None = None):
    """Work items and split records; whole rows of a bin by ascending rank
    (ascending id without one)."""
    ptr = np.asarray(ptr, dtype=np.int64)
    n = ptr.size - 1
    deg = np.diff(ptr)
    rows = np.arange(n, dtype=np.int64)

    heavy = rows[deg > chunk]
    nk = (deg[heavy] + chunk - 1) // chunk
    first = np.concatenate([[0], np.cumsum(nk)[:-1]]).astype(np.int64) if heavy.size else np.zeros(0, np.int64)
    splits = np.zeros(heavy.size, dtype=SPLIT)
    splits["row"] = heavy
    splits["first_slot"] = first
    splits["nslots"] = nk

    crow = np.repeat(heavy, nk)
    k = np.arange(crow.size, dtype=np.int64) - np.repeat(first, nk)
    chunks = np.zeros(crow.size, dtype=WORK_ITEM)
    chunks["begin"] = ptr[crow] + k * chunk
    chunks["len"] = np.minimum(chunk, ptr[crow + 1] - chunks["begin"])
    chunks["row"] = crow
    chunks["slot"] = np.arange(crow.size)
    chunks["flags"] = (k == 0).astype(np.int32)

    light = rows[deg <= chunk]
    b = floor_log2(deg[light])
    key2 = light if rank is None else np.asarray(rank, dtype=np.int64)[light]
    order = np.lexsort((key2, -b))        # bin descending, then rank (or row) ascending
    light = light[order]
    whole = np.zeros(light.size, dtype=WORK_ITEM)
    whole["begin"] = ptr[light]
    whole["len"] = deg[light]
    whole["row"] = light
    whole["slot"] = -1
    whole["flags"] = 1
    return np.concatenate([chunks, whole]), splits, int(crow.size)


def transpose(rowptr: np.ndarray, colidx: np.ndarray, edge_ids: bool = False):
    """(colptr, rowidx) of the transposed CSR; with edge_ids also the CSR edge
    id of every transposed entry."""
    rowptr = np.asarray(rowptr, dtype=np.int64)
    colidx = np.asarray(colidx, dtype=np.int64)
    n = rowptr.size - 1
    dst = np.repeat(np.arange(n, dtype=np.int64), np.diff(rowptr))
    order = np.argsort(colidx, kind="stable")
    colptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(np.bincount(colidx, minlength=n), out=colptr[1:])
    if edge_ids:
        return colptr, dst[order].astype(np.int32), order.astype(np.int32)
    return colptr, dst[order].astype(np.int32)


def expand_pointer(ptr: np.ndarray) -> np.ndarray:
    """The row of every entry of a CSR-like pointer array."""
    ptr = np.asarray(ptr, dtype=np.int64)
    return np.repeat(np.arange(ptr.size - 1, dtype=np.int64), np.diff(ptr)).astype(np.int32)


def transposed_positions(col_edge: np.ndarray) -> np.ndarray:
    """Position in the transposed CSR of every CSR edge: entry q of the
    transposed CSR is CSR edge col_edge[q], so edge col_edge[q] sits at q."""
    col_edge = np.asarray(col_edge, dtype=np.int64)
    out = np.empty(col_edge.size, dtype=np.int32)
    out[col_edge] = np.arange(col_edge.size, dtype=np.int32)
    return out


def tiles(rowptr: np.ndarray, colidx: np.ndarray, min_nnz: int):
    rowptr = np.asarray(rowptr, dtype=np.int64)
    src = np.asarray(colidx, dtype=np.int64)
    n = rowptr.size - 1
    E = src.size
    nbr = (n + 15) // 16
    dst = np.repeat(np.arange(n, dtype=np.int64), np.diff(rowptr))
    pair = dst * max(n, 1) + src
    _, first_idx = np.unique(pair, return_index=True)
    is_first = np.zeros(E, dtype=bool)
    is_first[first_idx] = True

    nbc = max(nbr, 1)
    key = (dst // 16) * nbc + (src // 16)
    keys, counts = np.unique(key[is_first], return_counts=True)
    dense_keys = keys[counts >= min_nnz]
    pos = np.searchsorted(dense_keys, key)
    if dense_keys.size:
        in_dense = dense_keys[np.minimum(pos, dense_keys.size - 1)] == key
    else:
        in_dense = np.zeros(E, dtype=bool)
    in_tile = is_first & in_dense

    tile_rowptr = np.zeros(nbr + 1, dtype=np.int64)
    np.cumsum(np.bincount(dense_keys // nbc, minlength=nbr), out=tile_rowptr[1:])
    tile_col = (dense_keys % nbc).astype(np.int32)
    mask = np.zeros((dense_keys.size, 16), dtype=np.uint16)
    sel = np.nonzero(in_tile)[0]
    np.bitwise_or.at(mask, (pos[sel], dst[sel] % 16),
                     (np.uint16(1) << (src[sel] % 16).astype(np.uint16)).astype(np.uint16))

    res = ~in_tile
    res_rowptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(np.bincount(dst[res], minlength=n), out=res_rowptr[1:])
    res_colidx = src[res].astype(np.int32)
    return tile_rowptr, tile_col, mask.reshape(-1), res_rowptr, res_colidx, int(in_tile.sum())


def tile_columns(n: int, tile_rowptr: np.ndarray, tile_col: np.ndarray):
    nb = (n + 15) // 16
    tile_row = np.repeat(np.arange(nb, dtype=np.int64), np.diff(tile_rowptr)).astype(np.int32)
    order = np.lexsort((tile_row, tile_col))      # column, then row
    tile_colptr = np.zeros(nb + 1, dtype=np.int64)
    np.cumsum(np.bincount(tile_col, minlength=nb), out=tile_colptr[1:])
    return tile_row, tile_colptr, order.astype(np.int32)
