"""Host preprocessing (CSR validation, work lists, transposed CSR, 16x16 tiles):
the library's arrays must equal an independent numpy statement of the same
specification byte for byte, and satisfy the structural invariants."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import plan_spec as S
from sparse_graph_attention_csr_amd import binding as B
from sparse_graph_attention_csr_amd import inputs as I


def check_plan(rowptr, colidx, chunk, tmin=0, bs=False, loc=False, order=2):
    p = B.Plan(rowptr, colidx, chunk=chunk, tile_min_nnz=tmin, block_sparse=bs, locality=loc,
               edge_order=order)
    C = p.stats()["chunk"]
    rank = S.cuthill_mckee_rank(rowptr, colidx) if loc else None
    items, splits, nslots = S.work_list(rowptr, C, rank)
    assert p.export(B.ARR_ROW_ITEMS).tobytes() == items.tobytes()
    assert p.export(B.ARR_ROW_SPLITS).tobytes() == splits.tobytes()
    colptr, rowidx, col_edge = S.transpose(rowptr, colidx, edge_ids=True)
    assert np.array_equal(p.export(B.ARR_COLPTR), colptr)
    assert np.array_equal(p.export(B.ARR_ROWIDX), rowidx)
    assert np.array_equal(p.export(B.ARR_COL_EDGE), col_edge)
    # the inverse map is built for edge order 2 (and for 0 above 2^21 edges)
    tpos = p.export(B.ARR_ROW_TPOS)
    if order == 2:
        assert np.array_equal(tpos, S.transposed_positions(col_edge))
    else:
        assert tpos.size == 0
    citems, csplits, cslots = S.work_list(colptr, C, rank)
    assert p.export(B.ARR_COL_ITEMS).tobytes() == citems.tobytes()
    assert p.export(B.ARR_COL_SPLITS).tobytes() == csplits.tobytes()
    st_ = p.stats()
    assert st_["row_slots"] == nslots and st_["col_slots"] == cslots
    if bs:
        tr, tc, tm, rr, rc, te = S.tiles(rowptr, colidx, tmin or 32)
        assert np.array_equal(p.export(B.ARR_TILE_ROWPTR), tr)
        assert np.array_equal(p.export(B.ARR_TILE_COL), tc)
        assert np.array_equal(p.export(B.ARR_TILE_MASK), tm)
        assert np.array_equal(p.export(B.ARR_RES_ROWPTR), rr)
        assert np.array_equal(p.export(B.ARR_RES_COLIDX), rc)
        assert st_["tile_edges"] == te
        n = rowptr.size - 1
        trow, tcp, tbc = S.tile_columns(n, tr, tc)
        assert np.array_equal(p.export(B.ARR_TILE_ROW), trow)
        assert np.array_equal(p.export(B.ARR_TILE_COLPTR), tcp)
        assert np.array_equal(p.export(B.ARR_TILE_BYCOL), tbc)
        rcp, rri, rce = S.transpose(rr, rc, edge_ids=True)
        assert np.array_equal(p.export(B.ARR_RES_COLPTR), rcp)
        assert np.array_equal(p.export(B.ARR_RES_ROWIDX), rri)
        assert np.array_equal(p.export(B.ARR_RES_COL_EDGE), rce)
        assert np.array_equal(p.export(B.ARR_RES_ROW), S.expand_pointer(rr))
        assert np.array_equal(p.export(B.ARR_RES_COLSRC), S.expand_pointer(rcp))
        assert np.array_equal(p.export(B.ARR_TILE_ROW_BYCOL), trow[tbc])
    return p


def invariants(p, rowptr, colidx):
    n = rowptr.size - 1
    E = colidx.size
    deg = np.diff(rowptr)
    for arr, ptr in ((B.ARR_ROW_ITEMS, rowptr), (B.ARR_COL_ITEMS, p.export(B.ARR_COLPTR))):
        items = p.export(arr)
        # every edge covered exactly once, every row present
        cover = np.zeros(E, dtype=np.int64)
        for it in items:
            cover[it["begin"]:it["begin"] + it["len"]] += 1
        assert np.all(cover == 1)
        assert set(items["row"].tolist()) == set(range(n))
        lens = np.bincount(items["row"], weights=items["len"], minlength=n)
        assert np.array_equal(lens.astype(np.int64), np.diff(ptr))
    # the transposed CSR is a permutation of the edge multiset
    colptr = p.export(B.ARR_COLPTR)
    rowidx = p.export(B.ARR_ROWIDX)
    dst = np.repeat(np.arange(n), deg)
    a = np.sort(dst.astype(np.int64) * n + colidx)
    b = np.sort(rowidx.astype(np.int64) * n + np.repeat(np.arange(n), np.diff(colptr)))
    assert np.array_equal(a, b)
    # each transposed entry names its CSR edge: same source and destination
    ce = p.export(B.ARR_COL_EDGE)
    assert np.array_equal(np.sort(ce), np.arange(E))
    assert np.array_equal(colidx[ce], np.repeat(np.arange(n), np.diff(colptr)))
    assert np.array_equal(dst[ce], rowidx)


GRAPHS = {
    "random": dict(n=60, max_deg=12),
    "empty_rows_dups": dict(n=70, max_deg=9, empty_frac=0.3, dup_frac=0.3),
    "heavy": dict(n=50, max_deg=5, heavy_rows=3, heavy_deg=140),
    "ragged_n": dict(n=37, max_deg=30, heavy_rows=2, heavy_deg=37),
}


@pytest.mark.parametrize("name", list(GRAPHS))
@pytest.mark.parametrize("chunk", [1, 7, 16, 0])
@pytest.mark.parametrize("loc", [False, True])
def test_plan_matches_spec(name, chunk, loc):
    rp, ci = I.random_csr(rng=np.random.default_rng(sum(map(ord, name))), **GRAPHS[name])
    p = check_plan(rp, ci, chunk, tmin=3, bs=True, loc=loc, order=2 if chunk else 1)
    invariants(p, rp, ci)


def test_transposed_positions_invert_the_transpose():
    """Every CSR edge p sits at position tpos[p] of the transposed CSR: same
    source and destination there, and tpos is a permutation."""
    rp, ci = I.random_csr(200, 15, np.random.default_rng(5), empty_frac=0.1, dup_frac=0.2)
    p = B.Plan(rp, ci, edge_order=2)
    tpos = p.export(B.ARR_ROW_TPOS).astype(np.int64)
    n, E = rp.size - 1, ci.size
    assert np.array_equal(np.sort(tpos), np.arange(E))
    colptr, rowidx = p.export(B.ARR_COLPTR), p.export(B.ARR_ROWIDX)
    src_of_pos = np.repeat(np.arange(n), np.diff(colptr))
    assert np.array_equal(src_of_pos[tpos], ci)
    assert np.array_equal(rowidx[tpos], np.repeat(np.arange(n), np.diff(rp)))
    # automatic order: no map for a small graph
    assert B.Plan(rp, ci).export(B.ARR_ROW_TPOS).size == 0


def test_cuthill_mckee_visits_components_breadth_first():
    # two components: a path 0-1-2-3 and a star 4-(5,6,7); self-loops ignored
    rows = [[1], [0, 2], [1, 3, 3], [2, 3], [5, 6, 7], [4], [4], [4, 7]]
    rp = np.zeros(len(rows) + 1, dtype=np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.array([j for r in rows for j in r], dtype=np.int32)
    rank = S.cuthill_mckee_rank(rp, ci)
    order = np.argsort(rank)
    # least degree first (node 0, degree 1; ties by id), then breadth first
    assert order.tolist()[:4] == [0, 1, 2, 3]
    assert set(order.tolist()[4:]) == {4, 5, 6, 7} and order[4] == 5
    check_plan(rp, ci, 0, loc=True)


def test_plan_on_workload_graph():
    rp, ci, _ = I.make_graph("gt_er1k_h4d32_f32")
    for chunk in (4, 8, 0):
        for tmin in (1, 2, 32):
            check_plan(rp, ci, chunk, tmin=tmin, bs=True)


def test_dense_community_tiles():
    # four fully connected 16-node blocks plus a few cross edges: every block a tile
    n = 64
    dst, src = [], []
    for c in range(4):
        for i in range(16):
            for j in range(16):
                dst.append(16 * c + i)
                src.append(16 * c + j)
    dst += [0, 1, 63]
    src += [40, 50, 2]
    rp, ci = I.csr_from_edges(n, np.array(dst), np.array(src), self_loops=False)
    p = check_plan(rp, ci, 0, tmin=16, bs=True)
    s = p.stats()
    assert s["tiles"] == 4 and s["tile_edges"] == 4 * 256 and s["residual_edges"] == 3
    assert np.all(p.export(B.ARR_TILE_MASK) == 0xFFFF)


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 40), max_deg=st.integers(1, 25), chunk=st.integers(1, 20),
       tmin=st.integers(1, 40), empty=st.floats(0, 0.5), dup=st.floats(0, 0.5),
       seed=st.integers(0, 2**31 - 1))
def test_plan_property(n, max_deg, chunk, tmin, empty, dup, seed):
    rp, ci = I.random_csr(n, max_deg, np.random.default_rng(seed), empty_frac=empty, dup_frac=dup)
    p = check_plan(rp, ci, chunk, tmin=tmin, bs=True, loc=bool(seed & 1))
    invariants(p, rp, ci)
    s = p.stats()
    assert s["tile_edges"] + s["residual_edges"] == ci.size


def test_empty_graphs():
    for n in (0, 5):
        rp = np.zeros(n + 1, dtype=np.int64)
        ci = np.zeros(0, dtype=np.int32)
        p = check_plan(rp, ci, 0, tmin=1, bs=True)
        assert p.stats()["row_items"] == n


@pytest.mark.parametrize("case", ["first", "monotone", "last", "col_hi", "col_neg"])
def test_invalid_csr_rejected(case):
    rp = np.array([0, 2, 3, 5], dtype=np.int64)
    ci = np.array([0, 1, 2, 1, 0], dtype=np.int32)
    if case == "first":
        rp = rp + 1
    elif case == "monotone":
        rp = np.array([0, 3, 2, 5])
    elif case == "last":
        ci = ci[:4]
    elif case == "col_hi":
        ci = ci.copy(); ci[2] = 3
    else:
        ci = ci.copy(); ci[0] = -1
    with pytest.raises(B.SgatError) as e:
        B.Plan(rp, ci)
    assert e.value.status == 2


def test_invalid_options_rejected():
    rp = np.array([0, 1], dtype=np.int64)
    ci = np.array([0], dtype=np.int32)
    for kw in (dict(chunk=-1), dict(tile_min_nnz=-2), dict(tile_min_nnz=257),
               dict(edge_order=3), dict(edge_order=-1)):
        with pytest.raises(B.SgatError) as e:
            B.Plan(rp, ci, **kw)
        assert e.value.status == 1
