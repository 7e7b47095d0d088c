"""Node orderings for the graph reordering study: every ordering is a
permutation, and relabelling keeps the edge multiset and moves each node's
rows with it (CPU), and the library's results move with the labels (GPU)."""
import numpy as np
import pytest

import oracle
from sparse_graph_attention_csr_amd import inputs as I


def small_workload(seed=0):
    rng = np.random.default_rng(seed)
    rp, ci = I.random_csr(300, 12, rng, empty_frac=0.05, dup_frac=0.1, heavy_rows=2, heavy_deg=400)
    n = rp.size - 1
    t = {k: I.normal_tensor(rng, (n, 4, 64), I.BF16) for k in ("q", "k", "v", "dout")}
    return dict(rowptr=rp, colidx=ci, **t)


@pytest.mark.parametrize("kind", I.ORDERINGS)
def test_relabel_is_a_consistent_renaming(kind):
    w = small_workload()
    order = I.node_order(w["rowptr"], w["colidx"], kind)
    n = w["rowptr"].size - 1
    assert np.array_equal(np.sort(order), np.arange(n))
    r = I.relabel(w, order)
    new_id = np.empty(n, dtype=np.int64)
    new_id[order] = np.arange(n)
    dst = np.repeat(np.arange(n), np.diff(w["rowptr"]))
    a = np.sort(new_id[dst] * n + new_id[w["colidx"]])
    dst2 = np.repeat(np.arange(n), np.diff(r["rowptr"]))
    b = np.sort(dst2 * n + r["colidx"].astype(np.int64))
    assert np.array_equal(a, b)
    assert np.array_equal(r["q"][new_id], w["q"])
    if kind == "degree":
        assert np.all(np.diff(np.diff(r["rowptr"])) <= 0)


def test_relabel_equivariance_of_the_oracle():
    w = small_workload(1)
    r = I.relabel(w, I.node_order(w["rowptr"], w["colidx"], "rcm"))
    new_id = np.empty(w["rowptr"].size - 1, dtype=np.int64)
    new_id[r["order"]] = np.arange(new_id.size)
    o1, l1 = oracle.gt_fwd(w["rowptr"], w["colidx"], w["q"], w["k"], w["v"])
    o2, l2 = oracle.gt_fwd(r["rowptr"], r["colidx"], r["q"], r["k"], r["v"])
    assert np.abs(o2[new_id] - o1).max() <= 1e-12 * max(1.0, np.abs(o1).max())


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["degree", "rcm"])
def test_gpu_results_move_with_the_labels(kind):
    from tests.gpu_util import TOL, Runner, dev, host, note, rel_err
    note(f"reorder {kind}")
    w = small_workload(2)
    r = I.relabel(w, I.node_order(w["rowptr"], w["colidx"], kind))
    n = w["rowptr"].size - 1
    new_id = np.empty(n, dtype=np.int64)
    new_id[r["order"]] = np.arange(n)
    res = []
    for x in (w, r):
        run = Runner(x["rowptr"], x["colidx"], chunk=64)
        q, k, v, do = (dev(x[key]) for key in ("q", "k", "v", "dout"))
        out, lse = run.gt_fwd(q, k, v)
        res.append([host(t) for t in (out, lse, *run.gt_bwd(q, k, v, out, lse, do))])
    for a, b in zip(*res):
        assert rel_err(b[new_id], a) <= TOL["bf16"]
    ro, _ = oracle.gt_fwd(r["rowptr"], r["colidx"], r["q"], r["k"], r["v"])
    assert rel_err(res[1][0], ro) <= TOL["bf16"]
