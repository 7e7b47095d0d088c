"""Pins for the fp64 CPU oracle, from directions other than the oracle itself.

Each test states what fixes the expected value: a hand-derived closed form
(tests/golden), the masked dense matrix form, fp64 autograd of the dense form,
central finite differences, or an identity of the softmax (weights summing to
one, single-neighbour rows, permutation and relabelling invariance, the
uniform-attention closed form, the key-shift identity, the linear regime of
LeakyReLU, head independence).
"""
import os

import numpy as np
import pytest
import scipy.sparse as sp

from sparse_graph_attention_csr_amd import inputs as I
from tests import dense_ref as R

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / scale


def rand_graph(seed, n=30, max_deg=6, **kw):
    rng = np.random.default_rng(seed)
    return I.random_csr(n, max_deg, rng, **kw)


def feats(seed, n, H, D, scale=1.0):
    rng = np.random.default_rng(seed)
    return [scale * rng.standard_normal((n, H, D)) for _ in range(4)]


def read_golden(name):
    d = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            d[key] = np.array([float(x) for x in vals])
    return d


# ---------------------------------------------------------------------------
# hand-worked closed forms
# ---------------------------------------------------------------------------

def test_gt_golden_closed_form(oracle_mod):
    g = read_golden("gt_two_node_closed_form.txt")
    n, H, D = int(g["n"][0]), int(g["heads"][0]), int(g["dim"][0])
    rp, ci = g["rowptr"].astype(np.int64), g["colidx"].astype(np.int32)
    sh = (n, H, D)
    q, k, v, do = (g[x].reshape(sh) for x in ("q", "k", "v", "dout"))
    out, lse = oracle_mod.gt_fwd(rp, ci, q, k, v)
    np.testing.assert_allclose(out, g["out"].reshape(sh), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, g["lse"].reshape(n, H), rtol=0, atol=1e-15)
    dq, dk, dv = oracle_mod.gt_bwd(rp, ci, q, k, v, do)
    np.testing.assert_allclose(dq, g["dq"].reshape(sh), rtol=0, atol=1e-15)
    np.testing.assert_allclose(dk, g["dk"].reshape(sh), rtol=0, atol=1e-15)
    np.testing.assert_allclose(dv, g["dv"].reshape(sh), rtol=0, atol=1e-15)


def test_gat_golden_closed_form(oracle_mod):
    g = read_golden("gatv2_two_node_closed_form.txt")
    n, H, D = int(g["n"][0]), int(g["heads"][0]), int(g["dim"][0])
    slope = float(g["slope"][0])
    rp, ci = g["rowptr"].astype(np.int64), g["colidx"].astype(np.int32)
    sh = (n, H, D)
    xs, xt, do = (g[x].reshape(sh) for x in ("xs", "xt", "dout"))
    a = g["a"].reshape(H, D)
    out, lse = oracle_mod.gat_fwd(rp, ci, xs, xt, a, slope)
    np.testing.assert_allclose(out, g["out"].reshape(sh), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, g["lse"].reshape(n, H), rtol=0, atol=1e-14)
    dxs, dxt, da = oracle_mod.gat_bwd(rp, ci, xs, xt, a, do, slope)
    np.testing.assert_allclose(dxs, g["dxs"].reshape(sh), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dxt, g["dxt"].reshape(sh), rtol=0, atol=1e-14)
    np.testing.assert_allclose(da, g["da"].reshape(H, D), rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# dense forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["complete", "sparse", "multigraph_empty"])
def test_gt_matches_masked_dense(oracle_mod, case):
    n, H, D = 24, 3, 8
    if case == "complete":
        # every j -> i including i -> i: plain dense softmax attention
        rp = np.arange(0, n * n + 1, n, dtype=np.int64)
        ci = np.tile(np.arange(n, dtype=np.int32), n)
    elif case == "sparse":
        rp, ci = rand_graph(1, n=n, max_deg=7)
    else:
        rp, ci = rand_graph(2, n=n, max_deg=7, empty_frac=0.2, dup_frac=0.3)
    q, k, v, _ = feats(3, n, H, D)
    out, lse = oracle_mod.gt_fwd(rp, ci, q, k, v)
    ro, rl = R.gt_dense_np(rp, ci, q, k, v)
    assert rel(out, ro) < 1e-12
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin)
    assert rel(lse[fin], rl[fin]) < 1e-12


@pytest.mark.parametrize("case", ["complete", "multigraph_empty"])
def test_gat_matches_masked_dense(oracle_mod, case):
    n, H, D = 20, 2, 8
    if case == "complete":
        rp = np.arange(0, n * n + 1, n, dtype=np.int64)
        ci = np.tile(np.arange(n, dtype=np.int32), n)
    else:
        rp, ci = rand_graph(4, n=n, max_deg=6, empty_frac=0.2, dup_frac=0.3)
    xs, xt, _, _ = feats(5, n, H, D)
    a = np.random.default_rng(6).standard_normal((H, D)) / np.sqrt(D)
    out, lse = oracle_mod.gat_fwd(rp, ci, xs, xt, a, 0.2)
    ro, rl = R.gat_dense_np(rp, ci, xs, xt, a, 0.2)
    assert rel(out, ro) < 1e-12
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin)
    assert rel(lse[fin], rl[fin]) < 1e-12


def test_gt_backward_matches_dense_autograd(oracle_mod):
    n, H, D = 28, 2, 8
    rp, ci = rand_graph(7, n=n, max_deg=8, empty_frac=0.1, dup_frac=0.2)
    q, k, v, do = feats(8, n, H, D)
    dq, dk, dv = oracle_mod.gt_bwd(rp, ci, q, k, v, do)
    tq, tk, tv = R.gt_dense_grads_torch(rp, ci, q, k, v, do)
    assert rel(dq, tq) < 1e-10
    assert rel(dk, tk) < 1e-10
    assert rel(dv, tv) < 1e-10


def test_gat_backward_matches_dense_autograd(oracle_mod):
    n, H, D = 24, 2, 8
    rp, ci = rand_graph(9, n=n, max_deg=8, empty_frac=0.1, dup_frac=0.2)
    xs, xt, _, do = feats(10, n, H, D)
    a = np.random.default_rng(11).standard_normal((H, D)) / np.sqrt(D)
    dxs, dxt, da = oracle_mod.gat_bwd(rp, ci, xs, xt, a, do, 0.2)
    ts, tt, ta = R.gat_dense_grads_torch(rp, ci, xs, xt, a, do, 0.2)
    assert rel(dxs, ts) < 1e-10
    assert rel(dxt, tt) < 1e-10
    assert rel(da, ta) < 1e-10


# ---------------------------------------------------------------------------
# finite differences
# ---------------------------------------------------------------------------

def tiny_multigraph():
    # 7 nodes: a deg-1 row (row 1 <- 4), self-loops, a repeated edge (3 -> 0 twice),
    # an empty row (row 6) and a source (5) with several out-edges.
    rows = [[0, 3, 3, 5], [4], [2, 5, 0], [3, 1, 5, 6], [4, 5], [5, 2], []]
    rp = np.zeros(len(rows) + 1, dtype=np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.array([j for r in rows for j in r], dtype=np.int32)
    return rp, ci


def fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    flat = x.reshape(-1)
    gf = g.reshape(-1)
    for t in range(flat.size):
        old = flat[t]
        flat[t] = old + h
        fp = f()
        flat[t] = old - h
        fm = f()
        flat[t] = old
        gf[t] = (fp - fm) / (2 * h)
    return g


def test_gt_backward_finite_differences(oracle_mod):
    rp, ci = tiny_multigraph()
    n, H, D = 7, 2, 4
    q, k, v, do = feats(12, n, H, D)

    def loss():
        out, _ = oracle_mod.gt_fwd(rp, ci, q, k, v)
        return float((out * do).sum())

    dq, dk, dv = oracle_mod.gt_bwd(rp, ci, q, k, v, do)
    assert rel(dq, fd_grad(loss, q)) < 1e-6
    assert rel(dk, fd_grad(loss, k)) < 1e-6
    assert rel(dv, fd_grad(loss, v)) < 1e-6


def test_gat_backward_finite_differences(oracle_mod):
    rp, ci = tiny_multigraph()
    n, H, D = 7, 2, 4
    rng = np.random.default_rng(13)
    # keep every z = xs_i + xt_j away from the LeakyReLU kink
    while True:
        xs, xt, do = (rng.standard_normal((n, H, D)) for _ in range(3))
        z = xs[:, None] + xt[None, :]
        if np.abs(z).min() > 1e-3:
            break
    a = rng.standard_normal((H, D)) / 2

    def loss():
        out, _ = oracle_mod.gat_fwd(rp, ci, xs, xt, a, 0.2)
        return float((out * do).sum())

    dxs, dxt, da = oracle_mod.gat_bwd(rp, ci, xs, xt, a, do, 0.2)
    assert rel(dxs, fd_grad(loss, xs)) < 1e-6
    assert rel(dxt, fd_grad(loss, xt)) < 1e-6
    assert rel(da, fd_grad(loss, a)) < 1e-6


# ---------------------------------------------------------------------------
# identities of the softmax
# ---------------------------------------------------------------------------

def test_weights_sum_to_one(oracle_mod):
    n, H, D = 40, 2, 8
    rp, ci = rand_graph(14, n=n, max_deg=9, dup_frac=0.2)
    q, k, _, _ = feats(15, n, H, D, scale=3.0)
    ones = np.ones((n, H, D))
    out, _ = oracle_mod.gt_fwd(rp, ci, q, k, ones)
    assert np.abs(out - 1.0).max() < 1e-14
    # GATv2 aggregates Xt itself; a constant Xt makes every row's weights uniform
    xs = feats(16, n, H, D)[0]
    a = np.random.default_rng(17).standard_normal((H, D))
    out, lse = oracle_mod.gat_fwd(rp, ci, xs, 2.5 * ones, a, 0.2)
    assert np.abs(out - 2.5).max() < 1e-14


def test_single_neighbour_row(oracle_mod):
    n, H, D = 12, 2, 8
    rp = np.arange(n + 1, dtype=np.int64)
    ci = np.random.default_rng(18).integers(0, n, size=n).astype(np.int32)
    q, k, v, _ = feats(19, n, H, D)
    out, lse = oracle_mod.gt_fwd(rp, ci, q, k, v)
    assert np.array_equal(out, v[ci])
    s = np.einsum("nhd,nhd->nh", q, k[ci]) / np.sqrt(D)
    assert np.abs(lse - s).max() < 1e-14
    a = np.random.default_rng(20).standard_normal((H, D))
    out, _ = oracle_mod.gat_fwd(rp, ci, q, k, a, 0.2)
    assert np.array_equal(out, k[ci])


def test_neighbour_order_invariance(oracle_mod):
    n, H, D = 50, 2, 8
    rp, ci = rand_graph(21, n=n, max_deg=10, empty_frac=0.1, dup_frac=0.2)
    rng = np.random.default_rng(22)
    ci2 = ci.copy()
    for i in range(n):
        rng.shuffle(ci2[rp[i]:rp[i + 1]])
    q, k, v, do = feats(23, n, H, D)
    o1, l1 = oracle_mod.gt_fwd(rp, ci, q, k, v)
    o2, l2 = oracle_mod.gt_fwd(rp, ci2, q, k, v)
    assert rel(o1, o2) < 1e-12
    g1 = oracle_mod.gt_bwd(rp, ci, q, k, v, do)
    g2 = oracle_mod.gt_bwd(rp, ci2, q, k, v, do)
    for x, y in zip(g1, g2):
        assert rel(x, y) < 1e-12


def test_relabelling_equivariance(oracle_mod):
    n, H, D = 40, 2, 8
    rp, ci = rand_graph(24, n=n, max_deg=8, dup_frac=0.1)
    pi = np.random.default_rng(25).permutation(n)
    # node i becomes pi[i]; rebuild CSR for the relabelled graph
    dst = np.repeat(np.arange(n), np.diff(rp))
    rp2, ci2 = I.csr_from_edges(n, pi[dst], pi[ci], self_loops=False, dedup=False)
    q, k, v, do = feats(26, n, H, D)
    inv = np.argsort(pi)
    q2, k2, v2, do2 = q[inv], k[inv], v[inv], do[inv]   # row pi[i] holds old row i
    o1, l1 = oracle_mod.gt_fwd(rp, ci, q, k, v)
    o2, l2 = oracle_mod.gt_fwd(rp2, ci2, q2, k2, v2)
    assert rel(o2[pi], o1) < 1e-12
    assert rel(l2[pi], l1) < 1e-12
    g1 = oracle_mod.gt_bwd(rp, ci, q, k, v, do)
    g2 = oracle_mod.gt_bwd(rp2, ci2, q2, k2, v2, do2)
    for x, y in zip(g1, g2):
        assert rel(y[pi], x) < 1e-12


def test_uniform_attention_closed_form(oracle_mod):
    """Q = 0 (GT) or a = 0 (GATv2): every weight is 1/deg, out is the neighbour
    mean (a row-normalised sparse product), lse = ln(deg), and dV = A_norm^T dOut."""
    n, H, D = 60, 2, 8
    rp, ci = rand_graph(27, n=n, max_deg=9, empty_frac=0.1, dup_frac=0.2)
    deg = np.diff(rp).astype(np.float64)
    _, k, v, do = feats(28, n, H, D)
    q = np.zeros_like(k)
    vals = np.repeat(np.where(deg > 0, 1.0 / np.maximum(deg, 1), 0.0), np.diff(rp))
    A = sp.csr_matrix((vals, ci, rp), shape=(n, n))
    out, lse = oracle_mod.gt_fwd(rp, ci, q, k, v)
    for h in range(H):
        assert rel(out[:, h, :], A @ v[:, h, :]) < 1e-13
    nz = deg > 0
    assert np.abs(lse[nz] - np.log(deg[nz])[:, None]).max() < 1e-13
    dq, dk, dv = oracle_mod.gt_bwd(rp, ci, q, k, v, do)
    assert np.abs(dk).max() == 0.0
    for h in range(H):
        assert rel(dv[:, h, :], A.T @ do[:, h, :]) < 1e-13
    xs = feats(29, n, H, D)[0]
    out, lse = oracle_mod.gat_fwd(rp, ci, xs, v, np.zeros((H, D)), 0.2)
    for h in range(H):
        assert rel(out[:, h, :], A @ v[:, h, :]) < 1e-13
    assert np.abs(lse[nz] - np.log(deg[nz])[:, None]).max() < 1e-13


def test_key_shift_identity(oracle_mod):
    """K_j -> K_j + c for all j adds Q_i.c/sqrt(D) to every score of row i:
    out is unchanged and lse shifts by that amount; dV is unchanged."""
    n, H, D = 40, 2, 8
    rp, ci = rand_graph(30, n=n, max_deg=8, dup_frac=0.1)
    q, k, v, do = feats(31, n, H, D)
    c = np.random.default_rng(32).standard_normal((1, H, D))
    o1, l1 = oracle_mod.gt_fwd(rp, ci, q, k, v)
    o2, l2 = oracle_mod.gt_fwd(rp, ci, q, k + c, v)
    assert rel(o2, o1) < 1e-12
    assert np.abs(l2 - l1 - (q * c).sum(-1) / np.sqrt(D)).max() < 1e-12
    _, _, dv1 = oracle_mod.gt_bwd(rp, ci, q, k, v, do)
    _, _, dv2 = oracle_mod.gt_bwd(rp, ci, q, k + c, v, do)
    assert rel(dv2, dv1) < 1e-12


def test_gat_linear_regime(oracle_mod):
    """All Xs, Xt > 0: LeakyReLU is the identity, so alpha_ij = softmax_j(a.Xt_j)
    does not depend on Xs. All < 0: the scores are scaled by the slope."""
    n, H, D = 40, 2, 8
    rp, ci = rand_graph(33, n=n, max_deg=8)
    rng = np.random.default_rng(34)
    xs = rng.random((n, H, D)) + 0.1
    xt = rng.random((n, H, D)) + 0.1
    a = rng.standard_normal((H, D))
    at = np.einsum("jhd,hd->jh", xt, a)          # a_h . Xt_j
    out, lse = oracle_mod.gat_fwd(rp, ci, xs, xt, a, 0.2)
    out2, _ = oracle_mod.gat_fwd(rp, ci, 3 * xs, xt, a, 0.2)
    assert rel(out2, out) < 1e-12
    ref = np.zeros((n, H, D))
    for i in range(n):
        js = ci[rp[i]:rp[i + 1]]
        w = np.exp(at[js] - at[js].max(0))
        w /= w.sum(0)
        ref[i] = np.einsum("jh,jhd->hd", w, xt[js])
    assert rel(out, ref) < 1e-12
    # negative regime: score = slope * (a.Xs_i + a.Xt_j)
    outn, lsen = oracle_mod.gat_fwd(rp, ci, -xs, -xt, a, 0.2)
    as_ = np.einsum("ihd,hd->ih", -xs, a)
    for i in range(n):
        js = ci[rp[i]:rp[i + 1]]
        s = 0.2 * (as_[i][None, :] + np.einsum("jhd,hd->jh", -xt[js], a))
        m = s.max(0)
        assert np.abs(lsen[i] - (m + np.log(np.exp(s - m).sum(0)))).max() < 1e-12


def test_head_independence(oracle_mod):
    n, H, D = 30, 3, 8
    rp, ci = rand_graph(35, n=n, max_deg=8, dup_frac=0.1)
    q, k, v, do = feats(36, n, H, D)
    out, lse = oracle_mod.gt_fwd(rp, ci, q, k, v)
    dq, dk, dv = oracle_mod.gt_bwd(rp, ci, q, k, v, do)
    for h in range(H):
        sl = slice(h, h + 1)
        o, l = oracle_mod.gt_fwd(rp, ci, q[:, sl], k[:, sl], v[:, sl])
        assert np.array_equal(o, out[:, sl]) and np.array_equal(l, lse[:, sl])
        g = oracle_mod.gt_bwd(rp, ci, q[:, sl], k[:, sl], v[:, sl], do[:, sl])
        assert np.array_equal(g[0], dq[:, sl]) and np.array_equal(g[1], dk[:, sl])
        assert np.array_equal(g[2], dv[:, sl])


def test_empty_rows(oracle_mod):
    n, H, D = 10, 2, 4
    rp = np.array([0, 0, 2, 2, 3, 3, 3, 4, 4, 4, 4], dtype=np.int64)
    ci = np.array([1, 3, 5, 2], dtype=np.int32)
    q, k, v, do = feats(37, n, H, D)
    out, lse = oracle_mod.gt_fwd(rp, ci, q, k, v)
    empty = np.diff(rp) == 0
    assert np.all(out[empty] == 0) and np.all(np.isneginf(lse[empty]))
    dq, dk, dv = oracle_mod.gt_bwd(rp, ci, q, k, v, do)
    assert np.all(dq[empty] == 0)
    nosrc = np.bincount(ci, minlength=n) == 0
    assert np.all(dk[nosrc] == 0) and np.all(dv[nosrc] == 0)
    # a graph with no edges at all
    rp0 = np.zeros(n + 1, dtype=np.int64)
    ci0 = np.zeros(0, dtype=np.int32)
    out, lse = oracle_mod.gt_fwd(rp0, ci0, q, k, v)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_row_selection_matches_full(oracle_mod):
    n, H, D = 50, 2, 8
    rp, ci = rand_graph(38, n=n, max_deg=9)
    q, k, v, do = feats(39, n, H, D)
    rows = np.array([3, 0, 49, 17, 17])
    o, l = oracle_mod.gt_fwd(rp, ci, q, k, v)
    os_, ls = oracle_mod.gt_fwd(rp, ci, q, k, v, rows=rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls, l[rows])
    g = oracle_mod.gt_bwd(rp, ci, q, k, v, do)
    gs = oracle_mod.gt_bwd(rp, ci, q, k, v, do, dst_rows=rows, src_rows=rows[::-1])
    assert np.array_equal(gs[0], g[0][rows])
    assert np.array_equal(gs[1], g[1][rows[::-1]]) and np.array_equal(gs[2], g[2][rows[::-1]])
    a = np.random.default_rng(40).standard_normal((H, D))
    gg = oracle_mod.gat_bwd(rp, ci, q, k, a, do)
    ggs = oracle_mod.gat_bwd(rp, ci, q, k, a, do, dst_rows=rows, src_rows=rows)
    assert np.array_equal(ggs[0], gg[0][rows]) and np.array_equal(ggs[1], gg[1][rows])
    assert np.array_equal(ggs[2], gg[2])


def test_stored_types_widen_exactly(oracle_mod):
    """fp32 and bf16 inputs give the same result as their exact fp64 values."""
    n, H, D = 30, 2, 8
    rp, ci = rand_graph(41, n=n, max_deg=8)
    rng = np.random.default_rng(42)
    q32, k32, v32 = (rng.standard_normal((n, H, D)).astype(np.float32) for _ in range(3))
    o32, l32 = oracle_mod.gt_fwd(rp, ci, q32, k32, v32)
    o64, l64 = oracle_mod.gt_fwd(rp, ci, *(x.astype(np.float64) for x in (q32, k32, v32)))
    assert np.array_equal(o32, o64) and np.array_equal(l32, l64)
    bits = [I.f32_to_bf16_bits(x) for x in (q32, k32, v32)]
    widened = [(b.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for b in bits]
    ob, lb = oracle_mod.gt_fwd(rp, ci, *bits)
    ow, lw = oracle_mod.gt_fwd(rp, ci, *widened)
    assert np.array_equal(ob, ow) and np.array_equal(lb, lw)


def test_invalid_graph_rejected(oracle_mod):
    q = np.zeros((3, 1, 4))
    with pytest.raises(RuntimeError):
        oracle_mod.gt_fwd(np.array([0, 1, 2, 3]), np.array([0, 5, 1]), q, q, q)
