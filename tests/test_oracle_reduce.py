"""Pins for the oracle's min/max reduction aggregation (CPU only).

Each test fixes the expected result from outside the oracle: a hand-worked
multigraph with ties (tests/golden), numpy's own minimum/maximum and
argmin/argmax (which return the first occurrence, the tie rule) row by row,
torch.autograd of the masked dense form on tie-free inputs, central finite
differences (exact for a piecewise-linear function away from ties), the
identity max(x) = -min(-x) with the same winners, and conservation of the
gradient (each (i, f) with a winner passes dout[i, f] to exactly one source).
"""
import numpy as np
import pytest
import torch

from sparse_graph_attention_csr_amd import inputs as I
from tests.test_oracle import read_golden


def graph(seed, n=40, max_deg=7, **kw):
    return I.random_csr(n, max_deg, np.random.default_rng(seed), **kw)


@pytest.mark.parametrize("op", ["min", "max"])
def test_reduce_golden_ties(oracle_mod, op):
    g = read_golden("minmax_ties_by_hand.txt")
    n, F = int(g["n"][0]), int(g["feat"][0])
    rp, ci = g["rowptr"].astype(np.int64), g["colidx"].astype(np.int32)
    x = g["x"].reshape(n, F)
    out, arg = oracle_mod.reduce_fwd(rp, ci, x, op)
    np.testing.assert_array_equal(out, g[f"{op}_out"].reshape(n, F))
    np.testing.assert_array_equal(arg, g[f"{op}_arg"].reshape(n, F).astype(np.int64))
    dx = oracle_mod.reduce_bwd(rp, ci, arg, g["dout"].reshape(n, F))
    np.testing.assert_array_equal(dx, g[f"{op}_dx"].reshape(n, F))


@pytest.mark.parametrize("op", ["min", "max"])
@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_reduce_matches_numpy_first_occurrence(oracle_mod, op, dtype):
    """Few distinct values, so ties are everywhere; np.argmin/argmax pick the
    first occurrence."""
    rp, ci = graph(1, empty_frac=0.15, dup_frac=0.3, heavy_rows=2, heavy_deg=50)
    n, F = rp.size - 1, 13
    rng = np.random.default_rng(2)
    xv = rng.integers(-3, 4, size=(n, F)).astype(np.float64) / 2
    x = {"f64": xv, "f32": xv.astype(np.float32), "bf16": I.f32_to_bf16_bits(xv.astype(np.float32))}[dtype]
    out, arg = oracle_mod.reduce_fwd(rp, ci, x, op)
    red, pick = (np.min, np.argmin) if op == "min" else (np.max, np.argmax)
    for i in range(n):
        b, e = rp[i], rp[i + 1]
        if b == e:
            assert np.all(out[i] == 0) and np.all(arg[i] == -1)
            continue
        rows = xv[ci[b:e]]
        np.testing.assert_array_equal(out[i], red(rows, axis=0))
        np.testing.assert_array_equal(arg[i], b + pick(rows, axis=0))


def test_reduce_row_selection(oracle_mod):
    rp, ci = graph(3, empty_frac=0.1)
    x = np.random.default_rng(4).standard_normal((rp.size - 1, 8))
    out, arg = oracle_mod.reduce_fwd(rp, ci, x, "min")
    sel = np.array([5, 0, 17, 17, 39])
    o2, a2 = oracle_mod.reduce_fwd(rp, ci, x, "min", rows=sel)
    np.testing.assert_array_equal(o2, out[sel])
    np.testing.assert_array_equal(a2, arg[sel])


def test_max_is_negated_min(oracle_mod):
    rp, ci = graph(5, empty_frac=0.1, dup_frac=0.2)
    x = np.random.default_rng(6).integers(-2, 3, size=(rp.size - 1, 9)).astype(np.float64)
    mo, ma = oracle_mod.reduce_fwd(rp, ci, -x, "min")
    xo, xa = oracle_mod.reduce_fwd(rp, ci, x, "max")
    np.testing.assert_array_equal(xa, ma)
    np.testing.assert_array_equal(xo, -mo + 0.0)


def dense_mask(rp, ci, n):
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        m[i, ci[rp[i]:rp[i + 1]]] = True
    return m


@pytest.mark.parametrize("op", ["min", "max"])
def test_reduce_backward_matches_dense_autograd(oracle_mod, op):
    """Simple graph (no repeated edges) and continuous values: no ties, so the
    subgradient torch.amin/amax returns is the one the definition gives."""
    rp, ci = graph(7, n=30, empty_frac=0.1)
    n, F = rp.size - 1, 6
    for i in range(n):               # drop repeated edges of each row
        s = np.unique(ci[rp[i]:rp[i + 1]])
        ci[rp[i]:rp[i] + s.size] = s
        ci[rp[i] + s.size:rp[i + 1]] = -1
    keep = ci >= 0
    deg = np.add.reduceat(keep.astype(np.int64), rp[:-1]) * (np.diff(rp) > 0)
    rp = np.concatenate([[0], np.cumsum(deg)]).astype(np.int64)
    ci = ci[keep].astype(np.int32)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((n, F))
    dout = rng.standard_normal((n, F))
    out, arg = oracle_mod.reduce_fwd(rp, ci, x, op)
    dx = oracle_mod.reduce_bwd(rp, ci, arg, dout)

    m = torch.tensor(dense_mask(rp, ci, n))
    X = torch.tensor(x, requires_grad=True)
    fill = float("inf") if op == "min" else float("-inf")
    G = torch.where(m[:, :, None], X[None, :, :], torch.tensor(fill, dtype=torch.float64))
    R = G.amin(1) if op == "min" else G.amax(1)
    has = m.any(1)[:, None]
    R = torch.where(has, R, torch.zeros_like(R))
    (R * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(out, R.detach().numpy(), rtol=0, atol=0)
    np.testing.assert_allclose(dx, X.grad.numpy(), rtol=0, atol=1e-14)


def test_reduce_backward_finite_differences(oracle_mod):
    rp, ci = graph(9, n=25, empty_frac=0.1, dup_frac=0.2)
    n, F = rp.size - 1, 5
    rng = np.random.default_rng(10)
    x = rng.standard_normal((n, F))
    dout = rng.standard_normal((n, F))
    _, arg = oracle_mod.reduce_fwd(rp, ci, x, "min")
    dx = oracle_mod.reduce_bwd(rp, ci, arg, dout)
    h = 1e-7
    for j, f in [(0, 0), (3, 2), (7, 4), (11, 1), (24, 3)]:
        xp, xm = x.copy(), x.copy()
        xp[j, f] += h
        xm[j, f] -= h
        lp = (oracle_mod.reduce_fwd(rp, ci, xp, "min")[0] * dout).sum()
        lm = (oracle_mod.reduce_fwd(rp, ci, xm, "min")[0] * dout).sum()
        assert abs((lp - lm) / (2 * h) - dx[j, f]) <= 1e-6 * (1 + abs(dx[j, f]))


def test_reduce_gradient_is_conserved(oracle_mod):
    rp, ci = graph(11, empty_frac=0.2, dup_frac=0.3)
    n, F = rp.size - 1, 7
    rng = np.random.default_rng(12)
    x = rng.integers(-2, 3, size=(n, F)).astype(np.float64)
    dout = rng.standard_normal((n, F))
    _, arg = oracle_mod.reduce_fwd(rp, ci, x, "max")
    dx = oracle_mod.reduce_bwd(rp, ci, arg, dout)
    has = (np.diff(rp) > 0)[:, None]
    np.testing.assert_allclose(dx.sum(0), (dout * has).sum(0), rtol=1e-13, atol=1e-13)


def test_reduce_bwd_rejects_foreign_winner(oracle_mod):
    rp = np.array([0, 1, 2], dtype=np.int64)
    ci = np.array([1, 0], dtype=np.int32)
    arg = np.array([[1], [1]], dtype=np.int64)      # edge 1 belongs to row 1, not row 0
    with pytest.raises(RuntimeError):
        oracle_mod.reduce_bwd(rp, ci, arg, np.ones((2, 1)))
