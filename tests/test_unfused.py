"""The unfused comparison formulations compute the same functions as the fused
library: run on the CPU in fp64, their forwards and torch.autograd backwards
match the fp64 oracle (so the latency and peak-memory ratios compare like
with like). CPU only."""
import numpy as np
import pytest
import torch

import bench_unfused as U
from sparse_graph_attention_csr_amd import inputs as I


def graph(seed):
    rng = np.random.default_rng(seed)
    return I.random_csr(120, 12, rng, empty_frac=0.1, dup_frac=0.1, heavy_rows=2, heavy_deg=90)


def t64(x, grad=True):
    return torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=grad)


@pytest.mark.parametrize("seed", [1, 2])
def test_unfused_gt_matches_oracle(oracle_mod, seed):
    rp, ci = graph(seed)
    n, H, D = rp.size - 1, 3, 16
    rng = np.random.default_rng(seed + 10)
    q, k, v, do = (rng.standard_normal((n, H, D)).astype(np.float32) for _ in range(4))
    dst, src = U.edge_index(torch.from_numpy(rp), torch.from_numpy(ci))
    Q, K, V = t64(q), t64(k), t64(v)
    out, lse = U.gt(dst, src, Q, K, V)
    (out * t64(do, False)).sum().backward()
    ro, rl = oracle_mod.gt_fwd(rp, ci, q, k, v)
    np.testing.assert_allclose(out.detach().numpy(), ro, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse.numpy()), np.isneginf(rl))
    fin = np.isfinite(rl)
    np.testing.assert_allclose(lse.numpy()[fin], rl[fin], rtol=0, atol=1e-12)
    for t, r in zip((Q, K, V), oracle_mod.gt_bwd(rp, ci, q, k, v, do)):
        np.testing.assert_allclose(t.grad.numpy(), r, rtol=0, atol=1e-11)


def test_unfused_gatv2_matches_oracle(oracle_mod):
    rp, ci = graph(3)
    n, H, D = rp.size - 1, 2, 16
    rng = np.random.default_rng(13)
    xs, xt, do = (rng.standard_normal((n, H, D)).astype(np.float32) for _ in range(3))
    a = (rng.standard_normal((H, D)) / 4).astype(np.float32)
    dst, src = U.edge_index(torch.from_numpy(rp), torch.from_numpy(ci))
    Xs, Xt, A = t64(xs), t64(xt), t64(a)
    out, lse = U.gatv2(dst, src, Xs, Xt, A, 0.2)
    (out * t64(do, False)).sum().backward()
    ro, rl = oracle_mod.gat_fwd(rp, ci, xs, xt, a, 0.2)
    np.testing.assert_allclose(out.detach().numpy(), ro, rtol=0, atol=1e-12)
    for t, r in zip((Xs, Xt, A), oracle_mod.gat_bwd(rp, ci, xs, xt, a, do, 0.2)):
        np.testing.assert_allclose(t.grad.numpy(), r, rtol=0, atol=1e-10)


@pytest.mark.parametrize("op", ["min", "max"])
def test_unfused_minmax_matches_oracle(oracle_mod, op):
    rp, ci = graph(4)
    n, F = rp.size - 1, 9
    for i in range(n):                       # distinct sources per row: no ties
        row = ci[rp[i]:rp[i + 1]]
        ci[rp[i]:rp[i + 1]] = np.random.default_rng(i).permutation(n)[:row.size]
    rng = np.random.default_rng(14)
    x, do = rng.standard_normal((n, F)), rng.standard_normal((n, F))
    dst, src = U.edge_index(torch.from_numpy(rp), torch.from_numpy(ci))
    X = t64(x)
    out = U.minmax(dst, src, X, op)
    (out * t64(do, False)).sum().backward()
    ro, ra = oracle_mod.reduce_fwd(rp, ci, x, op)
    np.testing.assert_array_equal(out.detach().numpy(), ro)
    np.testing.assert_allclose(X.grad.numpy(), oracle_mod.reduce_bwd(rp, ci, ra, do), rtol=0,
                               atol=1e-14)
