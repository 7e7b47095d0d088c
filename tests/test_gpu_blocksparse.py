"""GPU parity of the block-sparse (16x16 tiles on bf16 MFMA) path.

The tile path is a different execution of the same result: it must match the
fp64 oracle within the bf16 bar and agree with the gather path, for several
tile thresholds (including tau = 1, where every occupied tile is dense, and a
tau so high that every edge is residual), ragged N, repeated edges, empty rows
and head counts that are not a multiple of the four waves of a workgroup."""
import numpy as np
import pytest

import oracle
from sparse_graph_attention_csr_amd import inputs as I
from tests.gpu_util import TOL, TOL_LSE, Runner, dev, host, note, rel_err, widen

pytestmark = pytest.mark.gpu


def community_graph(n_comm, seed, extra_dup=False, empty_rows=0):
    rng = np.random.default_rng(seed)
    dst, src = I.community_pairs(n_comm, 64, 0.5, 2, rng)
    n = n_comm * 64
    if extra_dup:
        k = rng.integers(0, dst.size, size=dst.size // 20)
        dst, src = np.concatenate([dst, dst[k]]), np.concatenate([src, src[k]])
    rp, ci = I.csr_from_edges(n, dst, src, self_loops=True, dedup=not extra_dup)
    if empty_rows:
        keep = np.ones(n, dtype=bool)
        keep[rng.choice(n, size=empty_rows, replace=False)] = False
        deg = np.diff(rp) * keep
        ci = np.concatenate([ci[rp[i]:rp[i + 1]] for i in range(n) if keep[i]]).astype(np.int32)
        rp = np.zeros(n + 1, dtype=np.int64)
        np.cumsum(deg, out=rp[1:])
    return rp, ci


def run_tiles(r, q, k, v):
    import torch
    B, g = r.B, r.g
    n, H, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((n, H), dtype=torch.float32, device=q.device)
    ws = g.workspace(B.OP_GT_FWD, H, D, B.BF16)
    B.gt_fwd(g.plan, g.rowptr, g.colidx, q, k, v, out, lse, ws, use_tiles=True)
    return out, lse


def run_tiles_bwd(r, q, k, v, out, lse, do):
    import torch
    B, g = r.B, r.g
    n, H, D = q.shape
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = g.workspace(B.OP_GT_BWD, H, D, B.BF16)
    B.gt_bwd(g.plan, g.rowptr, g.colidx, q, k, v, out, lse, do, dq, dk, dv, ws, use_tiles=True)
    return dq, dk, dv


def check_bwd(r, rp, ci, q, k, v, do, out, lse):
    """Tile backward vs the oracle and vs the gather backward on the same inputs."""
    Q, K, V, DO = dev(q), dev(k), dev(v), dev(do)
    g = [host(x) for x in run_tiles_bwd(r, Q, K, V, out, lse, DO)]
    ref = oracle.gt_bwd(rp, ci, q, k, v, do)
    for x, y in zip(g, ref):
        assert rel_err(x, y) <= TOL["bf16"]
    gather = [host(x) for x in r.gt_bwd(Q, K, V, out, lse, DO)]
    for x, y in zip(g, gather):
        assert rel_err(x, y) <= TOL["bf16"]


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("H", [1, 4, 5, 16])
def test_tiles_match_oracle(H, D):
    """Each wave owns one head of a block: H = 5 puts three idle waves in a
    block's second workgroup, H = 16 (the largest H) gives each block four."""
    note(f"tiles community H={H} D={D}")
    rp, ci = community_graph(8, seed=H * 10 + D)
    n = rp.size - 1
    rng = np.random.default_rng(3)
    q, k, v, do = (I.normal_tensor(rng, (n, H, D), I.BF16) for _ in range(4))
    r = Runner(rp, ci, block_sparse=True)
    s = r.g.plan.stats()
    assert s["tiles"] > 0 and s["residual_edges"] > 0
    out, lse = run_tiles(r, dev(q), dev(k), dev(v))
    ro, rl = oracle.gt_fwd(rp, ci, q, k, v)
    assert rel_err(host(out), ro) <= TOL["bf16"]
    assert rel_err(host(lse), rl) <= TOL_LSE
    go, gl = r.gt_fwd(dev(q), dev(k), dev(v))
    assert rel_err(host(out), host(go)) <= TOL["bf16"]
    check_bwd(r, rp, ci, q, k, v, do, out, lse)


@pytest.mark.parametrize("tmin", [1, 8, 32, 200])
def test_tiles_thresholds_ragged_dups_empty(tmin):
    note(f"tiles tau={tmin}, ragged n, repeats, empty rows")
    rp, ci = community_graph(5, seed=tmin, extra_dup=True, empty_rows=7)
    # drop the last 13 nodes' rows and edges to make N not a multiple of 16
    n = rp.size - 1 - 13
    keep_e = rp[n]
    ci = ci[:keep_e]
    rp = rp[:n + 1]
    ci = np.where(ci < n, ci, ci % n).astype(np.int32)
    H, D = 4, 64
    rng = np.random.default_rng(4)
    q, k, v, do = (I.normal_tensor(rng, (n, H, D), I.BF16) for _ in range(4))
    r = Runner(rp, ci, block_sparse=True, tile_min_nnz=tmin)
    out, lse = run_tiles(r, dev(q), dev(k), dev(v))
    ro, rl = oracle.gt_fwd(rp, ci, q, k, v)
    assert rel_err(host(out), ro) <= TOL["bf16"]
    assert rel_err(host(lse), rl) <= TOL_LSE
    empty = np.diff(rp) == 0
    assert empty.any() and np.all(host(out)[empty] == 0)
    check_bwd(r, rp, ci, q, k, v, do, out, lse)


def test_tiles_random_graph_and_single_neighbour():
    note("tiles on a random graph; one-edge rows")
    rng = np.random.default_rng(5)
    rp, ci = I.random_csr(333, 30, rng, empty_frac=0.05, dup_frac=0.1)
    H, D = 3, 128
    q, k, v, do = (I.normal_tensor(rng, (333, H, D), I.BF16) for _ in range(4))
    r = Runner(rp, ci, block_sparse=True, tile_min_nnz=2)
    out, lse = run_tiles(r, dev(q), dev(k), dev(v))
    ro, rl = oracle.gt_fwd(rp, ci, q, k, v)
    assert rel_err(host(out), ro) <= TOL["bf16"]
    assert rel_err(host(lse), rl) <= TOL_LSE
    check_bwd(r, rp, ci, q, k, v, do, out, lse)
    # every row with one in-edge: weight 1 exactly, out = that neighbour's V
    n = 200
    rp1 = np.arange(n + 1, dtype=np.int64)
    ci1 = rng.integers(0, n, size=n).astype(np.int32)
    q, k, v = (I.normal_tensor(rng, (n, 4, 64), I.BF16) for _ in range(3))
    r = Runner(rp1, ci1, block_sparse=True, tile_min_nnz=1)
    out, _ = run_tiles(r, dev(q), dev(k), dev(v))
    assert np.array_equal(host(out), widen(v)[ci1])


def test_tiles_bitwise_deterministic():
    note("tiles determinism")
    rp, ci = community_graph(4, seed=9)
    n = rp.size - 1
    rng = np.random.default_rng(6)
    q, k, v, do = (dev(I.normal_tensor(rng, (n, 4, 128), I.BF16)) for _ in range(4))
    r = Runner(rp, ci, block_sparse=True)
    res = []
    for _ in range(2):
        out, lse = run_tiles(r, q, k, v)
        res.append([host(x) for x in (out, lse, *run_tiles_bwd(r, q, k, v, out, lse, do))])
    assert all(np.array_equal(x, y) for x, y in zip(*res))


def test_tiles_rejected_without_layout_or_fp32():
    import torch
    from sparse_graph_attention_csr_amd import binding as B
    rp, ci = community_graph(2, seed=1)
    n = rp.size - 1
    r = Runner(rp, ci)              # no tile layout built
    q = torch.zeros(n, 4, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.SgatError) as e:
        run_tiles(r, q, q, q)
    assert e.value.status == 8
    r = Runner(rp, ci, block_sparse=True)
    q32 = torch.zeros(n, 4, 64, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q32)
    lse = torch.empty(n, 4, device="cuda")
    with pytest.raises(B.SgatError) as e:
        B.gt_fwd(r.g.plan, r.g.rowptr, r.g.colidx, q32, q32, q32, out, lse,
                 r.g.workspace(B.OP_GT_FWD, 4, 64, B.F32), use_tiles=True)
    assert e.value.status == 8
