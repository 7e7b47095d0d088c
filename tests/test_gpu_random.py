"""Seeded randomized parity sweeps. The gather path: small graphs of random size and degree mix
(empty rows, single-edge rows, rows just under and over the short-item bound
and the chunk size, repeated edges), random layouts among those compiled,
random chunk sizes and GATv2 slopes; the Graph Transformer and GATv2 forward
and backward of each against the fp64 oracle, every output element.

Bar: the same as the fixed parity cases (max |gpu - oracle| / max |oracle|
<= 1e-4 for fp32 inputs, <= 2e-2 for bf16; lse <= 1e-4), except for gradients
that vanish exactly: GATv2's dXs at slope 1, and on graphs whose rows each have
one distinct in-neighbour dQ, dK, dXs and da, which are held to the dV or dXt
scale instead. The tile path:
random 16x16-block structures with random tile thresholds and layouts. Min/max
aggregation: random graphs, widths, dtypes, operations and chunk sizes.

SGAT_RANDOM_FIRST and SGAT_RANDOM_SCALE (environment, default 0 and 1) move
the case numbers and multiply the case counts, for a longer sweep on other
seeds; the defaults are the cases the suite runs."""
import os

import numpy as np
import pytest

import oracle
from sparse_graph_attention_csr_amd import inputs as I
from tests.gpu_util import TOL, TOL_LSE, Runner, dev, host, note, rel_err

pytestmark = pytest.mark.gpu

FIRST = int(os.environ.get("SGAT_RANDOM_FIRST", "0"))
SCALE = int(os.environ.get("SGAT_RANDOM_SCALE", "1"))


def cases(n):
    return range(FIRST, FIRST + n * SCALE)


LAYOUTS = [("f32", 4, 32), ("f32", 2, 64), ("f32", 1, 128), ("f32", 3, 64),
           ("bf16", 4, 128), ("bf16", 8, 64), ("bf16", 2, 64), ("bf16", 1, 32),
           ("bf16", 5, 32), ("bf16", 16, 128), ("bf16", 3, 64), ("bf16", 16, 64)]


def random_graph(rng):
    n = int(rng.integers(1, 700))
    kinds = rng.choice(5, size=n, p=[0.1, 0.15, 0.5, 0.15, 0.1])
    deg = np.where(kinds == 0, 0,
          np.where(kinds == 1, 1,
          np.where(kinds == 2, rng.integers(2, 40, size=n),
          np.where(kinds == 3, rng.integers(120, 136, size=n), rng.integers(200, 1500, size=n)))))
    rp = np.zeros(n + 1, dtype=np.int64)
    rp[1:] = np.cumsum(deg)
    ci = rng.integers(0, n, size=int(rp[-1])).astype(np.int32)   # repeats allowed
    return rp, ci


@pytest.mark.parametrize("case", cases(64))
def test_random_graphs(case):
    rng = np.random.default_rng(9000 + case)
    rp, ci = random_graph(rng)
    n = rp.size - 1
    dt, H, D = LAYOUTS[int(rng.integers(len(LAYOUTS)))]
    chunk = int(rng.choice([0, 1, 3, 64, 128, 500]))
    slope = float(rng.choice([0.2, 0.0, 1.0, -0.3]))
    order = 1 + case % 2          # dS handed over in CSR or in transposed order
    note(f"random case {case}: n={n} nnz={rp[-1]} dt={dt} H={H} D={D} chunk={chunk} "
         f"slope={slope} edge_order={order}")
    t = {nm: I.normal_tensor(rng, (n, H, D), dt) for nm in ("q", "k", "v", "dout")}
    a = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    r = Runner(rp, ci, chunk=chunk, edge_order=order)
    q, k, v, do = (dev(t[x]) for x in ("q", "k", "v", "dout"))

    out, lse = r.gt_fwd(q, k, v)
    dq, dk, dv = r.gt_bwd(q, k, v, out, lse, do)
    ro, rl = oracle.gt_fwd(rp, ci, t["q"], t["k"], t["v"])
    rq, rk, rv = oracle.gt_bwd(rp, ci, t["q"], t["k"], t["v"], t["dout"])
    # A graph whose every non-empty row has one distinct in-neighbour gives
    # equal scores in each row, out = that neighbour's row and dS = dE = 0
    # exactly: dQ, dK, dXs and da vanish (the oracle returns 0 to fp64
    # rounding, the library the rounding residue of Delta from its stored
    # output). There they are checked against the dV / dXt scale instead.
    degenerate = all(np.unique(ci[rp[i]:rp[i + 1]]).size <= 1 for i in range(n))

    def check(name, got, ref, scale_ref=None):
        g = host(got)
        if scale_ref is None:
            assert rel_err(g, ref) <= (TOL_LSE if name.endswith("lse") else TOL[dt]), name
        else:
            assert np.isfinite(g).all(), name
            scale = max(np.abs(ref).max(initial=0.0), np.abs(scale_ref).max(initial=0.0), 1e-30)
            assert np.abs(g - ref).max(initial=0.0) <= TOL[dt] * scale, name

    for name, got, ref in (("gt.out", out, ro), ("gt.lse", lse, rl), ("gt.dv", dv, rv)):
        check(name, got, ref)
    check("gt.dq", dq, rq, rv if degenerate else None)
    check("gt.dk", dk, rk, rv if degenerate else None)

    ad = dev(a)
    gout, glse = r.gat_fwd(q, k, ad, slope=slope)
    dxs, dxt, da = r.gat_bwd(q, k, ad, gout, glse, do, slope=slope)
    go, gl = oracle.gat_fwd(rp, ci, t["q"], t["k"], a, slope)
    gs, gt, ga = oracle.gat_bwd(rp, ci, t["q"], t["k"], a, t["dout"], slope)
    for name, got, ref in (("gat.out", gout, go), ("gat.lse", glse, gl), ("gat.dxt", dxt, gt)):
        check(name, got, ref)
    check("gat.da", da, ga, gt if degenerate else None)
    # with slope 1 the scores do not depend on Xs (a . (Xs_i + Xt_j) shifts a
    # whole row), so dXs vanishes exactly, as on a degenerate graph: then the
    # dXt scale; otherwise dXs against its own scale
    check("gat.dxs", dxs, gs, gt if (degenerate or slope == 1.0) else None)


def random_block_graph(rng):
    """Random 16x16-block structure: a few blocks dense at random densities
    (they become tiles above the threshold), scattered edges elsewhere, a
    ragged node count, some empty rows and repeated edges."""
    n = int(rng.integers(17, 600))
    nb = (n + 15) // 16
    dst, src = [], []
    for _ in range(int(rng.integers(1, 3 * nb + 2))):
        br, bc = int(rng.integers(nb)), int(rng.integers(nb))
        dens = float(rng.choice([0.05, 0.2, 0.5, 0.9, 1.0]))
        m = rng.random((16, 16)) < dens
        r_, c_ = np.nonzero(m)
        r_, c_ = r_ + 16 * br, c_ + 16 * bc
        ok = (r_ < n) & (c_ < n)
        dst.append(r_[ok]), src.append(c_[ok])
    k = int(rng.integers(0, 4 * n))
    dst.append(rng.integers(0, n, size=k)), src.append(rng.integers(0, n, size=k))
    dst, src = np.concatenate(dst), np.concatenate(src)
    rp, ci = I.csr_from_edges(n, dst, src, self_loops=bool(rng.integers(2)), dedup=bool(rng.integers(2)))
    return rp, ci


@pytest.mark.parametrize("case", cases(32))
def test_random_tile_graphs(case):
    """The 16x16 tile path (bf16 MFMA) on random block structures, random
    tile thresholds and layouts: forward and backward against the oracle."""
    import torch
    rng = np.random.default_rng(7000 + case)
    rp, ci = random_block_graph(rng)
    n = rp.size - 1
    H = int(rng.choice([1, 2, 4, 5, 8]))
    D = int(rng.choice([32, 64, 128]))
    tau = int(rng.choice([1, 8, 32, 100]))
    note(f"random tile case {case}: n={n} nnz={rp[-1]} H={H} D={D} tau={tau}")
    t = {nm: I.normal_tensor(rng, (n, H, D), I.BF16) for nm in ("q", "k", "v", "dout")}
    r = Runner(rp, ci, block_sparse=True, tile_min_nnz=tau)
    B, g = r.B, r.g
    q, k, v, do = (dev(t[x]) for x in ("q", "k", "v", "dout"))
    out = torch.empty_like(q)
    lse = torch.empty((n, H), dtype=torch.float32, device=q.device)
    B.gt_fwd(g.plan, g.rowptr, g.colidx, q, k, v, out, lse, g.workspace(B.OP_GT_FWD, H, D, B.BF16),
             use_tiles=True)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    B.gt_bwd(g.plan, g.rowptr, g.colidx, q, k, v, out, lse, do, dq, dk, dv,
             g.workspace(B.OP_GT_BWD, H, D, B.BF16), use_tiles=True)
    ro, rl = oracle.gt_fwd(rp, ci, t["q"], t["k"], t["v"])
    rq, rk, rv = oracle.gt_bwd(rp, ci, t["q"], t["k"], t["v"], t["dout"])
    for name, got, ref in (("out", out, ro), ("lse", lse, rl), ("dq", dq, rq), ("dk", dk, rk),
                           ("dv", dv, rv)):
        assert rel_err(host(got), ref) <= (TOL_LSE if name == "lse" else TOL["bf16"]), name


@pytest.mark.parametrize("case", cases(32))
def test_random_minmax(case):
    """Min/max aggregation on random graphs, feature widths (any multiple of
    the fragment up to 2048), dtypes, chunk sizes and tie-heavy or continuous
    values: values and winners bit-exact, dX to the bar of the fixed cases."""
    from tests.test_gpu_reduce import run_case
    rng = np.random.default_rng(5000 + case)
    rp, ci = random_graph(rng)
    n = rp.size - 1
    dt = str(rng.choice(["f32", "bf16"]))
    vec = 4 if dt == "f32" else 8
    F = vec * int(rng.integers(1, 2048 // vec + 1))
    op = str(rng.choice(["min", "max"]))
    chunk = int(rng.choice([0, 1, 5, 64, 300]))
    ties = bool(rng.integers(2))
    note(f"random min/max case {case}: n={n} nnz={rp[-1]} dt={dt} F={F} op={op} chunk={chunk} ties={ties}")
    x = (rng.integers(-4, 5, size=(n, F)) / 4.0) if ties else rng.standard_normal((n, F))
    x = x.astype(np.float32)
    if dt == "bf16":
        x = I.f32_to_bf16_bits(x)
    dout = rng.standard_normal((n, F)).astype(np.float32)
    if dt == "bf16":
        dout = I.f32_to_bf16_bits(dout)
    run_case(rp, ci, x, dout, dt, op, chunk)
