"""GPU parity at the full sizes of the five workloads, in the launch
configuration bench.py times (default plan options).

Every output tensor is checked for finiteness everywhere; sampled rows are
compared with the fp64 oracle, which computes exactly those rows: the rows of
the first work items (split chunks of the heaviest rows first), the
highest-degree rows and sources, and seeded random rows and sources. Heavy rows
are also checked per (row, head) against their own scale, since one dropped
chunk of a 200k-edge hub would hide under the global scale. GATv2's da is
compared in full."""
import numpy as np
import pytest

import oracle
from sparse_graph_attention_csr_amd import binding as B
from sparse_graph_attention_csr_amd import inputs as I
from tests.gpu_util import TOL, Runner, dev, host, note, rel_err, row_rel_err

pytestmark = pytest.mark.gpu


def samples(rp, plan, seed=0, n_rand=200, n_top=16):
    n = rp.size - 1
    deg = np.diff(rp)
    rng = np.random.default_rng(seed)
    items = plan.export(B.ARR_ROW_ITEMS)
    first = np.unique(items["row"][:32])
    top = np.argsort(-deg, kind="stable")[:n_top]
    dst = np.unique(np.concatenate([first, top, rng.choice(n, size=min(n, n_rand), replace=False)]))
    colptr = plan.export(B.ARR_COLPTR)
    odeg = np.diff(colptr)
    ctop = np.argsort(-odeg, kind="stable")[:n_top]
    src = np.unique(np.concatenate([ctop, rng.choice(n, size=min(n, n_rand), replace=False)]))
    heavy = np.unique(top)
    return dst, src, heavy, ctop


def finite(*ts):
    import torch
    for t in ts:
        assert bool(torch.isfinite(t).all()), "non-finite output"


def pick(t, idx):
    """Rows `idx` of a device tensor, as fp64 on the host (index on the device)."""
    import torch
    return host(t[torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(t.device)])


def check(name, gpu, ref, dt):
    e = rel_err(gpu, ref)
    note(f"  {name}: rel err {e:.3e} (tol {TOL[dt]:.0e})")
    assert e <= TOL[dt], name


def run_gt(name):
    note(f"{name}: generating")
    w = I.make_workload(name)
    spec = w["spec"]
    rp, ci = w["rowptr"], w["colidx"]
    note(f"{name}: N={rp.size - 1} E={ci.size} H={spec.heads} D={spec.dim}")
    r = Runner(rp, ci)
    q, k, v = dev(w["q"]), dev(w["k"]), dev(w["v"])
    out, lse = r.gt_fwd(q, k, v)
    finite(out)
    deg = np.diff(rp)
    lse_h = host(lse)
    assert np.all(np.isfinite(lse_h[deg > 0]))
    dst, src, heavy, ctop = samples(rp, r.g.plan)
    note(f"{name}: oracle forward on {dst.size} rows")
    ro, rl = oracle.gt_fwd(rp, ci, w["q"], w["k"], w["v"], rows=dst)
    out_h = pick(out, dst)
    dt = spec.dtype
    check("out", out_h, ro, dt)
    check("lse", lse_h[dst], rl, dt)
    hv = np.searchsorted(dst, heavy)
    e = row_rel_err(out_h[hv], ro[hv])
    note(f"  heavy rows per (row, head): {e:.3e}")
    assert e <= TOL[dt]
    if spec.passes != "fwd+bwd":
        return
    do = dev(w["dout"])
    dq, dk, dv = r.gt_bwd(q, k, v, out, lse, do)
    finite(dq, dk, dv)
    note(f"{name}: oracle backward on {dst.size} rows / {src.size} sources")
    rq, rk, rv = oracle.gt_bwd(rp, ci, w["q"], w["k"], w["v"], w["dout"], dst_rows=dst,
                               src_rows=src)
    check("dQ", pick(dq, dst), rq, dt)
    dk_h, dv_h = pick(dk, src), pick(dv, src)
    check("dK", dk_h, rk, dt)
    check("dV", dv_h, rv, dt)
    cv = np.searchsorted(src, ctop)
    e = max(row_rel_err(dk_h[cv], rk[cv]), row_rel_err(dv_h[cv], rv[cv]))
    note(f"  heavy sources per (row, head): {e:.3e}")
    assert e <= TOL[dt]


def test_gt_powerlaw_full_size():
    run_gt("gt_powerlaw200k_h4d128_bf16")


@pytest.mark.timeout(600)
def test_gt_community_full_size():
    run_gt("gt_community262k_h4d128_bf16")


@pytest.mark.timeout(600)
def test_gt_community_tiles_full_size():
    """The community workload on the 16x16 tile (MFMA) path, forward and backward."""
    import torch
    name = "gt_community262k_h4d128_bf16"
    note(f"{name} tiles: generating")
    w = I.make_workload(name)
    rp, ci = w["rowptr"], w["colidx"]
    r = Runner(rp, ci, block_sparse=True)
    st = r.g.plan.stats()
    note(f"  tiles={st['tiles']} tile_edges={st['tile_edges']} residual={st['residual_edges']}")
    q, k, v, do = dev(w["q"]), dev(w["k"]), dev(w["v"]), dev(w["dout"])
    n, H, D = q.shape
    B_ = r.B
    out = torch.empty_like(q)
    lse = torch.empty(n, H, dtype=torch.float32, device=q.device)
    B_.gt_fwd(r.g.plan, r.g.rowptr, r.g.colidx, q, k, v, out, lse,
              r.g.workspace(B_.OP_GT_FWD, H, D, B_.BF16), use_tiles=True)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    B_.gt_bwd(r.g.plan, r.g.rowptr, r.g.colidx, q, k, v, out, lse, do, dq, dk, dv,
              r.g.workspace(B_.OP_GT_BWD, H, D, B_.BF16), use_tiles=True)
    finite(out, dq, dk, dv)
    dst, src, heavy, ctop = samples(rp, r.g.plan)
    ro, rl = oracle.gt_fwd(rp, ci, w["q"], w["k"], w["v"], rows=dst)
    check("out", pick(out, dst), ro, "bf16")
    check("lse", pick(lse, dst), rl, "bf16")
    rq, rk, rv = oracle.gt_bwd(rp, ci, w["q"], w["k"], w["v"], w["dout"], dst_rows=dst,
                               src_rows=src)
    check("dQ", pick(dq, dst), rq, "bf16")
    check("dK", pick(dk, src), rk, "bf16")
    check("dV", pick(dv, src), rv, "bf16")


@pytest.mark.timeout(900)
def test_gt_hubs_full_size():
    run_gt("gt_hubs2m_h8d64_bf16")


@pytest.mark.timeout(600)
def test_gatv2_powerlaw_full_size():
    name = "gatv2_powerlaw500k_h2d64_bf16"
    note(f"{name}: generating")
    w = I.make_workload(name)
    spec = w["spec"]
    rp, ci = w["rowptr"], w["colidx"]
    note(f"{name}: N={rp.size - 1} E={ci.size} H={spec.heads} D={spec.dim}")
    r = Runner(rp, ci)
    xs, xt, a = dev(w["xs"]), dev(w["xt"]), dev(w["a"])
    out, lse = r.gat_fwd(xs, xt, a)
    finite(out)
    dst, src, heavy, ctop = samples(rp, r.g.plan)
    ro, rl = oracle.gat_fwd(rp, ci, w["xs"], w["xt"], w["a"], 0.2, rows=dst)
    out_h = pick(out, dst)
    check("out", out_h, ro, spec.dtype)
    check("lse", pick(lse, dst), rl, spec.dtype)
    hv = np.searchsorted(dst, heavy)
    e = row_rel_err(out_h[hv], ro[hv])
    note(f"  heavy rows per (row, head): {e:.3e}")
    assert e <= TOL[spec.dtype]
    do = dev(w["dout"])
    dxs, dxt, da = r.gat_bwd(xs, xt, a, out, lse, do)
    finite(dxs, dxt, da)
    note(f"{name}: oracle backward")
    rs, rt, ra = oracle.gat_bwd(rp, ci, w["xs"], w["xt"], w["a"], w["dout"], 0.2, dst_rows=dst,
                                src_rows=src)
    check("dXs", pick(dxs, dst), rs, spec.dtype)
    dxt_h = pick(dxt, src)
    check("dXt", dxt_h, rt, spec.dtype)
    check("da", host(da), ra, spec.dtype)
    e = row_rel_err(dxt_h[np.searchsorted(src, ctop)], rt[np.searchsorted(src, ctop)])
    note(f"  heavy sources per (row, head): {e:.3e}")
    assert e <= TOL[spec.dtype]
