"""GPU parity at the full sizes of the five workloads, in the launch
configuration bench.py times (default plan options), element by element.

The fp64 oracle computes every output row of the whole graph (its backward
forms every edge's weight and dS in any case); every element of every output
tensor is compared, the device tensors brought to the host in row blocks.
Bar: max |gpu - oracle| / max |oracle| per tensor <= 2e-2 for bf16 inputs
(1e-4 for fp32), and lse, an fp32 output computed in fp32 from the exact
input values, <= 1e-4 in every case. Heavy rows and sources (split across
wavefronts and merged) are also checked per (row, head) against their own
scale, since one dropped chunk of a 200k-edge hub would hide under the
global scale. GATv2's da is compared in full."""
import numpy as np
import pytest

import oracle
from sparse_graph_attention_csr_amd import binding as B
from sparse_graph_attention_csr_amd import inputs as I
from tests.gpu_util import TOL, TOL_LSE, Runner, dev, host, note, rel_err, row_rel_err

pytestmark = pytest.mark.gpu

BLOCK = 1 << 17   # rows brought to the host at a time


def heavy(rp, plan, n_top=16):
    """The highest-degree rows and the sources with the most out-edges."""
    deg = np.diff(rp)
    odeg = np.diff(plan.export(B.ARR_COLPTR))
    return (np.sort(np.argsort(-deg, kind="stable")[:n_top]),
            np.sort(np.argsort(-odeg, kind="stable")[:n_top]))


def pick(t, idx):
    """Rows `idx` of a device tensor, as fp64 on the host (index on the device)."""
    import torch
    return host(t[torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(t.device)])


def check_full(name, t, ref, tol):
    """Every element of device tensor t against the oracle's ref: the same
    non-finite entries (lse of empty rows), and max |t - ref| / max |ref|
    over the finite ones within tol."""
    import torch
    fin = np.isfinite(ref)
    scale = float(np.abs(ref[fin]).max()) if fin.any() else 0.0
    worst = 0.0
    for a in range(0, ref.shape[0], BLOCK):
        b = min(ref.shape[0], a + BLOCK)
        g = host(t[a:b])
        f = fin[a:b]
        assert np.array_equal(np.isfinite(g), f), f"{name}: non-finite entries differ"
        assert np.array_equal(g[~f], ref[a:b][~f]), f"{name}: non-finite values differ"
        if f.any():
            worst = max(worst, float(np.abs(g[f] - ref[a:b][f]).max()))
    e = worst / scale if scale > 0 else worst
    note(f"  {name}: rel err {e:.3e} over {ref.size} elements (tol {tol:.0e})")
    assert e <= tol, name


def check_heavy(name, t, ref, rows, tol):
    e = row_rel_err(pick(t, rows), ref[rows])
    note(f"  {name} per (row, head) on {rows.size} heavy rows: {e:.3e}")
    assert e <= tol, name


_REF = {}


def gt_reference(name):
    """The workload and the oracle's full forward and backward (kept for the
    tests that share a workload)."""
    if name not in _REF:
        note(f"{name}: generating")
        w = I.make_workload(name)
        rp, ci = w["rowptr"], w["colidx"]
        note(f"{name}: oracle on N={rp.size - 1} E={ci.size} ({oracle.num_threads()} threads)")
        ro, rl = oracle.gt_fwd(rp, ci, w["q"], w["k"], w["v"])
        grads = (oracle.gt_bwd(rp, ci, w["q"], w["k"], w["v"], w["dout"])
                 if w["spec"].passes == "fwd+bwd" else None)
        _REF.clear()
        _REF[name] = (w, ro, rl, grads)
    return _REF[name]


def run_gt(name, use_tiles=False):
    import torch
    w, ro, rl, grads = gt_reference(name)
    spec = w["spec"]
    dt = spec.dtype
    rp, ci = w["rowptr"], w["colidx"]
    r = Runner(rp, ci, block_sparse=use_tiles)
    g = r.g
    q, k, v = dev(w["q"]), dev(w["k"]), dev(w["v"])
    n, H, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty(n, H, dtype=torch.float32, device=q.device)
    B.gt_fwd(g.plan, g.rowptr, g.colidx, q, k, v, out, lse,
             g.workspace(B.OP_GT_FWD, H, D, B._dtype_code(q)), use_tiles=use_tiles)
    torch.cuda.synchronize()
    hrows, hsrc = heavy(rp, g.plan)
    check_full("out", out, ro, TOL[dt])
    check_full("lse", lse, rl, TOL_LSE)
    check_heavy("out", out, ro, hrows, TOL[dt])
    if grads is None:
        return
    rq, rk, rv = grads
    do = dev(w["dout"])
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    B.gt_bwd(g.plan, g.rowptr, g.colidx, q, k, v, out, lse, do, dq, dk, dv,
             g.workspace(B.OP_GT_BWD, H, D, B._dtype_code(q)), use_tiles=use_tiles)
    torch.cuda.synchronize()
    check_full("dQ", dq, rq, TOL[dt])
    check_full("dK", dk, rk, TOL[dt])
    check_full("dV", dv, rv, TOL[dt])
    check_heavy("dQ", dq, rq, hrows, TOL[dt])
    check_heavy("dK", dk, rk, hsrc, TOL[dt])
    check_heavy("dV", dv, rv, hsrc, TOL[dt])


def test_gt_er_forward_full_size():
    run_gt("gt_er1k_h4d32_f32")


@pytest.mark.timeout(600)
def test_gt_powerlaw_full_size():
    run_gt("gt_powerlaw200k_h4d128_bf16")


@pytest.mark.timeout(900)
def test_gt_community_full_size():
    run_gt("gt_community262k_h4d128_bf16")


@pytest.mark.timeout(900)
def test_gt_community_tiles_full_size():
    """The community workload on the 16x16 tile (MFMA) path, forward and
    backward, against the same oracle results."""
    run_gt("gt_community262k_h4d128_bf16", use_tiles=True)


@pytest.mark.timeout(1200)
def test_gt_hubs_full_size():
    run_gt("gt_hubs2m_h8d64_bf16")


@pytest.mark.timeout(900)
def test_gatv2_powerlaw_full_size():
    name = "gatv2_powerlaw500k_h2d64_bf16"
    note(f"{name}: generating")
    w = I.make_workload(name)
    spec = w["spec"]
    dt = spec.dtype
    rp, ci = w["rowptr"], w["colidx"]
    note(f"{name}: oracle on N={rp.size - 1} E={ci.size}")
    ro, rl = oracle.gat_fwd(rp, ci, w["xs"], w["xt"], w["a"], 0.2)
    rs, rt, ra = oracle.gat_bwd(rp, ci, w["xs"], w["xt"], w["a"], w["dout"], 0.2)
    r = Runner(rp, ci)
    xs, xt, a = dev(w["xs"]), dev(w["xt"]), dev(w["a"])
    out, lse = r.gat_fwd(xs, xt, a)
    hrows, hsrc = heavy(rp, r.g.plan)
    check_full("out", out, ro, TOL[dt])
    check_full("lse", lse, rl, TOL_LSE)
    check_heavy("out", out, ro, hrows, TOL[dt])
    do = dev(w["dout"])
    dxs, dxt, da = r.gat_bwd(xs, xt, a, out, lse, do)
    check_full("dXs", dxs, rs, TOL[dt])
    check_full("dXt", dxt, rt, TOL[dt])
    e = rel_err(host(da), ra)
    note(f"  da: rel err {e:.3e}")
    assert e <= TOL[dt]
    check_heavy("dXs", dxs, rs, hrows, TOL[dt])
    check_heavy("dXt", dxt, rt, hsrc, TOL[dt])
