"""The library's calls can be captured into a HIP graph: they allocate nothing,
synchronise nothing and issue no memset. One step of every family (Graph
Transformer on the gather path and on tiles, GATv2, min aggregation; forward
and backward) is captured once and replayed several times, with eager work
and synchronisations between the replays that overwrite every output; each
replay must reproduce the eager results bit for bit (the kernels are
deterministic)."""
import numpy as np
import pytest

from sparse_graph_attention_csr_amd import inputs as I
from tests.gpu_util import dev, note

pytestmark = pytest.mark.gpu


def test_graph_capture_replays_match_eager():
    import torch
    from sparse_graph_attention_csr_amd import binding as B
    note("graph capture")
    rng = np.random.default_rng(0)
    rp, ci = I.random_csr(300, 16, rng, empty_frac=0.05, dup_frac=0.1, heavy_rows=2,
                          heavy_deg=700)
    n, H, D, F = rp.size - 1, 4, 64, 128
    g = B.DeviceGraph(rp, ci, chunk=64, block_sparse=True)
    q, k, v, do, xs, xt = (dev(I.normal_tensor(rng, (n, H, D), I.BF16)) for _ in range(6))
    a = dev((rng.standard_normal((H, D)) / 8).astype(np.float32))
    x = dev(rng.standard_normal((n, F)).astype(np.float32))
    dx_in = dev(rng.standard_normal((n, F)).astype(np.float32))

    def e(t):
        return torch.empty_like(t)

    outs = {
        "gt_out": e(q), "gt_lse": torch.empty(n, H, device="cuda"),
        "gt_dq": e(q), "gt_dk": e(q), "gt_dv": e(q),
        "bs_out": e(q), "bs_lse": torch.empty(n, H, device="cuda"),
        "bs_dq": e(q), "bs_dk": e(q), "bs_dv": e(q),
        "gat_out": e(q), "gat_lse": torch.empty(n, H, device="cuda"),
        "gat_dxs": e(q), "gat_dxt": e(q), "gat_da": torch.empty(H, D, device="cuda"),
        "min_out": e(x), "min_arg": torch.empty(n, F, dtype=torch.int32, device="cuda"),
        "min_dx": e(x),
    }
    ws = {op: g.workspace(op, h, d, dt) for op, h, d, dt in (
        (B.OP_GT_FWD, H, D, B.BF16), (B.OP_GT_BWD, H, D, B.BF16), (B.OP_GAT_FWD, H, D, B.BF16),
        (B.OP_GAT_BWD, H, D, B.BF16), (B.OP_REDUCE_FWD, 1, F, B.F32), (B.OP_REDUCE_BWD, 1, F, B.F32))}
    o = outs

    def step():
        B.gt_fwd(g.plan, g.rowptr, g.colidx, q, k, v, o["gt_out"], o["gt_lse"], ws[B.OP_GT_FWD])
        B.gt_bwd(g.plan, g.rowptr, g.colidx, q, k, v, o["gt_out"], o["gt_lse"], do, o["gt_dq"],
                 o["gt_dk"], o["gt_dv"], ws[B.OP_GT_BWD])
        B.gt_fwd(g.plan, g.rowptr, g.colidx, q, k, v, o["bs_out"], o["bs_lse"], ws[B.OP_GT_FWD],
                 use_tiles=True)
        B.gt_bwd(g.plan, g.rowptr, g.colidx, q, k, v, o["bs_out"], o["bs_lse"], do, o["bs_dq"],
                 o["bs_dk"], o["bs_dv"], ws[B.OP_GT_BWD], use_tiles=True)
        B.gat_fwd(g.plan, g.rowptr, g.colidx, xs, xt, a, 0.2, o["gat_out"], o["gat_lse"],
                  ws[B.OP_GAT_FWD])
        B.gat_bwd(g.plan, g.rowptr, g.colidx, xs, xt, a, 0.2, o["gat_out"], o["gat_lse"], do,
                  o["gat_dxs"], o["gat_dxt"], o["gat_da"], ws[B.OP_GAT_BWD])
        B.reduce_fwd(g.plan, g.rowptr, g.colidx, x, "min", o["min_out"], o["min_arg"],
                     ws[B.OP_REDUCE_FWD])
        B.reduce_bwd(g.plan, g.rowptr, g.colidx, o["min_arg"], dx_in, o["min_dx"],
                     ws[B.OP_REDUCE_BWD])

    step()
    torch.cuda.synchronize()
    eager = {name: t.clone() for name, t in o.items()}

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for r in range(3):
        for t in o.values():                    # eager work between replays
            if t.dtype == torch.int32:
                t.fill_(-7)
            else:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in o.items():
            ref = eager[name]
            same = torch.equal(t, ref) if t.dtype == torch.int32 else bool(
                torch.equal(torch.nan_to_num(t.float(), nan=7.0, neginf=-9.0),
                            torch.nan_to_num(ref.float(), nan=7.0, neginf=-9.0)))
            assert same, f"replay {r}: {name} differs from the eager result"
