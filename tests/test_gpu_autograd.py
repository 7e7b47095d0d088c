"""torch.autograd integration: gradients through the fused functions and the
projection layers match the oracle (and the chain rule through the
projections, written out in numpy fp64)."""
import numpy as np
import pytest

import oracle
from sparse_graph_attention_csr_amd import inputs as I
from tests.gpu_util import TOL, note, rel_err

pytestmark = pytest.mark.gpu


def graph(seed, n=256):
    rng = np.random.default_rng(seed)
    return I.random_csr(n, 16, rng, empty_frac=0.05, dup_frac=0.1, heavy_rows=2, heavy_deg=600)


def test_gt_attention_gradients_fp32():
    import torch
    from sparse_graph_attention_csr_amd import binding as B
    from sparse_graph_attention_csr_amd.autograd import gt_attention
    note("autograd gt fp32")
    rp, ci = graph(1)
    n, H, D = rp.size - 1, 4, 32
    rng = np.random.default_rng(2)
    q, k, v, do = (rng.standard_normal((n, H, D)).astype(np.float32) for _ in range(4))
    g = B.DeviceGraph(rp, ci, chunk=64)
    Q, K, V = (torch.tensor(x, device="cuda", requires_grad=True) for x in (q, k, v))
    out, lse = gt_attention(g, Q, K, V, return_lse=True)
    (out * torch.tensor(do, device="cuda")).sum().backward()
    ro, rl = oracle.gt_fwd(rp, ci, q, k, v)
    rq, rk, rv = oracle.gt_bwd(rp, ci, q, k, v, do)
    assert rel_err(out.detach().cpu().numpy(), ro) <= TOL["f32"]
    assert rel_err(lse.cpu().numpy(), rl) <= TOL["f32"]
    for t, r in ((Q, rq), (K, rk), (V, rv)):
        assert rel_err(t.grad.cpu().numpy(), r) <= TOL["f32"]


def test_gatv2_attention_gradients_bf16():
    import torch
    from sparse_graph_attention_csr_amd import binding as B
    from sparse_graph_attention_csr_amd.autograd import gatv2_attention
    note("autograd gatv2 bf16")
    rp, ci = graph(3)
    n, H, D = rp.size - 1, 2, 64
    rng = np.random.default_rng(4)
    xs, xt, do = (I.normal_tensor(rng, (n, H, D), I.BF16) for _ in range(3))
    a = (rng.standard_normal((H, D)) / 8).astype(np.float32)
    g = B.DeviceGraph(rp, ci, chunk=64)

    def bf(x):
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16).requires_grad_(True)

    Xs, Xt = bf(xs), bf(xt)
    A = torch.tensor(a, device="cuda", requires_grad=True)
    out = gatv2_attention(g, Xs, Xt, A, 0.2)
    dO = torch.from_numpy(do.view(np.int16)).cuda().view(torch.bfloat16)
    (out.float() * dO.float()).sum().backward()
    rs, rt, ra = oracle.gat_bwd(rp, ci, xs, xt, a, do, 0.2)
    assert rel_err(Xs.grad.float().cpu().numpy(), rs) <= TOL["bf16"]
    assert rel_err(Xt.grad.float().cpu().numpy(), rt) <= TOL["bf16"]
    assert rel_err(A.grad.cpu().numpy(), ra) <= TOL["bf16"]


def test_layers_gradients_through_projections():
    import torch
    from sparse_graph_attention_csr_amd import binding as B
    from sparse_graph_attention_csr_amd.autograd import GATv2Attention, GraphTransformerAttention
    note("autograd layers")
    rp, ci = graph(5)
    n, F, H, D = rp.size - 1, 48, 4, 32
    rng = np.random.default_rng(6)
    x = rng.standard_normal((n, F)).astype(np.float32)
    dy = rng.standard_normal((n, H * D)).astype(np.float32)
    g = B.DeviceGraph(rp, ci, chunk=64)
    torch.manual_seed(0)

    # Graph Transformer layer
    layer = GraphTransformerAttention(F, H, D, device="cuda")
    X = torch.tensor(x, device="cuda")
    y = layer(g, X)
    (y * torch.tensor(dy, device="cuda")).sum().backward()
    proj = {nm: getattr(layer, nm) for nm in ("q", "k", "v")}
    qkv = {nm: (x @ p.weight.detach().cpu().numpy().T + p.bias.detach().cpu().numpy()).astype(np.float32)
           for nm, p in proj.items()}
    shp = (n, H, D)
    grads = oracle.gt_bwd(rp, ci, *(qkv[nm].reshape(shp) for nm in ("q", "k", "v")),
                          dy.reshape(shp).astype(np.float32))
    for nm, gr in zip(("q", "k", "v"), grads):
        gflat = gr.reshape(n, H * D)
        assert rel_err(proj[nm].weight.grad.cpu().numpy(), gflat.T @ x.astype(np.float64)) <= 1e-4
        # the K bias gradient is exactly zero (a common shift of all keys leaves
        # every softmax unchanged), so measure bias errors on the gradient's scale
        db = proj[nm].bias.grad.cpu().numpy()
        assert np.abs(db - gflat.sum(0)).max() <= 1e-4 * max(np.abs(gflat).sum(0).max(), 1e-30)

    # GATv2 layer
    layer = GATv2Attention(F, H, D, device="cuda")
    y = layer(g, X)
    (y * torch.tensor(dy, device="cuda")).sum().backward()
    xd = (x @ layer.dst.weight.detach().cpu().numpy().T + layer.dst.bias.detach().cpu().numpy()).astype(np.float32)
    xn = (x @ layer.nbr.weight.detach().cpu().numpy().T + layer.nbr.bias.detach().cpu().numpy()).astype(np.float32)
    a = layer.a.detach().cpu().numpy()
    gs, gt, ga = oracle.gat_bwd(rp, ci, xd.reshape(shp), xn.reshape(shp), a,
                                dy.reshape(shp).astype(np.float32), 0.2)
    assert rel_err(layer.a.grad.cpu().numpy(), ga) <= 1e-4
    assert rel_err(layer.dst.weight.grad.cpu().numpy(), gs.reshape(n, -1).T @ x) <= 1e-4
    assert rel_err(layer.nbr.weight.grad.cpu().numpy(), gt.reshape(n, -1).T @ x) <= 1e-4


def test_gt_attention_tiles_bf16():
    import torch
    from sparse_graph_attention_csr_amd import binding as B
    from sparse_graph_attention_csr_amd.autograd import gt_attention
    note("autograd gt tiles")
    dst, src = I.community_pairs(4, 64, 0.5, 2, np.random.default_rng(7))
    rp, ci = I.csr_from_edges(256, dst, src)
    n, H, D = 256, 4, 64
    rng = np.random.default_rng(8)
    q, k, v, do = (I.normal_tensor(rng, (n, H, D), I.BF16) for _ in range(4))
    g = B.DeviceGraph(rp, ci, block_sparse=True)

    def bf(x):
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16).requires_grad_(True)

    Q, K, V = bf(q), bf(k), bf(v)
    out = gt_attention(g, Q, K, V, use_tiles=True)
    dO = torch.from_numpy(do.view(np.int16)).cuda().view(torch.bfloat16)
    (out.float() * dO.float()).sum().backward()
    rq, rk, rv = oracle.gt_bwd(rp, ci, q, k, v, do)
    for t, r in ((Q, rq), (K, rk), (V, rv)):
        assert rel_err(t.grad.float().cpu().numpy(), r) <= TOL["bf16"]


@pytest.mark.parametrize("op", ["min", "max"])
def test_minmax_aggregate_gradients(op):
    import torch
    from sparse_graph_attention_csr_amd import binding as B
    from sparse_graph_attention_csr_amd.autograd import MinMaxAggregation
    note(f"autograd {op} aggregation")
    rp, ci = graph(9)
    n, F = rp.size - 1, 96
    rng = np.random.default_rng(10)
    x = rng.standard_normal((n, F)).astype(np.float32)
    do = rng.standard_normal((n, F)).astype(np.float32)
    g = B.DeviceGraph(rp, ci, chunk=64)
    X = torch.tensor(x, device="cuda", requires_grad=True)
    out = MinMaxAggregation(op)(g, X)
    (out * torch.tensor(do, device="cuda")).sum().backward()
    ro, ra = oracle.reduce_fwd(rp, ci, x, op)
    assert np.array_equal(out.detach().cpu().numpy().astype(np.float64), ro)
    assert rel_err(X.grad.cpu().numpy(), oracle.reduce_bwd(rp, ci, ra, do)) <= 1e-6
    with torch.no_grad():                   # no winners kept when no gradient is needed
        o2 = MinMaxAggregation(op)(g, X)
    assert torch.equal(o2, out.detach())
