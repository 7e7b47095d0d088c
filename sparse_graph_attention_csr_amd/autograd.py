"""PyTorch autograd integration of the fused attention (DF-GNN, Abstract: the
fused AT-GNN kernels are used from PyTorch).

``gt_attention`` and ``gatv2_attention`` are differentiable functions whose
forward and backward are the library's gt_fwd/gt_bwd and gat_fwd/gat_bwd;
``GraphTransformerAttention`` and ``GATv2Attention`` are layers that add the
input projections (plain torch Linear layers) around them.
``minmax_aggregate`` / ``MinMaxAggregation`` are min or max pooling over the
in-neighbours (reduce_fwd / reduce_bwd; IO-aware layers abstract: the
reduction-based aggregation family). Only argument marshalling happens here:
every step runs in libsgattn.so.
"""
from __future__ import annotations

import torch

from . import binding as B


def _dt(t: torch.Tensor) -> int:
    return B._dtype_code(t)


class _GTFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, graph, q, k, v, use_tiles):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        n, H, D = q.shape
        out = torch.empty_like(q)
        lse = torch.empty((n, H), dtype=torch.float32, device=q.device)
        B.gt_fwd(graph.plan, graph.rowptr, graph.colidx, q, k, v, out, lse,
                 graph.workspace(B.OP_GT_FWD, H, D, _dt(q)), use_tiles=use_tiles)
        ctx.graph, ctx.use_tiles = graph, use_tiles
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse = ctx.saved_tensors
        g = ctx.graph
        n, H, D = q.shape
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        B.gt_bwd(g.plan, g.rowptr, g.colidx, q, k, v, out, lse, dout.contiguous(), dq, dk, dv,
                 g.workspace(B.OP_GT_BWD, H, D, _dt(q)), use_tiles=ctx.use_tiles)
        return None, dq, dk, dv, None


class _GATFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, graph, x_dst, x_nbr, a, negative_slope):
        x_dst, x_nbr = x_dst.contiguous(), x_nbr.contiguous()
        a32 = a.detach().to(torch.float32).contiguous()
        n, H, D = x_dst.shape
        out = torch.empty_like(x_dst)
        lse = torch.empty((n, H), dtype=torch.float32, device=x_dst.device)
        B.gat_fwd(graph.plan, graph.rowptr, graph.colidx, x_dst, x_nbr, a32, negative_slope, out,
                  lse, graph.workspace(B.OP_GAT_FWD, H, D, _dt(x_dst)))
        ctx.graph, ctx.slope, ctx.a_dtype = graph, negative_slope, a.dtype
        ctx.save_for_backward(x_dst, x_nbr, a32, out, lse)
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        x_dst, x_nbr, a32, out, lse = ctx.saved_tensors
        g = ctx.graph
        n, H, D = x_dst.shape
        dxs, dxt = torch.empty_like(x_dst), torch.empty_like(x_nbr)
        da = torch.empty((H, D), dtype=torch.float32, device=x_dst.device)
        B.gat_bwd(g.plan, g.rowptr, g.colidx, x_dst, x_nbr, a32, ctx.slope, out, lse,
                  dout.contiguous(), dxs, dxt, da, g.workspace(B.OP_GAT_BWD, H, D, _dt(x_dst)))
        return None, dxs, dxt, da.to(ctx.a_dtype), None


def gt_attention(graph: B.DeviceGraph, q, k, v, use_tiles: bool = False, return_lse: bool = False):
    """Graph Transformer attention over ``graph`` (a DeviceGraph): q, k, v are
    [N, H, D] fp32 or bf16; returns out [N, H, D] (and lse [N, H] if asked)."""
    out, lse = _GTFunction.apply(graph, q, k, v, bool(use_tiles))
    return (out, lse) if return_lse else out


def gatv2_attention(graph: B.DeviceGraph, x_dst, x_nbr, a, negative_slope: float = 0.2,
                    return_lse: bool = False):
    """GATv2 attention: x_dst indexed by destination, x_nbr gathered by
    neighbour ([N, H, D]), a [H, D]; returns out [N, H, D] (and lse)."""
    out, lse = _GATFunction.apply(graph, x_dst, x_nbr, a, float(negative_slope))
    return (out, lse) if return_lse else out


class GraphTransformerAttention(torch.nn.Module):
    """x [N, in_dim] -> Q, K, V projections -> fused attention -> [N, H*D]."""

    def __init__(self, in_dim: int, heads: int, head_dim: int, bias: bool = True,
                 use_tiles: bool = False, device=None, dtype=None):
        super().__init__()
        kw = dict(device=device, dtype=dtype)
        self.heads, self.head_dim, self.use_tiles = heads, head_dim, use_tiles
        self.q = torch.nn.Linear(in_dim, heads * head_dim, bias=bias, **kw)
        self.k = torch.nn.Linear(in_dim, heads * head_dim, bias=bias, **kw)
        self.v = torch.nn.Linear(in_dim, heads * head_dim, bias=bias, **kw)

    def forward(self, graph: B.DeviceGraph, x: torch.Tensor) -> torch.Tensor:
        n = x.shape[0]
        shape = (n, self.heads, self.head_dim)
        out = gt_attention(graph, self.q(x).view(shape), self.k(x).view(shape),
                           self.v(x).view(shape), use_tiles=self.use_tiles)
        return out.reshape(n, self.heads * self.head_dim)


class GATv2Attention(torch.nn.Module):
    """x [N, in_dim] -> destination and neighbour projections -> fused GATv2
    attention with attention vector a [H, D] -> [N, H*D]."""

    def __init__(self, in_dim: int, heads: int, head_dim: int, negative_slope: float = 0.2,
                 bias: bool = True, device=None, dtype=None):
        super().__init__()
        kw = dict(device=device, dtype=dtype)
        self.heads, self.head_dim, self.negative_slope = heads, head_dim, negative_slope
        self.dst = torch.nn.Linear(in_dim, heads * head_dim, bias=bias, **kw)
        self.nbr = torch.nn.Linear(in_dim, heads * head_dim, bias=bias, **kw)
        self.a = torch.nn.Parameter(torch.randn(heads, head_dim, device=device,
                                                dtype=torch.float32) / head_dim ** 0.5)

    def forward(self, graph: B.DeviceGraph, x: torch.Tensor) -> torch.Tensor:
        n = x.shape[0]
        shape = (n, self.heads, self.head_dim)
        out = gatv2_attention(graph, self.dst(x).view(shape), self.nbr(x).view(shape), self.a,
                              self.negative_slope)
        return out.reshape(n, self.heads * self.head_dim)


class _ReduceFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, graph, x, op):
        x = x.contiguous()
        n, F = x.shape
        out = torch.empty_like(x)
        arg = (torch.empty((n, F), dtype=torch.int32, device=x.device)
               if ctx.needs_input_grad[1] else None)
        B.reduce_fwd(graph.plan, graph.rowptr, graph.colidx, x, op, out, arg,
                     graph.workspace(B.OP_REDUCE_FWD, 1, F, _dt(x)))
        ctx.graph = graph
        if arg is not None:
            ctx.save_for_backward(arg)
        return out

    @staticmethod
    def backward(ctx, dout):
        (arg,) = ctx.saved_tensors
        g = ctx.graph
        dout = dout.contiguous()
        n, F = dout.shape
        dx = torch.empty_like(dout)
        B.reduce_bwd(g.plan, g.rowptr, g.colidx, arg, dout, dx,
                     g.workspace(B.OP_REDUCE_BWD, 1, F, _dt(dout)))
        return None, dx, None


def minmax_aggregate(graph: B.DeviceGraph, x, op: str = "min"):
    """out[i] = elementwise min (or max) of x[j] over the in-neighbours j of i;
    x [N, F] fp32 or bf16; rows without in-edges give 0. The gradient goes to
    the winning edge's source (the first edge of the row on ties)."""
    if op not in B.REDUCE_OPS:
        raise ValueError("op must be 'min' or 'max'")
    return _ReduceFunction.apply(graph, x, B.REDUCE_OPS[op])


class MinMaxAggregation(torch.nn.Module):
    """Min or max pooling over the in-neighbours of every node."""

    def __init__(self, op: str = "min"):
        super().__init__()
        if op not in B.REDUCE_OPS:
            raise ValueError("op must be 'min' or 'max'")
        self.op = op

    def forward(self, graph: B.DeviceGraph, x: torch.Tensor) -> torch.Tensor:
        return minmax_aggregate(graph, x, self.op)
