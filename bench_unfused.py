"""Unfused comparison formulations, in plain PyTorch: the two attention layers
and min/max aggregation.

This is the baseline that ``bench.py --compare-unfused`` times and measures
the peak memory of, beside the fused library. It is the message-passing form
an unfused GNN layer takes (DF-GNN, Abstract: without kernel fusion the
layer's operations run as separate kernels with heavy data movement between
them; IO-aware layers paper, Abstract: message-passing frameworks materialise
edge-wise intermediates, so every per-edge score and weight sits in device
memory): gather the endpoint rows
per edge, score each edge, take the softmax over each destination's in-edges
with scatter reductions, weight the gathered value rows and scatter-add them
into the destinations. torch.autograd supplies the backward, which keeps the
per-edge tensors alive until it has run. No part of the fused library calls
this module, and it calls no part of the library.

Arithmetic: products in the input dtype; score sums, softmax and output
accumulation in fp32 (fp64 for fp64 inputs); output in the input dtype.
"""
from __future__ import annotations

import math

import torch


def edge_index(rowptr: torch.Tensor, colidx: torch.Tensor):
    """(dst, src) int64 edge lists of a CSR by destination."""
    n = rowptr.numel() - 1
    deg = (rowptr[1:] - rowptr[:-1]).long()
    dst = torch.repeat_interleave(torch.arange(n, device=rowptr.device), deg)
    return dst, colidx.long()


def _edge_softmax(s: torch.Tensor, dst: torch.Tensor, n: int):
    """Softmax of the [E, H] scores over each destination's in-edges; also the
    [n, H] natural log-sum-exp (-inf for rows without edges)."""
    H = s.shape[1]
    idx = dst[:, None].expand(-1, H)
    m = torch.full((n, H), -math.inf, dtype=s.dtype, device=s.device)
    m = m.scatter_reduce(0, idx, s.detach(), "amax", include_self=True)
    p = torch.exp(s - m[dst])
    l = torch.zeros((n, H), dtype=s.dtype, device=s.device).index_add(0, dst, p)
    return p / l[dst], (m + torch.log(l)).detach()


def gt(dst, src, q, k, v):
    """Graph Transformer attention: score q_i . k_j / sqrt(D) on edge j -> i,
    out_i = sum_j alpha_ij v_j. q, k, v [n, H, D]; returns (out, lse)."""
    n, H, D = q.shape
    acc = torch.promote_types(q.dtype, torch.float32)
    s = (q[dst] * k[src]).sum(-1, dtype=acc) * (1.0 / math.sqrt(D))
    alpha, lse = _edge_softmax(s, dst, n)
    out = torch.zeros((n, H, D), dtype=acc, device=q.device)
    out = out.index_add(0, dst, alpha[..., None] * v[src])
    return out.to(q.dtype), lse


def gatv2(dst, src, x_dst, x_nbr, a, negative_slope=0.2):
    """GATv2 attention: score a . LeakyReLU(x_dst_i + x_nbr_j) on edge j -> i,
    out_i = sum_j alpha_ij x_nbr_j. a [H, D] fp32; returns (out, lse)."""
    n, H, D = x_dst.shape
    acc = torch.promote_types(x_dst.dtype, torch.float32)
    z = torch.nn.functional.leaky_relu(x_dst[dst] + x_nbr[src], negative_slope)
    s = (z * a.to(z.dtype)).sum(-1, dtype=acc)
    alpha, lse = _edge_softmax(s, dst, n)
    out = torch.zeros((n, H, D), dtype=acc, device=x_dst.device)
    out = out.index_add(0, dst, alpha[..., None] * x_nbr[src])
    return out.to(x_dst.dtype), lse


def minmax(dst, src, x, op="min"):
    """Min or max aggregation: gather x[src] per edge, scatter-reduce into the
    destinations (rows without edges keep 0). torch's backward of the
    scatter reduction splits a gradient evenly between tied edges; with
    distinct values it is the winner's alone, as in the fused library."""
    n, F = x.shape
    out = torch.zeros((n, F), dtype=x.dtype, device=x.device)
    return out.scatter_reduce(0, dst[:, None].expand(-1, F), x[src],
                              "amin" if op == "min" else "amax", include_self=False)
