"""Masked dense forms of Graph Transformer and GATv2 attention (test pins).

These restate the layers as dense matrix expressions over an [N, N] score
matrix with -inf on non-edges, so they can pin the edge-by-edge oracle from an
independent direction. Repeated edges are folded in as log-multiplicities: a
pair (j -> i) that occurs c times contributes c * exp(s_ij) to row i's softmax,
which is softmax over s_ij + ln c_ij.
"""
from __future__ import annotations

import numpy as np
import torch


def multiplicity(rowptr, colidx, n):
    c = np.zeros((n, n), dtype=np.float64)
    for i in range(n):
        for e in range(rowptr[i], rowptr[i + 1]):
            c[i, colidx[e]] += 1.0
    return c


def _logc(c):
    with np.errstate(divide="ignore"):
        return np.log(c)


def gt_dense_np(rowptr, colidx, q, k, v):
    n, H, D = q.shape
    logc = _logc(multiplicity(rowptr, colidx, n))
    out = np.zeros((n, H, D))
    lse = np.full((n, H), -np.inf)
    for h in range(H):
        s = q[:, h, :] @ k[:, h, :].T / np.sqrt(D) + logc
        m = s.max(axis=1, keepdims=True)
        ok = np.isfinite(m[:, 0])
        p = np.zeros_like(s)
        p[ok] = np.exp(s[ok] - m[ok])
        l = p.sum(axis=1)
        out[ok, h, :] = (p[ok] / l[ok, None]) @ v[:, h, :]
        lse[ok, h] = m[ok, 0] + np.log(l[ok])
    return out, lse


def gat_scores_np(xs, xt, a, slope):
    """e[h, i, j] = sum_d a[h,d] LeakyReLU(xs[i,h,d] + xt[j,h,d]) by broadcasting."""
    z = xs.transpose(1, 0, 2)[:, :, None, :] + xt.transpose(1, 0, 2)[:, None, :, :]
    u = np.where(z > 0, z, slope * z)
    return np.einsum("hijd,hd->hij", u, a)


def gat_dense_np(rowptr, colidx, xs, xt, a, slope=0.2):
    n, H, D = xs.shape
    logc = _logc(multiplicity(rowptr, colidx, n))
    e = gat_scores_np(xs, xt, a, slope)
    out = np.zeros((n, H, D))
    lse = np.full((n, H), -np.inf)
    for h in range(H):
        s = e[h] + logc
        m = s.max(axis=1, keepdims=True)
        ok = np.isfinite(m[:, 0])
        p = np.zeros_like(s)
        p[ok] = np.exp(s[ok] - m[ok])
        l = p.sum(axis=1)
        out[ok, h, :] = (p[ok] / l[ok, None]) @ xt[:, h, :]
        lse[ok, h] = m[ok, 0] + np.log(l[ok])
    return out, lse


def _masked_softmax_t(s, logc_t):
    s = s + logc_t
    ok = torch.isfinite(s).any(dim=-1, keepdim=True)
    s = torch.where(ok, s, torch.zeros_like(s))
    p = torch.softmax(s, dim=-1)
    return torch.where(ok, p, torch.zeros_like(p))


def gt_dense_grads_torch(rowptr, colidx, q, k, v, dout):
    """(dQ, dK, dV) of L = sum(out * dout) by fp64 autograd over the dense form."""
    n, H, D = q.shape
    logc = torch.from_numpy(_logc(multiplicity(rowptr, colidx, n)))
    Q = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    K = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    V = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    outs = []
    for h in range(H):
        s = Q[:, h, :] @ K[:, h, :].T / np.sqrt(D)
        outs.append(_masked_softmax_t(s, logc) @ V[:, h, :])
    out = torch.stack(outs, dim=1)
    (out * torch.from_numpy(np.asarray(dout, dtype=np.float64))).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def gat_dense_grads_torch(rowptr, colidx, xs, xt, a, dout, slope=0.2):
    """(dXs, dXt, da) of L = sum(out * dout) by fp64 autograd over the dense form."""
    n, H, D = xs.shape
    logc = torch.from_numpy(_logc(multiplicity(rowptr, colidx, n)))
    Xs = torch.tensor(xs, dtype=torch.float64, requires_grad=True)
    Xt = torch.tensor(xt, dtype=torch.float64, requires_grad=True)
    A = torch.tensor(a, dtype=torch.float64, requires_grad=True)
    outs = []
    for h in range(H):
        z = Xs[:, h, None, :] + Xt[None, :, h, :]
        u = torch.nn.functional.leaky_relu(z, negative_slope=slope)
        s = (u * A[h]).sum(-1)
        outs.append(_masked_softmax_t(s, logc) @ Xt[:, h, :])
    out = torch.stack(outs, dim=1)
    (out * torch.from_numpy(np.asarray(dout, dtype=np.float64))).sum().backward()
    return Xs.grad.numpy(), Xt.grad.numpy(), A.grad.numpy()
