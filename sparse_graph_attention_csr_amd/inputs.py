"""Seeded synthetic workloads for fused graph attention.

This module only draws random graphs and dense feature tensors. It holds none of
the attention arithmetic, so both the HIP path and the fp64 CPU oracle can take
their inputs from here without sharing any of the method.

Graphs are returned as CSR by destination: row ``i`` lists the in-neighbours
``j`` of node ``i`` (edges ``j -> i``), rows ascending, sources ascending within
a row, one self-loop per node. ``rowptr`` is int64 ``[N+1]``, ``colidx`` int32
``[E]``.

bf16 tensors are returned as their raw bit patterns (numpy ``uint16``), drawn in
fp32 and rounded to nearest-even, so both sides consume identical values.

The five named workloads are the ones the attention-GNN studies describe in
words ("Graph Transformer" and "GATv2" layers on power-law, community and
super-node graphs; the DF-GNN abstract, and the IO-aware layers abstract and its
Graph Transformer (H=4, D=128) and GATv2 (H=2, D=64) figure captions). The
published studies used real datasets; these synthetic graphs stand in for them.
"""
from __future__ import annotations

import dataclasses
import numpy as np

F32 = "f32"
BF16 = "bf16"

# Fixed order of sub-streams spawned from one SeedSequence.
_STREAMS = ("graph", "q", "k", "v", "dout", "a")


def _streams(seed: int) -> dict:
    ss = np.random.SeedSequence(seed)
    return {name: np.random.Generator(np.random.PCG64(s))
            for name, s in zip(_STREAMS, ss.spawn(len(_STREAMS)))}


# ----------------------------------------------------------------------------
# dtype helpers (input preparation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def normal_tensor(rng: np.random.Generator, shape, dtype: str, std: float = 1.0,
                  chunk: int = 1 << 26) -> np.ndarray:
    """N(0, std^2) draws in fp32, returned as fp32 or as bf16 bits (uint16).

    Drawn in chunks so that very large tensors never hold a full fp32 copy.
    """
    n = int(np.prod(shape))
    if dtype == F32:
        out = rng.standard_normal(n, dtype=np.float32)
        if std != 1.0:
            out *= np.float32(std)
        return out.reshape(shape)
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = f32_to_bf16_bits(x)
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# graph assembly
# ----------------------------------------------------------------------------

def csr_from_edges(n: int, dst: np.ndarray, src: np.ndarray,
                   self_loops: bool = True, dedup: bool = True):
    """CSR by destination from an edge list, rows ascending, sources ascending.

    With ``dedup`` repeated (dst, src) pairs are kept once. With ``self_loops``
    exactly one edge i -> i is added per node (the random edges never contain
    one).
    """
    dst = np.asarray(dst, dtype=np.int64)
    src = np.asarray(src, dtype=np.int64)
    if self_loops:
        ids = np.arange(n, dtype=np.int64)
        dst = np.concatenate([dst, ids])
        src = np.concatenate([src, ids])
    code = dst * np.int64(n) + src
    if dedup:
        code = np.unique(code)
    else:
        code = np.sort(code, kind="stable")
    d = code // n
    s = code - d * n
    counts = np.bincount(d, minlength=n).astype(np.int64)
    rowptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=rowptr[1:])
    return rowptr, s.astype(np.int32)


def _first_unique_in_order(codes: np.ndarray) -> np.ndarray:
    """Distinct values of ``codes`` in order of first appearance."""
    _, idx = np.unique(codes, return_index=True)
    idx.sort()
    return codes[idx]


def er_pairs(n: int, m: int, rng: np.random.Generator):
    """G(n, m): exactly m distinct ordered pairs (src != dst), uniform.

    A pair is coded as ``dst*(n-1) + k`` with ``src = k if k < dst else k+1``,
    so self pairs never occur. Draws are taken with replacement in batches and
    de-duplicated in draw order until m distinct pairs exist.
    """
    total = n * (n - 1)
    if m > total:
        raise ValueError("more edges than ordered pairs")
    got = np.empty(0, dtype=np.int64)
    while got.size < m:
        need = m - got.size
        batch = rng.integers(0, total, size=int(need * 1.05) + 64, dtype=np.int64)
        got = _first_unique_in_order(np.concatenate([got, batch]))
    got = got[:m]
    dst = got // (n - 1)
    k = got - dst * (n - 1)
    src = np.where(k < dst, k, k + 1)
    return dst, src


def chung_lu_weights(n: int, gamma: float, mean: float, cap: float | None):
    """Expected degrees w_k proportional to (k+1)^(-1/(gamma-1)), mean ``mean``.

    With ``cap`` the weights are clamped at ``cap`` and the rest rescaled,
    repeated until the mean is ``mean`` and no weight exceeds ``cap``.
    """
    w = (np.arange(n, dtype=np.float64) + 1.0) ** (-1.0 / (gamma - 1.0))
    w *= mean * n / w.sum()
    if cap is not None:
        for _ in range(100):
            over = w >= cap
            w[over] = cap
            free = ~over
            rest = mean * n - cap * over.sum()
            w[free] *= rest / w[free].sum()
            if w.max() <= cap * (1 + 1e-12):
                break
        w = np.minimum(w, cap)
    return w


def chung_lu_pairs(n: int, gamma: float, mean: float, cap: int | None,
                   rng: np.random.Generator):
    """Directed Chung-Lu graph with exactly n*mean distinct edges.

    src and dst are drawn independently with probability proportional to the
    weights, self pairs dropped, duplicates dropped (first draw kept), and with
    ``cap`` a draw into a row that already holds ``cap`` edges is dropped.
    Edges are kept in draw order until n*mean of them exist. Node ids are then
    relabelled by a seeded random permutation so hubs are not at low ids.
    """
    m = int(round(n * mean))
    w = chung_lu_weights(n, gamma, mean, cap)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]

    def draw(k):
        s = np.searchsorted(cdf, rng.random(k), side="right")
        d = np.searchsorted(cdf, rng.random(k), side="right")
        np.minimum(s, n - 1, out=s)
        np.minimum(d, n - 1, out=d)
        return d.astype(np.int64) * n + s.astype(np.int64)

    codes = np.empty(0, dtype=np.int64)
    accepted = np.empty(0, dtype=np.int64)
    batch = int(m * 1.25) + 1024
    while True:
        c = draw(batch)
        d = c // n
        c = c[d != (c - d * n)]
        codes = _first_unique_in_order(np.concatenate([codes, c]))
        if cap is not None:
            dd = codes // n
            order = np.argsort(dd, kind="stable")
            sd = dd[order]
            starts = np.searchsorted(sd, sd, side="left")
            rank = np.empty_like(order)
            rank[order] = np.arange(order.size) - starts
            accepted = codes[rank < cap]
        else:
            accepted = codes
        if accepted.size >= m:
            break
        batch = int((m - accepted.size) * 1.5) + 1024
    accepted = accepted[:m]
    dst = accepted // n
    src = accepted - dst * n
    perm = rng.permutation(n).astype(np.int64)
    return perm[dst], perm[src]


def community_pairs(n_comm: int, size: int, p: float, n_inter: int,
                    rng: np.random.Generator):
    """Communities of ``size`` consecutive ids.

    Each ordered pair (j -> i), j != i, inside a community is an edge with
    probability p, drawn independently. Each node also receives ``n_inter``
    distinct in-neighbours drawn uniformly from outside its own community.
    """
    n = n_comm * size
    mask = rng.random((n_comm, size, size)) < p          # [c, dst, src]
    eye = np.eye(size, dtype=bool)
    mask &= ~eye[None]
    c, r, s = np.nonzero(mask)
    dst_in = c.astype(np.int64) * size + r
    src_in = c.astype(np.int64) * size + s
    outside = n - size
    picks = np.empty((n, n_inter), dtype=np.int64)
    for k in range(n_inter):
        col = rng.integers(0, outside, size=n, dtype=np.int64)
        while True:
            clash = np.zeros(n, dtype=bool)
            for q in range(k):
                clash |= col == picks[:, q]
            if not clash.any():
                break
            col[clash] = rng.integers(0, outside, size=int(clash.sum()), dtype=np.int64)
        picks[:, k] = col
    node = np.arange(n, dtype=np.int64)
    base = (node // size) * size
    src_out = np.where(picks < base[:, None], picks, picks + size)
    dst_out = np.repeat(node, n_inter)
    return (np.concatenate([dst_in, dst_out]),
            np.concatenate([src_in, src_out.reshape(-1)]))


def hub_pairs(n: int, mean: float, n_hubs: int, hub_in: int, hub_out: int,
              rng: np.random.Generator):
    """G(n, n*mean) background plus super nodes.

    ``n_hubs`` distinct hub ids are drawn uniformly; each receives ``hub_in``
    distinct in-neighbours and sends ``hub_out`` distinct out-edges, both drawn
    uniformly among the other nodes. The union is de-duplicated by the CSR
    assembly.
    """
    dst, src = er_pairs(n, int(round(n * mean)), rng)
    hubs = rng.choice(n, size=n_hubs, replace=False).astype(np.int64)
    dl, sl = [dst], [src]
    for h in hubs:
        ins = rng.choice(n - 1, size=hub_in, replace=False).astype(np.int64)
        ins += ins >= h
        dl.append(np.full(hub_in, h, dtype=np.int64))
        sl.append(ins)
        outs = rng.choice(n - 1, size=hub_out, replace=False).astype(np.int64)
        outs += outs >= h
        dl.append(outs)
        sl.append(np.full(hub_out, h, dtype=np.int64))
    return np.concatenate(dl), np.concatenate(sl), hubs


# ----------------------------------------------------------------------------
# named workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    op: str            # "gt", "gat" or "reduce" (min aggregation; heads = 1, dim = F)
    passes: str        # "fwd" or "fwd+bwd"
    n: int
    heads: int
    dim: int
    dtype: str
    graph: str         # human description


WORKLOADS = {
    "gt_er1k_h4d32_f32": Workload(
        "gt_er1k_h4d32_f32", "gt", "fwd", 1000, 4, 32, F32,
        "Erdos-Renyi G(n,m), n=1000, mean in-degree 8, plus self-loops"),
    "gt_powerlaw200k_h4d128_bf16": Workload(
        "gt_powerlaw200k_h4d128_bf16", "gt", "fwd+bwd", 200_000, 4, 128, BF16,
        "Chung-Lu power law, exponent 2.1, mean in-degree 15, in-degree cap 20000, plus self-loops"),
    "gatv2_powerlaw500k_h2d64_bf16": Workload(
        "gatv2_powerlaw500k_h2d64_bf16", "gat", "fwd+bwd", 500_000, 2, 64, BF16,
        "Chung-Lu power law, exponent 2.3, mean in-degree 20, plus self-loops"),
    "gt_community262k_h4d128_bf16": Workload(
        "gt_community262k_h4d128_bf16", "gt", "fwd+bwd", 262_144, 4, 128, BF16,
        "4096 communities of 64 consecutive ids, p_intra=0.5, 2 inter-community in-edges per node, plus self-loops"),
    "gt_hubs2m_h8d64_bf16": Workload(
        "gt_hubs2m_h8d64_bf16", "gt", "fwd+bwd", 2_000_000, 8, 64, BF16,
        "Erdos-Renyi mean in-degree 10 plus 64 hubs (200000 in-edges, 50000 out-edges each), plus self-loops"),
    "minagg_powerlaw500k_d512_f32": Workload(
        "minagg_powerlaw500k_d512_f32", "reduce", "fwd+bwd", 500_000, 1, 512, F32,
        "Chung-Lu power law, exponent 2.3, mean in-degree 20, plus self-loops"),
}

# The workload order used when a list of all of them is wanted.
WORKLOAD_ORDER = list(WORKLOADS)


def make_graph(name: str, seed: int = 0):
    """(rowptr, colidx, extra) of a named workload's graph."""
    w = WORKLOADS[name]
    rng = _streams(seed)["graph"]
    extra = {}
    if name == "gt_er1k_h4d32_f32":
        dst, src = er_pairs(w.n, 8 * w.n, rng)
    elif name == "gt_powerlaw200k_h4d128_bf16":
        dst, src = chung_lu_pairs(w.n, 2.1, 15.0, 20_000, rng)
    elif name in ("gatv2_powerlaw500k_h2d64_bf16", "minagg_powerlaw500k_d512_f32"):
        dst, src = chung_lu_pairs(w.n, 2.3, 20.0, None, rng)
    elif name == "gt_community262k_h4d128_bf16":
        dst, src = community_pairs(4096, 64, 0.5, 2, rng)
    elif name == "gt_hubs2m_h8d64_bf16":
        dst, src, hubs = hub_pairs(w.n, 10.0, 64, 200_000, 50_000, rng)
        extra["hubs"] = hubs
    else:
        raise KeyError(name)
    rowptr, colidx = csr_from_edges(w.n, dst, src, self_loops=True, dedup=True)
    return rowptr, colidx, extra


def make_tensors(name: str, seed: int = 0, with_grad: bool = True) -> dict:
    """Feature tensors of a named workload (fp32 arrays or bf16 bits).

    Graph Transformer: q, k, v (and dout), each [N, H, D].
    GATv2: xs (indexed by destination), xt (gathered by neighbour), a [H, D]
    in fp32 drawn N(0, 1/D), and dout.
    Min aggregation: x (and dout), each [N, F].
    """
    w = WORKLOADS[name]
    st = _streams(seed)
    shape = (w.n, w.heads, w.dim) if w.op != "reduce" else (w.n, w.dim)
    # (name, stream, shape, dtype, std): each tensor has a stream of its own,
    # so drawing them on parallel threads gives the same bytes as in turn
    jobs = []
    if w.op == "reduce":
        jobs.append(("x", "q", shape, w.dtype, 1.0))
    elif w.op == "gt":
        jobs += [("q", "q", shape, w.dtype, 1.0), ("k", "k", shape, w.dtype, 1.0),
                 ("v", "v", shape, w.dtype, 1.0)]
    else:
        jobs += [("xs", "q", shape, w.dtype, 1.0), ("xt", "k", shape, w.dtype, 1.0),
                 ("a", "a", (w.heads, w.dim), F32, w.dim ** -0.5)]
    if with_grad and w.passes == "fwd+bwd":
        jobs.append(("dout", "dout", shape, w.dtype, 1.0))
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(jobs)) as ex:
        arrs = list(ex.map(lambda j: normal_tensor(st[j[1]], j[2], j[3], std=j[4]), jobs))
    return {j[0]: a for j, a in zip(jobs, arrs)}


def make_workload(name: str, seed: int = 0, with_grad: bool = True) -> dict:
    rowptr, colidx, extra = make_graph(name, seed)
    d = {"spec": WORKLOADS[name], "rowptr": rowptr, "colidx": colidx}
    d.update(extra)
    d.update(make_tensors(name, seed, with_grad))
    return d


# ----------------------------------------------------------------------------
# small random cases for tests
# ----------------------------------------------------------------------------

def random_csr(n: int, max_deg: int, rng: np.random.Generator,
               empty_frac: float = 0.0, dup_frac: float = 0.0,
               heavy_rows: int = 0, heavy_deg: int = 0):
    """A small CSR by destination for tests.

    Degrees are uniform in [1, max_deg]; a fraction ``empty_frac`` of rows gets
    no edges; ``heavy_rows`` random rows get ``heavy_deg`` in-edges; a fraction
    ``dup_frac`` of each row's edges is replaced by repeats of earlier edges of
    that row (multigraph). Sources within a row come in random order.
    """
    deg = rng.integers(1, max_deg + 1, size=n)
    if empty_frac > 0:
        deg[rng.random(n) < empty_frac] = 0
    if heavy_rows:
        deg[rng.choice(n, size=min(heavy_rows, n), replace=False)] = heavy_deg
    rowptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(deg, out=rowptr[1:])
    col = rng.integers(0, n, size=int(rowptr[-1]), dtype=np.int64)
    if dup_frac > 0:
        for i in range(n):
            a, b = rowptr[i], rowptr[i + 1]
            for e in range(a + 1, b):
                if rng.random() < dup_frac:
                    col[e] = col[rng.integers(a, e)]
    return rowptr, col.astype(np.int32)


def degree_stats(rowptr: np.ndarray) -> dict:
    deg = np.diff(rowptr)
    if deg.size == 0:
        return {"n": 0, "e": 0}
    return {
        "n": int(deg.size), "e": int(rowptr[-1]),
        "min": int(deg.min()), "median": float(np.median(deg)),
        "p99": float(np.percentile(deg, 99)), "p999": float(np.percentile(deg, 99.9)),
        "max": int(deg.max()), "mean": float(deg.mean()),
    }


# ----------------------------------------------------------------------------
# node orderings (graph reordering study)
# ----------------------------------------------------------------------------

ORDERINGS = ("none", "random", "degree", "rcm")


def node_order(rowptr: np.ndarray, colidx: np.ndarray, kind: str, seed: int = 0) -> np.ndarray:
    """order[k] = the old id of the node placed at new position k.

    "none": the ids as generated; "random": a seeded uniform permutation;
    "degree": in-degree descending (ties by id); "rcm": reverse Cuthill-McKee
    on the structure of A + A^T.
    """
    n = rowptr.size - 1
    if kind == "none":
        return np.arange(n, dtype=np.int64)
    if kind == "random":
        return np.random.default_rng(seed).permutation(n).astype(np.int64)
    if kind == "degree":
        return np.argsort(-np.diff(rowptr), kind="stable").astype(np.int64)
    if kind == "rcm":
        import scipy.sparse as sp
        from scipy.sparse.csgraph import reverse_cuthill_mckee
        A = sp.csr_matrix((np.ones(colidx.size, dtype=np.int8), colidx, rowptr), shape=(n, n))
        return np.asarray(reverse_cuthill_mckee(A, symmetric_mode=False), dtype=np.int64)
    raise KeyError(kind)


def relabel(w: dict, order: np.ndarray) -> dict:
    """The same workload with node order[k] renamed k: the graph is rebuilt
    (rows ascending, sources ascending, every edge and repeat kept) and every
    per-node tensor permuted; per-head parameters are unchanged."""
    rp, ci = w["rowptr"], w["colidx"]
    n = rp.size - 1
    new_id = np.empty(n, dtype=np.int64)
    new_id[order] = np.arange(n, dtype=np.int64)
    dst = np.repeat(np.arange(n, dtype=np.int64), np.diff(rp))
    rp2, ci2 = csr_from_edges(n, new_id[dst], new_id[ci.astype(np.int64)], self_loops=False,
                              dedup=False)
    out = dict(w)
    out["rowptr"], out["colidx"] = rp2, ci2
    out["order"] = order
    for key in ("q", "k", "v", "xs", "xt", "dout"):
        if key in w:
            out[key] = np.ascontiguousarray(w[key][order])
    return out
