"""Benchmark: fused graph attention forward+backward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one forward and one backward pass of the whole fused layer over the
workload's graph, inputs already resident in device memory. The default
workload is the largest of the five: the super-node stress graph (N =
2,000,000, Erdos-Renyi background of mean in-degree 10 plus 64 hubs with
200,000 in-edges and 50,000 out-edges each, self-loops; Graph Transformer,
H = 8, D = 64; bf16 inputs, fp32 accumulation).

Prints one JSON line. ``value`` is E*H / step time in GEdge.head/s (E counts
self-loops), the step timed with a cold cache: 1 GiB is written between
steps, outside the timing, so no input survives in the Infinity Cache;
``warm`` holds the same steps run back to back. ``roofline`` is for the
kernel with the largest share of the step: algorithmic bytes per launch (the
per-edge and per-node traffic model of that kernel) over its mean launch
time, timed with HIP events recorded by the library on the launch stream
during the timed steps, against the 8 TB/s specification and against the
ceiling this GPU measured in the same run (``hbm_ceiling``: a read-only
stream and a random gather of rows of the workload's row size, both over
4 GiB). ``configs`` holds the cold and warm step times of the power-law Graph
Transformer and GATv2 workloads and of the community workload on the tile
path, measured in the same run. ``cpu_baseline`` times the fp64 CPU oracle on
a bounded sample of the headline workload (rows 0..r-1 of the CSR, the rest
emptied) on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK = 2.5e15   # dense bf16 matrix-core flop/s
DEFAULT_WORKLOAD = "gt_hubs2m_h8d64_bf16"
# timed beside the default workload in the same run: (workload, tile path)
EXTRA_CONFIGS = [("gt_powerlaw200k_h4d128_bf16", False), ("gatv2_powerlaw500k_h2d64_bf16", False),
                 ("gt_community262k_h4d128_bf16", True)]
_CSRC = "sparse_graph_attention_csr_amd/csrc/"
# the sources each kernel family is compiled from (a counter summary is valid
# only for the sources it was taken on)
KERNEL_SOURCES = {
    "gather": [_CSRC + f for f in ("device.hpp", "gather.hpp", "launch.hpp", "launch_gt.hip",
                                   "launch_gat.hip")],
    "tiles": [_CSRC + f for f in ("device.hpp", "blocksparse.hpp", "launch.hpp", "launch_bs.hip")],
    "reduce": [_CSRC + f for f in ("device.hpp", "reduce.hpp", "launch.hpp", "launch_reduce.hip")],
}


def kernel_family(kernel: str) -> str:
    if kernel.startswith("gt_bs_"):
        return "tiles"
    return "reduce" if kernel.startswith("reduce_") else "gather"


def _code_only(text: str) -> str:
    """C++ source without comments, blank lines or trailing spaces (so that a
    comment edit does not disown counters taken on the same code)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code of the sources a kernel family is built from; counter
    summaries under profiles/ record it, and bench.py uses a summary's HBM
    traffic only while the code still hashes the same."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel_family(kernel)]:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def tile_work(plan) -> dict:
    """Tile and pseudo-tile counts of a block-sparse plan (pseudo-tiles pack 16
    residual edges of one 16-row block each)."""
    import numpy as np
    from sparse_graph_attention_csr_amd import binding as B
    rr = plan.export(B.ARR_RES_ROWPTR)
    n = rr.size - 1
    res_blocks = np.diff(rr[np.minimum(np.arange(0, ((n + 15) // 16) * 16 + 1, 16), n)])
    pseudo = int(((res_blocks + 15) // 16).sum())
    s = plan.stats()
    return {"tiles": s["tiles"], "pseudo_tiles": pseudo, "residual_edges": s["residual_edges"]}


def mfma_flops(kernel: str, H: int, D: int, tw: dict) -> float | None:
    """Issued MFMA flops: per tile (dense or pseudo) and head, S (16x16xD) and
    the weighted sum (16xDx16), 2 flops per multiply-add each."""
    if not tw:
        return None
    per = {"gt_bs_fwd": 2, "gt_bs_bwd_rows": 3, "gt_bs_bwd_cols": 2}.get(kernel)
    if per is None:
        return None
    # forward: S, PV; rows: S, dP, dS K; cols: dS^T Q, P^T dO (P and dS come
    # from the row pass)
    return float((tw["tiles"] + tw["pseudo_tiles"]) * H * per * (2 * 16 * 16 * D))


def gat_record_bytes(H: int, D: int, b: int) -> int:
    """Bytes per edge of the records the GATv2 CSR backward pass leaves for the
    transposed pass: per head group of hg heads (the lanes of one edge group)
    a float2 (p, dE) per head and one byte of sign bits per lane, in whole
    dword pairs."""
    vec = 16 // b
    sph = D // vec
    want = min(H, 64 // sph)
    hg = 1
    while hg < want:
        hg *= 2
    n_hg = -(-H // hg)
    lanes = hg * sph
    return n_hg * 4 * (2 * hg + ((lanes // 4 + 1) & ~1))


# Work items shorter than this many edges at the end of the work list run
# several to a wavefront (the library's default short-item bound).
SHORT_ITEM_EDGES = 128


def edge_groups(H: int, D: int, b: int) -> int:
    """Edges a wavefront holds side by side for this layout (64-lane waves,
    16-byte fragments, head groups of a power of two heads)."""
    sph = D // (16 // b)
    want = min(H, 64 // sph)
    hg = 1
    while hg < want:
        hg *= 2
    return 64 // (hg * sph)


def row_item_split(plan) -> dict:
    """Items and edges of the CSR work list before and from the short suffix
    (the first item from which every item has fewer than SHORT_ITEM_EDGES)."""
    import numpy as np
    from sparse_graph_attention_csr_amd import binding as B
    ln = plan.export(B.ARR_ROW_ITEMS)["len"].astype(np.int64)
    long_at = np.flatnonzero(ln >= SHORT_ITEM_EDGES)
    first_short = int(long_at[-1]) + 1 if long_at.size else 0
    return {"long_items": first_short, "long_edges": int(ln[:first_short].sum()),
            "short_items": int(ln.size - first_short), "short_edges": int(ln[first_short:].sum())}


# sgat_plan_opts.edge_order 0: the Graph Transformer backward hands dS over
# in transposed order when it takes more than this many bytes
DS_TRANSPOSED_BYTES = 128 << 20


def gt_ds_transposed(plan, H: int) -> bool:
    """Whether the library's Graph Transformer backward keeps dS in
    transposed order for this plan and H (the rule documented with
    sgat_plan_opts.edge_order)."""
    from sparse_graph_attention_csr_amd import binding as B
    if plan.edge_order == 1 or plan.export(B.ARR_ROW_TPOS).size == 0:
        return False
    return plan.edge_order == 2 or plan.nnz * H * 4 > DS_TRANSPOSED_BYTES


def algorithmic_bytes(kernel: str, n: int, e: int, H: int, D: int, b: int,
                      tw: dict | None = None, split: dict | None = None,
                      tpos: bool = False) -> int | None:
    """Bytes a kernel must move: neighbour-row gathers per edge plus the
    per-node reads and writes of its own rows (R = H*D*b bytes per node row).
    The GATv2 CSR backward pass runs as two kernels when a wavefront holds
    several edges (long items, then short items several to a wave): each
    is charged its own edges and items (an item reads and writes its
    destination's row data like a node). The per-workgroup da partials of
    the GATv2 backward (H*D*4 bytes each, under 1% of either pass) are not
    counted. With `tpos` the Graph Transformer backward hands dS over in
    transposed order: its transposed pass reads no CSR edge ids and its CSR
    pass reads each edge's transposed position instead."""
    R = H * D * b
    if kernel in ("gat_bwd_rows", "gat_bwd_rows_short") and split is not None:
        which = "short" if kernel.endswith("_short") else "long"
        e, n = split[f"{which}_edges"], split[f"{which}_items"]
        kernel = "gat_bwd_rows"
    if kernel == "gt_bs_fwd" and tw:
        # dense tiles read each node's Q, K, V row once and write out and lse;
        # residual edges gather K_j and V_j; each tile reads its column and mask
        return (4 * R + 4 * H + 16) * n + (2 * R + 4) * tw["residual_edges"] + 36 * tw["tiles"]
    if kernel == "gt_bs_bwd_rows" and tw:
        # Q, dO, O, lse read and dQ written per node; K, V once per node through
        # the tiles; residual edges gather K_j, V_j; P and dS written for the
        # column pass: 2 x 512 bytes per (tile, head), 4 bytes per (residual edge, head)
        return ((6 * R + 4 * H + 16) * n + (2 * R + 4 + 4 * H) * tw["residual_edges"]
                + (36 + 1024 * H) * tw["tiles"])
    if kernel == "gt_bs_bwd_cols" and tw:
        # dK, dV written per node; Q, dO once per node through the tiles, with
        # the tiles' P and dS; residual edges gather Q_i, dO_i and read their
        # destination, residual edge id and (P, dS)
        return ((4 * R + 16) * n + (2 * R + 8 + 4 * H) * tw["residual_edges"]
                + (8 + 1024 * H) * tw["tiles"])
    model = {
        # K_j, V_j and colidx per edge; Q_i read, out_i and lse_i written per node
        "gt_fwd_rows": (2 * R + 4, 2 * R + 4 * H + 8),
        # O_i, dO_i, lse_i read and (lse, Delta) written per node
        "gt_bwd_delta": (0, 2 * R + 12 * H),
        # Q_i, dO_i, (lse_i, Delta_i), rowidx, edge id read and dS written per edge;
        # K_j, V_j read, dK_j, dV_j written per node
        "gt_bwd_cols": (2 * R + 12 * H + (4 if tpos else 8), 4 * R + 8),
        # K_j, colidx, dS (and with tpos its position) per edge; dQ_i written per node
        "gt_bwd_rows": (R + (8 if tpos else 4) + 4 * H, R + 8),
        # Xt_j and colidx per edge; Xs_i read, out_i, lse_i written
        "gat_fwd_rows": (R + 4, 2 * R + 4 * H + 8),
        # Xt_j, colidx read and the edge record written per edge; Xs_i, dO_i,
        # O_i, lse_i read, dXs_i written
        "gat_bwd_rows": (R + 4 + gat_record_bytes(H, D, b), 4 * R + 4 * H + 8),
        # dO_i, rowidx, edge id and the edge record per edge; Xt_j read (for
        # its da term) and dXt_j written per node
        "gat_bwd_cols": (R + 8 + gat_record_bytes(H, D, b), 2 * R + 8),
        # min/max aggregation (H = 1, D = F): X_j and colidx per edge; out_i and
        # the int32 winners arg_i written per node
        "reduce_fwd_rows": (R + 4, R + 4 * D),
        # per node: arg_i and dO_i read, the (feature, dout) pairs written; per
        # edge: its (start, count) written
        "reduce_bwd_route": (4, 4 * D + R + D * (4 if b == 2 else 8) + 16),
        # per edge: rowidx, edge id, (start, count); per node: its pairs read
        # once (by the edges that won them) and dX_j written
        "reduce_bwd_gather": (12, D * (4 if b == 2 else 8) + R),
    }.get(kernel)
    if model is None:
        return None
    per_edge, per_node = model
    return per_edge * e + per_node * n


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernel sources as they are now."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"kernel_source_hash:\s*(\w+)", txt)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not t or m.group(1) != kernel_source_hash(kernel):
        return None
    return float(t.group(1))


def cpu_baseline(w, seconds: float):
    """The oracle on rows 0..r-1 of the workload (other rows emptied), sized to
    about `seconds` of host time; returns a dict for the JSON line."""
    import numpy as np

    import oracle
    spec = w["spec"]
    rp, ci = w["rowptr"], w["colidx"]
    n = rp.size - 1

    split = [0.0, 0.0]   # forward and backward seconds of the runs that count

    def run(r):
        sub = rp.copy()
        sub[r + 1:] = rp[r]
        e = int(sub[-1])
        bwd = spec.passes == "fwd+bwd"
        t0 = time.perf_counter()
        if spec.op == "reduce":
            _, arg = oracle.reduce_fwd(sub, ci[:e], w["x"], "min", rows=np.arange(r))
            t1 = time.perf_counter()
            if bwd:
                full = np.full((n, spec.dim), -1, dtype=np.int64)
                full[:r] = arg
                oracle.reduce_bwd(sub, ci[:e], full, w["dout"])
        elif spec.op == "gt":
            oracle.gt_fwd(sub, ci[:e], w["q"], w["k"], w["v"], rows=np.arange(r))
            t1 = time.perf_counter()
            if bwd:
                oracle.gt_bwd(sub, ci[:e], w["q"], w["k"], w["v"], w["dout"],
                              dst_rows=np.arange(r), src_rows=np.unique(ci[:e]))
        else:
            oracle.gat_fwd(sub, ci[:e], w["xs"], w["xt"], w["a"], 0.2, rows=np.arange(r))
            t1 = time.perf_counter()
            if bwd:
                oracle.gat_bwd(sub, ci[:e], w["xs"], w["xt"], w["a"], w["dout"], 0.2,
                               dst_rows=np.arange(r), src_rows=np.unique(ci[:e]))
        t2 = time.perf_counter()
        split[0], split[1] = t1 - t0, t2 - t1
        return e, t2 - t0


    r = min(n, 2000)
    e, t = run(r)
    while t < seconds / 8 and r < n:        # grow the probe until it is long enough to scale
        r = min(n, r * 4)
        e, t = run(r)
    for _ in range(2):                      # scale to the target; cost per edge is not flat
        if r >= n or t >= seconds * 0.6:
            break
        target = e * seconds / max(t, 1e-9)
        r = int(min(n, max(r + 1, np.searchsorted(rp, target))))
        e, t = run(r)
    reps = 1
    tf, tb = split
    if r == n and t < seconds / 2:          # the whole workload is quick: repeat it
        reps = int(np.ceil(seconds / max(t, 1e-9)))
        t = tf = tb = 0.0
        for _ in range(reps):
            t += run(r)[1]
            tf, tb = tf + split[0], tb + split[1]
    rate = reps * e * spec.heads / t / 1e9
    return {"value": rate, "unit": "GEdge\u00b7head/s", "cores": oracle.num_threads(),
            "cpu": cpu_model(), "fwd_seconds": round(tf, 3), "bwd_seconds": round(tb, 3),
            "kind": "oracle",
            "sample": f"destination rows 0..{r - 1} of {n} ({e} of {int(rp[-1])} edges), "
                      f"{spec.passes}, fp64, {reps} run(s), {t:.1f} s"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def per_step_ms(step, reps: int, flush=None) -> dict:
    """Each step timed alone with events on the stream the library launches
    on (torch's current stream); `flush`, if given, runs before each step,
    outside its events. Median and minimum over the reps, in ms."""
    import statistics

    import torch
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    return {"median": round(statistics.median(times), 4), "min": round(min(times), 4),
            "reps": reps}


def load_workload(name: str, cache_dir: str) -> dict:
    """The seeded workload, generated or (with a cache directory) loaded from
    the .npz an earlier run saved there."""
    import numpy as np

    from sparse_graph_attention_csr_amd import inputs as I
    if not cache_dir:
        return I.make_workload(name)
    path = os.path.join(cache_dir, name + ".npz")
    if os.path.exists(path):
        with np.load(path, allow_pickle=False) as z:
            w = {k: z[k] for k in z.files}
    else:
        w = I.make_workload(name)
        os.makedirs(cache_dir, exist_ok=True)
        tmp = path + ".tmp.npz"
        np.savez(tmp, **{k: v for k, v in w.items() if isinstance(v, np.ndarray)})
        os.replace(tmp, path)
    w["spec"] = I.WORKLOADS[name]
    return w


def compare_unfused(spec, g, fused_step, fused_owned, inputs, fused_out, bwd, fused_ms,
                    steps, warmup):
    """Latency and peak device memory of one step of the unfused PyTorch
    formulation against the fused library on the same resident inputs.

    Memory counts what a step needs beyond the inputs and the device CSR, which
    both share: for the fused library the plan, workspaces, outputs and
    gradients (all allocated once, reused every step) plus anything allocated
    during a step; for the unfused formulation the peak of torch's allocator
    over a step (edge lists, per-edge tensors kept for autograd, outputs and
    gradients)."""
    import torch

    import bench_unfused as U

    def nbytes(t):
        return t.numel() * t.element_size()

    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    fused_step()
    torch.cuda.synchronize()
    fused_bytes = sum(nbytes(t) for t in fused_owned) + torch.cuda.max_memory_allocated() - base

    E, H, D = g.colidx.numel(), spec.heads, spec.dim
    est = E * H * D * (16 if inputs[0].element_size() == 2 else 28)
    free = torch.cuda.mem_get_info()[0]
    if est > 0.8 * free:
        return {"skipped": f"estimated unfused peak {est / 2**30:.0f} GiB exceeds the free "
                           f"device memory ({free / 2**30:.0f} GiB)"}

    n_in = 1 if spec.op == "reduce" else 3

    def unfused_step():
        leaves = [t.detach().requires_grad_(bwd) for t in inputs[:n_in]]
        dst, src = U.edge_index(g.rowptr, g.colidx)
        if spec.op == "reduce":
            o = U.minmax(dst, src, leaves[0], "min")
        elif spec.op == "gt":
            o, _ = U.gt(dst, src, *leaves)
        else:
            o, _ = U.gatv2(dst, src, *leaves, 0.2)
        if bwd:
            o.backward(inputs[n_in])
        return o.detach(), [t.grad for t in leaves]

    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o, grads = unfused_step()
    torch.cuda.synchronize()
    unfused_bytes = torch.cuda.max_memory_allocated() - base
    diff = ((o.float() - fused_out.float()).abs().max() / fused_out.float().abs().max()).item()
    del o, grads
    for _ in range(warmup):
        unfused_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        unfused_step()
    torch.cuda.synchronize()
    unfused_ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"ms_per_step": round(unfused_ms, 3), "fused_ms_per_step": round(fused_ms, 3),
            "latency_ratio": round(unfused_ms / fused_ms, 2),
            "peak_mib": round(unfused_bytes / 2**20, 1),
            "fused_mib": round(fused_bytes / 2**20, 1),
            "memory_ratio": round(unfused_bytes / fused_bytes, 2),
            "output_max_rel_diff": diff}


def hbm_ceiling(dev, row_bytes: int, gib: float) -> dict:
    """What this GPU's memory delivers, measured with the library's probes:
    a read-only stream over `gib` GiB (the best of three grid sizes) and a
    gather of whole rows of `row_bytes` bytes at uniform random indices over a
    `gib` GiB table (a footprint no cache holds, like the hub workload's K and
    V), each the best of 5 launches after one warm-up."""
    import torch

    from sparse_graph_attention_csr_amd import binding as B

    def best(fn):
        B.trace_clear()
        B.trace_enable(True)
        for _ in range(6):
            fn()
        torch.cuda.synchronize()
        B.trace_enable(False)
        ms = [t for _, t in B.trace_read()][1:]
        B.trace_clear()
        return min(ms)

    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    nb = int(gib * (1 << 30)) // 16 * 16
    buf = torch.ones(nb // 4, dtype=torch.int32, device=dev)
    read = {blocks: nb / (best(lambda: B.probe_read(buf, sink, blocks)) * 1e-3) / 1e9
            for blocks in (16384, 32768, 65536)}
    del buf
    rb = row_bytes if row_bytes in (256, 512, 1024) else 1024
    rows = nb // rb
    table = torch.ones(rows, rb // 4, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    n_idx = 64 << 20
    idx = torch.randint(0, rows, (n_idx,), dtype=torch.int32, device=dev, generator=gen)
    gather = n_idx * rb / (best(lambda: B.probe_gather(table, idx, sink)) * 1e-3) / 1e9
    del table, idx
    torch.cuda.empty_cache()
    top = max(read, key=read.get)
    return {"stream_read_gbs": round(read[top], 1), "stream_read_blocks": top,
            "gather_gbs": round(gather, 1), "gather_row_bytes": rb,
            "footprint_gib": gib, "spec_gbs": HBM_PEAK_GBS}


def edge_handoff_bytes(spec, n_e: int, H: int, D: int, b: int, tw: dict | None) -> int:
    """Bytes of the per-edge values the first backward pass leaves in the
    workspace for the second: dS per (edge, head) for the Graph Transformer
    gather path, the (p, dE, signs) record per edge for GATv2, P and dS per
    (tile, head) and per (residual edge, head) on the tile path."""
    if spec.op == "reduce" or spec.passes != "fwd+bwd":
        return 0
    if tw:
        return tw["tiles"] * H * 1024 + tw["residual_edges"] * H * 4
    if spec.op == "gt":
        return n_e * H * 4
    return n_e * gat_record_bytes(H, D, b)


class Bench:
    """One workload set up on the device: its plan, resident inputs, outputs,
    workspaces and the step closure."""

    def __init__(self, name: str, dev, chunk: int = 0, tiles: bool = False, reorder: str = "none",
                 locality: int = 0, cache_dir: str = ""):
        import numpy as np
        import torch

        from sparse_graph_attention_csr_amd import binding as B
        from sparse_graph_attention_csr_amd import inputs as I

        self.name = name
        self.spec = spec = I.WORKLOADS[name]
        w = load_workload(name, cache_dir)
        if reorder != "none":
            w = I.relabel(w, I.node_order(w["rowptr"], w["colidx"], reorder))
        self.w = w
        rp, ci = w["rowptr"], w["colidx"]
        self.n, self.e = n, e = rp.size - 1, int(rp[-1])
        self.H, self.D = H, D = spec.heads, spec.dim
        self.dt = dt = B.BF16 if spec.dtype == I.BF16 else B.F32
        self.nbytes = 2 if dt == B.BF16 else 4
        self.tiles = tiles

        t0 = time.perf_counter()
        g = self.g = B.DeviceGraph(rp, ci, device=dev, chunk=chunk, block_sparse=tiles,
                                   locality=bool(locality))
        self.tw = tile_work(g.plan) if tiles else None
        self.split = (row_item_split(g.plan)
                      if spec.op == "gat" and edge_groups(H, D, self.nbytes) > 1 else None)
        self.tpos = spec.op == "gt" and not tiles and gt_ds_transposed(g.plan, H)
        torch.cuda.synchronize()
        self.plan_ms = (time.perf_counter() - t0) * 1e3

        def todev(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        bwd = self.bwd = spec.passes == "fwd+bwd"
        lse = torch.empty(n, H, dtype=torch.float32, device=dev) if spec.op != "reduce" else None
        if spec.op == "reduce":
            X = todev(w["x"])
            out = torch.empty_like(X)
            arg = torch.empty((n, D), dtype=torch.int32, device=dev) if bwd else None
            wsf = g.workspace(B.OP_REDUCE_FWD, 1, D, dt)
            if bwd:
                dO = todev(w["dout"])
                dX = torch.empty_like(X)
                wsb = g.workspace(B.OP_REDUCE_BWD, 1, D, dt)
            outs = [out] + ([arg, dX] if bwd else [])
            inputs = [X] + ([dO] if bwd else [])

            def step():
                B.reduce_fwd(g.plan, g.rowptr, g.colidx, X, "min", out, arg, wsf)
                if bwd:
                    B.reduce_bwd(g.plan, g.rowptr, g.colidx, arg, dO, dX, wsb)
        elif spec.op == "gt":
            Q, K, V = todev(w["q"]), todev(w["k"]), todev(w["v"])
            out = torch.empty_like(Q)
            wsf = g.workspace(B.OP_GT_FWD, H, D, dt)
            if bwd:
                dO = todev(w["dout"])
                dQ, dK, dV = (torch.empty_like(Q) for _ in range(3))
                wsb = g.workspace(B.OP_GT_BWD, H, D, dt)
            outs = [out, lse] + ([dQ, dK, dV] if bwd else [])
            inputs = [Q, K, V] + ([dO] if bwd else [])

            def step():
                B.gt_fwd(g.plan, g.rowptr, g.colidx, Q, K, V, out, lse, wsf, use_tiles=tiles)
                if bwd:
                    B.gt_bwd(g.plan, g.rowptr, g.colidx, Q, K, V, out, lse, dO, dQ, dK, dV, wsb,
                             use_tiles=tiles)
        else:
            Xs, Xt = todev(w["xs"]), todev(w["xt"])
            A = torch.from_numpy(w["a"]).to(dev)
            out = torch.empty_like(Xs)
            wsf = g.workspace(B.OP_GAT_FWD, H, D, dt)
            if bwd:
                dO = todev(w["dout"])
                dXs, dXt = torch.empty_like(Xs), torch.empty_like(Xs)
                dA = torch.empty(H, D, dtype=torch.float32, device=dev)
                wsb = g.workspace(B.OP_GAT_BWD, H, D, dt)
            outs = [out, lse] + ([dXs, dXt, dA] if bwd else [])
            inputs = [Xs, Xt, A] + ([dO] if bwd else [])

            def step():
                B.gat_fwd(g.plan, g.rowptr, g.colidx, Xs, Xt, A, 0.2, out, lse, wsf)
                if bwd:
                    B.gat_bwd(g.plan, g.rowptr, g.colidx, Xs, Xt, A, 0.2, out, lse, dO, dXs, dXt,
                              dA, wsb)
        self.step, self.out, self.inputs = step, out, inputs
        self.ws = [wsf] + ([wsb] if bwd else [])
        self.owned = outs + self.ws

        def nb_(t):
            return t.numel() * t.element_size()
        self.memory = {
            "inputs_bytes": sum(nb_(t) for t in inputs),
            "outputs_bytes": sum(nb_(t) for t in outs),
            "plan_bytes": nb_(g.plan_buf),
            "workspace_bytes": {"fwd": g.plan.workspace_bytes(
                                    B.OP_REDUCE_FWD if spec.op == "reduce" else
                                    B.OP_GT_FWD if spec.op == "gt" else B.OP_GAT_FWD,
                                    1 if spec.op == "reduce" else H, D, dt)},
            "edge_handoff_bytes": edge_handoff_bytes(spec, e, H, D, self.nbytes, self.tw),
        }
        if bwd:
            self.memory["workspace_bytes"]["bwd"] = g.plan.workspace_bytes(
                B.OP_REDUCE_BWD if spec.op == "reduce" else
                B.OP_GT_BWD if spec.op == "gt" else B.OP_GAT_BWD,
                1 if spec.op == "reduce" else H, D, dt)

    def kernel_table(self, steps: int) -> dict:
        """Every kernel timed with events over `steps` untimed steps."""
        import torch

        from sparse_graph_attention_csr_amd import binding as B
        B.trace_clear()
        B.trace_enable(True)
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        B.trace_enable(False)
        recs = B.trace_read()
        B.trace_clear()
        per = {}
        for name, ms in recs:
            d = per.setdefault(name, [0.0, 0])
            d[0] += ms
            d[1] += 1
        total = max(sum(v[0] for v in per.values()), 1e-12)
        kernels = {}
        for name, (tot, cnt) in per.items():
            avg = tot / cnt
            ab = algorithmic_bytes(name, self.n, self.e, self.H, self.D, self.nbytes, self.tw,
                                   self.split, self.tpos)
            k = kernels[name] = {"ms": round(avg, 4), "launches_per_step": cnt / steps,
                                 "share": round(tot / total, 4)}
            if ab is not None:
                k["algorithmic_bytes"] = ab
                k["achieved_gbs"] = round(ab / (avg * 1e-3) / 1e9, 1)
            fl = mfma_flops(name, self.H, self.D, self.tw)
            if fl is not None:
                k["mfma_tflops"] = round(fl / (avg * 1e-3) / 1e12, 2)
                k["mfma_utilisation"] = round(fl / (avg * 1e-3) / MFMA_BF16_PEAK, 5)
        return kernels

    def timed(self, steps: int, dom: str, flush_buf) -> dict:
        """The timed regions. Cold: K steps, each bracketed by events on the
        launch stream, with `flush_buf` (1 GiB) written before each step
        outside its events; warm: K steps back to back between two
        synchronisations. The dominant kernel's launches carry events in both
        (the library's trace restricted to that kernel)."""
        import torch

        from sparse_graph_attention_csr_amd import binding as B
        B.trace_clear()
        B.trace_only(dom)
        B.trace_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs = []
        for _ in range(steps):
            flush_buf.fill_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            self.step()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        cold_wall = time.perf_counter() - t0
        cold = [a.elapsed_time(b) for a, b in evs]
        n_cold = B.trace_read()
        B.trace_clear()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        warm_ms = (time.perf_counter() - t0) * 1e3 / steps
        n_warm = B.trace_read()
        B.trace_enable(False)
        B.trace_only(None)
        B.trace_clear()
        dom_cold = [ms for name, ms in n_cold if name == dom]
        dom_warm = [ms for name, ms in n_warm if name == dom]
        return {"cold_ms": sum(cold) / steps, "cold_wall_s": cold_wall,
                "cold_median_ms": sorted(cold)[len(cold) // 2], "warm_ms": warm_ms,
                "dom_ms": sum(dom_cold + dom_warm) / len(dom_cold + dom_warm),
                "dom_cold_ms": sum(dom_cold) / len(dom_cold),
                "dom_warm_ms": sum(dom_warm) / len(dom_warm)}

    def rate(self, ms: float) -> float:
        return self.e * self.H / (ms * 1e-3) / 1e9

    def run(self, steps: int, warmup: int, flush_buf, ceiling: dict | None) -> dict:
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        kernels = self.kernel_table(steps)
        dom = max((k for k in kernels if "algorithmic_bytes" in kernels[k]),
                  key=lambda k: kernels[k]["ms"] * kernels[k]["launches_per_step"])
        t = self.timed(steps, dom, flush_buf)
        dk = kernels[dom]
        achieved = dk["algorithmic_bytes"] / (t["dom_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(dom, self.name),
                "algorithmic_bytes": dk["algorithmic_bytes"], "kernel_ms": round(t["dom_ms"], 4),
                "kernel_ms_cold": round(t["dom_cold_ms"], 4),
                "kernel_ms_warm": round(t["dom_warm_ms"], 4),
                # algorithmic bytes over time above the specification can only
                # mean that caches served part of the modelled gathers
                "cache_served": achieved > HBM_PEAK_GBS}
        if ceiling:
            roof["ceiling_gbs"] = ceiling["gather_gbs"]
            roof["frac_of_ceiling"] = round(achieved / ceiling["gather_gbs"], 4)
        if roof["traffic"] is not None:
            # the counter-measured bytes (L2 misses, Infinity Cache hits included) over the
            # same kernel's time: what the kernel actually pulled through the fabric
            tr = roof["traffic"] / (t["dom_ms"] * 1e-3) / 1e9
            roof["traffic_gbs"] = round(tr, 1)
            roof["traffic_frac"] = round(tr / HBM_PEAK_GBS, 4)
        step_bytes = sum(k["algorithmic_bytes"] * k["launches_per_step"]
                         for k in kernels.values() if "algorithmic_bytes" in k)
        step_gbs = step_bytes / (t["cold_ms"] * 1e-3) / 1e9
        return {"ms_per_step": t["cold_ms"], "cold_median_ms": t["cold_median_ms"],
                "cold_wall_s": t["cold_wall_s"], "warm_ms": t["warm_ms"], "roofline": roof,
                "kernels": kernels,
                "step_model": {"bytes": step_bytes, "gbs": round(step_gbs, 1),
                               "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                               "cache_served": step_gbs > HBM_PEAK_GBS}}

    def release(self):
        import torch
        for a in ("g", "step", "out", "inputs", "ws", "owned"):
            setattr(self, a, None)
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tiles", action="store_true",
                    help="Graph Transformer forward and backward on the 16x16 tile (MFMA) path")
    ap.add_argument("--reorder", default="none", choices=["none", "random", "degree", "rcm"],
                    help="relabel the nodes before timing (graph reordering study)")
    ap.add_argument("--locality", type=int, default=0, choices=[0, 1],
                    help="1: the plan orders rows of a degree bin by Cuthill-McKee rank")
    ap.add_argument("--compare-unfused", action="store_true",
                    help="also time the unfused PyTorch formulation (bench_unfused.py) and "
                         "report latency and peak-memory ratios")
    ap.add_argument("--step-times", action="store_true",
                    help="also time each step alone, warm and cold, and report median and "
                         "minimum over the steps")
    ap.add_argument("--extra", default="auto",
                    help="workloads timed beside the headline in the same run: 'auto' (the "
                         "power-law GT and GATv2 workloads and the community workload on tiles "
                         "when the headline is the default), 'none', or a comma list of names "
                         "(a name ending in ':tiles' runs on the tile path)")
    ap.add_argument("--probe-gib", type=float, default=4.0,
                    help="footprint of the memory-ceiling probes (0: skip them)")
    ap.add_argument("--cache-dir", default="",
                    help="keep the generated workload arrays here (.npz) and reuse them on the "
                         "next run (inputs only; the timed work is unchanged)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB three times "
                         "(calibrates the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_graph_attention_csr_amd import binding as B

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib:
        nb = args.copy_probe_mib << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": nb, "copy_probe_bytes_written": nb,
                          "launches": 3}), flush=True)
        return
    from sparse_graph_attention_csr_amd import inputs as I
    spec = I.WORKLOADS[args.workload]
    row_bytes = spec.heads * spec.dim * (2 if spec.dtype == I.BF16 else 4)
    ceiling = hbm_ceiling(dev, row_bytes, args.probe_gib) if args.probe_gib > 0 else None
    # 1 GiB written between cold steps (outside their timing)
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    hb = Bench(args.workload, dev, chunk=args.chunk, tiles=args.tiles, reorder=args.reorder,
               locality=args.locality, cache_dir=args.cache_dir)
    r = hb.run(args.steps, args.warmup, flush_buf, ceiling)
    ms_per_step = r["ms_per_step"]
    line = {
        "metric": "fused graph-attn fwd+bwd GEdge\u00b7head/s; achieved HBM GB/s vs MI355X peak",
        "value": round(hb.rate(ms_per_step), 4),
        "unit": "GEdge\u00b7head/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if hb.dt == B.BF16 else "f32",
        "data": "synthetic (seeded generator, seed 0)",
        "config": {"workload": args.workload, "graph": spec.graph, "nodes": hb.n,
                   "edges": hb.e, "heads": hb.H, "head_dim": hb.D, "passes": spec.passes,
                   "chunk": hb.g.plan.stats()["chunk"], "tiles": bool(args.tiles),
                   "reorder": args.reorder, "locality": args.locality,
                   "ds_order": "transposed" if hb.tpos else "csr",
                   "timing": "cold: 1 GiB written between steps, outside the timing"},
        "warm": {"ms_per_step": round(r["warm_ms"], 4), "value": round(hb.rate(r["warm_ms"]), 4)},
        "roofline": r["roofline"],
        "hbm_ceiling": ceiling,
        "step_model": r["step_model"],
        "memory": hb.memory,
        "kernels": r["kernels"],
        "plan_ms": round(hb.plan_ms, 1),
    }
    if args.step_times:
        line["steps_ms"] = {"warm": per_step_ms(hb.step, args.steps),
                            "cold": per_step_ms(hb.step, args.steps,
                                                flush=lambda: flush_buf.fill_(1.0))}
        for v in line["steps_ms"].values():
            v["value"] = round(hb.rate(v["median"]), 4)
    if args.compare_unfused:
        line["unfused"] = compare_unfused(spec, hb.g, hb.step, hb.owned + [hb.g.plan_buf],
                                          hb.inputs, hb.out, hb.bwd, r["warm_ms"], args.steps,
                                          args.warmup)
    w_head = hb.w
    hb.release()

    extra = args.extra
    if extra == "auto":
        extra = EXTRA_CONFIGS if (args.workload == DEFAULT_WORKLOAD and not args.tiles) else []
    elif extra == "none":
        extra = []
    else:
        extra = [(x.split(":")[0], x.endswith(":tiles")) for x in extra.split(",") if x]
    if extra:
        line["configs"] = {}
    for name, tiles in extra:
        eb = Bench(name, dev, tiles=tiles, cache_dir=args.cache_dir)
        er = eb.run(args.steps, args.warmup, flush_buf, None)
        key = name + (":tiles" if tiles else "")
        roof = er["roofline"]
        c = {"ms_per_step": round(er["ms_per_step"], 4), "value": round(eb.rate(er["ms_per_step"]), 4),
             "warm_ms_per_step": round(er["warm_ms"], 4), "warm_value": round(eb.rate(er["warm_ms"]), 4),
             "edges": eb.e, "dominant": {k: roof[k] for k in ("kernel", "kernel_ms", "achieved",
                                                                "frac", "cache_served")},
             "step_model": er["step_model"], "memory": eb.memory,
             "kernels": {k: {f: v[f] for f in ("ms", "achieved_gbs", "mfma_utilisation") if f in v}
                         for k, v in er["kernels"].items()}}
        line["configs"][key] = c
        eb.release()
        del eb

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w_head, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
