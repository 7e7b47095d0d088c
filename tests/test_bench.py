"""Host-side helpers of bench.py: the lane layout it assumes, the split of the
CSR work list into long items (one per wavefront) and the short suffix, and
that the two row-pass kernels are charged exactly the edges and items of the
whole pass between them. CPU only."""
import re

import numpy as np

import bench
from sparse_graph_attention_csr_amd import binding as B
from sparse_graph_attention_csr_amd import inputs as I


def test_edge_groups():
    # 64 lanes of 16-byte fragments; a head group is a power of two of heads
    assert bench.edge_groups(2, 64, 2) == 4      # bf16 2x64: 16 lanes per edge
    assert bench.edge_groups(4, 128, 2) == 1     # bf16 4x128: a whole wave per edge
    assert bench.edge_groups(8, 64, 2) == 1
    assert bench.edge_groups(1, 32, 2) == 16
    assert bench.edge_groups(3, 32, 2) == 4      # 3 heads padded to 4
    assert bench.edge_groups(4, 32, 4) == 2      # fp32: 8 lanes per 32-channel head


def test_record_bytes():
    assert bench.gat_record_bytes(2, 64, 2) == 32   # (p, dE) x 2 heads + 16 sign bytes
    assert bench.gat_record_bytes(8, 128, 2) == 192  # two head groups of 4 heads


def test_row_item_split_partitions_the_work_list():
    rng = np.random.default_rng(3)
    deg = rng.choice([0, 1, 5, 127, 128, 129, 600], size=700)
    rp = np.zeros(deg.size + 1, dtype=np.int64)
    rp[1:] = np.cumsum(deg)
    ci = rng.integers(0, deg.size, size=int(rp[-1])).astype(np.int32)
    plan = B.Plan(rp, ci, chunk=256)
    items = plan.export(B.ARR_ROW_ITEMS)
    sp = bench.row_item_split(plan)
    assert sp["long_items"] + sp["short_items"] == items.size
    assert sp["long_edges"] + sp["short_edges"] == rp[-1]
    lens = items["len"]
    assert np.all(lens[sp["long_items"]:] < bench.SHORT_ITEM_EDGES)
    assert lens[sp["long_items"] - 1] >= bench.SHORT_ITEM_EDGES
    # the two kernels together are charged what one pass over every item is
    n_items, e = int(items.size), int(rp[-1])
    both = sum(bench.algorithmic_bytes(k, deg.size, e, 2, 64, 2, None, sp)
               for k in ("gat_bwd_rows", "gat_bwd_rows_short"))
    assert both == bench.algorithmic_bytes("gat_bwd_rows", n_items, e, 2, 64, 2)


def test_cpu_baseline_samples_a_prefix_of_rows():
    """cpu_baseline on a workload the oracle cannot finish within the time it
    is given: it times destination rows 0..r-1 only (the other rows emptied),
    with r scaled towards the time target, and reports that sample."""
    import dataclasses
    rng = np.random.default_rng(7)
    n, H, D = 20000, 2, 32
    rp, ci = I.random_csr(n, 40, rng)
    spec = dataclasses.replace(I.WORKLOADS["gt_er1k_h4d32_f32"], name="test", n=n, heads=H, dim=D)
    w = {"spec": spec, "rowptr": rp, "colidx": ci}
    for key in ("q", "k", "v", "dout"):
        w[key] = rng.standard_normal((n, H, D))
    cb = bench.cpu_baseline(w, 0.01)
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    m = re.match(r"destination rows 0\.\.(\d+) of (\d+) \((\d+) of (\d+) edges\)", cb["sample"])
    assert m, cb["sample"]
    last, n_all, e, e_all = (int(x) for x in m.groups())
    assert n_all == n and e_all == rp[-1]
    assert 0 < last + 1 < n and e == rp[last + 1]
    assert cb["fwd_seconds"] >= 0 and cb["bwd_seconds"] >= 0   # rounded to ms
