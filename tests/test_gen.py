"""The seeded input generators: deterministic for a seed, and the graphs have
the structure each workload specifies (exact edge counts, one self-loop per
node, no repeated pair, the degree cap, community and hub structure). CPU
only; about a minute and a half for the five graphs."""
import numpy as np
import pytest

from sparse_graph_attention_csr_amd import inputs as I


@pytest.fixture(scope="module")
def graphs():
    cache = {}

    def get(name):
        if name not in cache:
            cache[name] = I.make_graph(name)
        return cache[name]
    return get


def rows_of(rp):
    return np.repeat(np.arange(rp.size - 1), np.diff(rp))


def check_simple_with_self_loops(rp, ci):
    """One self-loop per row and no repeated (destination, source) pair."""
    n = rp.size - 1
    dst = rows_of(rp)
    assert np.array_equal(np.bincount(dst[ci == dst], minlength=n), np.ones(n, dtype=np.int64))
    key = dst.astype(np.int64) * n + ci
    assert np.unique(key).size == key.size
    assert ci.min() >= 0 and ci.max() < n


def test_same_seed_same_bytes():
    a = I.make_workload("gt_er1k_h4d32_f32")
    b = I.make_workload("gt_er1k_h4d32_f32")
    for k in ("rowptr", "colidx", "q", "k", "v"):
        assert np.array_equal(a[k], b[k]), k
    c = I.make_workload("gt_er1k_h4d32_f32", seed=1)
    assert not np.array_equal(a["colidx"], c["colidx"])
    r1 = I.random_csr(500, 30, np.random.default_rng(5), empty_frac=0.1, dup_frac=0.2)
    r2 = I.random_csr(500, 30, np.random.default_rng(5), empty_frac=0.1, dup_frac=0.2)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


def test_er_graph(graphs):
    rp, ci, _ = graphs("gt_er1k_h4d32_f32")
    assert rp.size - 1 == 1000 and rp[-1] == 9000          # 8,000 distinct pairs + 1,000 self-loops
    check_simple_with_self_loops(rp, ci)
    w = I.make_tensors("gt_er1k_h4d32_f32")
    q = w["q"].astype(np.float64)
    assert w["q"].dtype == np.float32 and abs(q.mean()) < 0.02 and abs(q.std() - 1) < 0.02


def test_powerlaw_200k(graphs):
    rp, ci, _ = graphs("gt_powerlaw200k_h4d128_bf16")
    deg = np.diff(rp)
    assert rp.size - 1 == 200_000 and rp[-1] == 3_200_000   # exactly N*mean + N self-loops
    check_simple_with_self_loops(rp, ci)
    assert deg.max() <= 20_000 + 1                          # in-degree cap (+ the self-loop)
    assert 4 <= np.median(deg) <= 8 and deg.max() > 5_000   # heavy tail
    t = I.make_tensors("gt_powerlaw200k_h4d128_bf16")
    assert t["q"].dtype == np.uint16 and t["q"].shape == (200_000, 4, 128) and "dout" in t


def test_community_graph(graphs):
    rp, ci, _ = graphs("gt_community262k_h4d128_bf16")
    n = rp.size - 1
    assert n == 4096 * 64
    check_simple_with_self_loops(rp, ci)
    dst = rows_of(rp)
    outside = (ci // 64) != (dst // 64)
    assert np.array_equal(np.bincount(dst[outside], minlength=n), np.full(n, 2))
    intra = np.bincount(dst[~outside & (ci != dst)], minlength=n)   # Binomial(63, 0.5) each
    assert abs(intra.mean() - 31.5) < 0.1 and intra.max() <= 63


def test_gatv2_powerlaw_500k(graphs):
    rp, ci, _ = graphs("gatv2_powerlaw500k_h2d64_bf16")
    deg = np.diff(rp)
    assert rp.size - 1 == 500_000 and rp[-1] == 10_500_000
    check_simple_with_self_loops(rp, ci)
    assert 7 <= np.median(deg) <= 13 and deg.max() > 20_000  # no cap: the hubs are large


def test_hub_graph(graphs):
    rp, ci, extra = graphs("gt_hubs2m_h8d64_bf16")
    n = rp.size - 1
    hubs = extra["hubs"]
    assert n == 2_000_000 and hubs.size == 64 and np.unique(hubs).size == 64
    check_simple_with_self_loops(rp, ci)
    indeg = np.diff(rp)
    outdeg = np.bincount(ci, minlength=n)
    assert np.all(indeg[hubs] >= 200_000) and np.all(outdeg[hubs] >= 50_000)
    others = np.setdiff1d(np.arange(n), hubs)
    # background mean 10, the self-loop, and the hubs' 64 x 50,000 out-edges spread over the rest
    expect = 10 + 1 + 64 * 50_000 / others.size
    assert abs(indeg[others].mean() - expect) < 0.1
